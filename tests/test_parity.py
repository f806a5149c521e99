"""GPU parity: every libsmoe call against the CPU oracle on the same seeded
inputs. Integer results (expert IDs, alignment, ELB counts and plans) must
be bit-exact; router logits too (same float32 order on both sides); floating
outputs must be within the stated tolerances. Needs an MI355X."""

import numpy as np
import pytest
import torch

import oracle
from workload import get_config, make_activations, make_layer, make_router, quantize_rtn_int4
from workload.configs import MoEConfig
from workload.gen import zipf_bias

pytestmark = pytest.mark.gpu

# Layer-output tolerance: per token (or slot) row, max |gpu - ref| / max |ref|.
# The GPU computes in FP16 x FP16 -> FP32 with the intermediate activation
# and the output in FP16; expected error is ~1e-3.
ROW_TOL = 2e-2
# Routing weights: float32 softmax (expf, float32 sum) vs float64.
W_RTOL = 2e-5


@pytest.fixture(scope="module")
def smoe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from quantized_speculative_expert_amd import _lib  # fails loudly if not built
    return _lib


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def row_rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return (num / den).max() if len(num) else 0.0


_LAYERS = {}
_REFS = {}


def layer(name, seed=0, layer_idx=0):
    key = (name, seed, layer_idx)
    if key not in _LAYERS:
        _LAYERS[key] = make_layer(get_config(name), seed=seed, layer=layer_idx)
    return _LAYERS[key]


def ref_layer(name, pass_="draft", seed=0, layer_idx=0):
    """oracle.moe_layer of a generated layer, computed once per session."""
    key = (name, pass_, seed, layer_idx)
    if key not in _REFS:
        _REFS[key] = oracle.moe_layer(layer(name, seed, layer_idx), pass_)
    return _REFS[key]


def run_route(smoe, x, w, bias, k, flags=0, gate_w=None):
    T, E = x.shape[0], w.shape[0]
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    wt = torch.empty((T, k), dtype=torch.float32, device="cuda")
    lg = torch.empty((T, E), dtype=torch.float32, device="cuda")
    gate = torch.empty(T, dtype=torch.float32, device="cuda") if gate_w is not None else None
    smoe.smoe_route_topk(dev(x), dev(w), None if bias is None else dev(bias), k, flags, ids, wt,
                         lg, None if gate_w is None else dev(gate_w), gate)
    return host(ids), host(wt), host(lg), (host(gate) if gate is not None else None)


def run_align(smoe, ids, E):
    T, k = ids.shape
    S = T * k
    out = dict(counts=torch.full((E,), -7, dtype=torch.int32, device="cuda"),
               offsets=torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
               sorted_slots=torch.full((max(S, 1),), -7, dtype=torch.int32, device="cuda"),
               active=torch.full((E,), -7, dtype=torch.int32, device="cuda"),
               n_active=torch.full((1,), -7, dtype=torch.int32, device="cuda"))
    smoe.smoe_align_by_expert(dev(ids.astype(np.int32)), E, out["counts"], out["offsets"],
                              out["sorted_slots"][:S], out["active"], out["n_active"])
    res = {k_: host(v) for k_, v in out.items()}
    res["sorted_slots"] = res["sorted_slots"][:S]
    return res


def check_align(got, ref):
    for key in ("counts", "offsets", "sorted_slots", "active"):
        assert np.array_equal(got[key], ref[key]), key
    assert int(got["n_active"][0]) == int(ref["n_active"])


# ------------------------------------------------------------------ router

@pytest.mark.parametrize("name", ["tiny", "dsv2", "qwen", "phi", "dsv2_t1"])
def test_route_matches_oracle(smoe, name):
    L = layer(name)
    cfg = L.cfg
    ids, wt, lg, gate = run_route(smoe, L.x, L.w_router, L.router_bias, cfg.k,
                                  gate_w=L.shared_gate_w)
    ref_lg = oracle.router_logits_f32(L.x, L.w_router, L.router_bias)
    assert np.array_equal(lg.view(np.uint32), ref_lg.view(np.uint32))
    ref_ids = oracle.topk_experts(ref_lg, cfg.k)
    assert np.array_equal(ids, ref_ids)
    ref_w = oracle.routing_weights(ref_lg, ref_ids)
    assert np.allclose(wt, ref_w, rtol=W_RTOL, atol=1e-9)
    if L.shared_gate_w is not None:
        assert np.allclose(gate, oracle.shared_gate(L.x, L.shared_gate_w), rtol=1e-5, atol=1e-7)


def test_route_batched_zipf_layer(smoe):
    L = layer("batch", layer_idx=3)
    ids, wt, lg, _ = run_route(smoe, L.x, L.w_router, L.router_bias, L.cfg.k)
    ref_lg = oracle.router_logits_f32(L.x, L.w_router, L.router_bias)
    assert np.array_equal(lg.view(np.uint32), ref_lg.view(np.uint32))
    assert np.array_equal(ids, oracle.topk_experts(ref_lg, L.cfg.k))
    assert np.allclose(wt, oracle.routing_weights(ref_lg, ids), rtol=W_RTOL, atol=1e-9)


def test_route_golden_order(smoe):
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                    "router_order_handworked.json")))
    x = np.zeros((1, g["H"]), np.float16)
    for h, v in g["x_nonzero"].items():
        x[0, int(h)] = v
    w = np.zeros((g["E"], g["H"]), np.float32)
    for e, row in enumerate(g["w_nonzero"]):
        for h, v in row.items():
            w[e, int(h)] = v
    ids, wt, lg, _ = run_route(smoe, x, w, None, 1)
    assert lg[0].tolist() == g["expected_logits"]
    assert ids[0, 0] == 0


def test_route_ties_renorm_and_k_equals_E(smoe):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((33, 256)).astype(np.float16)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    w[5] = w[2]          # exact ties between experts 2 and 5
    w[7] = w[2]
    for k in (1, 3, 8):
        for flags in (0, 1):
            ids, wt, lg, _ = run_route(smoe, x, w, None, k, flags)
            ref_lg = oracle.router_logits_f32(x, w)
            ref_ids = oracle.topk_experts(ref_lg, k)
            assert np.array_equal(ids, ref_ids)
            ref_w = oracle.routing_weights(ref_lg, ref_ids, renorm=bool(flags))
            assert np.allclose(wt, ref_w, rtol=W_RTOL, atol=1e-9)


def test_route_single_token_and_large_E(smoe):
    rng = np.random.default_rng(8)
    x = rng.standard_normal((1, 512)).astype(np.float16)
    w = (rng.standard_normal((256, 512)) * 0.02).astype(np.float32)
    ids, wt, lg, _ = run_route(smoe, x, w, None, 8)
    ref_lg = oracle.router_logits_f32(x, w)
    assert np.array_equal(lg.view(np.uint32), ref_lg.view(np.uint32))
    assert np.array_equal(ids, oracle.topk_experts(ref_lg, 8))


@pytest.mark.parametrize("T", [1, 17, 29, 57, 64, 85, 100, 113, 150])
def test_route_token_tiles(smoe, T):
    # the logits kernel's token tile follows the window (one token per
    # workgroup at short windows, up to four at long ones): T = 57..113 at
    # 64 experts and a gate row gives tiles of 2 and 3 with ragged last
    # tiles; the logits stay bit-identical to the oracle's fixed order
    rng = np.random.default_rng(100 + T)
    x = rng.standard_normal((T, 2048)).astype(np.float16)
    w = (rng.standard_normal((64, 2048)) * 0.02).astype(np.float32)
    gw = (rng.standard_normal(2048) * 0.02).astype(np.float32)
    ids, wt, lg, gate = run_route(smoe, x, w, None, 6, gate_w=gw)
    ref_lg = oracle.router_logits_f32(x, w)
    assert np.array_equal(lg.view(np.uint32), ref_lg.view(np.uint32))
    assert np.array_equal(ids, oracle.topk_experts(ref_lg, 6))
    ref_gate = oracle.shared_gate(x, gw)
    assert np.allclose(gate, ref_gate, rtol=1e-5, atol=1e-7)


# ------------------------------------------------------------------ fused routing call

def _routing_buffers(T, k, E, gated, L, M):
    i32 = dict(dtype=torch.int32, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    b = dict(ids=torch.full((T, k), -7, **i32), w=torch.full((T, k), -7.0, **f32),
             lg=torch.full((T, E), -7.0, **f32),
             gate=torch.full((T,), -7.0, **f32) if gated else None,
             counts=torch.full((E,), -7, **i32), offsets=torch.full((E + 1,), -7, **i32),
             sorted=torch.full((max(T * k, 1),), -7, **i32), active=torch.full((E,), -7, **i32),
             n_active=torch.full((1,), -7, **i32))
    if L:
        b["cnt"] = torch.arange(L * E, **i32).reshape(L, E) % 5   # non-zero starting counts
        b["plan"] = torch.full((L, max(M, 1)), -7, **i32)
        b["plan_cnt"] = torch.full((L, max(M, 1)), -7, **i32)
    return b


def _run_routing(smoe, fused, x, w, bias, k, flags, gate_w, elb):
    T, E = x.shape[0], w.shape[0]
    L, layer, M, clear = elb if elb else (0, 0, 0, 0)
    b = _routing_buffers(T, k, E, gate_w is not None, L, M)
    S = T * k
    xd, wd = dev(x), dev(w)
    bd = None if bias is None else dev(bias)
    gd = None if gate_w is None else dev(gate_w)
    if fused:
        smoe.smoe_route_align_elb(xd, wd, bd, k, flags, b["ids"], b["w"], b["lg"], gd, b["gate"],
                                  b["counts"], b["offsets"], b["sorted"][:S], b["active"],
                                  b["n_active"], elb_counts=b.get("cnt"), layer=layer, M=M,
                                  plan_ids=b["plan"] if L and M else None,
                                  plan_counts=b["plan_cnt"] if L and M else None,
                                  elb_flags=clear)
    else:
        smoe.smoe_route_topk(xd, wd, bd, k, flags, b["ids"], b["w"], b["lg"], gd, b["gate"])
        smoe.smoe_align_by_expert(b["ids"], E, b["counts"], b["offsets"], b["sorted"][:S],
                                  b["active"], b["n_active"])
        if L:
            smoe.smoe_elb_accumulate_topm(b["cnt"], b["ids"][None], layer, M,
                                          b["plan"] if M else None, b["plan_cnt"] if M else None,
                                          clear)
    return {k_: host(v) for k_, v in b.items() if v is not None}


@pytest.mark.parametrize("name,elb", [("tiny", None), ("dsv2", (1, 0, 32, 0)),
                                      ("qwen", (3, 1, 8, 1)), ("phi", (2, 1, 4, 0)),
                                      ("dsv2", (26, 20, 32, 1)),   # more layers than waves
                                      ("batch", (26, 3, 32, 0))])
def test_route_align_elb_equals_separate_calls(smoe, name, elb):
    # one call == route_topk, align_by_expert, elb_accumulate_topm one after
    # the other, bit for bit (the batch window takes the three-call path)
    L = layer(name, layer_idx=3 if name == "batch" else 0)
    cfg = L.cfg
    args = (L.x, L.w_router, L.router_bias, cfg.k, 0, L.shared_gate_w, elb)
    got = _run_routing(smoe, True, *args)
    ref = _run_routing(smoe, False, *args)
    assert got.keys() == ref.keys()
    for key in ref:
        assert np.array_equal(got[key].view(np.uint32) if got[key].dtype == np.float32 else got[key],
                              ref[key].view(np.uint32) if ref[key].dtype == np.float32 else ref[key]), key
    assert np.array_equal(got["ids"], oracle.topk_experts(
        oracle.router_logits_f32(L.x, L.w_router, L.router_bias), cfg.k))


def test_route_align_elb_ties_and_renorm(smoe):
    rng = np.random.default_rng(11)
    x = rng.standard_normal((33, 256)).astype(np.float16)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    w[5] = w[2]
    for k, flags in ((1, 0), (3, 1), (8, 0)):
        args = (x, w, None, k, flags, None, (2, 0, 4, 1))
        got = _run_routing(smoe, True, *args)
        ref = _run_routing(smoe, False, *args)
        for key in ref:
            assert np.array_equal(got[key], ref[key]), (k, key)


@pytest.mark.parametrize("T,k,E,elb", [(64, 8, 256, (20, 5, 64, 0)),   # 512 slots, E = 256
                                       (1, 1, 1, (3, 2, 1, 1)),          # one slot, one expert
                                       (65, 7, 100, (16, 15, 100, 1))])  # M = E, ragged chunks
def test_route_align_elb_window_limits(smoe, T, k, E, elb):
    rng = np.random.default_rng(T * 1000 + E)
    x = rng.standard_normal((T, 256)).astype(np.float16)
    w = (rng.standard_normal((E, 256)) * 0.02).astype(np.float32)
    args = (x, w, None, k, 0, None, elb)
    got = _run_routing(smoe, True, *args)
    ref = _run_routing(smoe, False, *args)
    for key in ref:
        assert np.array_equal(got[key], ref[key]), key


# ------------------------------------------------------------------ alignment

@pytest.mark.parametrize("E,k,T,seed", [(8, 2, 17, 0), (64, 6, 17, 1), (60, 4, 9, 2),
                                        (16, 2, 17, 3), (64, 6, 544, 4), (256, 8, 4096, 5),
                                        (7, 1, 1, 6)])
def test_align_matches_oracle(smoe, E, k, T, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    check_align(run_align(smoe, ids, E), oracle.align_by_expert(ids, E))


def test_align_edge_cases(smoe):
    for ids, E in [(np.full((17, 1), 3, np.int32), 8),                   # one expert
                   (np.zeros((0, 2), np.int32), 8),                      # empty window
                   (np.array([[0, 9], [-1, 2], [2, 2]], np.int32), 8),   # dropped IDs
                   (np.tile(np.arange(4, dtype=np.int32), (300, 1)), 4)]:  # k = E
        check_align(run_align(smoe, ids, E), oracle.align_by_expert(ids, E))


def test_align_is_deterministic(smoe):
    rng = np.random.default_rng(12)
    ids = rng.integers(0, 64, size=(544, 6)).astype(np.int32)
    a = run_align(smoe, ids, 64)
    b = run_align(smoe, ids, 64)
    for key in a:
        assert np.array_equal(a[key], b[key])


# ------------------------------------------------------------------ ELB

def test_elb_golden_and_clear(smoe):
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "elb_handworked.json")))
    cnt = torch.zeros((g["L"], g["E"]), dtype=torch.int32, device="cuda")
    ids = dev(np.array(g["ids"], np.int32))
    plan = torch.empty((g["L"], 3), dtype=torch.int32, device="cuda")
    pc = torch.empty((g["L"], 3), dtype=torch.int32, device="cuda")
    smoe.smoe_elb_accumulate_topm(cnt, ids, 0, 3, plan, pc, 0)
    assert host(cnt).tolist() == g["expected_counts"]
    assert host(plan).tolist() == g["expected_top3_ids"]
    assert host(pc).tolist() == g["expected_top3_counts"]
    plan4 = torch.empty((g["L"], 4), dtype=torch.int32, device="cuda")
    smoe.smoe_elb_accumulate_topm(cnt, None, 0, 4, plan4, None, smoe.SMOE_ELB_CLEAR_AFTER)
    assert host(plan4)[0].tolist() == g["expected_top4_ids_layer0"]
    assert not host(cnt).any()
    tie = dev(np.array(g["tie_counts"], np.int32))
    plan1 = torch.empty((1, 3), dtype=torch.int32, device="cuda")
    smoe.smoe_elb_accumulate_topm(tie, None, 0, 3, plan1, None, 0)
    assert host(plan1).tolist() == g["tie_expected_top3"]


def test_elb_random_layers_and_split_calls(smoe):
    rng = np.random.default_rng(4)
    L, E, T, k, M = 26, 64, 17, 6, 32
    ids = np.stack([np.stack([rng.permutation(E)[:k] for _ in range(T)])
                    for _ in range(L)]).astype(np.int32)
    ref = oracle.elb_accumulate(np.zeros((L, E), np.int32), ids, 0)
    ref_ids, ref_cnt = oracle.elb_topm(ref, M)
    cnt = torch.zeros((L, E), dtype=torch.int32, device="cuda")
    plan = torch.empty((L, M), dtype=torch.int32, device="cuda")
    pc = torch.empty((L, M), dtype=torch.int32, device="cuda")
    smoe.smoe_elb_accumulate_topm(cnt, dev(ids), 0, M, plan, pc, 0)
    assert np.array_equal(host(cnt), ref)
    assert np.array_equal(host(plan), ref_ids) and np.array_equal(host(pc), ref_cnt)
    # token by token, one layer per call, accumulate only: same counter
    cnt2 = torch.zeros((L, E), dtype=torch.int32, device="cuda")
    for t in range(T):
        for l in range(0, L, 5):
            smoe.smoe_elb_accumulate_topm(cnt2, dev(np.ascontiguousarray(ids[l:l + 5, t:t + 1])),
                                          l, 0, None, None, 0)
    assert np.array_equal(host(cnt2), ref)


# ------------------------------------------------------------------ expert FFN

def oracle_slots_int4(L, ids, slots=None):
    cfg = L.cfg

    def load(e):
        return (oracle.dequant_int4(L.wg_q[e], L.wg_s[e], cfg.G),
                oracle.dequant_int4(L.wu_q[e], L.wu_s[e], cfg.G),
                oracle.dequant_int4(L.wd_q[e], L.wd_s[e], cfg.G))
    return oracle.routed_ffn_expertwise(L.x, ids, load)


def tile_dev(smoe, w, s, E, N, K, G):
    """Device copies of a row-major [E][N][K] weight (and its INT4 scales)
    in the tiled layout, made by smoe_tile_weights."""
    w = dev(w) if isinstance(w, np.ndarray) else w
    s = dev(s) if isinstance(s, np.ndarray) else s
    wt = torch.empty_like(w)
    st = torch.empty_like(s) if s is not None else None
    smoe.smoe_tile_weights(w, s, E, N, K, G, wt, st)
    return wt, st


def tiled_layout_np(w, s, G):
    """The tiled layout written out from its definition with numpy index
    arithmetic: w uint32 words [E][N][nb * 16] (K = 128 nb INT4 codes, or
    32 nb FP16 values as words), s [E][N][nb * 128 / G] or None. INT4 words
    get their nibbles unzipped (k = 8w + 2p in position p, k = 8w + 2p + 1 in
    position 4 + p)."""
    if G != 0:
        nib = [(w >> np.uint32(4 * j)) & np.uint32(0xF) for j in range(8)]
        w = np.zeros_like(w)
        for j in range(8):
            pos = 4 + j // 2 if j % 2 else j // 2
            w |= nib[j] << np.uint32(4 * pos)
    E, N, words = w.shape
    nb = words // 16
    Gw = 128 if G == 0 else G
    per = Gw // 32
    wt = np.empty(E * N * words, np.uint32)
    o = 0
    for e in range(E):
        for sl in range(N // 16):
            for b in range(nb):
                for g in range(4):
                    for r in range(16):
                        for q in range(4):
                            word = (q // per) * (Gw // 8) + g * per + q % per
                            wt[o] = w[e, 16 * sl + r, 16 * b + word]
                            o += 1
    if s is None:
        return wt, None
    nq = 128 // G
    st = np.empty(s.size, s.dtype)
    o = 0
    for e in range(E):
        for sl in range(N // 16):
            for b in range(nb):
                for r in range(16):
                    st[o:o + nq] = s[e, 16 * sl + r, nq * b:nq * (b + 1)]
                    o += nq
    return wt, st


@pytest.mark.parametrize("G", [0, 32, 64, 128])
def test_tile_weights_layout(smoe, G):
    """smoe_tile_weights matches the layout's definition bit for bit
    (two experts, 48 rows, K = 256: three row slices, several blocks)."""
    E, N, K = 2, 48, 256
    rng = np.random.default_rng(G + 1)
    if G:
        w = rng.integers(0, 2**32, (E, N, K // 8), dtype=np.uint64).astype(np.uint32)
        s = rng.standard_normal((E, N, K // G)).astype(np.float16)
    else:
        w = rng.standard_normal((E, N, K)).astype(np.float16)
        s = None
    wt, st = tile_dev(smoe, w, s, E, N, K, G)
    w_words = w if G else w.view(np.uint32)
    ref_w, ref_s = tiled_layout_np(w_words.reshape(E, N, -1), s, G)
    got_w = host(wt).reshape(-1).view(np.uint32)
    assert np.array_equal(got_w, ref_w)
    if G:
        assert np.array_equal(host(st).reshape(-1).view(np.uint16), ref_s.view(np.uint16))


def test_tile_weights_argument_checks(smoe):
    w = torch.zeros(2 * 16 * 32, dtype=torch.int32, device="cuda")
    s = torch.zeros(2 * 16 * 2, dtype=torch.float16, device="cuda")
    out, so = torch.empty_like(w), torch.empty_like(s)
    with pytest.raises(smoe.SmoeError, match="multiple"):
        smoe.smoe_tile_weights(w, s, 2, 8, 256, 128, out, so)      # N not a multiple of 16
    with pytest.raises(smoe.SmoeError, match="group size"):
        smoe.smoe_tile_weights(w, s, 2, 16, 256, 256, out, so)
    with pytest.raises(smoe.SmoeError, match="overlap"):
        smoe.smoe_tile_weights(w, s, 2, 16, 256, 128, w, so)
    smoe.smoe_tile_weights(w, s, 0, 16, 256, 128, out, so)         # nothing to do


def _shared_dev(shared, T, H, smoe=None, tiled=False):
    if shared is None:
        return None, None, 0
    sg, su, sd = shared
    out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    Is = sg.shape[0]
    if tiled:
        return (tile_dev(smoe, sg, None, 1, Is, H, 0)[0], tile_dev(smoe, su, None, 1, Is, H, 0)[0],
                tile_dev(smoe, sd, None, 1, H, Is, 0)[0]), out, Is
    return (dev(sg), dev(su), dev(sd)), out, Is


def run_w4a16(smoe, x, ids, E, I, G, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, shared=None, calls=1,
              tiled=False):
    """slot_out (and shared_out when shared = (sg, su, sd) fp16 is given);
    with calls > 1 the same workspace serves that many calls in a row and
    the last call's outputs are returned. tiled: every weight tiled by
    smoe_tile_weights and the tiled-layout call used."""
    T, k = ids.shape
    H = x.shape[1]
    al = oracle.align_by_expert(ids, E)
    sh, sh_out, Is = _shared_dev(shared, T, H, smoe, tiled)
    ws = torch.zeros(smoe.smoe_ffn_workspace_bytes(T, k, E, H, I, Is), dtype=torch.uint8,
                     device="cuda")
    args = [dev(a) for a in (x, wg_q, wg_s, wu_q, wu_s, wd_q, wd_s, al["sorted_slots"],
                             al["offsets"])]
    fn = smoe.smoe_w4a16_expert_ffn
    if tiled:
        args[1:3] = tile_dev(smoe, args[1], args[2], E, I, H, G)
        args[3:5] = tile_dev(smoe, args[3], args[4], E, I, H, G)
        args[5:7] = tile_dev(smoe, args[5], args[6], E, H, I, G)
        fn = smoe.smoe_w4a16_expert_ffn_tiled
    for _ in range(calls):
        out = torch.full((T * k, H), float("nan"), dtype=torch.float32, device="cuda")
        if sh_out is not None:
            sh_out.fill_(float("nan"))
        fn(args[0], k, E, I, G, *args[1:7], args[7], args[8], ws, out,
           shared=sh, shared_out=sh_out)
    if shared is None:
        return host(out)
    return host(out), host(sh_out)


@pytest.mark.parametrize("tiled", [False, True], ids=["rows", "tiled"])
@pytest.mark.parametrize("name", ["tiny", "dsv2", "qwen"])
def test_w4a16_ffn_matches_oracle(smoe, name, tiled):
    L = layer(name)
    cfg = L.cfg
    ids = oracle.topk_experts(oracle.router_logits_f32(L.x, L.w_router, L.router_bias), cfg.k)
    got = run_w4a16(smoe, L.x, ids, cfg.E, cfg.I, cfg.G, L.wg_q, L.wg_s, L.wu_q, L.wu_s,
                    L.wd_q, L.wd_s, tiled=tiled)
    ref = oracle_slots_int4(L, ids)
    assert np.isfinite(got).all()
    err = row_rel_err(got, ref)
    assert err <= ROW_TOL, err


@pytest.mark.parametrize("name", ["tiny", "dsv2"])
def test_w4a16_ffn_one_expert_per_call(smoe, name):
    """A call may cover a subset of the experts with the window's k (here
    E = 1 < k): the expert's weights, the full sorted slot list and the
    expert's [begin, end) offsets. Its slots' rows equal the oracle's."""
    L = layer(name)
    cfg = L.cfg
    ids = oracle.topk_experts(oracle.router_logits_f32(L.x, L.w_router, L.router_bias), cfg.k)
    ref = oracle_slots_int4(L, ids)
    al = oracle.align_by_expert(ids, cfg.E)
    off = al["offsets"]
    T, H = L.x.shape
    ws = torch.zeros(smoe.smoe_ffn_workspace_bytes(T, cfg.k, 1, H, cfg.I), dtype=torch.uint8,
                     device="cuda")
    x, ss = dev(L.x), dev(al["sorted_slots"])
    w = {n: dev(getattr(L, n)) for n in ("wg_q", "wg_s", "wu_q", "wu_s", "wd_q", "wd_s")}
    active = [e for e in range(cfg.E) if off[e + 1] > off[e]][:8]
    for e in active:
        out = torch.full((T * cfg.k, H), float("nan"), dtype=torch.float32, device="cuda")
        sl = slice(e, e + 1)
        o = torch.tensor([off[e], off[e + 1]], dtype=torch.int32, device="cuda")
        smoe.smoe_w4a16_expert_ffn(x, cfg.k, 1, cfg.I, cfg.G, *(w[n][sl] for n in (
            "wg_q", "wg_s", "wu_q", "wu_s", "wd_q", "wd_s")), ss, o, ws, out)
        rows = al["sorted_slots"][off[e]:off[e + 1]]
        got = host(out)[rows]
        assert np.isfinite(got).all(), e
        err = row_rel_err(got, ref[rows])
        assert err <= ROW_TOL, (e, err)


def _synthetic_int4(E, H, I, G, seed):
    rng = np.random.default_rng(seed)
    q = {}
    for nm, (n, kk) in (("wg", (I, H)), ("wu", (I, H)), ("wd", (H, I))):
        codes, scales = zip(*[quantize_rtn_int4(
            (rng.standard_normal((n, kk)) * 0.02).astype(np.float32), G) for _ in range(E)])
        q[nm + "_q"], q[nm + "_s"] = np.stack(codes), np.stack(scales)
    return q


@pytest.mark.parametrize("E,k,T,H,I,G", [
    (8, 2, 17, 256, 512, 32),        # G = 32 path
    (8, 2, 128, 256, 384, 64),       # 32 slots per expert: two 16-slot MFMA groups
    (4, 2, 150, 256, 256, 128),      # 75 slots per expert: 64-slot chunks, several per expert
    (16, 1, 1, 384, 256, 128),       # a single token
    (6, 3, 40, 128, 128, 64),        # minimal sizes, ragged chunks
    (256, 8, 33, 128, 128, 32),      # the limits: 256 experts, top-8, g32
    (8, 2, 17, 256, 512, 64),        # x resident in LDS for the gate/up stage, g64
])
@pytest.mark.parametrize("tiled", [False, True], ids=["rows", "tiled"])
def test_w4a16_ffn_shapes(smoe, E, k, T, H, I, G, tiled):
    rng = np.random.default_rng(T * 7 + E)
    x = rng.standard_normal((T, H)).astype(np.float16)
    q = _synthetic_int4(E, H, I, G, seed=E + H)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    got = run_w4a16(smoe, x, ids, E, I, G, q["wg_q"], q["wg_s"], q["wu_q"], q["wu_s"],
                    q["wd_q"], q["wd_s"], tiled=tiled)

    def load(e):
        return tuple(oracle.dequant_int4(q[n + "_q"][e], q[n + "_s"][e], G) for n in ("wg", "wu", "wd"))
    ref = oracle.routed_ffn_expertwise(x, ids, load)
    err = row_rel_err(got, ref)
    assert err <= ROW_TOL, err


def _long_window_ids(rng, T, k, E, skew, drop):
    # Zipf-skewed routing (some experts take several 64-slot chunks, some
    # none), optionally with dropped slots
    p = 1.0 / np.arange(1, E + 1) ** skew
    p /= p.sum()
    perm = rng.permutation(E)
    ids = np.stack([perm[rng.choice(E, k, replace=False, p=p)] for _ in range(T)]).astype(np.int32)
    if drop:
        ids[rng.random(ids.shape) < drop] = -1
    return ids


@pytest.mark.parametrize("E,k,T,H,I,G,Is,drop", [
    (8, 2, 600, 256, 384, 128, 0, 0.0),      # 150 slots per expert: 3 chunks each
    (16, 4, 300, 384, 256, 64, 256, 0.0),    # with the shared expert (5 chunks of 64 tokens)
    (64, 6, 200, 256, 256, 32, 384, 0.02),   # skewed, g32, dropped slots
    (64, 6, 200, 256, 256, 32, 0, 0.0),      # g32 alone (wrong rows once, with per-column-group branches)
    (32, 8, 512, 128, 128, 128, 128, 0.0),   # 4096 slots, the longest window taken
])
def test_w4a16_ffn_long_window(smoe, E, k, T, H, I, G, Is, drop):
    # windows of at least 1024 slots over tiled weights take the long-window
    # FFN: every slot row against the oracle
    rng = np.random.default_rng(T + E)
    q = _synthetic_int4(E, H, I, G, seed=E + T)
    x = rng.standard_normal((T, H)).astype(np.float16)
    ids = _long_window_ids(rng, T, k, E, 1.1, drop)
    shared = None
    if Is:
        shared = tuple((rng.standard_normal(sh) * 0.02).astype(np.float16)
                       for sh in ((Is, H), (Is, H), (H, Is)))
    got = run_w4a16(smoe, x, ids, E, I, G, q["wg_q"], q["wg_s"], q["wu_q"], q["wu_s"],
                    q["wd_q"], q["wd_s"], shared=shared, calls=2, tiled=True)
    if shared is not None:
        got, got_s = got
        assert row_rel_err(got_s, oracle.shared_ffn(x, *shared)) <= ROW_TOL
    ref = oracle.routed_ffn_expertwise(x, ids, lambda e: tuple(
        oracle.dequant_int4(q[n + "_q"][e], q[n + "_s"][e], G) for n in ("wg", "wu", "wd")))
    assert np.isfinite(got).all()
    assert row_rel_err(got, ref) <= ROW_TOL
    dropped = ids.reshape(-1) < 0
    assert (got[dropped] == 0).all()


def _wide_items(ids, E, T, n, tiles, shared_tiles):
    # items of one long-window stage: 64-position chunks of every expert's
    # slots times the row tiles, plus the shared expert's chunks times its
    # tiles (shared_tiles = (tokens per chunk, tiles), or None)
    cnt = np.bincount(ids[ids >= 0].reshape(-1), minlength=E)
    items = int(np.sum((cnt + n - 1) // n)) * tiles
    if shared_tiles is not None:
        ch, st = shared_tiles
        items += (T + ch - 1) // ch * st
    return items


@pytest.mark.parametrize("stage,H,I,Is", [
    (1, 128, 8320, 256),     # gate/up: 64 chunks x 65 row tiles
    (2, 16384, 128, 128),    # down: 64 chunks x 64 tiles of 256 rows, 8 x 128 shared
])
def test_w4a16_ffn_long_window_static_split(smoe, stage, H, I, Is):
    # Launches with more than 16 items per workgroup (past the LDS item
    # tables' room at 256 workgroups) cut every item into static ranges
    # instead of claiming the routed ones at run time.
    E, k, T, G = 8, 8, 512, 128
    rng = np.random.default_rng(31 + stage)
    q = _synthetic_int4(E, H, I, G, seed=40 + stage)
    x = rng.standard_normal((T, H)).astype(np.float16)
    ids = _long_window_ids(rng, T, k, E, 0.0, 0.02)
    if stage == 1:
        n_items = _wide_items(ids, E, T, 64, I // 128, (128, Is // 128))
    else:
        n_items = _wide_items(ids, E, T, 64, (H // 16 + 15) // 16, (64, H // 128))
    assert n_items > 16 * 256, n_items
    shared = tuple((rng.standard_normal(sh) * 0.02).astype(np.float16)
                   for sh in ((Is, H), (Is, H), (H, Is)))
    got, got_s = run_w4a16(smoe, x, ids, E, I, G, q["wg_q"], q["wg_s"], q["wu_q"], q["wu_s"],
                           q["wd_q"], q["wd_s"], shared=shared, calls=2, tiled=True)
    assert row_rel_err(got_s, oracle.shared_ffn(x, *shared)) <= ROW_TOL
    ref = oracle.routed_ffn_expertwise(x, ids, lambda e: tuple(
        oracle.dequant_int4(q[n + "_q"][e], q[n + "_s"][e], G) for n in ("wg", "wu", "wd")))
    dropped = ids.reshape(-1) < 0
    assert np.isfinite(got).all()
    assert row_rel_err(got[~dropped], ref[~dropped]) <= ROW_TOL
    assert (got[dropped] == 0).all()


def test_w4a16_ffn_long_window_claims_across_calls(smoe):
    # The long-window FFN hands its routed items out at run time from
    # counters in the workspace, which each launch leaves at zero. Calls in
    # a row on one workspace with different routings (different numbers of
    # items), eagerly and replayed from a HIP graph: every call's rows equal
    # the oracle's, and the same call gives the same bits however its items
    # fell to the workgroups.
    E, k, T, H, I, G, Is = 16, 4, 300, 256, 256, 128, 256
    rng = np.random.default_rng(5)
    q = _synthetic_int4(E, H, I, G, seed=21)
    x = rng.standard_normal((T, H)).astype(np.float16)
    shared = tuple((rng.standard_normal(sh) * 0.02).astype(np.float16)
                   for sh in ((Is, H), (Is, H), (H, Is)))
    sh, sh_out, _ = _shared_dev(shared, T, H, smoe, True)
    ws = torch.zeros(smoe.smoe_ffn_workspace_bytes(T, k, E, H, I, Is), dtype=torch.uint8,
                     device="cuda")
    xd = dev(x)
    w = [dev(q[n]) for n in ("wg_q", "wg_s", "wu_q", "wu_s", "wd_q", "wd_s")]
    w[0:2] = tile_dev(smoe, w[0], w[1], E, I, H, G)
    w[2:4] = tile_dev(smoe, w[2], w[3], E, I, H, G)
    w[4:6] = tile_dev(smoe, w[4], w[5], E, H, I, G)
    out = torch.empty((T * k, H), dtype=torch.float32, device="cuda")

    def call(ss, off):
        smoe.smoe_w4a16_expert_ffn_tiled(xd, k, E, I, G, *w, ss, off, ws, out,
                                         shared=sh, shared_out=sh_out)

    def ref_of(ids):
        return oracle.routed_ffn_expertwise(x, ids, lambda e: tuple(
            oracle.dequant_int4(q[n + "_q"][e], q[n + "_s"][e], G) for n in ("wg", "wu", "wd")))

    routings = [_long_window_ids(rng, T, k, E, s, 0.0) for s in (0.0, 1.5, 0.7)]
    aligned = [oracle.align_by_expert(ids, E) for ids in routings]
    dev_al = [(dev(al["sorted_slots"]), dev(al["offsets"])) for al in aligned]
    first = []
    for ids, (ss, off) in zip(routings, dev_al):
        out.fill_(float("nan"))
        call(ss, off)
        got = host(out)
        assert np.isfinite(got).all()
        assert row_rel_err(got, ref_of(ids)) <= ROW_TOL
        first.append(got)
    assert row_rel_err(host(sh_out), oracle.shared_ffn(x, *shared)) <= ROW_TOL
    # graph replays of the second routing, with eager calls of the others between
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        call(*dev_al[1])
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            call(*dev_al[1])
    torch.cuda.current_stream().wait_stream(s)
    for i in range(3):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out), first[1]), i
        call(*dev_al[(i % 2) * 2])
        torch.cuda.synchronize()
        assert np.array_equal(host(out), first[(i % 2) * 2]), i


@pytest.mark.parametrize("Is", [0, 256])
def test_fp16_ffn_long_window(smoe, Is):
    E, k, T, H, I = 12, 4, 300, 256, 384
    rng = np.random.default_rng(77 + Is)
    x = rng.standard_normal((T, H)).astype(np.float16)
    wg = (rng.standard_normal((E, I, H)) * 0.02).astype(np.float16)
    wu = (rng.standard_normal((E, I, H)) * 0.02).astype(np.float16)
    wd = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float16)
    ids = _long_window_ids(rng, T, k, E, 1.1, 0.0)
    shared = None
    if Is:
        shared = tuple((rng.standard_normal(sh) * 0.02).astype(np.float16)
                       for sh in ((Is, H), (Is, H), (H, Is)))
    got = run_fp16(smoe, x, ids, E, I, wg, wu, wd, shared=shared, calls=2, tiled=True)
    if shared is not None:
        got, got_s = got
        assert row_rel_err(got_s, oracle.shared_ffn(x, *shared)) <= ROW_TOL
    ref = oracle.routed_ffn_expertwise(x, ids, lambda e: (wg[e], wu[e], wd[e]))
    assert row_rel_err(got, ref) <= ROW_TOL


def test_w4a16_ffn_one_hot_expert(smoe):
    # every slot on one expert: many chunks of the same expert
    E, k, T, H, I, G = 8, 1, 300, 256, 256, 64
    rng = np.random.default_rng(3)
    x = rng.standard_normal((T, H)).astype(np.float16)
    q = _synthetic_int4(E, H, I, G, seed=1)
    ids = np.full((T, k), 6, np.int32)
    got = run_w4a16(smoe, x, ids, E, I, G, q["wg_q"], q["wg_s"], q["wu_q"], q["wu_s"],
                    q["wd_q"], q["wd_s"])

    def load(e):
        return tuple(oracle.dequant_int4(q[n + "_q"][e], q[n + "_s"][e], G) for n in ("wg", "wu", "wd"))
    assert row_rel_err(got, oracle.routed_ffn_expertwise(x, ids, load)) <= ROW_TOL


def run_fp16(smoe, x, ids, E, I, wg, wu, wd, shared=None, calls=1, tiled=False):
    T, k = ids.shape
    H = x.shape[1]
    al = oracle.align_by_expert(ids, E)
    sh, sh_out, Is = _shared_dev(shared, T, H, smoe, tiled)
    ws = torch.zeros(smoe.smoe_ffn_workspace_bytes(T, k, E, H, I, Is), dtype=torch.uint8,
                     device="cuda")
    args = [dev(a) for a in (x, wg, wu, wd, al["sorted_slots"], al["offsets"])]
    fn = smoe.smoe_fp16_expert_ffn
    if tiled:
        args[1] = tile_dev(smoe, args[1], None, E, I, H, 0)[0]
        args[2] = tile_dev(smoe, args[2], None, E, I, H, 0)[0]
        args[3] = tile_dev(smoe, args[3], None, E, H, I, 0)[0]
        fn = smoe.smoe_fp16_expert_ffn_tiled
    for _ in range(calls):
        out = torch.full((T * k, H), float("nan"), dtype=torch.float32, device="cuda")
        if sh_out is not None:
            sh_out.fill_(float("nan"))
        fn(args[0], k, E, I, *args[1:4], args[4], args[5], ws, out,
           shared=sh, shared_out=sh_out)
    if shared is None:
        return host(out)
    return host(out), host(sh_out)


def test_fp16_ffn_shared_expert_dsv2(smoe):
    L = layer("dsv2")
    T = L.cfg.T
    ids = np.zeros((T, 1), np.int32)
    got = run_fp16(smoe, L.x, ids, 1, L.sg16.shape[0], L.sg16[None], L.su16[None], L.sd16[None])
    ref = oracle.shared_ffn(L.x, L.sg16, L.su16, L.sd16)
    assert row_rel_err(got, ref) <= ROW_TOL


@pytest.mark.parametrize("name", ["dsv2", "qwen"])
@pytest.mark.parametrize("tiled", [False, True], ids=["rows", "tiled"])
def test_w4a16_ffn_with_shared_expert(smoe, name, tiled):
    # routed INT4 experts and the FP16 shared expert(s) in the same launches,
    # three calls in a row on one workspace
    L = layer(name)
    cfg = L.cfg
    ids = oracle.topk_experts(oracle.router_logits_f32(L.x, L.w_router, L.router_bias), cfg.k)
    got, got_sh = run_w4a16(smoe, L.x, ids, cfg.E, cfg.I, cfg.G, L.wg_q, L.wg_s, L.wu_q,
                            L.wu_s, L.wd_q, L.wd_s, shared=(L.sg16, L.su16, L.sd16), calls=3,
                            tiled=tiled)
    assert np.isfinite(got).all() and np.isfinite(got_sh).all()
    assert row_rel_err(got, oracle_slots_int4(L, ids)) <= ROW_TOL
    assert row_rel_err(got_sh, oracle.shared_ffn(L.x, L.sg16, L.su16, L.sd16)) <= ROW_TOL


@pytest.mark.parametrize("E,k,T,H,I,G,Is", [
    (8, 2, 40, 256, 384, 64, 640),   # shared expert over two token chunks (32 + 8)
    (16, 1, 1, 384, 256, 128, 256),  # a single token
    (6, 3, 17, 128, 128, 32, 3072),  # shared rows staged in several k phases
    (8, 3, 200, 256, 384, 128, 512),  # wide chunks (128 slots): routed and shared, 72-row tail
    (32, 2, 97, 384, 256, 128, 384),  # wide chunks, a 97-token shared chunk (7 column groups)
    (16, 2, 9, 256, 256, 32, 512),   # x resident: g32 routed, FP16 shared in the INT4 k order
    (12, 3, 18, 512, 256, 64, 384),  # x resident: g64 routed, an 18-token shared chunk (2 groups)
    (64, 6, 19, 2048, 256, 128, 256),  # the widest window that keeps x resident at H = 2048
    (64, 6, 20, 2048, 256, 128, 256),  # one token more: x staged per chunk again
])
@pytest.mark.parametrize("tiled", [False, True], ids=["rows", "tiled"])
def test_w4a16_ffn_with_shared_shapes(smoe, E, k, T, H, I, G, Is, tiled):
    rng = np.random.default_rng(T + Is)
    x = rng.standard_normal((T, H)).astype(np.float16)
    q = _synthetic_int4(E, H, I, G, seed=E + Is)
    sg = (rng.standard_normal((Is, H)) * 0.02).astype(np.float16)
    su = (rng.standard_normal((Is, H)) * 0.02).astype(np.float16)
    sd = (rng.standard_normal((H, Is)) * 0.02).astype(np.float16)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    got, got_sh = run_w4a16(smoe, x, ids, E, I, G, q["wg_q"], q["wg_s"], q["wu_q"], q["wu_s"],
                            q["wd_q"], q["wd_s"], shared=(sg, su, sd), calls=2, tiled=tiled)

    def load(e):
        return tuple(oracle.dequant_int4(q[n + "_q"][e], q[n + "_s"][e], G) for n in ("wg", "wu", "wd"))
    assert row_rel_err(got, oracle.routed_ffn_expertwise(x, ids, load)) <= ROW_TOL
    assert row_rel_err(got_sh, oracle.shared_ffn(x, sg, su, sd)) <= ROW_TOL


@pytest.mark.parametrize("tiled", [False, True], ids=["rows", "tiled"])
def test_fp16_ffn_with_shared_expert(smoe, tiled):
    E, k, T, H, I, Is = 8, 2, 17, 256, 512, 768
    rng = np.random.default_rng(5)
    x = rng.standard_normal((T, H)).astype(np.float16)
    wg, wu = [(rng.standard_normal((E, I, H)) * 0.02).astype(np.float16) for _ in range(2)]
    wd = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float16)
    sg, su = [(rng.standard_normal((Is, H)) * 0.02).astype(np.float16) for _ in range(2)]
    sd = (rng.standard_normal((H, Is)) * 0.02).astype(np.float16)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    got, got_sh = run_fp16(smoe, x, ids, E, I, wg, wu, wd, shared=(sg, su, sd), calls=2,
                           tiled=tiled)
    ref = oracle.routed_ffn_expertwise(x, ids, lambda e: (wg[e], wu[e], wd[e]))
    assert row_rel_err(got, ref) <= ROW_TOL
    assert row_rel_err(got_sh, oracle.shared_ffn(x, sg, su, sd)) <= ROW_TOL


@pytest.mark.parametrize("E,k,T,H,I", [(8, 2, 17, 256, 512), (4, 2, 150, 256, 256),
                                       (16, 1, 1, 384, 256), (3, 3, 300, 256, 384)])
@pytest.mark.parametrize("tiled", [False, True], ids=["rows", "tiled"])
def test_fp16_ffn_shapes(smoe, E, k, T, H, I, tiled):
    rng = np.random.default_rng(E * T)
    x = rng.standard_normal((T, H)).astype(np.float16)
    wg = (rng.standard_normal((E, I, H)) * 0.02).astype(np.float16)
    wu = (rng.standard_normal((E, I, H)) * 0.02).astype(np.float16)
    wd = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float16)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    got = run_fp16(smoe, x, ids, E, I, wg, wu, wd, tiled=tiled)
    ref = oracle.routed_ffn_expertwise(x, ids, lambda e: (wg[e], wu[e], wd[e]))
    assert row_rel_err(got, ref) <= ROW_TOL


def _pool(smoe, wg, wu, wd, slot_of, M, tiled):
    """Device pool [M][3][I*H] fp16 holding expert e's (wg, wu, wd) at slot
    slot_of[e] (-1: not resident), and the three base views into it."""
    E, I, H = wg.shape
    msz = I * H
    pool = torch.zeros(M * 3 * msz, dtype=torch.float16, device="cuda")
    for e in range(E):
        s = int(slot_of[e])
        if s < 0:
            continue
        for j, w in enumerate((wg[e], wu[e], wd[e])):
            n, kk = w.shape
            t = dev(np.ascontiguousarray(w))
            if tiled:
                t = tile_dev(smoe, t, None, 1, n, kk, 0)[0]
            pool[(3 * s + j) * msz:(3 * s + j + 1) * msz] = t.reshape(-1)
    return pool, pool[0:], pool[msz:], pool[2 * msz:]


@pytest.mark.parametrize("tiled", [False, True], ids=["rows", "tiled"])
def test_fp16_ffn_mapped_disjoint_calls(smoe, tiled):
    # experts placed at scattered slots of a pool; a first call over some of
    # them (the resident ones), a second over the rest: together they fill
    # slot_out exactly like one unmapped call, and rows outside a call keep
    # what they held
    E, k, T, H, I, M = 8, 2, 17, 256, 384, 11
    rng = np.random.default_rng(7)
    x = rng.standard_normal((T, H)).astype(np.float16)
    wg = (rng.standard_normal((E, I, H)) * 0.02).astype(np.float16)
    wu = (rng.standard_normal((E, I, H)) * 0.02).astype(np.float16)
    wd = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float16)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    ids[3, 1] = -1  # a dropped slot: written by neither call
    slot_of = rng.permutation(M)[:E].astype(np.int32)
    pool, pg, pu, pd = _pool(smoe, wg, wu, wd, slot_of, M, tiled)
    al = oracle.align_by_expert(ids, E)
    ref = oracle.routed_ffn_expertwise(x, ids, lambda e: (wg[e], wu[e], wd[e]))
    first = np.zeros(E, bool)
    first[[0, 2, 3, 6]] = True
    tables = [np.where(first, 3 * slot_of, -1), np.where(~first, 3 * slot_of, -1)]
    ws = torch.zeros(smoe.smoe_ffn_workspace_bytes(T, k, E, H, I, 0), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((T * k, H), 7.0, dtype=torch.float32, device="cuda")
    xs, ss, offs = dev(x), dev(al["sorted_slots"]), dev(al["offsets"])
    slot_expert = ids.reshape(-1)
    for c, tab in enumerate(tables):
        smoe.smoe_fp16_expert_ffn_mapped(xs, k, E, I, pg, pu, pd, 3 * M - 2, tab, ss, offs, ws,
                                         out, tiled=tiled)
        got = host(out)
        done = np.isin(slot_expert, np.nonzero(first if c == 0 else np.ones(E, bool))[0])
        assert row_rel_err(got[done], ref[done]) <= ROW_TOL
        assert (got[~done] == 7.0).all()
    assert (host(out)[3 * k + 1] == 7.0).all()


def test_ffn_workspace_stamp_detects_a_shape_change(smoe):
    # a workspace zeroed for one window and then used for another without
    # zeroing again gives NaN outputs (not wrong sums) until it is cleared
    E, k, H, I = 8, 2, 256, 256
    rng = np.random.default_rng(3)
    wg = (rng.standard_normal((E, I, H)) * 0.02).astype(np.float16)
    wu = (rng.standard_normal((E, I, H)) * 0.02).astype(np.float16)
    wd = (rng.standard_normal((E, H, I)) * 0.02).astype(np.float16)
    W = [dev(w) for w in (wg, wu, wd)]
    ws = torch.zeros(smoe.smoe_ffn_workspace_bytes(17, k, E, H, I, 0), dtype=torch.uint8,
                     device="cuda")

    def call(T):
        x = rng.standard_normal((T, H)).astype(np.float16)
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        al = oracle.align_by_expert(ids, E)
        out = torch.zeros((T * k, H), dtype=torch.float32, device="cuda")
        smoe.smoe_fp16_expert_ffn(dev(x), k, E, I, *W, dev(al["sorted_slots"]),
                                  dev(al["offsets"]), ws, out)
        ref = oracle.routed_ffn_expertwise(x, ids, lambda e: (wg[e], wu[e], wd[e]))
        return host(out), ref

    for _ in range(2):  # the same shape twice: fine
        got, ref = call(17)
        assert row_rel_err(got, ref) <= ROW_TOL
    got, _ = call(9)  # another T on the same workspace: spoiled
    assert np.isnan(got).all()
    got, _ = call(17)  # stays spoiled, also for the first shape
    assert np.isnan(got).all()
    smoe.smoe_ffn_workspace_clear(ws)
    for T in (9, 9):  # zeroed: serves the new shape
        got, ref = call(T)
        assert row_rel_err(got, ref) <= ROW_TOL


@pytest.mark.parametrize("tiled", [False, True], ids=["rows", "tiled"])
def test_phi_draft_and_target(smoe, tiled):
    # both expert FFN calls of the Phi-shaped window against the oracle, on
    # every slot of every active expert (34 slots over the 15 experts the
    # window routes to)
    L = layer("phi")
    cfg = L.cfg
    ref_d, ref_t = ref_layer("phi", "draft"), ref_layer("phi", "target")
    ids = ref_d["ids"]
    assert np.array_equal(ref_t["ids"], ids)
    draft = run_w4a16(smoe, L.x, ids, cfg.E, cfg.I, cfg.G, L.wg_q, L.wg_s, L.wu_q, L.wu_s,
                      L.wd_q, L.wd_s, tiled=tiled)
    target = run_fp16(smoe, L.x, ids, cfg.E, cfg.I, L.wg16, L.wu16, L.wd16, tiled=tiled)
    assert np.isfinite(draft).all() and np.isfinite(target).all()
    assert draft.shape == ref_d["slot_out"].shape == (cfg.T * cfg.k, cfg.H)
    assert row_rel_err(draft, ref_d["slot_out"]) <= ROW_TOL
    assert row_rel_err(target, ref_t["slot_out"]) <= ROW_TOL
    # the two passes really differ (INT4 against FP16 weights)
    assert row_rel_err(draft, target) > 1e-3


# ------------------------------------------------------------------ combine

def test_combine_matches_oracle(smoe):
    rng = np.random.default_rng(31)
    for T, k, H, shared, gated in [(17, 6, 2048, True, False), (9, 4, 2048, True, True),
                                   (17, 2, 4096, False, False), (1, 1, 128, False, False)]:
        so = rng.standard_normal((T * k, H)).astype(np.float32)
        w = rng.random((T, k)).astype(np.float32)
        sh = rng.standard_normal((T, H)).astype(np.float32) if shared else None
        g = rng.random(T).astype(np.float32) if gated else None
        y = torch.empty((T, H), dtype=torch.float16, device="cuda")
        smoe.smoe_combine(dev(so), dev(w), None if sh is None else dev(sh),
                          None if g is None else dev(g), y)
        _, ref16 = oracle.combine(so, w, sh, g)
        y64 = oracle.combine(so, w, sh, g)[0]
        got = host(y).astype(np.float64)
        # fp16 output: within one fp16 rounding step of the float64 sum
        assert np.all(np.abs(got - y64) <= np.abs(y64) * 2.0 ** -10 + 1e-6)


def test_empty_window_is_a_noop(smoe):
    """T = 0: every call returns at once; the fused routing call still ranks
    the ELB counters, exactly as the separate calls do."""
    rng = np.random.default_rng(41)
    x = np.zeros((0, 256), np.float16)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    got = _run_routing(smoe, True, x, w, None, 2, 0, None, (2, 1, 3, 0))
    ref = _run_routing(smoe, False, x, w, None, 2, 0, None, (2, 1, 3, 0))
    for key in ref:
        assert np.array_equal(got[key], ref[key]), key
    assert not got["offsets"].any() and int(got["n_active"][0]) == 0
    q = _synthetic_int4(8, 256, 128, 64, seed=5)
    out = run_w4a16(smoe, x, np.zeros((0, 2), np.int32), 8, 128, 64, q["wg_q"], q["wg_s"],
                    q["wu_q"], q["wu_s"], q["wd_q"], q["wd_s"])
    assert out.shape == (0, 256)
    y = torch.empty((0, 256), dtype=torch.float16, device="cuda")
    smoe.smoe_combine(torch.empty((0, 256), dtype=torch.float32, device="cuda"),
                      torch.empty((0, 2), dtype=torch.float32, device="cuda"), None, None, y)
    torch.cuda.synchronize()


# ------------------------------------------------------------------ whole layer

_LAYER_MODES = ["fused", "fused-side", "separate", "separate-side", "three-routing-calls",
                "one-call", "fused-tiled", "separate-tiled", "one-call-tiled"]
# (the Phi-shaped layer has no shared expert, so its separate modes equal fused)
_LAYER_CASES = ([(n, m) for n in ("tiny", "dsv2", "qwen", "dsv2_t1") for m in _LAYER_MODES] +
                [("phi", m) for m in ("fused", "three-routing-calls", "one-call", "fused-tiled",
                                      "one-call-tiled")])


@pytest.mark.parametrize("name,mode", _LAYER_CASES)
def test_layer_draft_matches_oracle(smoe, name, mode):
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L = layer(name)
    ref = ref_layer(name, "draft")
    tiled = mode.endswith("-tiled")
    mode = mode[:-len("-tiled")] if tiled else mode
    d = DeviceLayer(L, tiled=tiled, with_target=False)
    if mode == "one-call":
        d.run(one_call=True)
    else:
        d.run(fuse_shared=not mode.startswith("separate"),
              fuse_routing=mode != "three-routing-calls",
              side_stream=torch.cuda.Stream() if mode.endswith("side") else None)
    assert np.array_equal(host(d.topk_ids), ref["ids"])
    assert np.array_equal(host(d.sorted_slots), ref["sorted_slots"])
    assert int(host(d.n_active)[0]) == int(ref["n_active"])
    err = row_rel_err(host(d.y), ref["y64"])
    assert err <= ROW_TOL, err
    assert row_rel_err(host(d.slot_out), ref["slot_out"]) <= ROW_TOL
    if L.cfg.elb_M:
        ref_cnt = oracle.elb_accumulate(np.zeros((1, L.cfg.E), np.int32), ref["ids"][None], 0)
        pid, pc = oracle.elb_topm(ref_cnt, L.cfg.elb_M)
        assert np.array_equal(host(d.elb_counts), ref_cnt)
        assert np.array_equal(host(d.plan_ids), pid) and np.array_equal(host(d.plan_counts), pc)


def test_layer_fused_separate_fused_on_one_layer(smoe):
    # the shared experts fused into the routed FFN, then in a call of their
    # own, then fused again, on one DeviceLayer: every run matches the oracle
    # (each mode keeps a workspace of its own shape)
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L = layer("dsv2")
    ref = ref_layer("dsv2", "draft")
    d = DeviceLayer(L, with_target=False)
    for fuse in (True, False, True, False):
        d.y.fill_(float("nan"))
        d.run(fuse_shared=fuse)
        y = host(d.y)
        assert np.isfinite(y).all()
        assert row_rel_err(y, ref["y64"]) <= ROW_TOL


@pytest.mark.parametrize("tiled", [False, True], ids=["rows", "tiled"])
def test_phi_target_layer_matches_oracle(smoe, tiled):
    # the FP16 target verification pass of the Phi-shaped layer through the
    # whole layer (route, align, FP16 expert FFN, combine): every slot and
    # all 17 rows of y against oracle.moe_layer(..., "target")
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L = layer("phi")
    ref = ref_layer("phi", "target")
    d = DeviceLayer(L, tiled=tiled)
    d.run(target=True)
    assert np.array_equal(host(d.topk_ids), ref["ids"])
    assert np.array_equal(host(d.sorted_slots), ref["sorted_slots"])
    assert row_rel_err(host(d.slot_out), ref["slot_out"]) <= ROW_TOL
    y = host(d.y)
    assert y.shape == (17, 4096) and np.isfinite(y).all()
    assert row_rel_err(y, ref["y64"]) <= ROW_TOL
    # the draft pass over the same tokens on the same runner picks the same
    # experts (one shared router) and matches the oracle's draft layer,
    # which is not the target output
    d.run(target=False)
    assert np.array_equal(host(d.topk_ids), ref["ids"])
    ref_d = ref_layer("phi", "draft")
    assert row_rel_err(host(d.y), ref_d["y64"]) <= ROW_TOL
    assert row_rel_err(ref_d["y64"], ref["y64"]) > 1e-3


def test_batch_stack_26_layers(smoe):
    # The batched stack: 26 layers of 544 tokens, each with its own
    # activations, router and Zipf(1.1) router skew, each run as the whole
    # draft layer (routing, alignment, ELB update of its own counter row,
    # W4A16 FFN with the shared experts, combine). The ELB accumulates over
    # the 26 layers and is ranked top-32 once at the end. Expert weights: the
    # generated weights of layer 0 serve every layer (the counter and plan
    # depend only on the routing inputs, which are per layer).
    from quantized_speculative_expert_amd.layer import DeviceLayer
    cfg = get_config("batch")
    L0 = layer("batch", layer_idx=0)
    d = DeviceLayer(L0, elb_layers=cfg.layers)
    ids_all = np.empty((cfg.layers, cfg.T, cfg.k), np.int32)
    y0 = None
    for l in range(cfg.layers):
        x = make_activations(cfg, 0, l)
        wr = make_router(cfg, 0, l)
        b = zipf_bias(cfg.E, cfg.zipf_s, 0, l)
        d.x.copy_(torch.from_numpy(x))
        d.w_router.copy_(torch.from_numpy(wr))
        d.router_bias.copy_(torch.from_numpy(b))
        d.run(layer=l, rank=False)
        ids = host(d.topk_ids)
        ref_ids = oracle.topk_experts(oracle.router_logits_f32(x, wr, b), cfg.k)
        assert np.array_equal(ids, ref_ids), l
        ids_all[l] = ids
        if l == 0:
            y0 = host(d.y).copy()
            assert np.array_equal(host(d.sorted_slots),
                                  oracle.align_by_expert(ref_ids, cfg.E)["sorted_slots"])
    # one ranking over all 26 counter rows, then compare with the oracle
    d.elb(layer=0, M=cfg.elb_M, accumulate=False)
    ref_cnt = oracle.elb_accumulate(np.zeros((cfg.layers, cfg.E), np.int32), ids_all, 0)
    pid, pc = oracle.elb_topm(ref_cnt, cfg.elb_M)
    assert np.array_equal(host(d.elb_counts), ref_cnt)
    assert np.array_equal(host(d.plan_ids), pid)
    assert np.array_equal(host(d.plan_counts), pc)
    assert ref_cnt.sum() == cfg.layers * cfg.T * cfg.k
    # every token of layer 0 against the oracle layer
    ref0 = ref_layer("batch", "draft", layer_idx=0)
    assert row_rel_err(y0, ref0["y64"]) <= ROW_TOL


@pytest.mark.parametrize("tiled", [False, True], ids=["rows", "tiled"])
def test_batch_layer_full_size_sampled(smoe, tiled):
    # the batched window (544 tokens, Zipf-skewed router, 32-slot chunks) at
    # full size through the whole layer; the oracle checks every slot of
    # three experts and the outputs of two tokens, computed one by one
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L = layer("batch", layer_idx=3)
    cfg = L.cfg
    d = DeviceLayer(L, elb_layers=cfg.layers, tiled=tiled)
    d.run()
    lg = oracle.router_logits_f32(L.x, L.w_router, L.router_bias)
    ids = oracle.topk_experts(lg, cfg.k)
    assert np.array_equal(host(d.topk_ids), ids)
    al = oracle.align_by_expert(ids, cfg.E)
    assert np.array_equal(host(d.sorted_slots), al["sorted_slots"])
    slot_out = host(d.slot_out)
    flat = ids.ravel()

    def expert(e):
        return (oracle.dequant_int4(L.wg_q[e], L.wg_s[e], cfg.G),
                oracle.dequant_int4(L.wu_q[e], L.wu_s[e], cfg.G),
                oracle.dequant_int4(L.wd_q[e], L.wd_s[e], cfg.G))
    counts = np.bincount(flat, minlength=cfg.E)
    busiest = int(np.argmax(counts))                  # more than one 32-slot chunk
    for e in sorted({busiest, int(np.argmin(np.where(counts > 0, counts, 1 << 30))), 7}):
        sl = np.flatnonzero(flat == e)
        if len(sl) == 0:
            continue
        ref = oracle.swiglu(L.x[sl // cfg.k].astype(np.float64), *expert(e))
        assert row_rel_err(slot_out[sl], ref) <= ROW_TOL, e
    assert counts[busiest] > 32
    w = oracle.routing_weights(lg, ids)
    y = host(d.y)
    for t in (0, 543):
        so = np.stack([oracle.swiglu(L.x[t:t + 1].astype(np.float64), *expert(int(e)))[0]
                       for e in ids[t]])
        sh = oracle.shared_ffn(L.x[t:t + 1], L.sg16, L.su16, L.sd16)
        ref = (w[t][:, None] * so).sum(0) + sh[0]
        assert row_rel_err(y[t:t + 1], ref[None]) <= ROW_TOL, t
    # the layer's row of the 26-layer activation counter and its top-32 plan
    cnt = np.zeros((cfg.layers, cfg.E), np.int32)
    cnt[0] = np.bincount(flat, minlength=cfg.E)
    pid, pc = oracle.elb_topm(cnt, cfg.elb_M)
    assert np.array_equal(host(d.elb_counts), cnt)
    assert np.array_equal(host(d.plan_ids), pid) and np.array_equal(host(d.plan_counts), pc)


@pytest.mark.parametrize("fused", [True, False, "one-call", "one-call-tiled"])
def test_layer_graph_replay_matches_eager(smoe, fused):
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L = layer("dsv2")
    d = DeviceLayer(L, tiled=fused == "one-call-tiled")
    one = fused in ("one-call", "one-call-tiled")
    d.run(elb=False, fuse_shared=bool(fused), one_call=one)
    eager = host(d.y).copy()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            # the ELB update runs on the side branch of the graph (or in line,
            # in one call)
            d.run(elb=True, fuse_shared=bool(fused), side_stream=None if one else side,
                  one_call=one)
    torch.cuda.current_stream().wait_stream(s)
    ids_eager = host(d.topk_ids).copy()
    once = np.bincount(ids_eager.ravel(), minlength=L.cfg.E)
    d.elb_counts.zero_()
    for rep in range(3):
        d.y.zero_()
        d.topk_ids.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(d.topk_ids), ids_eager)
        assert np.array_equal(host(d.elb_counts)[0], (rep + 1) * once)
        # split-K tiles add fp32 partial sums with device atomics, so the
        # float output may differ from the eager run in the last bits
        assert row_rel_err(host(d.y), eager) <= 1e-3


@pytest.mark.parametrize("name", ["tiny", "dsv2", "phi", "dsv2_t1"])
def test_tiled_layer_equals_row_major(smoe, name):
    """Tiling moves bytes, not values: the same layer over tiled weights
    gives the row-major layer's IDs and alignment, and its outputs up to the
    order in which split-K tiles add their partial sums."""
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L = layer(name)
    rows, tiled = DeviceLayer(L), DeviceLayer(L, tiled=True)
    for d in (rows, tiled):
        d.run()
    torch.cuda.synchronize()
    assert np.array_equal(host(rows.topk_ids), host(tiled.topk_ids))
    assert np.array_equal(host(rows.sorted_slots), host(tiled.sorted_slots))
    assert row_rel_err(host(tiled.slot_out), host(rows.slot_out)) <= 1e-3
    assert row_rel_err(host(tiled.y), host(rows.y)) <= 1e-3


def _layer_outputs(d):
    return dict(ids=host(d.topk_ids).copy(), w=host(d.topk_w).copy(), lg=host(d.logits).copy(),
                counts=host(d.counts).copy(), offsets=host(d.offsets).copy(),
                slots=host(d.sorted_slots).copy(), active=host(d.active).copy(),
                n_active=host(d.n_active).copy(), elb=host(d.elb_counts).copy(),
                plan=host(d.plan_ids).copy(), plan_c=host(d.plan_counts).copy(),
                y=host(d.y).astype(np.float64))


@pytest.mark.parametrize("name", ["tiny", "dsv2", "qwen", "phi", "dsv2_t1"])
def test_layer_one_call_equals_separate_calls(smoe, name):
    # the one-call layer against the separate calls on the device: integer
    # results bit for bit, y up to the order of the split-K float atomics
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L = layer(name)
    d = DeviceLayer(L)
    d.run()
    sep = _layer_outputs(d)
    d.elb_counts.zero_()
    for t in (d.topk_ids, d.counts, d.offsets, d.sorted_slots, d.active, d.n_active,
              d.plan_ids, d.plan_counts):
        t.fill_(-3)
    d.y.zero_()
    d.run(one_call=True)
    one = _layer_outputs(d)
    keys = ["ids", "lg", "counts", "offsets", "slots", "active", "n_active"]
    if L.cfg.elb_M > 0:  # (no ELB plan without M)
        keys += ["elb", "plan", "plan_c"]
    for key in keys:
        assert np.array_equal(one[key], sep[key]), key
    assert np.array_equal(one["w"], sep["w"])
    assert row_rel_err(one["y"], sep["y"]) <= 1e-3


def test_layer_one_call_interleaved_with_other_calls(smoe):
    # one-call layers mixed with separate-call layers on one FFN workspace
    # (whose call counter every FFN call advances) all match the oracle
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L = layer("dsv2")
    ref = oracle.moe_layer(L, "draft")
    d = DeviceLayer(L)
    for one in (True, False, True, True, False, False, True):
        d.topk_ids.fill_(-1)
        d.sorted_slots.fill_(-1)
        d.y.zero_()
        d.run(elb=False, one_call=one)
        assert np.array_equal(host(d.topk_ids), ref["ids"]), one
        assert np.array_equal(host(d.sorted_slots), ref["sorted_slots"]), one
        assert row_rel_err(host(d.y), ref["y64"]) <= ROW_TOL, one


def test_layer_one_call_batch_window(smoe):
    # 544 tokens x top-6 = 3264 slots, above the one-workgroup routing
    # limit (the routing takes its three separate launches inside the call)
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L = layer("batch", layer_idx=1)
    d = DeviceLayer(L, elb_layers=L.cfg.layers)
    d.run()
    sep = _layer_outputs(d)
    d.elb_counts.zero_()
    d.topk_ids.fill_(-1)
    d.sorted_slots.fill_(-1)
    d.run(one_call=True)
    one = _layer_outputs(d)
    for key in ("ids", "slots", "offsets", "elb", "plan"):
        assert np.array_equal(one[key], sep[key]), key
    assert row_rel_err(one["y"], sep["y"]) <= 1e-3
