"""Pins of the CPU reference (oracle/) against facts it does not compute itself:
hand-worked golden fixtures, closed forms, brute force on tiny inputs,
invariants and an independent float64 computation within a stated error
bound. CPU only.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from workload import get_config, make_activations, make_router, quantize_rtn_int4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- router logits

def _sparse_router_case():
    g = golden("router_order_handworked.json")
    H, E = g["H"], g["E"]
    x = np.zeros((1, H), np.float16)
    for h, v in g["x_nonzero"].items():
        x[0, int(h)] = v
    w = np.zeros((E, H), np.float32)
    for e, row in enumerate(g["w_nonzero"]):
        for h, v in row.items():
            w[e, int(h)] = v
    return g, x, w


def test_router_order_handworked():
    g, x, w = _sparse_router_case()
    # the fixture's values are exactly representable
    assert float(x[0, 66]) == 1.0 + 2.0 ** -10
    assert float(w[1, 2]) == 1.0 + 2.0 ** -10 + 2.0 ** -14
    lg = oracle.router_logits_f32(x, w)
    assert lg.dtype == np.float32
    assert lg[0].tolist() == g["expected_logits"]
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    assert exact[0].tolist() == g["exact_logits"]


def test_router_logits_exact_small_integers():
    # integers small enough that every partial sum is exact in float32
    rng = np.random.default_rng(11)
    T, E, H = 5, 7, 256
    x = rng.integers(-3, 4, size=(T, H)).astype(np.float16)
    w = rng.integers(-4, 5, size=(E, H)).astype(np.float32)
    lg = oracle.router_logits_f32(x, w)
    ref = np.zeros((T, E), np.int64)
    for t in range(T):
        for e in range(E):
            ref[t, e] = sum(int(x[t, h]) * int(w[e, h]) for h in range(H))
    assert np.array_equal(lg.astype(np.int64), ref)


@pytest.mark.parametrize("name", ["tiny", "dsv2", "phi"])
def test_router_logits_within_fp32_bound(name):
    cfg = get_config(name)
    x = make_activations(cfg, seed=3)
    w = make_router(cfg, seed=3)
    lg = oracle.router_logits_f32(x, w).astype(np.float64)
    x64, w64 = x.astype(np.float64), w.astype(np.float64)
    exact = x64 @ w64.T
    mag = np.abs(x64) @ np.abs(w64).T
    n_ops = cfg.H // 64 + 6 + 1
    bound = 1.01 * n_ops * 2.0 ** -24 * mag
    assert np.all(np.abs(lg - exact) <= bound)
    # and the error is not trivially zero everywhere (it is a float32 sum)
    assert np.any(lg != exact)


def test_router_bias_is_added_last():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 128)).astype(np.float16)
    w = (rng.standard_normal((6, 128)) * 0.02).astype(np.float32)
    b = rng.standard_normal(6).astype(np.float32)
    a = oracle.router_logits_f32(x, w)
    ab = oracle.router_logits_f32(x, w, b)
    assert np.array_equal(ab, (a + b[None, :]).astype(np.float32))


# ---------------------------------------------------------------- top-k

def _dominates(lg, a, b):
    """Expert a ranks ahead of expert b: larger logit, or equal and lower ID."""
    return lg[a] > lg[b] or (lg[a] == lg[b] and a < b)


def test_topk_golden_ties():
    g = golden("topk_ties_handworked.json")
    lg = np.array([float(v) for v in g["logits"]], np.float32)
    assert math.copysign(1.0, lg[1]) < 0  # the fixture holds a real -0.0
    for k, exp in g["expected"].items():
        ids = oracle.topk_experts(lg[None, :], int(k))
        assert ids[0].tolist() == exp


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_subsets(seed):
    rng = np.random.default_rng(seed)
    E, k, T = 7, 3, 9
    # coarse values force many exact ties
    lg = rng.integers(-2, 3, size=(T, E)).astype(np.float32) * np.float32(0.5)
    ids = oracle.topk_experts(lg, k)
    for t in range(T):
        # exactly one k-subset dominates its complement
        winners = [set(c) for c in itertools.combinations(range(E), k)
                   if all(_dominates(lg[t], a, b)
                          for a in c for b in range(E) if b not in c)]
        assert len(winners) == 1
        assert set(ids[t].tolist()) == winners[0]
        for j in range(k - 1):
            assert _dominates(lg[t], ids[t, j], ids[t, j + 1])


def test_topk_k_equals_E_is_permutation():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((4, 8)).astype(np.float32)
    ids = oracle.topk_experts(lg, 8)
    for t in range(4):
        assert sorted(ids[t].tolist()) == list(range(8))
        assert np.all(np.diff(lg[t, ids[t]]) <= 0)


def test_topk_duplicated_router_rows_pick_lower_id():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((6, 128)).astype(np.float16)
    w = (rng.standard_normal((5, 128)) * 0.02).astype(np.float32)
    w[3] = w[1]      # experts 1 and 3 always tie exactly
    lg = oracle.router_logits_f32(x, w)
    assert np.array_equal(lg[:, 1], lg[:, 3])
    ids = oracle.topk_experts(lg, 5)
    for t in range(6):
        order = ids[t].tolist()
        assert order.index(1) == order.index(3) - 1


@pytest.mark.parametrize("name", ["dsv2", "qwen"])
def test_topk_agrees_with_float64_where_separated(name):
    cfg = get_config(name)
    x = make_activations(cfg, seed=1)
    w = make_router(cfg, seed=1)
    lg = oracle.router_logits_f32(x, w)
    x64, w64 = x.astype(np.float64), w.astype(np.float64)
    exact = x64 @ w64.T
    bound = 1.01 * (cfg.H // 64 + 7) * 2.0 ** -24 * (np.abs(x64) @ np.abs(w64).T)
    ids = oracle.topk_experts(lg, cfg.k)
    checked = 0
    for t in range(cfg.T):
        order = np.argsort(-exact[t], kind="stable")
        kth, nxt = order[cfg.k - 1], order[cfg.k]
        if exact[t, kth] - exact[t, nxt] > bound[t, kth] + bound[t, nxt]:
            assert set(ids[t].tolist()) == set(order[:cfg.k].tolist())
            checked += 1
    assert checked >= cfg.T // 2


# ---------------------------------------------------------------- weights, gate

def test_routing_weights_closed_form():
    lg = np.log(np.array([[1.0, 2.0, 3.0, 4.0]])).astype(np.float32)
    ids = np.array([[3, 2, 1, 0]], np.int32)
    w = oracle.routing_weights(lg, ids)
    assert np.allclose(w[0], [0.4, 0.3, 0.2, 0.1], rtol=1e-6, atol=0)
    w2 = oracle.routing_weights(lg, ids[:, :2], renorm=True)
    assert np.allclose(w2[0], [4 / 7, 3 / 7], rtol=1e-6, atol=0)
    flat = oracle.routing_weights(np.zeros((1, 5), np.float32), np.array([[0, 4]]))
    assert np.array_equal(flat, [[0.2, 0.2]])


def test_routing_weights_sum_to_one_over_all_experts():
    rng = np.random.default_rng(4)
    lg = (rng.standard_normal((10, 16)) * 3).astype(np.float32)
    ids = oracle.topk_experts(lg, 16)
    w = oracle.routing_weights(lg, ids)
    assert np.allclose(w.sum(axis=1), 1.0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)


def test_shared_gate_closed_form():
    x = np.zeros((3, 64), np.float16)
    x[0, 5] = 1.0
    x[1, 5] = 2.0
    w = np.zeros(64, np.float32)
    w[5] = np.float32(np.log(3.0))
    g = oracle.shared_gate(x, w)
    assert abs(g[0] - 0.75) < 1e-7        # sigmoid(ln 3) = 3/4
    assert abs(g[1] - 0.9) < 1e-7         # sigmoid(2 ln 3) = 9/10
    assert g[2] == 0.5


# ---------------------------------------------------------------- alignment

def _check_alignment(ids, E):
    al = oracle.align_by_expert(ids, E)
    flat = np.asarray(ids).ravel()
    S = flat.size
    valid = [s for s in range(S) if 0 <= flat[s] < E]
    ref = sorted(valid, key=lambda s: (int(flat[s]), s))
    n = len(ref)
    assert al["sorted_slots"][:n].tolist() == ref
    assert np.all(al["sorted_slots"][n:] == -1)
    bc = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
    assert np.array_equal(al["counts"], bc)
    assert al["offsets"][0] == 0 and al["offsets"][E] == n
    assert np.array_equal(np.diff(al["offsets"]), bc)
    act = np.flatnonzero(bc)
    assert int(al["n_active"]) == act.size
    assert al["active"][:act.size].tolist() == act.tolist()
    assert np.all(al["active"][act.size:] == -1)
    for e in range(E):
        seg = al["sorted_slots"][al["offsets"][e]:al["offsets"][e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
    return al


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("E,k,T", [(8, 2, 17), (64, 6, 17), (60, 4, 9), (16, 2, 1)])
def test_align_matches_sorted(seed, E, k, T):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    _check_alignment(ids, E)


def test_align_edge_cases():
    _check_alignment(np.full((17, 1), 3, np.int32), 8)         # one expert only
    _check_alignment(np.zeros((0, 2), np.int32), 8)            # empty window
    bad = np.array([[0, 9], [-1, 2], [2, 2]], np.int32)          # dropped IDs
    al = _check_alignment(bad, 8)
    assert int(al["offsets"][8]) == 4


def test_expert_demand_single_token_golden():
    g = golden("expert_demand_k1.json")
    cfg = get_config("dsv2")
    assert (cfg.E, cfg.k) == (g["E"], g["top_k"])
    x = make_activations(cfg, seed=0)
    w = make_router(cfg, seed=0)
    for t in range(cfg.T):
        ids = oracle.topk_experts(oracle.router_logits_f32(x[t:t + 1], w), cfg.k)
        al = oracle.align_by_expert(ids, cfg.E)
        assert float(al["n_active"]) == g["experts_per_layer"]


# ---------------------------------------------------------------- INT4

def test_dequant_golden_words():
    g = golden("int4_pack_handworked.json")
    codes = np.array(g["words"], np.uint32).reshape(2, 1)
    scales = np.array(g["scales"], np.float16).reshape(2, 1)
    deq = oracle.dequant_int4(codes, scales, g["group"])
    assert deq.tolist() == g["expected"]


@pytest.mark.parametrize("G", [32, 64, 128])
def test_quantize_dequantize_within_half_step(G):
    rng = np.random.default_rng(G)
    W = (rng.standard_normal((24, 512)) * 0.02).astype(np.float32)
    W[3, :G] = 0.0                       # an all-zero group
    W[5, 7] = 0.5                        # an outlier dominating its group
    codes, s16 = quantize_rtn_int4(W, G)
    deq = oracle.dequant_int4(codes, s16, G)
    step = np.repeat(s16.astype(np.float64), G, axis=1)
    err = np.abs(deq - W.astype(np.float64))
    assert np.all(err <= step / 2 * (1 + 2.0 ** -20) + 1e-30)
    nib = np.stack([(codes >> (4 * j)) & 0xF for j in range(8)], axis=-1).reshape(W.shape)
    zero_group = nib[3, :G]
    assert np.all(zero_group == 8) and s16[3, 0] == 0
    live = np.ones_like(nib, bool)
    live[3, :G] = False
    assert nib[live].min() >= 1 and nib[live].max() <= 15
    # the group maximum maps to +-7 steps
    assert abs(deq[5, 7] - 0.5) <= step[5, 7] / 2
    assert nib[5, 7] == 15


# ---------------------------------------------------------------- expert MLP

def test_swiglu_golden():
    g = golden("swiglu_handworked.json")
    x = np.array(g["x"], np.float16)
    y = oracle.swiglu(x.astype(np.float64), np.array(g["wg"]), np.array(g["wu"]),
                      np.array(g["wd"]), act_fp16=True)
    assert y.tolist() == g["expected_y"]


def test_silu_closed_form():
    # x = [1], Wg = [ln 3] -> g = ln 3, SiLU(g) = (3/4) ln 3; up = 1, down = 1
    x = np.array([[1.0]])
    y = oracle.swiglu(x, np.array([[math.log(3.0)]]), np.array([[1.0]]),
                      np.array([[1.0]]), act_fp16=False)
    assert abs(y[0, 0] - 0.75 * math.log(3.0)) < 1e-15


def _dense_reference(x, wg, wu, wd):
    """Unit-by-unit float64 MLP with explicit sums (independent of the oracle)."""
    m, H = x.shape
    I = wg.shape[0]
    out = np.zeros((m, wd.shape[0]))
    for r in range(m):
        h = np.zeros(I)
        for i in range(I):
            g = math.fsum(x[r, q] * wg[i, q] for q in range(H))
            u = math.fsum(x[r, q] * wu[i, q] for q in range(H))
            h[i] = g / (1.0 + math.exp(-g)) * u
        for n in range(wd.shape[0]):
            out[r, n] = math.fsum(h[i] * wd[n, i] for i in range(I))
    return out


def test_swiglu_matches_unit_by_unit_sums():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((3, 24))
    wg, wu = rng.standard_normal((10, 24)), rng.standard_normal((10, 24))
    wd = rng.standard_normal((24, 10))
    y = oracle.swiglu(x, wg, wu, wd, act_fp16=False)
    assert np.allclose(y, _dense_reference(x, wg, wu, wd), rtol=1e-12, atol=1e-12)


def _tiny_int4_layer(seed=0):
    cfg = get_config("tiny")
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((cfg.T, cfg.H)).astype(np.float16)
    mats = {}
    for e in range(cfg.E):
        wg = (rng.standard_normal((cfg.I, cfg.H)) * 0.02).astype(np.float32)
        wu = (rng.standard_normal((cfg.I, cfg.H)) * 0.02).astype(np.float32)
        wd = (rng.standard_normal((cfg.H, cfg.I)) * 0.02).astype(np.float32)
        mats[e] = tuple(oracle.dequant_int4(*quantize_rtn_int4(m, cfg.G), cfg.G)
                        for m in (wg, wu, wd))
    ids = np.stack([rng.permutation(cfg.E)[:cfg.k] for _ in range(cfg.T)]).astype(np.int32)
    return cfg, x, ids, mats


def test_expertwise_equals_tokenwise():
    cfg, x, ids, mats = _tiny_int4_layer()
    a = oracle.routed_ffn_tokenwise(x, ids, lambda e: mats[e])
    b = oracle.routed_ffn_expertwise(x, ids, lambda e: mats[e])
    assert np.allclose(a, b, rtol=1e-12, atol=1e-15)


def test_dropped_slots_give_zero_rows():
    # a slot routed to no expert (ID -1, dropped by the alignment) receives
    # nothing: its row is zero in both forms, and every other row is the one
    # it would have without the drop (the loader is never asked for -1)
    cfg, x, ids, mats = _tiny_int4_layer(3)
    dropped = ids.copy()
    dropped[[0, 5, 9], [1, 0, 1]] = -1
    asked = []

    def load(e):
        asked.append(e)
        return mats[e]

    for fn in (oracle.routed_ffn_tokenwise, oracle.routed_ffn_expertwise):
        asked.clear()
        out = fn(x, dropped, load)
        full = fn(x, ids, lambda e: mats[e])
        gone = dropped.reshape(-1) < 0
        assert (out[gone] == 0).all() and -1 not in asked
        assert np.array_equal(out[~gone], full[~gone])


def test_routed_single_expert_is_dense_mlp():
    cfg, x, ids, mats = _tiny_int4_layer(1)
    ids1 = np.full((cfg.T, 1), 5, np.int32)
    out = oracle.routed_ffn_tokenwise(x[:3], ids1[:3], lambda e: mats[e], act_fp16=False)
    ref = _dense_reference(x[:3].astype(np.float64), *mats[5])
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- combine

def test_combine_identity_and_linearity():
    rng = np.random.default_rng(8)
    T, k, H = 5, 3, 16
    so = rng.standard_normal((T * k, H))
    y64, _ = oracle.combine(so[::k].copy(), np.ones((T, 1)))
    assert np.array_equal(y64, so[::k])
    w = rng.random((T, k))
    ya, _ = oracle.combine(so, w)
    yb, _ = oracle.combine(so, 2.5 * w)
    assert np.allclose(yb, 2.5 * ya, rtol=1e-14)
    manual = np.stack([sum(w[t, j] * so[t * k + j] for j in range(k)) for t in range(T)])
    assert np.allclose(ya, manual, rtol=1e-14)
    sh = rng.standard_normal((T, H))
    g = rng.random(T)
    yc, y16 = oracle.combine(so, w, sh, g)
    assert np.allclose(yc - ya, g[:, None] * sh, rtol=1e-12, atol=1e-14)
    yd, _ = oracle.combine(so, w, sh, None)
    assert np.allclose(yd - ya, sh, rtol=1e-12, atol=1e-14)
    assert y16.dtype == np.float16


# ---------------------------------------------------------------- ELB

def test_elb_golden():
    g = golden("elb_handworked.json")
    cnt = np.zeros((g["L"], g["E"]), np.int32)
    cnt = oracle.elb_accumulate(cnt, np.array(g["ids"]), 0)
    assert cnt.tolist() == g["expected_counts"]
    ids, vals = oracle.elb_topm(cnt, 3)
    assert ids.tolist() == g["expected_top3_ids"]
    assert vals.tolist() == g["expected_top3_counts"]
    ids4, _ = oracle.elb_topm(cnt, 4)
    assert ids4[0].tolist() == g["expected_top4_ids_layer0"]
    tids, _ = oracle.elb_topm(np.array(g["tie_counts"]), 3)
    assert tids.tolist() == g["tie_expected_top3"]


def test_elb_bincount_and_split_additivity():
    rng = np.random.default_rng(3)
    L, E, T, k = 4, 64, 17, 6
    ids = np.stack([np.stack([rng.permutation(E)[:k] for _ in range(T)])
                    for _ in range(L)]).astype(np.int32)
    whole = oracle.elb_accumulate(np.zeros((L, E), np.int32), ids, 0)
    for l in range(L):
        assert np.array_equal(whole[l], np.bincount(ids[l].ravel(), minlength=E))
        assert whole[l].sum() == T * k
    # token by token, layer by layer, gives the same counter
    step = np.zeros((L, E), np.int32)
    for t in range(T):
        for l in range(L):
            step = oracle.elb_accumulate(step, ids[l:l + 1, t:t + 1], l)
    assert np.array_equal(step, whole)
    # one token touches exactly k experts per layer
    one = oracle.elb_accumulate(np.zeros((L, E), np.int32), ids[:, :1], 0)
    assert np.all((one > 0).sum(axis=1) == k)


@pytest.mark.parametrize("seed", range(4))
def test_elb_topm_brute_force(seed):
    rng = np.random.default_rng(seed)
    L, E, M = 3, 9, 4
    cnt = rng.integers(0, 4, size=(L, E)).astype(np.int32)
    ids, vals = oracle.elb_topm(cnt, M)
    for l in range(L):
        c = cnt[l]
        winners = [set(s) for s in itertools.combinations(range(E), M)
                   if all(c[a] > c[b] or (c[a] == c[b] and a < b)
                          for a in s for b in range(E) if b not in s)]
        assert len(winners) == 1 and set(ids[l].tolist()) == winners[0]
        assert vals[l].tolist() == [int(c[e]) for e in ids[l]]
        for j in range(M - 1):
            a, b = ids[l, j], ids[l, j + 1]
            assert c[a] > c[b] or (c[a] == c[b] and a < b)
