"""GPU tests of the expert cache's verification FFN (smoe_cache_verify_layer):
experts copied from pinned host memory into a device slot pool on a copy
stream, hits computed first and misses as they land, checked against the
CPU oracle (every slot row and the shared experts), against the FFN without
a cache, and decision for decision against the CPU model of the cache."""

import copy

import numpy as np
import pytest
import torch

import oracle
from oracle import offload as O

pytestmark = pytest.mark.gpu

ROW_TOL = 2e-2  # per-row max |gpu - ref| / max |ref| (fp16 h, fp32 sums)


@pytest.fixture(scope="module")
def smoe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from quantized_speculative_expert_amd import _lib
    return _lib


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def row_rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return (num / den).max() if len(num) else 0.0


class Setup:
    def __init__(self, smoe, L, E, k, T, H, I, Is, M, tiled, seed):
        rng = np.random.default_rng(seed)
        self.L, self.E, self.k, self.T, self.H, self.I, self.Is, self.M = L, E, k, T, H, I, Is, M
        self.tiled = tiled
        self.rng = rng
        self.w = [[tuple((rng.standard_normal(sh) * 0.03).astype(np.float16)
                         for sh in ((I, H), (I, H), (H, I))) for _ in range(E)] for _ in range(L)]
        msz = I * H
        self.expert_bytes = 3 * msz * 2
        hostbuf = torch.empty(L * E * 3 * msz, dtype=torch.float16, pin_memory=True)
        for l in range(L):
            for e in range(E):
                for j, w in enumerate(self.w[l][e]):
                    t = torch.from_numpy(np.ascontiguousarray(w))
                    if tiled:  # each matrix tiled on the device, then back to the host store
                        td = t.cuda()
                        tt = torch.empty_like(td)
                        smoe.smoe_tile_weights(td, None, 1, w.shape[0], w.shape[1], 0, tt)
                        t = tt.cpu()
                    o = ((l * E + e) * 3 + j) * msz
                    hostbuf[o:o + msz] = t.reshape(-1)
        self.hostbuf = hostbuf
        self.pool = torch.zeros(L * M * 3 * msz, dtype=torch.float16, device="cuda")
        self.cache = smoe.smoe_cache_create(L, E, M, self.expert_bytes, self.pool, hostbuf)
        self.model = O.CacheModel(L, M)
        self.copy_stream = torch.cuda.Stream()
        dev = dict(dtype=torch.uint8, device="cuda")
        self.ws_routed = torch.zeros(smoe.smoe_ffn_workspace_bytes(T, k, E, H, I, 0), **dev)
        self.ws_shared = (torch.zeros(smoe.smoe_ffn_workspace_bytes(T, k, E, H, I, Is), **dev)
                          if Is else None)
        if Is:
            self.shared_np = tuple((rng.standard_normal(sh) * 0.03).astype(np.float16)
                                   for sh in ((Is, H), (Is, H), (H, Is)))
            self.shared = []
            for w in self.shared_np:
                t = torch.from_numpy(np.ascontiguousarray(w)).cuda()
                if tiled:
                    tt = torch.empty_like(t)
                    smoe.smoe_tile_weights(t, None, 1, w.shape[0], w.shape[1], 0, tt)
                    t = tt
                self.shared.append(t)

    def warm(self, smoe, slot_expert, last_use, clock):
        smoe.smoe_cache_set_state(self.cache, slot_expert, last_use, clock,
                                  copy_stream=self.copy_stream)
        self.model.slot_expert = [list(map(int, r)) for r in slot_expert]
        self.model.last_use = [list(map(int, r)) for r in last_use]
        self.model.clock = clock

    def verify(self, smoe, l, ids):
        T, k, E, H = self.T, self.k, self.E, self.H
        x = self.rng.standard_normal((T, H)).astype(np.float16)
        al = oracle.align_by_expert(ids, E)
        counts = np.bincount(ids[ids >= 0].reshape(-1), minlength=E).astype(np.int32)
        slot_out = torch.full((T * k, H), float("nan"), dtype=torch.float32, device="cuda")
        shared_out = (torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
                      if self.Is else None)
        xs = torch.from_numpy(x).cuda()
        sched = smoe.smoe_cache_verify_layer(
            self.cache, l, counts, xs, k, self.I, torch.from_numpy(al["sorted_slots"]).cuda(),
            torch.from_numpy(al["offsets"]).cuda(), self.ws_shared, self.ws_routed, slot_out,
            shared=tuple(self.shared) if self.Is else None, shared_out=shared_out,
            tiled=self.tiled, copy_stream=self.copy_stream)
        want = self.model.verify(l, [int(c) for c in counts])
        assert [tuple(r) for r in sched.tolist()] == want
        se, lu, _, clock = smoe.smoe_cache_state(self.cache, self.L, self.M)
        assert se.tolist() == self.model.slot_expert and clock == self.model.clock
        ref = oracle.routed_ffn_expertwise(x, ids, lambda e: self.w[l][e])
        got = host(slot_out)
        kept = (ids.reshape(-1) >= 0)
        assert np.isfinite(got[kept]).all()
        assert row_rel_err(got[kept], ref[kept]) <= ROW_TOL
        if self.Is:
            ref_s = oracle.shared_ffn(x, *self.shared_np)
            assert row_rel_err(host(shared_out), ref_s) <= ROW_TOL
        return x, al, got, sched

    def close(self, smoe):
        torch.cuda.synchronize()
        smoe.smoe_cache_destroy(self.cache)


def routed_ids(rng, T, k, E, hot=None):
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    p /= p.sum()
    perm = rng.permutation(E) if hot is None else hot
    return np.stack([perm[rng.choice(E, k, replace=False, p=p)] for _ in range(T)]).astype(
        np.int32)


@pytest.mark.parametrize("tiled", [False, True], ids=["rows", "tiled"])
@pytest.mark.parametrize("Is", [0, 256], ids=["routed", "shared"])
def test_verify_layer_hits_misses_and_reuse(smoe, tiled, Is):
    # 2 layers, 8 experts, 3 slots each: windows that need up to 8 experts
    # with 3 slots, so misses wait for slots released by earlier computations
    s = Setup(smoe, L=2, E=8, k=2, T=17, H=256, I=384, Is=Is, M=3, tiled=tiled, seed=11)
    s.warm(smoe, np.array([[5, -1, 2], [0, 1, 7]], np.int32),
           np.array([[3, 0, 4], [1, 2, 3]], np.int64), 4)
    waits = 0
    for rnd in range(6):
        l = rnd % 2
        ids = routed_ids(s.rng, s.T, s.k, s.E)
        _, _, _, sched = s.verify(smoe, l, ids)
        waits += int((sched[:, 4] >= 0).sum())
    assert waits > 0  # some misses really waited for a released slot
    s.close(smoe)


def test_verify_layer_equals_uncached_ffn(smoe):
    # the same window through the cache and through smoe_fp16_expert_ffn over
    # all experts at their own index
    s = Setup(smoe, L=1, E=8, k=2, T=17, H=256, I=256, Is=0, M=4, tiled=False, seed=5)
    ids = routed_ids(s.rng, s.T, s.k, s.E)
    x, al, got, _ = s.verify(smoe, 0, ids)
    wg = torch.from_numpy(np.stack([w[0] for w in s.w[0]])).cuda()
    wu = torch.from_numpy(np.stack([w[1] for w in s.w[0]])).cuda()
    wd = torch.from_numpy(np.stack([w[2] for w in s.w[0]])).cuda()
    ws = torch.zeros(smoe.smoe_ffn_workspace_bytes(s.T, s.k, s.E, s.H, s.I, 0),
                     dtype=torch.uint8, device="cuda")
    out = torch.zeros((s.T * s.k, s.H), dtype=torch.float32, device="cuda")
    smoe.smoe_fp16_expert_ffn(torch.from_numpy(x).cuda(), s.k, s.E, s.I, wg, wu, wd,
                              torch.from_numpy(al["sorted_slots"]).cuda(),
                              torch.from_numpy(al["offsets"]).cuda(), ws, out)
    assert row_rel_err(got, host(out)) <= 1e-3
    s.close(smoe)


def test_prefetch_then_verify_all_hits(smoe):
    # a top-M plan prefetched into the pool (copies on the copy stream); the
    # verification of a window routed to those experts is all hits
    s = Setup(smoe, L=2, E=8, k=2, T=9, H=256, I=256, Is=0, M=4, tiled=True, seed=3)
    plan_ids = np.array([[6, 1, 3, 0], [2, 4, 5, 7]], np.int32)
    plan_counts = np.array([[5, 4, 2, 1], [3, 3, 1, 1]], np.int32)
    smoe.smoe_cache_begin_window(s.cache)
    s.model.begin_window()
    loads, full = smoe.smoe_cache_prefetch(s.cache, plan_ids, plan_counts, 2, 4,
                                           copy_stream=s.copy_stream)
    want = []
    for l in range(2):
        want += s.model.prefetch(l, list(zip(plan_ids[l].tolist(), plan_counts[l].tolist())))
    assert [tuple(r) for r in loads.tolist()] == want and full
    for l in range(2):
        hot = np.concatenate([plan_ids[l], np.setdiff1d(np.arange(8), plan_ids[l])])
        ids = np.stack([s.rng.permutation(plan_ids[l])[:2] for _ in range(s.T)]).astype(np.int32)
        _, _, _, sched = s.verify(smoe, l, ids)
        assert (sched[:, 2] == O.HIT).all()
    s.close(smoe)


# ------------------------------------------------------------------ whole window

def test_speculative_window_with_prefetch_and_cached_verification(smoe):
    # 3 layers, 16 experts, top-2, a K=8 window, 6 slots per layer: the
    # draft's routing drives the prefetch exactly as the model's planner
    # decides; verification decisions equal the model's; y of every layer
    # equals the oracle's composition on the device's routing
    import dataclasses
    from quantized_speculative_expert_amd.offload import OffloadStack
    from workload import make_layer, make_router
    from workload.configs import MoEConfig
    from workload.gen import zipf_bias
    cfg = MoEConfig(name="offload-test", E=16, k=2, H=256, I=256, G=128, T=9, shared_I=256,
                    elb_M=6)
    L, M, K = 3, 6, cfg.T - 1
    draft_inp = make_layer(dataclasses.replace(cfg, T=1), seed=4, layer=0)
    zipf = [zipf_bias(cfg.E, 1.0, 4, l).astype(np.float32) for l in range(L)]
    routers = [make_router(cfg, 4, l) for l in range(L)]
    st = OffloadStack(cfg, draft_inp, L, M, zipf=zipf, routers=routers, seed=4, tiled=False)
    model = O.CacheModel(L, M)
    rng = np.random.default_rng(4)
    bw, us = 20.0, 150.0
    for w in range(3):
        xd = (rng.standard_normal((L, K, cfg.H)) * 1.0).astype(np.float16)
        xt = np.concatenate([xd + (0.05 * rng.standard_normal(xd.shape)).astype(np.float16),
                             rng.standard_normal((L, 1, cfg.H)).astype(np.float16)], axis=1)
        rec = torch.empty((K, L, cfg.k), dtype=torch.int32, device="cuda")
        out = st.draft_window(torch.from_numpy(xd).cuda(), True, 2, bw, us, record=rec)
        routing = host(rec)
        want = O.plan_window(routing, cfg.E, model, 2, st.expert_bytes, bw, us)
        assert out["chunks"] == want["chunks"]
        assert [(b, [tuple(x) for x in ld.tolist()]) for b, ld in out["loads"]] == \
            want["boundaries"]
        xt_dev = torch.from_numpy(np.ascontiguousarray(xt)).cuda()
        for l in range(L):
            sched = st.verify_layer(l, xt_dev[l])
            counts = host(st.t_counts)
            assert [tuple(r) for r in sched.tolist()] == model.verify(l, [int(c) for c in counts])
            ids, wts = host(st.t_ids), host(st.t_w)
            hw = st.host[l].numpy()
            load = lambda e: (hw[e, 0].reshape(cfg.I, cfg.H), hw[e, 1].reshape(cfg.I, cfg.H),
                              hw[e, 2].reshape(cfg.H, cfg.I))
            slot_ref = oracle.routed_ffn_expertwise(xt[l], ids, load)
            sh = tuple(draft_inp.__getattribute__(n) for n in ("sg16", "su16", "sd16"))
            y_ref = oracle.combine(slot_ref, wts, oracle.shared_ffn(xt[l], *sh))[0]
            assert row_rel_err(host(st.y[l]), y_ref) <= ROW_TOL
    st.close()
