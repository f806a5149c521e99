"""smoe_w4a16_expert_ffn_noalloc (the FFN over the library's static
workspace) against smoe_w4a16_expert_ffn with a caller workspace, through
the C ABI: two calls in a row on the same device, the second with a smaller
window, so that the second runs over what the first left in the shared
array. Needs an MI355X."""

import numpy as np
import pytest
import torch

import oracle
from workload import get_config, make_layer

pytestmark = pytest.mark.gpu

ROW_TOL = 2e-2     # against the oracle (fp16 activations, fp32 accumulation)
SAME_TOL = 1e-3    # against the workspace call: split tiles add fp32 partial
                   # sums with device atomics, so the last bits may differ


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


@pytest.fixture(scope="module")
def dsv2():
    return make_layer(get_config("dsv2"), seed=0)


def _window(L, T):
    """Device inputs of the first T tokens of the layer (oracle routing)."""
    cfg = L.cfg
    x = L.x[:T]
    ids = oracle.topk_experts(oracle.router_logits_f32(x, L.w_router), cfg.k)
    al = oracle.align_by_expert(ids, cfg.E)
    return dict(T=T, x=dev(x), ids=ids, slots=dev(al["sorted_slots"]),
                offsets=dev(al["offsets"]))


def _run(smoe, L, W, w, noalloc):
    cfg = L.cfg
    T, H = W["T"], cfg.H
    slot_out = torch.full((T * cfg.k, H), float("nan"), dtype=torch.float32, device="cuda")
    shared_out = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
    args = (W["x"], cfg.k, cfg.E, cfg.I, cfg.G, w["wg_q"], w["wg_s"], w["wu_q"], w["wu_s"],
            w["wd_q"], w["wd_s"], W["slots"], W["offsets"])
    shared = (w["sg"], w["su"], w["sd"])
    if noalloc:
        smoe.smoe_w4a16_expert_ffn_noalloc(*args, slot_out, shared=shared,
                                           shared_out=shared_out)
    else:
        ws = torch.zeros(smoe.smoe_ffn_workspace_bytes(T, cfg.k, cfg.E, H, cfg.I,
                                                       cfg.shared_I),
                         dtype=torch.uint8, device="cuda")
        smoe.smoe_w4a16_expert_ffn(*args, ws, slot_out, shared=shared, shared_out=shared_out)
    return host(slot_out), host(shared_out)


def test_noalloc_matches_workspace_call_twice(smoe, dsv2):
    L = dsv2
    w = {n: dev(getattr(L, n)) for n in ("wg_q", "wg_s", "wu_q", "wu_s", "wd_q", "wd_s")}
    w.update(sg=dev(L.sg16), su=dev(L.su16), sd=dev(L.sd16))
    windows = [_window(L, 17), _window(L, 5)]       # the second call is smaller
    refs = [_run(smoe, L, W, w, noalloc=False) for W in windows]
    outs = [_run(smoe, L, W, w, noalloc=True) for W in windows]   # back to back
    for W, (ref_so, ref_sh), (so, sh) in zip(windows, refs, outs):
        assert np.isfinite(so).all() and np.isfinite(sh).all(), W["T"]
        assert row_rel_err(so, ref_so) <= SAME_TOL, W["T"]
        assert row_rel_err(sh, ref_sh) <= SAME_TOL, W["T"]
        # and both against the oracle, on the slots of a few experts
        x = L.x[:W["T"]]
        flat = W["ids"].ravel()
        for e in sorted(set(flat.tolist()))[:4]:
            s = np.flatnonzero(flat == e)
            ref = oracle.swiglu(x[s // L.cfg.k].astype(np.float64),
                                oracle.dequant_int4(L.wg_q[e], L.wg_s[e], L.cfg.G),
                                oracle.dequant_int4(L.wu_q[e], L.wu_s[e], L.cfg.G),
                                oracle.dequant_int4(L.wd_q[e], L.wd_s[e], L.cfg.G))
            assert row_rel_err(so[s], ref) <= ROW_TOL, (W["T"], e)
        ref_sh = oracle.shared_ffn(x, L.sg16, L.su16, L.sd16)
        assert row_rel_err(sh, ref_sh) <= ROW_TOL, W["T"]


def test_noalloc_refuses_windows_above_its_workspace(smoe, dsv2):
    # 544 tokens x top-6 need about 98 MB of workspace, above the static 16 MiB
    L = dsv2
    cfg = L.cfg
    T = 544
    x = torch.zeros((T, cfg.H), dtype=torch.float16, device="cuda")
    slots = torch.zeros(T * cfg.k, dtype=torch.int32, device="cuda")
    offsets = torch.zeros(cfg.E + 1, dtype=torch.int32, device="cuda")
    slot_out = torch.zeros((T * cfg.k, cfg.H), dtype=torch.float32, device="cuda")
    w = {n: dev(getattr(L, n)) for n in ("wg_q", "wg_s", "wu_q", "wu_s", "wd_q", "wd_s")}
    with pytest.raises(smoe.SmoeError) as ei:
        smoe.smoe_w4a16_expert_ffn_noalloc(x, cfg.k, cfg.E, cfg.I, cfg.G, w["wg_q"], w["wg_s"],
                                           w["wu_q"], w["wu_s"], w["wd_q"], w["wd_s"], slots,
                                           offsets, slot_out)
    assert ei.value.status == smoe.SMOE_EUNSUPPORTED
    assert "static workspace" in str(ei.value)
    torch.cuda.synchronize()
    assert not slot_out.any()  # nothing was enqueued
