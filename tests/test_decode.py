"""GPU parity of the single-token draft layer: smoe_moe_layer_w4a16_tiled
with one token runs the router, top-k, alignment, ELB update, routed and
shared experts and the combine in two launches of its own. Every output of
the call is checked against the oracle (integers and logits bit for bit,
floats within the layer tolerance), against the step-by-step calls on the
same runner, and over repeated calls on one workspace (the words the
call's workgroups hand values over with must be back at zero after each
call). Needs an MI355X."""

import numpy as np
import pytest
import torch

import oracle
from workload import get_config, make_layer
from workload.configs import MoEConfig

pytestmark = pytest.mark.gpu

ROW_TOL = 2e-2   # per-row relative error of layer outputs (as the other layer tests)
W_RTOL = 2e-5    # routing weights: float32 softmax against float64

# single-token shapes: the DeepSeek-V2-Lite draft step, and synthetic ones
# that vary the group size, the shared expert and its gate, the router skew,
# E up to 256 and k up to 8
_CASES = {
    "dsv2_t1": get_config("dsv2_t1"),
    "g64_noshared": MoEConfig(name="g64_noshared", E=8, k=2, H=256, I=512, G=64, T=1),
    "g32_gate_skew": MoEConfig(name="g32_gate_skew", E=16, k=4, H=512, I=256, G=32, T=1,
                               shared_I=256, shared_gate=True, zipf_s=1.1, elb_M=4),
    "e256_k8": MoEConfig(name="e256_k8", E=256, k=8, H=1024, I=128, G=128, T=1,
                         shared_I=384, elb_M=16),
    "qwen_t1": MoEConfig(name="qwen_t1", E=60, k=4, H=2048, I=1408, G=128, T=1,
                         shared_I=5632, shared_gate=True),
}
_INPUTS = {}


@pytest.fixture(scope="module")
def smoe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from quantized_speculative_expert_amd import _lib  # fails loudly if not built
    return _lib


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def row_rel_err(got, ref):
    got = np.asarray(got, np.float64).reshape(len(got), -1)
    ref = np.asarray(ref, np.float64).reshape(len(ref), -1)
    num = np.abs(got - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return (num / den).max() if len(num) else 0.0


def case(name):
    if name not in _INPUTS:
        L = make_layer(_CASES[name], seed=3)
        _INPUTS[name] = (L, oracle.moe_layer(L, "draft"))
    return _INPUTS[name]


def outputs(d):
    out = {"logits": host(d.logits), "ids": host(d.topk_ids), "w": host(d.topk_w),
           "counts": host(d.counts), "offsets": host(d.offsets),
           "sorted_slots": host(d.sorted_slots), "n_active": host(d.n_active),
           "active": host(d.active),
           "slot_out": host(d.slot_out), "y": host(d.y),
           "elb_counts": host(d.elb_counts), "plan_ids": host(d.plan_ids),
           "plan_counts": host(d.plan_counts)}
    if d.shared_out is not None:
        out["shared_out"] = host(d.shared_out)
    if d.shared_gate is not None:
        out["gate"] = host(d.shared_gate)
    return out


def check_against_oracle(got, L, ref):
    cfg = L.cfg
    assert np.array_equal(got["logits"], ref["logits"])
    assert np.array_equal(got["ids"], ref["ids"])
    np.testing.assert_allclose(got["w"], ref["w"], rtol=W_RTOL, atol=1e-7)
    for key in ("counts", "offsets", "sorted_slots", "active"):
        assert np.array_equal(got[key], ref[key]), key
    assert int(got["n_active"][0]) == int(ref["n_active"])
    assert row_rel_err(got["slot_out"], ref["slot_out"]) <= ROW_TOL
    assert np.isfinite(got["y"]).all()
    assert row_rel_err(got["y"], ref["y64"]) <= ROW_TOL
    if cfg.shared_I:
        assert row_rel_err(got["shared_out"], ref["shared_out"]) <= ROW_TOL
    if cfg.shared_gate:
        np.testing.assert_allclose(got["gate"], ref["gate"], rtol=1e-5, atol=1e-7)


@pytest.mark.parametrize("name", list(_CASES))
def test_decode_layer_matches_oracle(smoe, name):
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L, ref = case(name)
    d = DeviceLayer(L, tiled=True, with_target=False)
    d.run(one_call=True)
    got = outputs(d)
    check_against_oracle(got, L, ref)
    if L.cfg.elb_M:
        cnt = oracle.elb_accumulate(np.zeros((1, L.cfg.E), np.int32), ref["ids"][None], 0)
        pid, pc = oracle.elb_topm(cnt, L.cfg.elb_M)
        assert np.array_equal(got["elb_counts"], cnt)
        assert np.array_equal(got["plan_ids"], pid) and np.array_equal(got["plan_counts"], pc)


@pytest.mark.parametrize("name", ["dsv2_t1", "g32_gate_skew"])
def test_decode_layer_equals_step_calls(smoe, name):
    # the same runner through the separate calls (route + align + ELB, the
    # split-K FFN, the combine): integer results and logits identical, the
    # floats within the tolerance of each other
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L, _ = case(name)
    d = DeviceLayer(L, tiled=True, with_target=False)
    d.run(one_call=True)
    a = outputs(d)
    d.elb_counts.zero_()
    d.run()
    b = outputs(d)
    for key in ("logits", "ids", "counts", "offsets", "sorted_slots", "active", "n_active",
                "elb_counts", "plan_ids", "plan_counts"):
        assert np.array_equal(a[key], b[key]), key
    np.testing.assert_allclose(a["w"], b["w"], rtol=1e-6, atol=0)
    assert row_rel_err(a["slot_out"], b["slot_out"]) <= ROW_TOL
    assert row_rel_err(a["y"], b["y"].astype(np.float64)) <= ROW_TOL


def test_decode_layer_repeats_bit_for_bit(smoe):
    # calls in a row on one workspace, eagerly and replayed from a HIP graph,
    # with the step-by-step calls in between: every call finds its hand-over
    # words at zero, and the sums have a fixed order, so every output is the
    # same bit for bit
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L, ref = case("dsv2_t1")
    d = DeviceLayer(L, tiled=True, with_target=False)

    def once():
        d.elb_counts.zero_()
        d.y.fill_(float("nan"))
        d.slot_out.fill_(float("nan"))
        d.run(one_call=True)
        return outputs(d)

    first = once()
    check_against_oracle(first, L, ref)
    for i in range(4):
        again = once()
        for key in first:
            assert np.array_equal(first[key], again[key], equal_nan=False), (i, key)
    d.run()  # the split-K FFN on the same workspace
    torch.cuda.synchronize()
    again = once()
    for key in first:
        assert np.array_equal(first[key], again[key]), key
    # graph replays (the counter reset is a kernel, not a memset)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        d.run(one_call=True)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            d.run(one_call=True)
    torch.cuda.current_stream().wait_stream(s)
    for i in range(5):
        d.y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(d.y), first["y"]), i
        assert np.array_equal(host(d.slot_out), first["slot_out"]), i


def test_decode_layer_rows_layout_takes_step_calls(smoe):
    # row-major weights keep the step-by-step path at T = 1 (the single-token
    # layer reads the tiled layout only); both agree with the oracle
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L, ref = case("g64_noshared")
    d = DeviceLayer(L, tiled=False, with_target=False)
    d.run(one_call=True)
    check_against_oracle(outputs(d), L, ref)


@pytest.mark.parametrize("flags,elb_flags", [(0, 0), (1, 1)], ids=["plain", "renorm-clear"])
def test_decode_layer_routing_outputs_multi_layer(smoe, flags, elb_flags):
    # The one-call layer at T = 1 with the routing flags, a three-layer
    # activation counter (this call's layer 1, random prior counts) and the
    # clear flag: every routing output, the counter and every layer's plan
    # equal those of smoe_route_align_elb from the same state, bit for bit
    # (weights within float32 rounding of the same formula)
    from quantized_speculative_expert_amd.layer import DeviceLayer
    L, _ = case("g32_gate_skew")
    d = DeviceLayer(L, tiled=True, with_target=False)
    cfg = L.cfg
    M = 4
    rng = np.random.default_rng(11)
    prior = torch.from_numpy(rng.integers(0, 3, (3, cfg.E)).astype(np.int32)).cuda()

    def bufs():
        return {"ids": torch.empty((1, cfg.k), dtype=torch.int32, device="cuda"),
                "w": torch.empty((1, cfg.k), dtype=torch.float32, device="cuda"),
                "lg": torch.empty((1, cfg.E), dtype=torch.float32, device="cuda"),
                "gate": torch.empty(1, dtype=torch.float32, device="cuda"),
                "counts": torch.empty(cfg.E, dtype=torch.int32, device="cuda"),
                "offsets": torch.empty(cfg.E + 1, dtype=torch.int32, device="cuda"),
                "sorted": torch.empty(cfg.k, dtype=torch.int32, device="cuda"),
                "active": torch.empty(cfg.E, dtype=torch.int32, device="cuda"),
                "nact": torch.empty(1, dtype=torch.int32, device="cuda"),
                "elb": prior.clone(),
                "pid": torch.full((3, M), -7, dtype=torch.int32, device="cuda"),
                "pc": torch.full((3, M), -7, dtype=torch.int32, device="cuda")}

    a, b = bufs(), bufs()
    d._call("smoe_moe_layer_w4a16")(
        d.x, d.w_router, d.router_bias, cfg.k, flags, a["ids"], a["w"], a["lg"],
        d.shared_gate_w, a["gate"], a["counts"], a["offsets"], a["sorted"], a["active"],
        a["nact"], a["elb"], 1, M, a["pid"], a["pc"], elb_flags, cfg.I, cfg.G, d.wg_q, d.wg_s,
        d.wu_q, d.wu_s, d.wd_q, d.wd_s, d.workspace, d.slot_out, d.y,
        shared=(d.sg16, d.su16, d.sd16), shared_out=d.shared_out)
    smoe.smoe_route_align_elb(d.x, d.w_router, d.router_bias, cfg.k, flags, b["ids"], b["w"],
                              b["lg"], d.shared_gate_w, b["gate"], b["counts"], b["offsets"],
                              b["sorted"], b["active"], b["nact"], elb_counts=b["elb"], layer=1,
                              M=M, plan_ids=b["pid"], plan_counts=b["pc"], elb_flags=elb_flags)
    for key in a:
        if key == "w":
            np.testing.assert_allclose(host(a[key]), host(b[key]), rtol=1e-6, atol=0)
        else:
            assert np.array_equal(host(a[key]), host(b[key])), key
    if elb_flags:
        assert not host(a["elb"]).any()
