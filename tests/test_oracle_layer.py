"""Pins of the oracle's whole-layer composition (oracle.moe_layer and
oracle.shared_ffn) on the CPU.

The per-step functions are pinned in test_oracle.py. Here the wiring between
them is pinned two ways, neither of which calls moe_layer to produce the
expected values:
  * a layer worked by hand (tests/golden/layer_handworked.json): router bias,
    top-1 of 2 experts, softmax weight, INT4 draft and different FP16 target
    experts, a gated FP16 shared expert, fp16 combine;
  * a token-by-token composition of the pinned pieces on random layers with
    every option switched on (bias, shared experts, gate, both passes).
A last test plants each plausible wiring mistake in the oracle and checks
that one of these pins catches it.
"""

import json
import os

import numpy as np
import pytest

import oracle
import oracle.moe as oracle_moe
from workload import make_layer
from workload.configs import MoEConfig
from workload.gen import LayerInputs, pack_int4_codes

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "layer_handworked.json")) as f:
        return json.load(f)


def _dense(shape, entries, dtype):
    a = np.zeros(shape, dtype)
    for ent in entries:
        a[tuple(int(i) for i in ent[:-1])] = ent[-1]
    return a


def _int4(shape, entries, G):
    """INT4 codes and unit scales for the listed integer values (code = v + 8)."""
    E, N, K = shape
    v = _dense(shape, entries, np.int64)
    assert np.all(np.abs(v) <= 7)
    codes = np.stack([pack_int4_codes((v[e] + 8).astype(np.uint8)) for e in range(E)])
    scales = np.ones((E, N, K // G), np.float16)
    return codes, scales


def golden_layer():
    """LayerInputs of the hand-worked layer."""
    g = _golden()
    s = g["shape"]
    E, H, I, G, T, Is = s["E"], s["H"], s["I"], s["G"], s["T"], s["shared_I"]
    cfg = MoEConfig(name="golden", E=E, k=s["k"], H=H, I=I, G=G, T=T, shared_I=Is,
                    shared_gate=True, target_fp16=True)
    wg_q, wg_s = _int4((E, I, H), g["draft"]["wg"], G)
    wu_q, wu_s = _int4((E, I, H), g["draft"]["wu"], G)
    wd_q, wd_s = _int4((E, H, I), g["draft"]["wd"], G)
    gw = np.zeros(H, np.float32)
    for h, v in g["shared_gate_w"]:
        gw[int(h)] = v
    return LayerInputs(
        cfg=cfg, seed=0, layer=0,
        x=_dense((T, H), g["x"], np.float16),
        w_router=_dense((E, H), g["w_router"], np.float32),
        router_bias=np.array(g["router_bias"], np.float32),
        shared_gate_w=gw,
        wg_q=wg_q, wg_s=wg_s, wu_q=wu_q, wu_s=wu_s, wd_q=wd_q, wd_s=wd_s,
        wg16=_dense((E, I, H), g["target"]["wg"], np.float16),
        wu16=_dense((E, I, H), g["target"]["wu"], np.float16),
        wd16=_dense((E, H, I), g["target"]["wd"], np.float16),
        sg16=_dense((Is, H), g["shared"]["sg"], np.float16),
        su16=_dense((Is, H), g["shared"]["su"], np.float16),
        sd16=_dense((H, Is), g["shared"]["sd"], np.float16))


def check_golden_layer(moe_layer=None):
    """Assert that moe_layer gives the hand-worked results in both passes."""
    moe_layer = moe_layer or oracle.moe_layer
    g = _golden()
    exp = g["expected"]
    L = golden_layer()
    for pass_ in ("draft", "target"):
        r = moe_layer(L, pass_)
        e = exp[pass_]
        assert r["ids"].tolist() == exp["ids"], pass_
        np.testing.assert_allclose(r["w"], exp["w"], rtol=1e-15, atol=0)
        np.testing.assert_allclose(r["gate"], exp["gate"], rtol=1e-15, atol=0)
        assert r["shared_out"][:, :3].tolist() == exp["shared_out_head"]
        assert r["slot_out"][:, :3].tolist() == e["slot_out_head"], pass_
        np.testing.assert_allclose(r["y64"][:, :3], e["y64_head"], rtol=1e-14, atol=1e-14)
        assert r["y"][:, :3].astype(np.float64).tolist() == e["y16_head"], pass_
        for key in ("slot_out", "shared_out", "y64"):
            assert not np.any(r[key][:, 3:]), key


def test_moe_layer_golden():
    check_golden_layer()


def test_shared_ffn_golden_argument_order():
    L = golden_layer()
    out = oracle.shared_ffn(L.x, L.sg16, L.su16, L.sd16)
    assert out[:, :3].tolist() == _golden()["expected"]["shared_out_head"]
    # gate and up play different roles: swapping them changes the result
    swapped = oracle.shared_ffn(L.x, L.su16, L.sg16, L.sd16)
    assert swapped[0, 0] == float(np.float16(0.5 / (1.0 + np.exp(-0.5)) * 20.0))


# ------------------------------------------------------------ hand composition

def _random_layer(seed, H=128, I=128, E=6, k=2, T=5, G=64, shared_I=128):
    """A small layer with every option on: router bias, gated shared
    experts, INT4 draft and FP16 target experts (seeded generator)."""
    cfg = MoEConfig(name="compose", E=E, k=k, H=H, I=I, G=G, T=T, shared_I=shared_I,
                    shared_gate=True, zipf_s=1.1, target_fp16=True)
    return make_layer(cfg, seed=seed)


def compose_by_token(L, pass_):
    """The layer token by token from the pinned pieces (no moe_layer)."""
    cfg = L.cfg
    lg = oracle.router_logits_f32(L.x, L.w_router, L.router_bias)
    y = np.zeros((cfg.T, cfg.H))
    slot_out = np.zeros((cfg.T * cfg.k, cfg.H))
    for t in range(cfg.T):
        ids = oracle.topk_experts(lg[t:t + 1], cfg.k)[0]
        p = np.exp(lg[t].astype(np.float64) - lg[t].max())
        p /= p.sum()
        xt = L.x[t:t + 1].astype(np.float64)
        for j, e in enumerate(ids):
            if pass_ == "draft":
                mats = (oracle.dequant_int4(L.wg_q[e], L.wg_s[e], cfg.G),
                        oracle.dequant_int4(L.wu_q[e], L.wu_s[e], cfg.G),
                        oracle.dequant_int4(L.wd_q[e], L.wd_s[e], cfg.G))
            else:
                mats = (L.wg16[e], L.wu16[e], L.wd16[e])
            so = oracle.swiglu(xt, *mats)[0]
            slot_out[t * cfg.k + j] = so
            y[t] += p[e] * so
        sh = oracle.swiglu(xt, L.sg16, L.su16, L.sd16)[0]
        gate = 1.0 / (1.0 + np.exp(-float(xt[0] @ L.shared_gate_w.astype(np.float64))))
        y[t] += gate * sh
    return slot_out, y


def check_composition(L, moe_layer=None):
    moe_layer = moe_layer or oracle.moe_layer
    for pass_ in ("draft", "target"):
        r = moe_layer(L, pass_)
        slot_out, y = compose_by_token(L, pass_)
        np.testing.assert_allclose(r["slot_out"], slot_out, rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(r["y64"], y, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_moe_layer_equals_token_by_token_composition(seed):
    check_composition(_random_layer(seed))


def test_moe_layer_passes_differ():
    # the target pass really reads the FP16 weights: its outputs differ from
    # the INT4 draft by about the quantisation error, not by zero
    L = _random_layer(0)
    d, t = oracle.moe_layer(L, "draft"), oracle.moe_layer(L, "target")
    assert np.array_equal(d["ids"], t["ids"])
    rel = np.abs(d["y64"] - t["y64"]).max() / np.abs(t["y64"]).max()
    assert 1e-4 < rel < 0.2


# ------------------------------------------------------------ planted mistakes

def _plant(monkeypatch, name, fn):
    monkeypatch.setattr(oracle_moe, name, fn)


_MISTAKES = ["swapped_shared_gate_up", "dropped_gate", "renorm_on", "target_loads_int4",
             "dropped_bias", "shared_term_dropped"]


@pytest.mark.parametrize("mistake", _MISTAKES)
def test_planted_mistake_fails_a_pin(monkeypatch, mistake):
    """Each wiring mistake, planted in the oracle on the CPU, fails the
    hand-worked golden and the token-by-token composition."""
    layer_fn = oracle_moe.moe_layer
    orig = {n: getattr(oracle_moe, n) for n in
            ("shared_ffn", "shared_gate", "routing_weights", "router_logits_f32", "combine")}
    if mistake == "swapped_shared_gate_up":
        _plant(monkeypatch, "shared_ffn",
               lambda x, sg, su, sd, act_fp16=True: orig["shared_ffn"](x, su, sg, sd, act_fp16))
    elif mistake == "dropped_gate":
        _plant(monkeypatch, "shared_gate", lambda x, w: np.ones(len(x)))
    elif mistake == "renorm_on":
        _plant(monkeypatch, "routing_weights",
               lambda lg, ids, renorm=False: orig["routing_weights"](lg, ids, renorm=True))
    elif mistake == "target_loads_int4":
        def layer_fn(inp, pass_="draft", **kw):
            return oracle_moe.moe_layer(inp, "draft", **kw)
    elif mistake == "dropped_bias":
        _plant(monkeypatch, "router_logits_f32",
               lambda x, w, bias=None: orig["router_logits_f32"](x, w, None))
    elif mistake == "shared_term_dropped":
        _plant(monkeypatch, "combine",
               lambda so, w, sh=None, g=None: orig["combine"](so, w, None, None))
    with pytest.raises(AssertionError):
        check_golden_layer(layer_fn)
    with pytest.raises(AssertionError):
        check_composition(_random_layer(0), layer_fn)
