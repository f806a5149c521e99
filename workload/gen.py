"""Seeded synthetic layer inputs and offline INT4 weight preparation.

Every array is drawn from its own counter-keyed PCG64 stream,
``numpy.random.default_rng([seed, layer, kind, index])``, so any one expert
can be regenerated on its own (the CPU reference only needs the experts a
window touches) and the draw order of one tensor never shifts another.

Value distributions: activations N(0, 1) rounded to fp16; router, gate and
expert weights N(0, 0.02) in fp32; routed experts are then quantised to
symmetric INT4 with fp16 group scales, FP16 weights (shared experts, the
target pass) are the fp16 rounding of the same fp32 draws.

Packed INT4 format (canonical, read by both the reference and the kernels):
for a weight matrix W[N][K], codes are uint32 [N][K/8]; word w of row n
holds the codes for k = 8w .. 8w+7 with the code for k = 8w+j in bits
4j .. 4j+3; scales are fp16 [N][K/G], one per G consecutive k of a row.
A stored code c stands for the integer c - 8 in [-7, 7].
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

from .configs import MoEConfig

WEIGHT_STD = np.float32(0.02)

# Stream keys: default_rng([seed, layer, KIND, index]).
_KIND_X = 0
_KIND_ROUTER = 1
_KIND_EXPERT = 2
_KIND_SHARED = 3
_KIND_SHARED_GATE = 4
_KIND_ZIPF = 5


def _rng(seed: int, layer: int, kind: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(layer), int(kind), int(index)])


def pack_int4_codes(codes: np.ndarray) -> np.ndarray:
    """Pack unsigned 4-bit codes [N][K] (values 0..15) into uint32 [N][K/8]."""
    codes = np.asarray(codes)
    n, k = codes.shape
    if k % 8:
        raise ValueError("K must be a multiple of 8")
    c = codes.astype(np.uint32).reshape(n, k // 8, 8)
    out = np.zeros((n, k // 8), dtype=np.uint32)
    for j in range(8):
        out |= c[:, :, j] << np.uint32(4 * j)
    return out


def quantize_rtn_int4(w: np.ndarray, group: int):
    """Round-to-nearest symmetric INT4 with fp16 per-group scales.

    For each row and each run of `group` consecutive reduction-dim entries:
    scale = fp16(max|w| / 7), q = clip(rint(w / scale), -7, 7) (ties to
    even), code = q + 8; an all-zero group gets scale 0 and code 8.
    Returns (codes uint32 [N][K/8], scales float16 [N][K/group]).
    This is the offline preparation step that GPTQ performs in the Specter
    paper's setup (symmetric INT4, group 128); GPTQ's calibration-driven
    error compensation needs trained weights and data, so plain rounding
    stands in for it.
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % group:
        raise ValueError("K must be a multiple of the group size")
    wg = w.reshape(n, k // group, group)
    amax = np.max(np.abs(wg), axis=2)
    s16 = (amax / np.float32(7.0)).astype(np.float16)
    s32 = s16.astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(wg / s32[:, :, None])
    q = np.where(s32[:, :, None] == 0, 0, q)
    q = np.clip(q, -7, 7).astype(np.int8)
    codes = (q + 8).astype(np.uint8).reshape(n, k)
    return pack_int4_codes(codes), s16


def zipf_bias(E: int, s: float, seed: int, layer: int) -> np.ndarray:
    """Per-expert log-prior -s*ln(r_e) for a seeded random rank permutation r.

    Adding it to router logits makes the prior routing probability of the
    expert of rank r proportional to r**-s (a Zipf(s) skew).
    """
    ranks = _rng(seed, layer, _KIND_ZIPF).permutation(E) + 1
    return (-float(s) * np.log(ranks.astype(np.float64))).astype(np.float32)


@dataclass
class ExpertWeights:
    """One routed expert: INT4 draft weights and optional FP16 target weights."""
    wg_q: np.ndarray        # uint32 [I][H/8]
    wg_s: np.ndarray        # float16 [I][H/G]
    wu_q: np.ndarray
    wu_s: np.ndarray
    wd_q: np.ndarray        # uint32 [H][I/8]
    wd_s: np.ndarray        # float16 [H][I/G]
    wg16: Optional[np.ndarray] = None   # float16 [I][H]
    wu16: Optional[np.ndarray] = None
    wd16: Optional[np.ndarray] = None   # float16 [H][I]


def make_expert(cfg: MoEConfig, e: int, seed: int = 0, layer: int = 0,
                want_fp16: Optional[bool] = None) -> ExpertWeights:
    """Generate and quantise routed expert `e` of one layer."""
    if want_fp16 is None:
        want_fp16 = cfg.target_fp16
    rng = _rng(seed, layer, _KIND_EXPERT, e)
    wg = rng.standard_normal((cfg.I, cfg.H), dtype=np.float32) * WEIGHT_STD
    wu = rng.standard_normal((cfg.I, cfg.H), dtype=np.float32) * WEIGHT_STD
    wd = rng.standard_normal((cfg.H, cfg.I), dtype=np.float32) * WEIGHT_STD
    wg_q, wg_s = quantize_rtn_int4(wg, cfg.G)
    wu_q, wu_s = quantize_rtn_int4(wu, cfg.G)
    wd_q, wd_s = quantize_rtn_int4(wd, cfg.G)
    out = ExpertWeights(wg_q, wg_s, wu_q, wu_s, wd_q, wd_s)
    if want_fp16:
        out.wg16 = wg.astype(np.float16)
        out.wu16 = wu.astype(np.float16)
        out.wd16 = wd.astype(np.float16)
    return out


@dataclass
class LayerInputs:
    cfg: MoEConfig
    seed: int
    layer: int
    x: np.ndarray                           # float16 [T][H]
    w_router: np.ndarray                    # float32 [E][H]
    router_bias: Optional[np.ndarray]       # float32 [E] or None
    shared_gate_w: Optional[np.ndarray]     # float32 [H] or None
    # routed experts, stacked over E (INT4 draft)
    wg_q: np.ndarray
    wg_s: np.ndarray
    wu_q: np.ndarray
    wu_s: np.ndarray
    wd_q: np.ndarray
    wd_s: np.ndarray
    # FP16 target weights for the verification pass (or None)
    wg16: Optional[np.ndarray] = None
    wu16: Optional[np.ndarray] = None
    wd16: Optional[np.ndarray] = None
    # FP16 shared expert(s), concatenated along the intermediate dim (or None)
    sg16: Optional[np.ndarray] = None       # [shared_I][H]
    su16: Optional[np.ndarray] = None       # [shared_I][H]
    sd16: Optional[np.ndarray] = None       # [H][shared_I]
    meta: Dict[str, object] = field(default_factory=dict)

    def expert(self, e: int) -> ExpertWeights:
        return ExpertWeights(
            self.wg_q[e], self.wg_s[e], self.wu_q[e], self.wu_s[e],
            self.wd_q[e], self.wd_s[e],
            None if self.wg16 is None else self.wg16[e],
            None if self.wu16 is None else self.wu16[e],
            None if self.wd16 is None else self.wd16[e])


def make_activations(cfg: MoEConfig, seed: int = 0, layer: int = 0) -> np.ndarray:
    return _rng(seed, layer, _KIND_X).standard_normal(
        (cfg.T, cfg.H), dtype=np.float32).astype(np.float16)


def make_router(cfg: MoEConfig, seed: int = 0, layer: int = 0) -> np.ndarray:
    return _rng(seed, layer, _KIND_ROUTER).standard_normal(
        (cfg.E, cfg.H), dtype=np.float32) * WEIGHT_STD


def make_shared(cfg: MoEConfig, seed: int = 0, layer: int = 0):
    if cfg.shared_I == 0:
        return None, None, None
    rng = _rng(seed, layer, _KIND_SHARED)
    sg = rng.standard_normal((cfg.shared_I, cfg.H), dtype=np.float32) * WEIGHT_STD
    su = rng.standard_normal((cfg.shared_I, cfg.H), dtype=np.float32) * WEIGHT_STD
    sd = rng.standard_normal((cfg.H, cfg.shared_I), dtype=np.float32) * WEIGHT_STD
    return sg.astype(np.float16), su.astype(np.float16), sd.astype(np.float16)


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_layer(cfg: MoEConfig, seed: int = 0, layer: int = 0,
               want_fp16: Optional[bool] = None) -> LayerInputs:
    """All inputs of one MoE layer (every routed expert generated)."""
    if want_fp16 is None:
        want_fp16 = cfg.target_fp16
    x = make_activations(cfg, seed, layer)
    w_router = make_router(cfg, seed, layer)
    bias = zipf_bias(cfg.E, cfg.zipf_s, seed, layer) if cfg.zipf_s else None
    gate_w = None
    if cfg.shared_gate:
        gate_w = _rng(seed, layer, _KIND_SHARED_GATE).standard_normal(
            cfg.H, dtype=np.float32) * WEIGHT_STD

    E, I, H, G = cfg.E, cfg.I, cfg.H, cfg.G
    wg_q = np.empty((E, I, H // 8), np.uint32)
    wu_q = np.empty((E, I, H // 8), np.uint32)
    wd_q = np.empty((E, H, I // 8), np.uint32)
    wg_s = np.empty((E, I, H // G), np.float16)
    wu_s = np.empty((E, I, H // G), np.float16)
    wd_s = np.empty((E, H, I // G), np.float16)
    wg16 = wu16 = wd16 = None
    if want_fp16:
        wg16 = np.empty((E, I, H), np.float16)
        wu16 = np.empty((E, I, H), np.float16)
        wd16 = np.empty((E, H, I), np.float16)

    def one(e: int) -> None:
        ew = make_expert(cfg, e, seed, layer, want_fp16)
        wg_q[e], wg_s[e], wu_q[e], wu_s[e] = ew.wg_q, ew.wg_s, ew.wu_q, ew.wu_s
        wd_q[e], wd_s[e] = ew.wd_q, ew.wd_s
        if want_fp16:
            wg16[e], wu16[e], wd16[e] = ew.wg16, ew.wu16, ew.wd16

    with ThreadPoolExecutor(max_workers=_threads()) as pool:
        list(pool.map(one, range(E)))

    sg16, su16, sd16 = make_shared(cfg, seed, layer)
    return LayerInputs(
        cfg=cfg, seed=seed, layer=layer, x=x, w_router=w_router, router_bias=bias,
        shared_gate_w=gate_w, wg_q=wg_q, wg_s=wg_s, wu_q=wu_q, wu_s=wu_s,
        wd_q=wd_q, wd_s=wd_s, wg16=wg16, wu16=wu16, wd16=wd16,
        sg16=sg16, su16=su16, sd16=sd16,
        meta={"generator": "numpy PCG64 default_rng([seed, layer, kind, index])",
              "seed": seed, "layer": layer})
