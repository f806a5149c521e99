"""Seeded input generator: packing format, determinism, shapes (CPU only)."""

import json
import os

import numpy as np

from workload import (get_config, make_expert, make_layer, pack_int4_codes,
                      quantize_rtn_int4, zipf_bias)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_pack_matches_golden_words():
    g = json.load(open(os.path.join(GOLDEN, "int4_pack_handworked.json")))
    codes = np.array([[1, 2, 3, 4, 5, 6, 7, 8], [8, 15, 0, 15, 0, 0, 0, 0]], np.uint8)
    assert pack_int4_codes(codes)[:, 0].tolist() == g["words"]


def test_quantizer_scale_rule():
    w = np.array([[0.7, -0.35, 0.1, 0.0, 0.0, 0.0, 0.0, 0.0]], np.float32)
    codes, s = quantize_rtn_int4(w, 8)
    assert s.dtype == np.float16 and s[0, 0] == np.float16(0.1)
    nib = [(int(codes[0, 0]) >> (4 * j)) & 0xF for j in range(8)]
    # scale s = fp16(0.7/7) = 0.0999755859375; 0.7/s = 7.0017 -> 7,
    # -0.35/s = -3.5009 -> -4, 0.1/s = 1.0002 -> 1; codes are q + 8
    assert nib[:3] == [15, 4, 9] and nib[3:] == [8] * 5


def test_generation_is_deterministic_and_per_expert():
    cfg = get_config("tiny")
    a = make_layer(cfg, seed=0)
    b = make_layer(cfg, seed=0)
    for name in ("x", "w_router", "wg_q", "wg_s", "wd_q", "wd_s"):
        assert np.array_equal(getattr(a, name), getattr(b, name))
    e3 = make_expert(cfg, 3, seed=0)
    assert np.array_equal(a.wu_q[3], e3.wu_q) and np.array_equal(a.wd_s[3], e3.wd_s)
    c = make_layer(cfg, seed=1)
    assert not np.array_equal(a.x, c.x)


def test_shapes_and_dtypes():
    cfg = get_config("tiny")
    L = make_layer(cfg, seed=0)
    assert L.x.shape == (17, 256) and L.x.dtype == np.float16
    assert L.w_router.shape == (8, 256) and L.w_router.dtype == np.float32
    assert L.wg_q.shape == (8, 512, 32) and L.wg_q.dtype == np.uint32
    assert L.wg_s.shape == (8, 512, 4) and L.wg_s.dtype == np.float16
    assert L.wd_q.shape == (8, 256, 64) and L.wd_s.shape == (8, 256, 8)
    assert L.sg16 is None and L.router_bias is None


def test_zipf_bias_is_log_rank_prior():
    b = zipf_bias(64, 1.1, seed=0, layer=2).astype(np.float64)
    ranks = np.rint(np.exp(-b / 1.1)).astype(int)
    assert sorted(ranks.tolist()) == list(range(1, 65))
    assert b.max() == 0.0
