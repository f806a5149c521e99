"""The native SpecFit selection (host code of libsmoe, no GPU needed) against
the brute-force model of oracle/specfit.py: the same subtree, the same ratio
bit for bit, and as many legal subtrees visited as exist, on the hand-worked
pool and on seeded random pools up to the pages' 18-node, K = 7 size."""

import json
import os

import numpy as np
import pytest

from oracle import specfit as SF
from test_oracle_specfit import G, random_pool, sets


@pytest.fixture(scope="module")
def lib():
    from quantized_speculative_expert_amd import _lib
    return _lib


def bitmaps(root, ne, E):
    W = (E + 63) // 64
    L = len(root)
    out = np.zeros((len(ne) + 1, L, W), np.uint64)
    for row, node in enumerate([root] + list(ne)):
        for l, es in enumerate(node):
            for e in es:
                out[row, l, e // 64] |= np.uint64(1) << np.uint64(e % 64)
    return out


def resident_bits(res, E):
    if res is None:
        return None
    return bitmaps(res, [], E)[0]


def native(lib, parent, prob, root, ne, K, b, beta, E, resident=None):
    return lib.smoe_specfit_select(np.asarray(parent, np.int32), np.asarray(prob, np.float64),
                                   bitmaps(root, ne, E), K, np.asarray(b, np.float64), beta,
                                   resident_bits=resident_bits(resident, E), E=E)


def test_native_golden(lib):
    root = [set(l) for l in G["root_experts"]]
    ne = sets(G["node_experts"])
    par, p, b, beta = G["parent"], G["path_prob"], G["intercepts"], G["beta"]
    sel, r, ev = native(lib, par, p, root, ne, 4, b, beta, 8)
    assert sel == G["expected_no_cache"] and r == G["expected_ratio_no_cache"]
    assert ev == G["expected_legal"]
    assert native(lib, par, p, root, ne, 4, b, beta, 8,
                  [set(l) for l in G["resident"]])[0] == G["expected_cached"]
    assert native(lib, par, p, root, ne, 1, b, beta, 8)[0] == G["expected_K1"]
    assert native(lib, par, G["tie_path_prob"], root, sets(G["tie_node_experts"]), 1, b, beta,
                  8)[0] == G["expected_tie_K1"]


def random_case(rng, n, L, E, k):
    parent, depth, prob, root, ne = random_pool(rng, n, L=L, E=E, k=k)
    n = len(parent)
    K = min(7, n)
    b = np.cumsum(rng.uniform(0.5, 2.0, K + 1)).tolist()
    beta = float(rng.choice([0.0, 0.01, 0.1, 1.0]))
    res = None
    if rng.random() < 0.5:
        res = [set(rng.choice(E, E // 2, replace=False).tolist()) for _ in range(L)]
    return parent, prob, root, ne, K, b, beta, res


@pytest.mark.parametrize("seed", range(40))
def test_native_matches_brute_force(lib, seed):
    rng = np.random.default_rng(300 + seed)
    n = int(rng.integers(1, 13))
    E = int(rng.choice([8, 64, 100, 128, 256]))
    parent, prob, root, ne, K, b, beta, res = random_case(rng, n, 3, E, 2)
    want, wr, legal = SF.select(parent, prob, root, ne, K, b, beta, res)
    got, gr, ev = native(lib, parent, prob, root, ne, K, b, beta, E, res)
    assert got == want and gr == wr and ev == legal


@pytest.mark.parametrize("seed", range(3))
def test_native_matches_brute_force_at_the_pages_pool_size(lib, seed):
    # 18 nodes, top-2 expansion, depth <= 5, K = 7
    rng = np.random.default_rng(400 + seed)
    parent, prob, root, ne, K, b, beta, res = random_case(rng, 18, 4, 128, 8)
    assert len(parent) == 18 and K == 7
    want, wr, legal = SF.select(parent, prob, root, ne, K, b, beta, res)
    got, gr, ev = native(lib, parent, prob, root, ne, K, b, beta, 128, res)
    assert got == want and gr == wr and ev == legal


def test_native_argument_checks(lib):
    bits = np.zeros((3, 1, 1), np.uint64)
    with pytest.raises(lib.SmoeError):  # a parent after its child
        lib.smoe_specfit_select(np.array([1, -1], np.int32), np.ones(2), bits, 2,
                                np.ones(3), 1.0, E=8)
    with pytest.raises(lib.SmoeError):  # a zero intercept
        lib.smoe_specfit_select(np.array([-1, 0], np.int32), np.ones(2), bits, 2,
                                np.array([1.0, 0.0, 1.0]), 1.0, E=8)
