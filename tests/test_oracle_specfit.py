"""CPU pins of the SpecFit selection model (oracle/specfit.py): a hand-worked
pool (tests/golden/specfit_handworked.json), closed forms (counts of legal
subtrees of a path and of a star; with a flat cost the best subtree is the K
most probable nodes), the coverage feature's monotone submodularity, and
planted mistakes that fail these pins."""

import json
import math
import os

import numpy as np
import pytest

from oracle import specfit as SF

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "specfit_handworked.json")))


def sets(x):
    return [[set(l) for l in node] for node in x]


def golden_checks(sel=SF.select):
    root = [set(l) for l in G["root_experts"]]
    ne = sets(G["node_experts"])
    par, p, b, beta = G["parent"], G["path_prob"], G["intercepts"], G["beta"]
    s0, r0, legal = sel(par, p, root, ne, 4, b, beta)
    s1, _, _ = sel(par, p, root, ne, 4, b, beta, resident=[set(l) for l in G["resident"]])
    s2, _, _ = sel(par, p, root, ne, 1, b, beta)
    s3, _, _ = sel(par, G["tie_path_prob"], root, sets(G["tie_node_experts"]), 1, b, beta)
    return (s0 == G["expected_no_cache"] and abs(r0 - G["expected_ratio_no_cache"]) < 1e-15
            and legal == G["expected_legal"] and s1 == G["expected_cached"]
            and s2 == G["expected_K1"] and s3 == G["expected_tie_K1"])


def test_golden_selection():
    assert golden_checks()


def test_golden_stop_rule():
    d = G["depth"]
    assert SF.keep_drafting([0, 2], d, 2) and not SF.keep_drafting([0], d, 2)


def random_pool(rng, n, depth_max=5, L=3, E=16, k=2):
    """Top-2 expansion: each node has at most two children, depth <= depth_max;
    path probabilities shrink down the tree."""
    parent, depth, prob = [], [], []
    frontier = [(-1, 0, 1.0)]  # (node, depth, path prob); -1 is the root
    kids = {}
    while len(parent) < n and frontier:
        i = int(rng.integers(0, len(frontier)))
        v, dv, pv = frontier[i]
        if kids.get(v, 0) >= 2 or dv >= depth_max:
            frontier.pop(i)
            continue
        kids[v] = kids.get(v, 0) + 1
        q = float(pv * rng.uniform(0.2, 0.95))
        parent.append(v)
        depth.append(dv + 1)
        prob.append(q)
        frontier.append((len(parent) - 1, dv + 1, q))
    root = [set(rng.choice(E, k, replace=False).tolist()) for _ in range(L)]
    ne = [[set(rng.choice(E, k, replace=False).tolist()) for _ in range(L)]
          for _ in range(len(parent))]
    return parent, depth, prob, root, ne


def count_legal(parent, K):
    n = len(parent)
    return sum(1 for s in range(K + 1) for S in __import__("itertools").combinations(range(n), s)
               if SF.is_legal(parent, set(S), K))


@pytest.mark.parametrize("n,K", [(5, 3), (7, 7), (6, 2)])
def test_legal_count_closed_forms(n, K):
    path = [-1] + list(range(n - 1))           # a chain: sizes 0..min(K, n), one each
    assert count_legal(path, K) == min(K, n) + 1
    star = [-1] * n                             # all children of the root: any subset
    assert count_legal(star, K) == sum(math.comb(n, j) for j in range(min(K, n) + 1))


@pytest.mark.parametrize("seed", range(8))
def test_flat_cost_takes_the_most_probable_nodes(seed):
    # beta = 0 and one intercept: the ratio is the reward, so the best legal
    # subtree is the min(K, n) nodes of largest path probability (path
    # probabilities never grow down the tree, so that set is ancestor-closed)
    rng = np.random.default_rng(seed)
    parent, depth, prob, root, ne = random_pool(rng, 9)
    K = min(7, len(parent))
    sel, _, _ = SF.select(parent, prob, root, ne, K, [2.0] * (K + 1), 0.0)
    top = sorted(sorted(range(len(prob)), key=lambda v: (-prob[v], v))[:K])
    assert sel == top


@pytest.mark.parametrize("seed", range(8))
def test_union_feature_is_monotone_submodular(seed):
    rng = np.random.default_rng(50 + seed)
    parent, depth, prob, root, ne = random_pool(rng, 10)
    n = len(parent)
    for _ in range(30):
        A = set(rng.choice(n, int(rng.integers(0, n)), replace=False).tolist())
        B = A | set(rng.choice(n, int(rng.integers(0, n)), replace=False).tolist())
        v = int(rng.integers(0, n))
        fa, fb = SF.union_feature(A, root, ne), SF.union_feature(B, root, ne)
        ga = SF.union_feature(A | {v}, root, ne) - fa
        gb = SF.union_feature(B | {v}, root, ne) - fb
        assert fb >= fa and ga >= gb >= 0


def test_heavy_expert_cost_prefers_nodes_that_add_no_experts():
    # with a huge beta only selections adding no experts beyond the root's
    # are competitive: node 1 shares the root's experts, the others do not
    root = [{0, 1}]
    ne = [[{2}], [{0, 1}], [{3}]]
    sel, _, _ = SF.select([-1, -1, 0], [0.5, 0.4, 0.3], root, ne, 3, [1.0] * 4, 1e6)
    assert sel == [1]


# planted mistakes: each breaks a pin above
def no_root_reward(parent, p, root, ne, K, b, beta, resident=None):
    return SF.select(parent, [x - 1.0 / max(1, len(p)) for x in p], root, ne, K, b, beta, resident)


def no_root_experts(parent, p, root, ne, K, b, beta, resident=None):
    return SF.select(parent, p, [set() for _ in root], ne, K, b, beta, resident)


def no_closure(parent, p, root, ne, K, b, beta, resident=None):
    return SF.select([-1] * len(parent), p, root, ne, K, b, beta, resident)


@pytest.mark.parametrize("bad", [no_root_reward, no_root_experts, no_closure])
def test_planted_mistakes_fail_the_golden(bad):
    assert not golden_checks(bad)
