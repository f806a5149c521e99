"""Plain model of SpecFit's verification-subtree selection (test
infrastructure only): brute force over every subset of the draft pool.

Source: the SpecFit page (its sections 3.1 to 3.3 and appendix A.2 / A.3):
  * a legal verification subtree is a set of draft nodes that contains every
    selected node's ancestors and has at most K nodes; the candidate pool of
    the pages has top-2 expansion, depth at most 5 and at most 18 nodes, and
    K = min(7, |pool|);
  * the estimated committed-token reward of a subtree is one (the root) plus
    the sum of its nodes' commit probabilities, estimated by the drafter's
    path probabilities;
  * the predicted cycle time is an intercept that depends on the node count
    plus beta times a per-layer expert-union feature: the experts that the
    subtree's tokens activate, counted once per layer (a coverage function:
    a node only pays for experts not already in the union);
  * the selector returns the legal subtree with the largest reward / time;
  * drafting continues after a level only if the selection contains a node
    of that level.

Readings where the page leaves a step open (each also listed in the
repository's design document):
  * the root (the committed token the tree grows from) is always verified:
    its experts are in every union, and the empty selection is legal;
  * with an expert cache the feature counts, per layer, the union's experts
    that are not resident (the ones the forward has to transfer); without a
    cache every expert counts;
  * reward = 1 + the path probabilities summed in ascending node index;
    time = intercept[|S|] + beta * F(S); the ratio is reward / time, all in
    IEEE double;
  * ties: the larger ratio, then fewer nodes, then the lexicographically
    smaller ascending node list.
"""

from __future__ import annotations

from itertools import combinations
from typing import List, Optional, Sequence, Set, Tuple


def ancestors(parent: Sequence[int], v: int) -> List[int]:
    out = []
    p = parent[v]
    while p >= 0:
        out.append(p)
        p = parent[p]
    return out


def is_legal(parent: Sequence[int], S: Set[int], K: int) -> bool:
    if len(S) > K:
        return False
    return all(set(ancestors(parent, v)) <= S for v in S)


def union_feature(S: Sequence[int], root_experts: Sequence[Set[int]],
                  node_experts: Sequence[Sequence[Set[int]]],
                  resident: Optional[Sequence[Set[int]]] = None) -> int:
    """Sum over layers of |(root's experts U experts of the nodes in S) minus
    the resident ones|. node_experts[v][l], root_experts[l]: sets of expert IDs."""
    F = 0
    for l in range(len(root_experts)):
        u = set(root_experts[l])
        for v in S:
            u |= set(node_experts[v][l])
        if resident is not None:
            u -= set(resident[l])
        F += len(u)
    return F


def score(S: Sequence[int], path_prob: Sequence[float], intercepts: Sequence[float], beta: float,
          root_experts, node_experts, resident=None) -> Tuple[float, float, float]:
    """(reward, time, reward / time) of the selection S."""
    reward = 1.0
    for v in sorted(S):
        reward += path_prob[v]
    F = union_feature(S, root_experts, node_experts, resident)
    t = intercepts[len(S)] + beta * F
    return reward, t, reward / t


def select(parent: Sequence[int], path_prob: Sequence[float], root_experts, node_experts,
           K: int, intercepts: Sequence[float], beta: float, resident=None):
    """The best legal subtree by brute force over every subset of the pool.
    Returns (sorted node list, ratio, number of legal subtrees)."""
    n = len(parent)
    best, best_key, legal = None, None, 0
    for size in range(0, min(K, n) + 1):
        for S in combinations(range(n), size):
            if not is_legal(parent, set(S), K):
                continue
            legal += 1
            _, _, r = score(S, path_prob, intercepts, beta, root_experts, node_experts, resident)
            key = (-r, len(S), list(S))
            if best_key is None or key < best_key:
                best_key, best = key, list(S)
    return best, -best_key[0], legal


def keep_drafting(selection: Sequence[int], depth: Sequence[int], level: int) -> bool:
    """After drafting `level`, drafting goes on only if the selection holds a
    node of that level."""
    return any(depth[v] == level for v in selection)
