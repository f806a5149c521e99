"""CPU pins of the expert-cache and prefetch-planner model (oracle/offload.py):
a hand-worked golden (tests/golden/cache_handworked.json), closed forms of
the boundary rule, and invariants that the pages fix (hits before misses, no
protected or claimed slot taken, causal snapshots, the phases of a window),
checked by brute force on random cases; planted mistakes fail them."""

import json
import math
import os

import numpy as np
import pytest

from oracle import offload as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "cache_handworked.json")))


def golden_verify(model_cls=O.CacheModel):
    g = GOLD["verify"]
    m = model_cls(g["L"], g["M"])
    m.slot_expert = [list(r) for r in g["slot_expert"]]
    m.last_use = [list(r) for r in g["last_use"]]
    m.clock = g["clock"]
    sched = m.verify(0, g["counts"])
    return m, sched


def check_golden_verify(model_cls=O.CacheModel):
    g = GOLD["verify"]
    m, sched = golden_verify(model_cls)
    return ([list(s) for s in sched] == g["expected_schedule"]
            and m.slot_expert == g["expected_slot_expert"]
            and m.last_use == g["expected_last_use"] and m.clock == g["expected_clock"])


def run_golden_planner():
    g = GOLD["planner"]
    m = O.CacheModel(g["L"], g["M"])
    outs = []
    for w in g["windows"]:
        outs.append(O.plan_window(np.array(w["routing"]), g["E"], m, g["b1"], g["expert_bytes"],
                                  g["h2d_gb_per_s"], g["draft_us_per_token"]))
    windows_state = [list(r) for r in m.slot_expert]
    sched = m.verify(g["verify_layer"], g["verify_counts"])
    return m, outs, sched, windows_state


def check_golden_planner():
    g = GOLD["planner"]
    m, outs, sched, windows_state = run_golden_planner()
    for w, out in zip(g["windows"], outs):
        if [list(c) for c in out["chunks"]] != w["expected_chunks"]:
            return False
        got = [[b, [list(x) for x in loads]] for b, loads in out["boundaries"]]
        if got != w["expected_boundaries"]:
            return False
    return (windows_state == g["expected_slot_expert"]
            and m.slot_expert == g["expected_slot_expert_after_verify"]
            and [list(s) for s in sched] == g["expected_verify_schedule"])


def test_verify_golden():
    assert check_golden_verify()


def test_planner_golden():
    assert check_golden_planner()


# ------------------------------------------------------------------ boundary rule

@pytest.mark.parametrize("n,expect", [(0, 3), (1, 3), (2, 3), (3, 4), (4, 4), (5, 5), (40, 10)])
def test_next_boundary_closed_form(n, expect):
    # 200 us per expert (1 MB at 5 GB/s), 400 us per draft token, b = 2, K = 10:
    # n experts need ceil(n / 2) tokens, at least one
    assert O.next_boundary(2, 10, n, 1e6, 5.0, 400.0) == expect
    assert expect == min(2 + max(1, math.ceil(n / 2)), 10)


def test_next_boundary_infinite_bandwidth_and_cap():
    assert O.next_boundary(0, 16, 50, 17.3e6, 1e18, 30.0) == 1
    assert O.next_boundary(15, 16, 50, 17.3e6, 1.0, 30.0) == 16
    assert O.next_boundary(16, 16, 0, 1.0, 1.0, 1.0) == 16


# ------------------------------------------------------------------ verification invariants

def random_state(rng, L, E, M):
    m = O.CacheModel(L, M)
    for l in range(L):
        k = rng.integers(0, M + 1)
        experts = rng.permutation(E)[:k]
        slots = rng.permutation(M)[:k]
        for e, s in zip(experts, slots):
            m.slot_expert[l][s] = int(e)
            m.last_use[l][s] = int(rng.integers(1, 20))
    m.clock = 20
    return m


def check_verify_invariants(before, counts, sched, l=0):
    M = before.M
    required = [e for e in range(len(counts)) if counts[e] > 0]
    cached = {before.slot_expert[l][s]: s for s in range(M) if before.slot_expert[l][s] >= 0}
    # every required expert exactly once; hits (ascending) then misses (ascending)
    assert sorted(s[0] for s in sched) == required
    kinds = [s[2] for s in sched]
    assert kinds == sorted(kinds)
    hits = [s for s in sched if s[2] == O.HIT]
    misses = [s for s in sched if s[2] == O.MISS]
    assert [h[0] for h in hits] == sorted(e for e in required if e in cached)
    assert [x[0] for x in misses] == sorted(e for e in required if e not in cached)
    assert all(h[1] == cached[h[0]] and h[4] == -1 for h in hits)
    protected = {h[1] for h in hits}
    # slot timeline: a slot is taken at once only if free or unprotected and not
    # yet taken in this call; otherwise it must have been used by the group
    # named in `wait`, and that group's computation is earlier in the order
    holder_group = {s: 0 for s in protected}  # slot -> group that last used it
    taken_now = set()
    for j, x in enumerate(misses):
        s, wait = x[1], x[4]
        if wait == -1:
            assert s not in protected and s not in taken_now
            taken_now.add(s)
        else:
            assert holder_group.get(s) == wait and wait < 1 + j
        holder_group[s] = 1 + j
    # LRU among the slots taken at once: empty ones first, then by last use
    free_slots = [s for s in range(M) if s not in protected]
    order = sorted(free_slots, key=lambda s: (before.slot_expert[l][s] >= 0,
                                              before.last_use[l][s], s))
    immediate = [x[1] for x in misses if x[4] == -1]
    assert immediate == order[:len(immediate)]
    # a wait is needed only when every unprotected slot is already taken
    if any(x[4] != -1 for x in misses):
        assert len(immediate) == len(free_slots)


@pytest.mark.parametrize("seed", range(40))
def test_verify_invariants_random(seed):
    rng = np.random.default_rng(seed)
    E, M = int(rng.integers(2, 12)), int(rng.integers(1, 7))
    m = random_state(rng, 1, E, M)
    import copy
    before = copy.deepcopy(m)
    counts = (rng.random(E) < 0.6) * rng.integers(1, 5, E)
    sched = m.verify(0, [int(c) for c in counts])
    check_verify_invariants(before, counts, sched)


def test_resident_expert_computed_while_missing_one_loads():
    # the pages' example: tokens route to a cached expert A and a missing B;
    # A's sub-batch goes first, B is copied into a free slot at once
    m = O.CacheModel(1, 2)
    m.slot_expert[0] = [7, -1]
    m.last_use[0] = [1, 0]
    m.clock = 1
    sched = m.verify(0, [0] * 7 + [2, 3])  # A = 7, B = 8
    assert sched == [(7, 0, O.HIT, 7, -1), (8, 1, O.MISS, -1, -1)]


# ------------------------------------------------------------------ planner invariants

def random_routing(rng, K, L, E, k, skew=1.2):
    p = 1.0 / np.arange(1, E + 1) ** skew
    p /= p.sum()
    out = np.zeros((K, L, k), np.int32)
    for l in range(L):
        perm = rng.permutation(E)
        for i in range(K):
            out[i, l] = perm[rng.choice(E, k, replace=False, p=p)]
    return out


def check_window(out, routing, E, m_before, m_after, b1, eb, bw, us):
    K, L = routing.shape[:2]
    chunks = out["chunks"]
    assert chunks[0] == (0, min(b1, K), O.COLD)
    for (a0, a1, _), (c0, c1, _) in zip(chunks, chunks[1:]):
        assert a1 == c0 and c0 < c1
    if K > b1:
        assert chunks[-1][1] == K and chunks[-1][2] == O.CLEANUP
        assert all(c[2] == O.OVERLAP for c in chunks[1:-1])
    assert len(out["boundaries"]) == len(chunks) - 1
    claimed_slots = [set() for _ in range(L)]
    for (b, loads), (c0, c1, ph) in zip(out["boundaries"], chunks[1:]):
        assert b == c0
        # snapshot uses tokens [0, b) only: the loaded experts have a positive
        # count there and rank within the layer's top-M
        cnt = np.zeros((L, E), np.int64)
        for i in range(b):
            for l in range(L):
                for e in routing[i][l]:
                    cnt[l][e] += 1
        for l, e, s, ev in loads:
            assert cnt[l][e] > 0
            rank = sorted(range(E), key=lambda x: (-cnt[l][x], x))
            assert rank.index(e) < m_after.M
            assert s not in claimed_slots[l]  # a claimed slot is never taken again
            claimed_slots[l].add(s)
        if ph == O.OVERLAP or (ph == O.CLEANUP and c1 == K and
                               not all(m_after.unclaimed(l) == 0 for l in range(L))):
            want = max(1, math.ceil(len(loads) * eb / (bw * 1000.0) / us))
            assert c1 - c0 == want or c1 == K


@pytest.mark.parametrize("seed", range(20))
def test_planner_invariants_random(seed):
    rng = np.random.default_rng(100 + seed)
    K, L, E, k = int(rng.integers(2, 17)), int(rng.integers(1, 4)), int(rng.integers(4, 20)), 2
    M = int(rng.integers(1, E))
    routing = random_routing(rng, K, L, E, k)
    m = random_state(rng, L, E, M)
    import copy
    before = copy.deepcopy(m)
    b1, eb, bw, us = int(rng.integers(1, 4)), 1e6, float(rng.uniform(1, 30)), 300.0
    out = O.plan_window(routing, E, m, b1, eb, bw, us)
    check_window(out, routing, E, before, m, b1, eb, bw, us)


@pytest.mark.parametrize("seed", range(10))
def test_planner_snapshot_is_causal(seed):
    # changing the routing of the tokens after a boundary changes nothing
    # decided at that boundary
    rng = np.random.default_rng(200 + seed)
    K, L, E, k, M = 12, 2, 10, 2, 4
    routing = random_routing(rng, K, L, E, k)
    a = O.plan_window(routing, E, O.CacheModel(L, M), 2, 1e6, 10.0, 100.0)
    b0 = a["boundaries"][0][0] if a["boundaries"] else K
    other = routing.copy()
    other[b0:] = random_routing(rng, K, L, E, k)[b0:]
    b = O.plan_window(other, E, O.CacheModel(L, M), 2, 1e6, 10.0, 100.0)
    if a["boundaries"]:
        assert a["boundaries"][0] == b["boundaries"][0]


def test_planner_fast_link_takes_one_token_chunks():
    # with an unlimited link every chunk after the first is one token long
    # until the cache is full or drafting ends
    rng = np.random.default_rng(5)
    routing = random_routing(rng, 10, 2, 32, 2)
    out = O.plan_window(routing, 32, O.CacheModel(2, 30), 2, 1e6, 1e15, 100.0)
    assert all(c1 - c0 == 1 for c0, c1, _ in out["chunks"][1:])


def test_planner_cold_start_covers_short_windows():
    routing = random_routing(np.random.default_rng(6), 2, 1, 8, 2)
    out = O.plan_window(routing, 8, O.CacheModel(1, 4), 4, 1e6, 10.0, 100.0)
    assert out["chunks"] == [(0, 2, O.COLD)] and out["boundaries"] == []


# ------------------------------------------------------------------ planted mistakes

class MRUCache(O.CacheModel):
    def _victims(self, l, exclude):
        v = super()._victims(l, exclude)
        empty = [s for s in v if self.slot_expert[l][s] < 0]
        used = [s for s in v if self.slot_expert[l][s] >= 0]
        return empty + used[::-1]


class MissesFirst(O.CacheModel):
    def verify(self, l, counts):
        out = super().verify(l, counts)
        return [x for x in out if x[2] == O.MISS] + [x for x in out if x[2] == O.HIT]


class NoProtection(O.CacheModel):
    def verify(self, l, counts):
        # hits' slots offered to the misses at once
        required = [e for e in range(len(counts)) if counts[e] > 0]
        hits = [e for e in required if self.slot_of(l, e) >= 0]
        misses = [e for e in required if self.slot_of(l, e) < 0]
        avail = self._victims(l, set())
        out = [(e, self.slot_of(l, e), O.HIT, e, -1) for e in hits]
        for e in misses:
            if not avail:
                avail = self._victims(l, set())
            s = avail.pop(0)
            out.append((e, s, O.MISS, self.slot_expert[l][s], -1))
            self.slot_expert[l][s] = e
        return out


@pytest.mark.parametrize("cls", [MRUCache, MissesFirst, NoProtection])
def test_planted_mistakes_fail_the_verify_pins(cls):
    caught = not check_golden_verify(cls)
    for seed in range(40):
        rng = np.random.default_rng(seed)
        E, M = int(rng.integers(2, 12)), int(rng.integers(1, 7))
        base = random_state(rng, 1, E, M)
        m = cls(1, M)
        m.slot_expert, m.last_use, m.clock = base.slot_expert, base.last_use, base.clock
        import copy
        before = copy.deepcopy(m)
        counts = (rng.random(E) < 0.6) * rng.integers(1, 5, E)
        try:
            check_verify_invariants(before, counts, m.verify(0, [int(c) for c in counts]))
        except AssertionError:
            caught = True
    assert caught


def test_planted_planner_mistakes_fail_the_golden(monkeypatch):
    # a floor instead of a ceil for the chunk length; the zero-count experts
    # treated as selected; no claim on cached experts
    orig_next = O.next_boundary

    def floor_next(b, K, n, eb, bw, us):
        t = n * eb / (bw * 1000.0)
        return min(b + max(1, int(math.floor(t / us))), K)

    monkeypatch.setattr(O, "next_boundary", floor_next)
    assert not check_golden_planner()
    monkeypatch.setattr(O, "next_boundary", orig_next)
    assert check_golden_planner()

    orig_prefetch = O.CacheModel.prefetch

    def zero_counts_too(self, l, ranked):
        return orig_prefetch(self, l, [(e, max(c, 1)) for e, c in ranked])

    monkeypatch.setattr(O.CacheModel, "prefetch", zero_counts_too)
    assert not check_golden_planner()
