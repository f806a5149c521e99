"""The native expert cache and prefetch planner (host code of libsmoe, no GPU
needed) against the CPU model of oracle/offload.py: every decision bit for
bit -- verification schedules, slot states, prefetch loads, chunk boundaries
and phases -- on the hand-worked golden and on seeded random windows."""

import copy
import json
import os

import numpy as np
import pytest

from oracle import offload as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "cache_handworked.json")))


@pytest.fixture(scope="module")
def lib():
    from quantized_speculative_expert_amd import _lib  # fails loudly if not built
    return _lib


class Native:
    """A decisions-only native cache (no device memory)."""

    def __init__(self, lib, L, E, M):
        self.lib, self.L, self.E, self.M = lib, L, E, M
        self.h = lib.smoe_cache_create(L, E, M, 0)

    def close(self):
        self.lib.smoe_cache_destroy(self.h)

    def set_from(self, m: O.CacheModel):
        self.lib.smoe_cache_set_state(self.h, np.array(m.slot_expert, np.int32).reshape(self.L, self.M),
                                      np.array(m.last_use, np.int64).reshape(self.L, self.M),
                                      m.clock)

    def state(self):
        se, lu, cl, clock = self.lib.smoe_cache_state(self.h, self.L, self.M)
        return se.tolist(), lu.tolist(), cl.tolist(), clock

    def verify(self, l, counts):
        return [tuple(r) for r in self.lib.smoe_cache_verify_plan(
            self.h, l, np.asarray(counts, np.int32)).tolist()]


def model_state(m: O.CacheModel):
    return (m.slot_expert, m.last_use, [[int(c) for c in r] for r in m.claimed], m.clock)


def native_window(lib, nat: Native, routing, E, b1, eb, bw, us):
    """The planner loop driven by the native calls (top-M snapshots taken
    here from the counts with a plain sort)."""
    K, L = routing.shape[:2]
    lib.smoe_cache_begin_window(nat.h)
    cnt = np.zeros((L, E), np.int64)

    def observe(i0, i1):
        for i in range(i0, i1):
            for l in range(L):
                for e in routing[i][l]:
                    if 0 <= e < E:
                        cnt[l][e] += 1

    b = min(max(b1, 0), K)
    chunks = [(0, b, O.COLD)]
    observe(0, b)
    boundaries = []
    M = nat.M
    while b < K:
        order = np.array([sorted(range(E), key=lambda e: (-cnt[l][e], e))[:M] for l in range(L)],
                         np.int32).reshape(L, M)
        counts = np.array([[cnt[l][e] for e in order[l]] for l in range(L)],
                          np.int32).reshape(L, M)
        loads, full = lib.smoe_cache_prefetch(nat.h, order, counts, L, M)
        loads = [tuple(x) for x in loads.tolist()]
        boundaries.append((b, loads))
        if full:
            chunks.append((b, K, O.CLEANUP))
            break
        nb = lib.smoe_prefetch_next_boundary(b, K, len(loads), eb, bw, us)
        chunks.append((b, nb, O.OVERLAP if nb < K else O.CLEANUP))
        observe(b, nb)
        b = nb
    return {"chunks": chunks, "boundaries": boundaries}


def test_native_verify_golden(lib):
    g = GOLD["verify"]
    m = O.CacheModel(g["L"], g["M"])
    m.slot_expert, m.last_use, m.clock = g["slot_expert"], g["last_use"], g["clock"]
    nat = Native(lib, g["L"], g["E"], g["M"])
    nat.set_from(m)
    assert [list(s) for s in nat.verify(0, g["counts"])] == g["expected_schedule"]
    se, lu, _, clock = nat.state()
    assert se == g["expected_slot_expert"] and lu == g["expected_last_use"]
    assert clock == g["expected_clock"]
    nat.close()


def test_native_planner_golden(lib):
    g = GOLD["planner"]
    nat = Native(lib, g["L"], g["E"], g["M"])
    for w in g["windows"]:
        out = native_window(lib, nat, np.array(w["routing"]), g["E"], g["b1"], g["expert_bytes"],
                            g["h2d_gb_per_s"], g["draft_us_per_token"])
        assert [list(c) for c in out["chunks"]] == w["expected_chunks"]
        assert [[b, [list(x) for x in ld]] for b, ld in out["boundaries"]] == \
            w["expected_boundaries"]
    assert nat.state()[0] == g["expected_slot_expert"]
    assert [list(s) for s in nat.verify(g["verify_layer"], g["verify_counts"])] == \
        g["expected_verify_schedule"]
    nat.close()


@pytest.mark.parametrize("seed", range(60))
def test_native_verify_matches_model(lib, seed):
    rng = np.random.default_rng(1000 + seed)
    L, E, M = int(rng.integers(1, 4)), int(rng.integers(2, 40)), int(rng.integers(1, 12))
    m = O.CacheModel(L, M)
    for l in range(L):
        k = int(rng.integers(0, min(M, E) + 1))
        for e, s in zip(rng.permutation(E)[:k], rng.permutation(M)[:k]):
            m.slot_expert[l][int(s)] = int(e)
            m.last_use[l][int(s)] = int(rng.integers(1, 5))  # many ties
    m.clock = 5
    nat = Native(lib, L, E, M)
    nat.set_from(m)
    for _ in range(4):  # a few layers' verifications in a row
        l = int(rng.integers(0, L))
        counts = ((rng.random(E) < 0.5) * rng.integers(1, 6, E)).astype(np.int32)
        assert nat.verify(l, counts) == m.verify(l, [int(c) for c in counts])
        assert nat.state() == model_state(m)
    nat.close()


@pytest.mark.parametrize("seed", range(30))
def test_native_windows_match_model(lib, seed):
    rng = np.random.default_rng(2000 + seed)
    L, E, k = int(rng.integers(1, 5)), int(rng.integers(4, 64)), int(rng.integers(1, 4))
    M = int(rng.integers(1, E))
    K = int(rng.integers(1, 18))
    m = O.CacheModel(L, M)
    nat = Native(lib, L, E, M)
    eb, bw, us = float(rng.choice([1e6, 17.3e6, 5.77e6])), float(rng.uniform(1, 64)), \
        float(rng.uniform(20, 900))
    for w in range(3):  # consecutive windows on one cache, then verification
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
        routing = np.array([[rng.choice(E, min(k, E), replace=False, p=p) for _ in range(L)]
                            for _ in range(K)], np.int32)
        b1 = int(rng.integers(0, 4))
        want = O.plan_window(routing, E, m, b1, eb, bw, us)
        got = native_window(lib, nat, routing, E, b1, eb, bw, us)
        assert got == want
        assert nat.state() == model_state(m)
        for l in range(L):
            counts = np.bincount(routing[:, l].reshape(-1), minlength=E).astype(np.int32)
            assert nat.verify(l, counts) == m.verify(l, [int(c) for c in counts])
    nat.close()


def test_native_next_boundary_matches_model(lib):
    rng = np.random.default_rng(9)
    for _ in range(2000):
        b = int(rng.integers(0, 20))
        K = b + int(rng.integers(0, 20))
        n = int(rng.integers(0, 70))
        eb = float(rng.choice([1e6, 17301504.0, 4460544.0]))
        bw, us = float(rng.uniform(0.5, 64)), float(rng.uniform(1, 1000))
        assert lib.smoe_prefetch_next_boundary(b, K, n, eb, bw, us) == \
            O.next_boundary(b, K, n, eb, bw, us)


def test_native_argument_checks(lib):
    with pytest.raises(lib.SmoeError):
        lib.smoe_cache_create(0, 4, 2, 0)
    h = lib.smoe_cache_create(1, 4, 2, 0)
    with pytest.raises(lib.SmoeError):  # an expert held twice
        lib.smoe_cache_set_state(h, np.array([[1, 1]], np.int32), np.zeros((1, 2), np.int64), 0)
    with pytest.raises(lib.SmoeError):  # a plan naming an expert outside [0, E)
        lib.smoe_cache_prefetch(h, np.array([[4, 0]], np.int32), np.ones((1, 2), np.int32), 1, 2)
    # decisions-only caches do no device work (refused before any HIP call)
    counts = np.ones(4, np.int32)
    raw = lib.raw_library()
    st = raw.smoe_cache_verify_layer(h, 0, counts.ctypes.data_as(lib.ctypes.c_void_p), None, 1, 1,
                                     128, 128, 0, None, None, 0, None, None, None, None, 0, None,
                                     0, None, None, None, None, None, None)
    assert st == lib.SMOE_EINVAL
    lib.smoe_cache_destroy(h)
    with pytest.raises(lib.SmoeError):
        lib.smoe_prefetch_next_boundary(3, 2, 0, 1.0, 1.0, 1.0)
