"""Plain model of the expert cache and the ELB-driven prefetch planner
(test infrastructure only: the decisions the native runtime must take,
written out in pure Python over small integer state).

Sources (cited by page title and paragraph):
  * "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step
    Speculative Offloading", paper body:
      - Layer-Aware Prefetch Planner paragraphs: three phases (Cold Start,
        Prefetch Overlap, Final Cleanup); no transfer before the predefined
        first boundary b_1; at each boundary a top-M snapshot of the ELB
        counters, the experts of that ranking not already cached form the
        next host-to-device batch, and the next boundary is chosen so that
        the draft compute of the chunk matches the batch's transfer time;
        the planner stops once a batch fills the remaining cache slots (or
        drafting ends), and the final chunk's routing is discarded;
      - Verification Expert Cache Residency Manager paragraph: the target
        router's experts of a layer are split into cache hits (computed
        first) and misses (loaded, then computed as they land); an expert's
        slot is protected while it waits for or runs its computation and
        becomes replaceable once its tokens are done; loaded experts are
        not replaced before they are used;
      - cache-aware execution schedule paragraph (resident expert's
        sub-batch computed while a missing expert is copied).
  * Specter repository design notes ("Design"), "Predictive I/O
    Orchestrator": expert_cache tracks resident experts, replacement order
    and slot ownership; residency is a per-layer slot budget.

Readings where the pages leave a step open (each also listed in the
repository's design document):
  * replacement order is least-recently-used: every slot carries the clock
    value of its last use; a use is one prefetch call on the layer (all
    slots it claims or loads), the hit group of a verification, or one
    miss's computation; the clock advances by one per use; ties go to the
    lower slot index; an empty slot is always taken before an occupied one;
  * the snapshot's selected experts are the top-M ranking entries with a
    positive count (a zero count is no routing evidence);
  * at a boundary the selected experts already cached are claimed first,
    then the missing ones are loaded in ranking order into unclaimed slots;
    a slot claimed in the current window is not given up in that window;
  * verification takes the hits in one computation (ascending expert ID)
    and the misses one by one in ascending expert ID; a miss takes an empty
    slot, else an unprotected one (LRU), else the first slot that a
    finished computation releases (the hit group's slots in slot order,
    then each miss's slot in compute order);
  * the next boundary is b + n with the smallest n >= 1 such that
    n * (draft time per token) >= transfer time of the batch, capped at K;
    the transfer time of n experts is n * expert_bytes / bandwidth;
  * "the batch fills the remaining slots" means that after the batch no
    layer has an unclaimed slot; reaching K also ends the planning; there
    is no snapshot at K.
"""

from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

HIT, MISS = 0, 1
COLD, OVERLAP, CLEANUP = 0, 1, 2


class CacheModel:
    """Slot state of an L-layer expert cache with M slots per layer."""

    def __init__(self, L: int, M: int):
        self.L, self.M = L, M
        self.slot_expert = [[-1] * M for _ in range(L)]
        self.last_use = [[0] * M for _ in range(L)]
        self.claimed = [[False] * M for _ in range(L)]
        self.clock = 0

    def slot_of(self, l: int, e: int) -> int:
        for s in range(self.M):
            if self.slot_expert[l][s] == e:
                return s
        return -1

    def begin_window(self) -> None:
        for l in range(self.L):
            for s in range(self.M):
                self.claimed[l][s] = False

    def _tick(self) -> int:
        self.clock += 1
        return self.clock

    def _victims(self, l: int, exclude) -> List[int]:
        """Slots a new expert may take, in the order it takes them: empty
        slots by index, then occupied ones by (last use, index)."""
        empty = [s for s in range(self.M) if self.slot_expert[l][s] < 0 and s not in exclude]
        used = [s for s in range(self.M) if self.slot_expert[l][s] >= 0 and s not in exclude]
        used.sort(key=lambda s: (self.last_use[l][s], s))
        return empty + used

    # ---- prefetch at a boundary (Layer-Aware Prefetch Planner)
    def prefetch(self, l: int, ranked: Sequence[Tuple[int, int]]) -> List[Tuple[int, int, int, int]]:
        """ranked: the layer's top-M snapshot as (expert, count) in ranking
        order. Returns the loads as (layer, expert, slot, evicted expert)."""
        selected = [e for e, c in ranked if c > 0][: self.M]
        now = self._tick()
        for e in selected:  # cached ones are claimed first
            s = self.slot_of(l, e)
            if s >= 0:
                self.claimed[l][s] = True
                self.last_use[l][s] = now
        loads = []
        for e in selected:
            if self.slot_of(l, e) >= 0:
                continue
            cand = self._victims(l, {s for s in range(self.M) if self.claimed[l][s]})
            if not cand:
                break
            s = cand[0]
            loads.append((l, e, s, self.slot_expert[l][s]))
            self.slot_expert[l][s] = e
            self.claimed[l][s] = True
            self.last_use[l][s] = now
        return loads

    def unclaimed(self, l: int) -> int:
        return sum(1 for s in range(self.M) if not self.claimed[l][s])

    # ---- verification of one layer (Residency Manager)
    def verify(self, l: int, counts: Sequence[int]) -> List[Tuple[int, int, int, int, int]]:
        """counts[e]: tokens the target router sent to expert e. Returns the
        compute order as (expert, slot, kind, evicted, wait) where wait is
        -1 (slot free at once), 0 (after the hit group) or 1 + j (after
        miss j's computation)."""
        required = [e for e in range(len(counts)) if counts[e] > 0]
        hits = [e for e in required if self.slot_of(l, e) >= 0]
        misses = [e for e in required if self.slot_of(l, e) < 0]
        if misses and self.M == 0:
            raise ValueError("no cache slots")
        protected = {self.slot_of(l, e) for e in hits}
        avail = self._victims(l, protected)
        releases: List[Tuple[int, int]] = [(s, 0) for s in sorted(protected)]
        out = []
        now = self._tick() if hits else None
        for e in hits:
            s = self.slot_of(l, e)
            self.last_use[l][s] = now
            out.append((e, s, HIT, e, -1))
        for j, e in enumerate(misses):
            if avail:
                s, wait = avail.pop(0), -1
            else:
                s, wait = releases.pop(0)
            out.append((e, s, MISS, self.slot_expert[l][s], wait))
            self.slot_expert[l][s] = e
            self.last_use[l][s] = self._tick()
            releases.append((s, 1 + j))
        return out


def next_boundary(b: int, K: int, n_transfer: int, expert_bytes: float, h2d_gb_per_s: float,
                  draft_us_per_token: float) -> int:
    """Smallest b + n (n >= 1) whose n draft tokens take at least the batch's
    transfer time, capped at K. Transfer time in microseconds:
    n_transfer * expert_bytes / (h2d_gb_per_s * 1000)."""
    t_io = n_transfer * expert_bytes / (h2d_gb_per_s * 1000.0)
    n = max(1, int(math.ceil(t_io / draft_us_per_token)))
    return min(b + n, K)


def elb_snapshot(cnt: np.ndarray, M: int) -> List[List[Tuple[int, int]]]:
    """Per layer, the top-M experts by count (descending), ties to the lower
    expert ID, with their counts (zero counts included, as ranked)."""
    out = []
    for row in cnt:
        order = sorted(range(len(row)), key=lambda e: (-int(row[e]), e))[:M]
        out.append([(e, int(row[e])) for e in order])
    return out


def plan_window(routing: np.ndarray, E: int, cache: CacheModel, b1: int,
                expert_bytes: float, h2d_gb_per_s: float, draft_us_per_token: float) -> Dict:
    """One draft window of K tokens: routing[i][l] holds the draft router's
    experts of token i in layer l (IDs outside [0, E) are not counted).
    Returns the chunks [(begin, end, phase)], the loads of each boundary
    [(boundary, [(layer, expert, slot, evicted)])] and the final counters."""
    K, L = routing.shape[0], routing.shape[1]
    cnt = np.zeros((L, E), np.int64)

    def observe(i0: int, i1: int) -> None:
        for i in range(i0, i1):
            for l in range(L):
                for e in routing[i][l]:
                    if 0 <= e < E:
                        cnt[l][e] += 1

    cache.begin_window()
    b = min(max(b1, 0), K)
    chunks = [(0, b, COLD)]
    observe(0, b)
    boundaries = []
    while b < K:
        snap = elb_snapshot(cnt, cache.M)
        loads = []
        for l in range(L):
            loads += cache.prefetch(l, snap[l])
        boundaries.append((b, loads))
        if all(cache.unclaimed(l) == 0 for l in range(L)):
            chunks.append((b, K, CLEANUP))
            break
        nb = next_boundary(b, K, len(loads), expert_bytes, h2d_gb_per_s, draft_us_per_token)
        chunks.append((b, nb, OVERLAP if nb < K else CLEANUP))
        observe(b, nb)
        b = nb
    return {"chunks": chunks, "boundaries": boundaries}
