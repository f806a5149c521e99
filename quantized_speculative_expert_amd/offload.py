"""A speculative window over a stack whose FP16 target experts live in host
memory: the draft proposes K tokens one by one through L draft layers (INT4
experts resident in HBM) while the activation counters (ELB) accumulate;
at chunk boundaries the prefetch planner copies the predicted FP16 experts
into the per-layer slot cache; then the target verifies the K+1 window
layer by layer with the cache (resident experts first, misses as their
copies land) and combines.

Specter paper: Incremental Routing Pattern Analyzer, Layer-Aware Prefetch
Planner, Verification Expert Cache Residency Manager, cache-aware execution
schedule and Overlap-Oriented Parallelism Optimizer paragraphs; Design page,
"Predictive I/O Orchestrator".

This module only sequences libsmoe calls (routing, ELB, FFNs, combine, the
cache's decisions, copies and events) and allocates buffers; every step of
the computation and every residency decision runs in the library.
"""

from __future__ import annotations

import copy
import dataclasses
import time
from typing import Dict, List, Optional

import numpy as np
import torch

from . import _lib
from .layer import DeviceLayer

COLD, OVERLAP, CLEANUP = 0, 1, 2


def _fp16_experts(E: int, I: int, H: int, gen: torch.Generator, device, tiled: bool,
                  std: float = 0.02) -> torch.Tensor:
    """FP16 target experts of one layer as [E][3][I*H] (wg, wu, wd; each
    matrix tiled on its own when `tiled`), generated on the device."""
    out = torch.empty((E, 3, I * H), dtype=torch.float16, device=device)
    for j, (n, k) in enumerate(((I, H), (I, H), (H, I))):
        w = (torch.randn((E, n, k), generator=gen, device=device) * std).to(torch.float16)
        if tiled:
            t = torch.empty_like(w)
            _lib.smoe_tile_weights(w, None, E, n, k, 0, t)
            w = t
        out[:, j] = w.reshape(E, -1)
    return out


class OffloadStack:
    """L MoE layers of one shape (cfg: T = K + 1 tokens in the verification
    window) with an expert cache of M slots per layer."""

    def __init__(self, cfg, draft_inp, L: int, M: int, zipf: Optional[List[np.ndarray]] = None,
                 routers: Optional[List[np.ndarray]] = None, seed: int = 0, tiled: bool = True,
                 device="cuda"):
        """draft_inp: workload.LayerInputs of the single-token draft layer
        (cfg with T = 1): its INT4 experts and shared experts serve every
        layer of the stack; routers[l] / zipf[l] give each layer its own
        router (and optional logit bias)."""
        self.cfg, self.L, self.M = cfg, L, M
        self.K = cfg.T - 1
        self.device = torch.device(device)
        self.tiled = tiled
        d = self.device
        E, I, H, k, T = cfg.E, cfg.I, cfg.H, cfg.k, cfg.T
        # draft layers: one set of INT4 experts, a router per layer, one
        # counter [L][E] and one top-M plan for the whole stack
        base = DeviceLayer(draft_inp, device=d, elb_layers=L, with_target=False, tiled=tiled)
        self.elb_counts = base.elb_counts
        self.plan_ids = torch.empty((L, M), dtype=torch.int32, device=d)
        self.plan_counts = torch.empty((L, M), dtype=torch.int32, device=d)
        self.draft: List[DeviceLayer] = []
        for l in range(L):
            dl = copy.copy(base)
            if routers is not None:
                dl.w_router = torch.from_numpy(np.ascontiguousarray(routers[l])).to(d)
            dl.router_bias = (torch.from_numpy(np.ascontiguousarray(zipf[l])).to(d)
                              if zipf is not None else base.router_bias)
            dl.plan_ids, dl.plan_counts = self.plan_ids, self.plan_counts
            self.draft.append(dl)
        # target: FP16 experts in pinned host memory, [L][E][3][I*H]
        self.expert_bytes = 3 * I * H * 2
        gen = torch.Generator(device=d)
        gen.manual_seed(seed)
        self.host = torch.empty((L, E, 3, I * H), dtype=torch.float16, pin_memory=True)
        for l in range(L):
            self.host[l].copy_(_fp16_experts(E, I, H, gen, d, tiled))
        torch.cuda.synchronize(d)
        self.pool = torch.zeros((L, M, 3, I * H), dtype=torch.float16, device=d)
        self.cache = _lib.smoe_cache_create(L, E, M, self.expert_bytes, self.pool, self.host)
        self.copy_stream = torch.cuda.Stream(device=d)
        # target window buffers (one layer at a time)
        i32 = dict(dtype=torch.int32, device=d)
        f32 = dict(dtype=torch.float32, device=d)
        S = T * k
        self.t_ids = torch.empty((T, k), **i32)
        self.t_w = torch.empty((T, k), **f32)
        self.t_logits = torch.empty((T, E), **f32)
        self.t_counts = torch.empty(E, **i32)
        self.t_offsets = torch.empty(E + 1, **i32)
        self.t_slots = torch.empty(S, **i32)
        self.t_active = torch.empty(E, **i32)
        self.t_nact = torch.empty(1, **i32)
        self.slot_out = torch.empty((S, H), **f32)
        self.Is = base.shared_I
        self.shared = (base.sg16, base.su16, base.sd16) if self.Is else None
        self.shared_out = torch.empty((T, H), **f32) if self.Is else None
        u8 = dict(dtype=torch.uint8, device=d)
        self.ws_routed = torch.zeros(_lib.smoe_ffn_workspace_bytes(T, k, E, H, I, 0), **u8)
        self.ws_shared = (torch.zeros(_lib.smoe_ffn_workspace_bytes(T, k, E, H, I, self.Is), **u8)
                          if self.Is else None)
        self.y = torch.empty((L, T, H), dtype=torch.float16, device=d)
        self.counts_host = torch.empty(E, dtype=torch.int32, pin_memory=True)
        self.plan_host = torch.empty((2, L, M), dtype=torch.int32, pin_memory=True)

    def close(self) -> None:
        torch.cuda.synchronize(self.device)
        if self.cache:
            _lib.smoe_cache_destroy(self.cache)
            self.cache = None

    # ------------------------------------------------------------------ draft
    def draft_token(self, x_draft: torch.Tensor, i: int,
                    record: Optional[torch.Tensor] = None) -> None:
        """Draft token i through every layer: routing with the ELB update of
        that layer's counter row, the W4A16 FFN (with the shared experts) and
        the combine. x_draft: fp16 [L][K][H] draft activations; record
        (optional, int32 [K][L][k] on the device) keeps the draft's expert IDs."""
        for l, dl in enumerate(self.draft):
            dl.x = x_draft[l, i:i + 1]
            dl.route_align_elb(elb=True, layer=l, rank=False)
            if record is not None:
                record[i, l].copy_(dl.topk_ids[0])
            dl.routed_ffn()
            dl.combine()

    def snapshot(self):
        """Top-M plan of every layer (ELB ranking on the device, copied back)."""
        _lib.smoe_elb_accumulate_topm(self.elb_counts, None, 0, self.M, self.plan_ids,
                                      self.plan_counts, 0)
        self.plan_host[0].copy_(self.plan_ids, non_blocking=True)
        self.plan_host[1].copy_(self.plan_counts, non_blocking=True)
        torch.cuda.current_stream(self.device).synchronize()
        return self.plan_host[0].numpy().copy(), self.plan_host[1].numpy().copy()

    def draft_window(self, x_draft: torch.Tensor, planner: bool, b1: int,
                     h2d_gb_per_s: float, draft_us_per_token: float,
                     record: Optional[torch.Tensor] = None) -> Dict:
        """The K draft tokens, with (planner=True) the ELB-driven prefetch at
        chunk boundaries. Ends with the counters cleared."""
        K = self.K
        _lib.smoe_cache_begin_window(self.cache)
        b = min(max(b1, 0), K) if planner else K
        chunks, loads_per_boundary = [(0, b, COLD)], []
        for i in range(b):
            self.draft_token(x_draft, i, record)
        while b < K:
            ids, cnts = self.snapshot()
            loads, full = _lib.smoe_cache_prefetch(self.cache, ids, cnts, self.L, self.M,
                                                   copy_stream=self.copy_stream)
            loads_per_boundary.append((b, loads))
            if full:
                nb, phase = K, CLEANUP
            else:
                nb = _lib.smoe_prefetch_next_boundary(b, K, len(loads), self.expert_bytes,
                                                      h2d_gb_per_s, draft_us_per_token)
                phase = OVERLAP if nb < K else CLEANUP
            chunks.append((b, nb, phase))
            for i in range(b, nb):
                self.draft_token(x_draft, i, record)
            b = nb
        # the final chunk's routing is not used: the counters start the next
        # window at zero
        _lib.smoe_elb_accumulate_topm(self.elb_counts, None, 0, 0, None, None,
                                      _lib.SMOE_ELB_CLEAR_AFTER)
        return {"chunks": chunks, "loads": loads_per_boundary}

    # ------------------------------------------------------------ verification
    def verify_layer(self, l: int, x_target: torch.Tensor) -> np.ndarray:
        """Target routing of layer l over the window, then the cached FFN and
        the combine into y[l]. Returns the cache's schedule."""
        dl = self.draft[l]
        _lib.smoe_route_align_elb(x_target, dl.w_router, dl.router_bias, self.cfg.k, 0,
                                  self.t_ids, self.t_w, self.t_logits, None, None,
                                  self.t_counts, self.t_offsets, self.t_slots, self.t_active,
                                  self.t_nact)
        self.counts_host.copy_(self.t_counts, non_blocking=True)
        torch.cuda.current_stream(self.device).synchronize()
        sched = _lib.smoe_cache_verify_layer(
            self.cache, l, self.counts_host.numpy(), x_target, self.cfg.k, self.cfg.I,
            self.t_slots, self.t_offsets, self.ws_shared, self.ws_routed, self.slot_out,
            shared=self.shared, shared_out=self.shared_out, tiled=self.tiled,
            copy_stream=self.copy_stream)
        _lib.smoe_combine(self.slot_out, self.t_w, self.shared_out, None, self.y[l])
        return sched

    def verify_window(self, x_target: torch.Tensor) -> List[np.ndarray]:
        return [self.verify_layer(l, x_target[l]) for l in range(self.L)]


def measure_h2d(device, mib: int = 256, reps: int = 3) -> float:
    """Pinned host to device copy bandwidth in GB/s (best of reps)."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(n, dtype=torch.uint8, device=device)
    best = 0.0
    for _ in range(reps):
        torch.cuda.synchronize(device)
        t0 = time.perf_counter()
        dst.copy_(src, non_blocking=True)
        torch.cuda.synchronize(device)
        best = max(best, n / (time.perf_counter() - t0) / 1e9)
    return best
