"""One MoE layer on the device: the libsmoe calls in order.

DeviceLayer holds the device copies of one layer's inputs (any object with
the attributes of workload.LayerInputs) and the output / scratch buffers,
and enqueues route -> align -> [ELB] -> expert FFN -> combine on a stream.
It only sequences calls of the HIP library and allocates buffers; all
arithmetic happens in the library.

Draft pass: INT4 (W4A16) routed experts (Specter paper, fused multi-expert
draft kernel paragraph). Target pass: FP16 routed experts with the same
expert-centric gather/scatter (expert-wise verification paragraphs). The
always-on shared experts are FP16 in both (hybrid-precision layout). By
default they run inside the routed FFN's two launches, so one weight stream
covers routed and shared experts; run(fuse_shared=False) runs them as a
call of their own instead, optionally on a side stream (they depend only on
x).
"""

from __future__ import annotations

import copy
from typing import Optional

import numpy as np
import torch

from . import _lib


def _dev(a: Optional[np.ndarray], device) -> Optional[torch.Tensor]:
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(device)


class DeviceLayer:
    def __init__(self, inp, device="cuda", elb_layers: int = 1, with_target: Optional[bool] = None,
                 tiled: bool = False):
        """tiled: hold every expert weight (routed INT4, FP16 target, FP16
        shared) in the tiled layout of smoe_tile_weights, tiled once here on
        the device, and run the *_tiled library calls."""
        cfg = inp.cfg
        self.cfg = cfg
        self.device = torch.device(device)
        d = self.device
        T, k, E, H, I = cfg.T, cfg.k, cfg.E, cfg.H, cfg.I
        S = T * k
        self.x = _dev(inp.x, d)
        self.w_router = _dev(inp.w_router, d)
        self.router_bias = _dev(inp.router_bias, d)
        self.shared_gate_w = _dev(inp.shared_gate_w, d)
        self.wg_q, self.wg_s = _dev(inp.wg_q, d), _dev(inp.wg_s, d)
        self.wu_q, self.wu_s = _dev(inp.wu_q, d), _dev(inp.wu_s, d)
        self.wd_q, self.wd_s = _dev(inp.wd_q, d), _dev(inp.wd_s, d)
        if with_target is None:
            with_target = inp.wg16 is not None
        self.wg16 = _dev(inp.wg16, d) if with_target else None
        self.wu16 = _dev(inp.wu16, d) if with_target else None
        self.wd16 = _dev(inp.wd16, d) if with_target else None
        self.sg16, self.su16, self.sd16 = (_dev(inp.sg16, d), _dev(inp.su16, d),
                                          _dev(inp.sd16, d))
        Is = self.sg16.shape[0] if self.sg16 is not None else 0
        self.shared_I = Is
        self.tiled = bool(tiled)
        if self.tiled:
            G = cfg.G
            self.wg_q, self.wg_s = self._tile(self.wg_q, self.wg_s, E, I, H, G)
            self.wu_q, self.wu_s = self._tile(self.wu_q, self.wu_s, E, I, H, G)
            self.wd_q, self.wd_s = self._tile(self.wd_q, self.wd_s, E, H, I, G)
            if self.wg16 is not None:
                self.wg16 = self._tile(self.wg16, None, E, I, H, 0)[0]
                self.wu16 = self._tile(self.wu16, None, E, I, H, 0)[0]
                self.wd16 = self._tile(self.wd16, None, E, H, I, 0)[0]
            if Is:
                self.sg16 = self._tile(self.sg16, None, 1, Is, H, 0)[0]
                self.su16 = self._tile(self.su16, None, 1, Is, H, 0)[0]
                self.sd16 = self._tile(self.sd16, None, 1, H, Is, 0)[0]
            torch.cuda.synchronize(d)

        i32 = dict(dtype=torch.int32, device=d)
        f32 = dict(dtype=torch.float32, device=d)
        self.topk_ids = torch.empty((T, k), **i32)
        self.topk_w = torch.empty((T, k), **f32)
        self.logits = torch.empty((T, E), **f32)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.sorted_slots = torch.empty(S, **i32)
        self.active = torch.empty(E, **i32)
        self.n_active = torch.empty(1, **i32)
        # zero-filled once; the FFN calls keep it consistent from then on. A
        # workspace serves one (T, k, I, shared_I): the routed calls with the
        # shared experts fused use this one, those without them their own
        ws = _lib.smoe_ffn_workspace_bytes(T, k, E, H, I, Is)
        self.workspace = torch.zeros(ws, dtype=torch.uint8, device=d)
        self.routed_ws = (torch.zeros(_lib.smoe_ffn_workspace_bytes(T, k, E, H, I, 0),
                                      dtype=torch.uint8, device=d) if Is else self.workspace)
        self.slot_out = torch.empty((S, H), **f32)
        self.y = torch.empty((T, H), dtype=torch.float16, device=d)
        self.shared_gate = torch.empty(T, **f32) if self.shared_gate_w is not None else None
        if Is:
            self.shared_out = torch.empty((T, H), **f32)
            # for the separate shared-expert call (E = 1, every token once)
            self.shared_ws = torch.zeros(_lib.smoe_ffn_workspace_bytes(T, 1, 1, H, Is),
                                         dtype=torch.uint8, device=d)
            self.shared_slots = torch.arange(T, **i32)
            self.shared_offsets = torch.tensor([0, T], **i32)
        else:
            self.shared_out = None
        self.elb_counts = torch.zeros((elb_layers, E), **i32)
        M = max(cfg.elb_M, 0)
        self.plan_ids = torch.empty((elb_layers, max(M, 1)), **i32)
        self.plan_counts = torch.empty((elb_layers, max(M, 1)), **i32)

    @staticmethod
    def _tile(w, s, E, N, K, G):
        wt = torch.empty_like(w)
        st = torch.empty_like(s) if s is not None else None
        _lib.smoe_tile_weights(w, s, E, N, K, G, wt, st)
        return wt, st

    def _call(self, name: str):
        """The library call `name`, or its tiled-layout form."""
        return getattr(_lib, name + "_tiled" if self.tiled else name)

    _WEIGHTS = ("w_router", "router_bias", "shared_gate_w", "wg_q", "wg_s", "wu_q", "wu_s",
                "wd_q", "wd_s", "wg16", "wu16", "wd16", "sg16", "su16", "sd16")

    def weight_bytes(self) -> int:
        """Device bytes held by this layer's weights (router, routed, shared)."""
        return sum(t.numel() * t.element_size() for t in
                   (getattr(self, n) for n in self._WEIGHTS) if t is not None)

    def with_weight_copy(self) -> "DeviceLayer":
        """A runner over fresh device copies of every weight tensor.

        Inputs, outputs and scratch buffers are shared with this runner (so
        the two must not run concurrently); only the weights get new
        addresses. Used to rotate several copies so that each call reads its
        weights from HBM rather than from a cache holding the previous call's.
        """
        other = copy.copy(self)
        for n in self._WEIGHTS:
            t = getattr(self, n)
            if t is not None:
                setattr(other, n, t.clone())
        return other

    # ---------------------------------------------------------------- steps
    def route(self, stream=None) -> None:
        _lib.smoe_route_topk(self.x, self.w_router, self.router_bias, self.cfg.k, 0,
                             self.topk_ids, self.topk_w, self.logits,
                             self.shared_gate_w, self.shared_gate, stream=stream)

    def route_align_elb(self, elb: bool = True, layer: int = 0, rank: bool = True,
                        stream=None) -> None:
        """route, align and (with elb) the ELB update of `layer` in one call;
        with rank, also the top-M plan of every layer of the counter."""
        M = self.cfg.elb_M if elb and rank else 0
        _lib.smoe_route_align_elb(self.x, self.w_router, self.router_bias, self.cfg.k, 0,
                                  self.topk_ids, self.topk_w, self.logits,
                                  self.shared_gate_w, self.shared_gate, self.counts,
                                  self.offsets, self.sorted_slots, self.active, self.n_active,
                                  elb_counts=self.elb_counts if elb else None, layer=layer, M=M,
                                  plan_ids=self.plan_ids if M > 0 else None,
                                  plan_counts=self.plan_counts if M > 0 else None,
                                  stream=stream)

    def align(self, stream=None) -> None:
        _lib.smoe_align_by_expert(self.topk_ids, self.cfg.E, self.counts, self.offsets,
                                  self.sorted_slots, self.active, self.n_active, stream=stream)

    def elb(self, layer: int = 0, M: Optional[int] = None, flags: int = 0, stream=None,
            accumulate: bool = True) -> None:
        """Add this window's IDs to row `layer` of the counter (unless not
        accumulate) and rank every layer's top-M (M = 0: no ranking)."""
        M = self.cfg.elb_M if M is None else M
        _lib.smoe_elb_accumulate_topm(self.elb_counts, self.topk_ids[None] if accumulate else None,
                                      layer, M,
                                      self.plan_ids if M > 0 else None,
                                      self.plan_counts if M > 0 else None, flags, stream=stream)

    def routed_ffn(self, target: bool = False, with_shared: bool = True, stream=None) -> None:
        """Routed experts (INT4 draft, or FP16 target) and, with_shared, the
        shared experts in the same two launches."""
        c = self.cfg
        shared = shared_out = None
        if with_shared and self.shared_out is not None:
            shared = (self.sg16, self.su16, self.sd16)
            shared_out = self.shared_out
        ws = self.workspace if shared is not None else self.routed_ws
        if target:
            self._call("smoe_fp16_expert_ffn")(self.x, c.k, c.E, c.I, self.wg16, self.wu16, self.wd16,
                                      self.sorted_slots, self.offsets, ws,
                                      self.slot_out, shared=shared, shared_out=shared_out,
                                      stream=stream)
        else:
            self._call("smoe_w4a16_expert_ffn")(self.x, c.k, c.E, c.I, c.G, self.wg_q, self.wg_s,
                                       self.wu_q, self.wu_s, self.wd_q, self.wd_s,
                                       self.sorted_slots, self.offsets, ws,
                                       self.slot_out, shared=shared, shared_out=shared_out,
                                       stream=stream)

    def shared_ffn(self, stream=None) -> None:
        """The shared experts alone: an FP16 FFN call with one expert that
        every token uses once."""
        if self.shared_out is None:
            return
        self._call("smoe_fp16_expert_ffn")(self.x, 1, 1, self.shared_I, self.sg16, self.su16, self.sd16,
                                  self.shared_slots, self.shared_offsets, self.shared_ws,
                                  self.shared_out, stream=stream)

    def combine(self, stream=None) -> None:
        _lib.smoe_combine(self.slot_out, self.topk_w, self.shared_out, self.shared_gate,
                          self.y, stream=stream)

    def layer_call(self, elb: bool = True, layer: int = 0, rank: bool = True,
                   stream=None) -> None:
        """The whole draft layer as one library call (smoe_moe_layer_w4a16),
        which checks every step's arguments before it enqueues anything."""
        c = self.cfg
        M = c.elb_M if elb and rank else 0
        shared = shared_out = None
        if self.shared_out is not None:
            shared = (self.sg16, self.su16, self.sd16)
            shared_out = self.shared_out
        self._call("smoe_moe_layer_w4a16")(
            self.x, self.w_router, self.router_bias, c.k, 0, self.topk_ids, self.topk_w,
            self.logits, self.shared_gate_w, self.shared_gate, self.counts, self.offsets,
            self.sorted_slots, self.active, self.n_active,
            self.elb_counts if elb else None, layer, M,
            self.plan_ids if M > 0 else None, self.plan_counts if M > 0 else None, 0,
            c.I, c.G, self.wg_q, self.wg_s, self.wu_q, self.wu_s, self.wd_q, self.wd_s,
            self.workspace, self.slot_out, self.y, shared=shared, shared_out=shared_out,
            stream=stream)

    # ---------------------------------------------------------------- whole layer
    def run(self, target: bool = False, elb: bool = True, fuse_shared: bool = True,
            fuse_routing: bool = True, side_stream=None, one_call: bool = False,
            layer: int = 0, rank: bool = True) -> None:
        """Enqueue the whole layer on the current stream.

        The ELB update adds this window's IDs to row `layer` of the counter;
        with rank it also writes every layer's top-M plan (a stack of layers
        can accumulate with rank=False and rank once at the end).

        one_call runs the draft layer as the single library call
        smoe_moe_layer_w4a16 (shared experts fused, no side stream).

        fuse_routing makes routing, alignment and the ELB update one call
        (smoe_route_align_elb); otherwise they are three. fuse_shared runs
        the shared experts inside the routed FFN call; otherwise they get a
        call of their own. With side_stream, the work off the layer's
        critical path runs there: the ELB update when routing is not fused
        (it needs only the routing) and a separate shared-expert call (it
        needs only x). The side stream forks from the current stream and
        joins it again before the layer ends (before the combine for the
        shared experts).
        """
        separate = not fuse_shared and self.shared_out is not None
        use_elb = elb and self.cfg.elb_M > 0 and not target
        if one_call:
            if target or separate or side_stream is not None:
                raise ValueError("one_call covers the draft layer with fused shared experts")
            self.layer_call(elb=use_elb, layer=layer, rank=rank)
            return
        main = torch.cuda.current_stream(self.device)
        side = side_stream

        def fork():
            ev = torch.cuda.Event()
            ev.record(main)
            side.wait_event(ev)

        def join():
            ev = torch.cuda.Event()
            ev.record(side)
            main.wait_event(ev)

        if separate:
            if side is not None:
                fork()
                self.shared_ffn(stream=side)
            else:
                self.shared_ffn()
        shared_done = None
        if separate and side is not None:
            shared_done = torch.cuda.Event()
            shared_done.record(side)
        side_elb = False
        if fuse_routing:
            self.route_align_elb(elb=use_elb, layer=layer, rank=rank)
        else:
            self.route()
            if use_elb:
                M = None if rank else 0
                if side is not None:
                    fork()
                    self.elb(layer=layer, M=M, stream=side)
                    side_elb = True
                else:
                    self.elb(layer=layer, M=M)
            self.align()
        self.routed_ffn(target=target, with_shared=not separate)
        if shared_done is not None:
            main.wait_event(shared_done)
        self.combine()
        if side is not None and (separate or side_elb):
            join()
