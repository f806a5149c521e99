"""ctypes binding of libsmoe (argument marshalling only).

Each function has the name of the C entry point it calls and takes torch
tensors for device memory (plus an optional torch stream); it checks dtypes,
devices and contiguity, passes raw pointers and sizes, and raises SmoeError
on a non-zero status. Every step of the computation runs in the HIP library.
If the library is missing or cannot be loaded, importing this module fails.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libsmoe.so not found at {LIB_PATH}; build it first with "
        "`python -m quantized_speculative_expert_amd.build` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t

_SIGNATURES = {
    "smoe_abi_version": (_i, []),
    "smoe_status_string": (ctypes.c_char_p, [_i]),
    "smoe_last_error": (ctypes.c_char_p, []),
    "smoe_route_topk": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p]),
    "smoe_align_by_expert": (_i, [_p, _i, _i, _i, _p, _p, _p, _p, _p, _p]),
    "smoe_route_align_elb": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p,
                                  _p, _p, _p, _p, _p, _p, _i, _i, _i, _p, _p, _i, _p]),
    "smoe_elb_accumulate_topm": (_i, [_p, _i, _i, _p, _i, _i, _i, _i, _i, _p, _p, _i, _p]),
    "smoe_ffn_workspace_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "smoe_w4a16_expert_ffn": (_i, [_p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p,
                                   _p, _p, _i, _p, _p, _p, _p, _sz, _p, _p, _p]),
    "smoe_fp16_expert_ffn": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _i, _p, _p, _p,
                                  _p, _sz, _p, _p, _p]),
    "smoe_combine": (_i, [_p, _p, _i, _i, _i, _p, _p, _p, _p]),
    "smoe_moe_layer_w4a16": (_i, [_p, _p, _p, _i, _i, _i, _i, _i,      # x .. flags
                                  _p, _p, _p, _p, _p,                  # topk_ids .. shared_gate
                                  _p, _p, _p, _p, _p,                  # counts .. n_active
                                  _p, _i, _i, _i, _p, _p, _i,          # elb_counts .. elb_flags
                                  _i, _i, _p, _p, _p, _p, _p, _p,      # I, G, routed weights
                                  _i, _p, _p, _p,                      # shared_I, shared weights
                                  _p, _sz, _p, _p, _p, _p]),           # workspace .. stream
    "smoe_tile_weights": (_i, [_p, _p, _i, _i, _i, _i, _p, _p, _p]),
    "smoe_w4a16_expert_ffn_noalloc": (_i, [_p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p,
                                           _p, _p, _i, _p, _p, _p, _p, _p, _p]),
    "smoe_fp16_expert_ffn_mapped": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p, _i, _i, _p,
                                         _p, _p, _i, _p, _p, _p, _p, _sz, _p, _p, _p]),
    "smoe_ffn_workspace_clear": (_i, [_p, _sz, _p]),
    "smoe_cache_create": (_i, [_i, _i, _i, _sz, _p, _p, _p]),
    "smoe_cache_destroy": (_i, [_p]),
    "smoe_cache_begin_window": (_i, [_p]),
    "smoe_cache_state": (_i, [_p, _p, _p, _p, _p]),
    "smoe_cache_set_state": (_i, [_p, _p, _p, ctypes.c_int64, _p]),
    "smoe_cache_prefetch": (_i, [_p, _p, _p, _i, _p, _p, _p, _p]),
    "smoe_prefetch_next_boundary": (_i, [_i, _i, _i, ctypes.c_double, ctypes.c_double,
                                         ctypes.c_double, _p]),
    "smoe_cache_verify_plan": (_i, [_p, _i, _p, _p, _p]),
    "smoe_specfit_select": (_i, [_i, _p, _p, _i, _i, _p, _p, _i, _p, ctypes.c_double, _p, _p,
                                 _p, _p]),
    "smoe_cache_verify_layer": (_i, [_p, _i, _p, _p, _i, _i, _i, _i, _i, _p, _p, _i, _p, _p, _p,
                                     _p, _sz, _p, _sz, _p, _p, _p, _p, _p, _p]),
}
# the tiled-layout calls take the same arguments as their row-major forms
for _name in ("smoe_w4a16_expert_ffn", "smoe_fp16_expert_ffn", "smoe_moe_layer_w4a16"):
    _SIGNATURES[_name + "_tiled"] = _SIGNATURES[_name]

for _name, (_res, _args) in _SIGNATURES.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

SMOE_OK = 0
SMOE_EINVAL = -1
SMOE_EUNSUPPORTED = -2
SMOE_EHIP = -3
SMOE_ROUTE_RENORM = 1
SMOE_ELB_CLEAR_AFTER = 1


class SmoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        detail = _lib.smoe_last_error().decode()
        super().__init__(f"{fn}: {_lib.smoe_status_string(status).decode()} ({detail})")


def exported_symbols():
    return sorted(_SIGNATURES)


def _check(fn: str, status: int) -> None:
    if status != SMOE_OK:
        raise SmoeError(fn, status)


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor") -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.data_ptr() if t.numel() else None


def _need(t: Optional[torch.Tensor], n: int, name: str) -> None:
    """The library reads or writes n elements behind t's pointer: refuse a
    smaller tensor here, before a kernel could run off its end."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {n}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def smoe_abi_version() -> int:
    return int(_lib.smoe_abi_version())


def smoe_ffn_workspace_bytes(T: int, k: int, E: int, H: int, I: int, shared_I: int = 0) -> int:
    return int(_lib.smoe_ffn_workspace_bytes(T, k, E, H, I, shared_I))


def _shared_args(shared, shared_out):
    """(shared_I, wg, wu, wd, out) pointers of the optional shared expert."""
    if shared is None:
        if shared_out is not None:
            raise ValueError("shared_out given without shared-expert weights")
        return 0, None, None, None, None
    sg, su, sd = shared
    if sg.dim() != 2 or su.shape != sg.shape or sd.dim() != 2 or sd.shape[1] != sg.shape[0]:
        raise ValueError("shared weights must be wg, wu [shared_I][H] and wd [H][shared_I]")
    return (sg.shape[0], _ptr(sg, torch.float16, "shared_wg"), _ptr(su, torch.float16, "shared_wu"),
            _ptr(sd, torch.float16, "shared_wd"), _ptr(shared_out, torch.float32, "shared_out"))


def _route_sizes(T, H, E, k, w_router, logit_bias, topk_ids, topk_w, logits, shared_gate_w,
                 shared_gate) -> None:
    _need(w_router, E * H, "w_router")
    _need(logit_bias, E, "logit_bias")
    _need(topk_ids, T * k, "topk_ids")
    _need(topk_w, T * k, "topk_w")
    _need(logits, T * E, "logits")
    _need(shared_gate_w, H, "shared_gate_w")
    _need(shared_gate, T, "shared_gate")


def _align_sizes(S, E, counts, offsets, sorted_slots, active, n_active) -> None:
    _need(counts, E, "expert_counts")
    _need(offsets, E + 1, "expert_offsets")
    _need(sorted_slots, S, "sorted_slots")
    _need(active, E, "active_experts")
    _need(n_active, 1, "n_active")


def smoe_route_topk(x, w_router, logit_bias, k: int, flags: int, topk_ids, topk_w, logits,
                    shared_gate_w=None, shared_gate=None, stream=None) -> None:
    T, H = x.shape
    E = w_router.shape[0]
    _route_sizes(T, H, E, k, w_router, logit_bias, topk_ids, topk_w, logits, shared_gate_w,
                 shared_gate)
    _check("smoe_route_topk", _lib.smoe_route_topk(
        _ptr(x, torch.float16, "x"), _ptr(w_router, torch.float32, "w_router"),
        _ptr(logit_bias, torch.float32, "logit_bias"), T, H, E, k, flags,
        _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_w, torch.float32, "topk_w"),
        _ptr(logits, torch.float32, "logits"),
        _ptr(shared_gate_w, torch.float32, "shared_gate_w"),
        _ptr(shared_gate, torch.float32, "shared_gate"), _stream(stream)))


def smoe_route_align_elb(x, w_router, logit_bias, k: int, flags: int, topk_ids, topk_w, logits,
                         shared_gate_w, shared_gate, expert_counts, expert_offsets, sorted_slots,
                         active_experts, n_active, elb_counts=None, layer: int = 0, M: int = 0,
                         plan_ids=None, plan_counts=None, elb_flags: int = 0,
                         stream=None) -> None:
    """smoe_route_topk, smoe_align_by_expert and (with elb_counts [L][E])
    smoe_elb_accumulate_topm for layer `layer`, in one call."""
    T, H = x.shape
    E = w_router.shape[0]
    L = elb_counts.shape[0] if elb_counts is not None else 0
    _route_sizes(T, H, E, k, w_router, logit_bias, topk_ids, topk_w, logits, shared_gate_w,
                 shared_gate)
    _align_sizes(T * k, E, expert_counts, expert_offsets, sorted_slots, active_experts, n_active)
    _need(elb_counts, L * E, "elb_counts")
    _need(plan_ids, L * M, "plan_ids")
    _need(plan_counts, L * M, "plan_counts")
    _check("smoe_route_align_elb", _lib.smoe_route_align_elb(
        _ptr(x, torch.float16, "x"), _ptr(w_router, torch.float32, "w_router"),
        _ptr(logit_bias, torch.float32, "logit_bias"), T, H, E, k, flags,
        _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_w, torch.float32, "topk_w"),
        _ptr(logits, torch.float32, "logits"),
        _ptr(shared_gate_w, torch.float32, "shared_gate_w"),
        _ptr(shared_gate, torch.float32, "shared_gate"),
        _ptr(expert_counts, torch.int32, "expert_counts"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"),
        _ptr(sorted_slots, torch.int32, "sorted_slots"),
        _ptr(active_experts, torch.int32, "active_experts"),
        _ptr(n_active, torch.int32, "n_active"),
        _ptr(elb_counts, torch.int32, "elb_counts"), L, layer, M,
        _ptr(plan_ids, torch.int32, "plan_ids"), _ptr(plan_counts, torch.int32, "plan_counts"),
        elb_flags, _stream(stream)))


def smoe_align_by_expert(topk_ids, E: int, expert_counts, expert_offsets, sorted_slots,
                         active_experts, n_active, stream=None) -> None:
    T, k = topk_ids.shape
    _align_sizes(T * k, E, expert_counts, expert_offsets, sorted_slots, active_experts, n_active)
    _check("smoe_align_by_expert", _lib.smoe_align_by_expert(
        _ptr(topk_ids, torch.int32, "topk_ids"), T, k, E,
        _ptr(expert_counts, torch.int32, "expert_counts"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"),
        _ptr(sorted_slots, torch.int32, "sorted_slots"),
        _ptr(active_experts, torch.int32, "active_experts"),
        _ptr(n_active, torch.int32, "n_active"), _stream(stream)))


def smoe_elb_accumulate_topm(elb_counts, topk_ids, layer_begin: int, M: int, plan_ids,
                             plan_counts=None, flags: int = 0, stream=None) -> None:
    """topk_ids: int32 [n_layers][T][k] or None (rank only)."""
    L, E = elb_counts.shape
    if topk_ids is not None:
        n_layers, T, k = topk_ids.shape
    else:
        n_layers, T, k = 0, 0, 1
    _need(plan_ids, L * M, "plan_ids")
    _need(plan_counts, L * M, "plan_counts")
    _check("smoe_elb_accumulate_topm", _lib.smoe_elb_accumulate_topm(
        _ptr(elb_counts, torch.int32, "elb_counts"), L, E,
        _ptr(topk_ids, torch.int32, "topk_ids"), layer_begin, n_layers, T, k, M,
        _ptr(plan_ids, torch.int32, "plan_ids"), _ptr(plan_counts, torch.int32, "plan_counts"),
        flags, _stream(stream)))


def _ffn_sizes(T, k, E, H, sI, sorted_slots, expert_offsets, slot_out, shared, shared_out):
    _need(sorted_slots, T * k, "sorted_slots")
    _need(expert_offsets, E + 1, "expert_offsets")
    _need(slot_out, T * k * H, "slot_out")
    if shared is not None:
        for name, t in zip(("shared_wg", "shared_wu", "shared_wd"), shared):
            _need(t, sI * H, name)
        _need(shared_out, T * H, "shared_out")


def smoe_w4a16_expert_ffn(x, k: int, E: int, I: int, group_size: int, wg_q, wg_s, wu_q, wu_s,
                          wd_q, wd_s, sorted_slots, expert_offsets, workspace, slot_out,
                          shared=None, shared_out=None, stream=None, *, _fn="") -> None:
    """shared: optional (wg, wu, wd) fp16 weights of the always-on shared expert."""
    fname = _fn or "smoe_w4a16_expert_ffn"
    T, H = x.shape
    sI, sg, su, sd, so = _shared_args(shared, shared_out)
    G = max(group_size, 1)
    for name, t in (("wg_q", wg_q), ("wu_q", wu_q)):
        _need(t, E * I * H // 8, name)
    for name, t in (("wg_s", wg_s), ("wu_s", wu_s)):
        _need(t, E * I * H // G, name)
    _need(wd_q, E * H * I // 8, "wd_q")
    _need(wd_s, E * H * I // G, "wd_s")
    _ffn_sizes(T, k, E, H, sI, sorted_slots, expert_offsets, slot_out, shared, shared_out)
    _check(fname, getattr(_lib, fname)(
        _ptr(x, torch.float16, "x"), T, k, E, H, I, group_size,
        _ptr(wg_q, torch.int32, "wg_q"), _ptr(wg_s, torch.float16, "wg_s"),
        _ptr(wu_q, torch.int32, "wu_q"), _ptr(wu_s, torch.float16, "wu_s"),
        _ptr(wd_q, torch.int32, "wd_q"), _ptr(wd_s, torch.float16, "wd_s"),
        _ptr(sorted_slots, torch.int32, "sorted_slots"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"), sI, sg, su, sd,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _ptr(slot_out, torch.float32, "slot_out"), so, _stream(stream)))


SMOE_NOALLOC_SCRATCH_BYTES = 16 << 20


def smoe_w4a16_expert_ffn_noalloc(x, k: int, E: int, I: int, group_size: int, wg_q, wg_s, wu_q,
                                  wu_s, wd_q, wd_s, sorted_slots, expert_offsets, slot_out,
                                  shared=None, shared_out=None, stream=None) -> None:
    """smoe_w4a16_expert_ffn with the library's static workspace (no
    workspace argument; the call allocates nothing)."""
    T, H = x.shape
    sI, sg, su, sd, so = _shared_args(shared, shared_out)
    G = max(group_size, 1)
    for name, t in (("wg_q", wg_q), ("wu_q", wu_q)):
        _need(t, E * I * H // 8, name)
    for name, t in (("wg_s", wg_s), ("wu_s", wu_s)):
        _need(t, E * I * H // G, name)
    _need(wd_q, E * H * I // 8, "wd_q")
    _need(wd_s, E * H * I // G, "wd_s")
    _ffn_sizes(T, k, E, H, sI, sorted_slots, expert_offsets, slot_out, shared, shared_out)
    _check("smoe_w4a16_expert_ffn_noalloc", _lib.smoe_w4a16_expert_ffn_noalloc(
        _ptr(x, torch.float16, "x"), T, k, E, H, I, group_size,
        _ptr(wg_q, torch.int32, "wg_q"), _ptr(wg_s, torch.float16, "wg_s"),
        _ptr(wu_q, torch.int32, "wu_q"), _ptr(wu_s, torch.float16, "wu_s"),
        _ptr(wd_q, torch.int32, "wd_q"), _ptr(wd_s, torch.float16, "wd_s"),
        _ptr(sorted_slots, torch.int32, "sorted_slots"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"), sI, sg, su, sd,
        _ptr(slot_out, torch.float32, "slot_out"), so, _stream(stream)))


def smoe_fp16_expert_ffn(x, k: int, E: int, I: int, wg, wu, wd, sorted_slots, expert_offsets,
                         workspace, slot_out, shared=None, shared_out=None, stream=None, *,
                         _fn="") -> None:
    """shared: optional (wg, wu, wd) fp16 weights of the always-on shared expert."""
    fname = _fn or "smoe_fp16_expert_ffn"
    T, H = x.shape
    sI, sg, su, sd, so = _shared_args(shared, shared_out)
    for name, t in (("wg", wg), ("wu", wu), ("wd", wd)):
        _need(t, E * I * H, name)
    _ffn_sizes(T, k, E, H, sI, sorted_slots, expert_offsets, slot_out, shared, shared_out)
    _check(fname, getattr(_lib, fname)(
        _ptr(x, torch.float16, "x"), T, k, E, H, I,
        _ptr(wg, torch.float16, "wg"), _ptr(wu, torch.float16, "wu"),
        _ptr(wd, torch.float16, "wd"),
        _ptr(sorted_slots, torch.int32, "sorted_slots"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"), sI, sg, su, sd,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _ptr(slot_out, torch.float32, "slot_out"), so, _stream(stream)))


def smoe_fp16_expert_ffn_mapped(x, k: int, E: int, I: int, wg, wu, wd, n_matrices: int,
                                expert_matrix, sorted_slots, expert_offsets, workspace,
                                slot_out, shared=None, shared_out=None, stream=None, *,
                                tiled: bool = False) -> None:
    """wg, wu, wd: fp16 bases of n_matrices matrices each (views into one pool
    may overlap); expert_matrix: host int32 [E] (a sequence or NumPy array),
    the matrix of each expert, -1 = not in this call."""
    T, H = x.shape
    sI, sg, su, sd, so = _shared_args(shared, shared_out)
    for name, t in (("wg", wg), ("wu", wu), ("wd", wd)):
        _need(t, n_matrices * I * H, name)
    table = (ctypes.c_int32 * E)(*[int(v) for v in list(expert_matrix)[:E]])
    if len(list(expert_matrix)) < E:
        raise ValueError(f"expert_matrix holds {len(list(expert_matrix))} entries, the call needs {E}")
    _ffn_sizes(T, k, E, H, sI, sorted_slots, expert_offsets, slot_out, shared, shared_out)
    _check("smoe_fp16_expert_ffn_mapped", _lib.smoe_fp16_expert_ffn_mapped(
        _ptr(x, torch.float16, "x"), T, k, E, H, I,
        _ptr(wg, torch.float16, "wg"), _ptr(wu, torch.float16, "wu"),
        _ptr(wd, torch.float16, "wd"), 1 if tiled else 0, n_matrices,
        ctypes.cast(table, ctypes.c_void_p),
        _ptr(sorted_slots, torch.int32, "sorted_slots"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"), sI, sg, su, sd,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _ptr(slot_out, torch.float32, "slot_out"), so, _stream(stream)))


def smoe_ffn_workspace_clear(workspace, stream=None) -> None:
    """Zero a FFN workspace with a fill kernel (graph-capturable)."""
    _check("smoe_ffn_workspace_clear", _lib.smoe_ffn_workspace_clear(
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream)))


def smoe_combine(slot_out, topk_w, shared_out, shared_gate, y, stream=None) -> None:
    T, k = topk_w.shape
    H = y.shape[1]
    _need(slot_out, T * k * H, "slot_out")
    _need(shared_out, T * H, "shared_out")
    _need(shared_gate, T, "shared_gate")
    _need(y, T * H, "y")
    _check("smoe_combine", _lib.smoe_combine(
        _ptr(slot_out, torch.float32, "slot_out"), _ptr(topk_w, torch.float32, "topk_w"),
        T, k, H, _ptr(shared_out, torch.float32, "shared_out"),
        _ptr(shared_gate, torch.float32, "shared_gate"),
        _ptr(y, torch.float16, "y"), _stream(stream)))


def raw_library() -> ctypes.CDLL:
    """The loaded CDLL (for tests that call the C ABI directly)."""
    return _lib


def smoe_moe_layer_w4a16(x, w_router, logit_bias, k: int, flags: int, topk_ids, topk_w, logits,
                         shared_gate_w, shared_gate, expert_counts, expert_offsets, sorted_slots,
                         active_experts, n_active, elb_counts, layer: int, M: int, plan_ids,
                         plan_counts, elb_flags: int, I: int, group_size: int, wg_q, wg_s, wu_q,
                         wu_s, wd_q, wd_s, workspace, slot_out, y, shared=None, shared_out=None,
                         stream=None, *, _fn="") -> None:
    """The whole draft layer in one call: smoe_route_align_elb,
    smoe_w4a16_expert_ffn and smoe_combine with the same arguments.
    elb_counts [L][E] or None; shared: optional (wg, wu, wd) fp16 weights."""
    fname = _fn or "smoe_moe_layer_w4a16"
    T, H = x.shape
    E = w_router.shape[0]
    L = elb_counts.shape[0] if elb_counts is not None else 0
    _route_sizes(T, H, E, k, w_router, logit_bias, topk_ids, topk_w, logits, shared_gate_w,
                 shared_gate)
    _align_sizes(T * k, E, expert_counts, expert_offsets, sorted_slots, active_experts, n_active)
    _need(elb_counts, L * E, "elb_counts")
    _need(plan_ids, L * M, "plan_ids")
    _need(plan_counts, L * M, "plan_counts")
    sI, sg, su, sd, so = _shared_args(shared, shared_out)
    G = max(group_size, 1)
    for name, t in (("wg_q", wg_q), ("wu_q", wu_q)):
        _need(t, E * I * H // 8, name)
    for name, t in (("wg_s", wg_s), ("wu_s", wu_s)):
        _need(t, E * I * H // G, name)
    _need(wd_q, E * H * I // 8, "wd_q")
    _need(wd_s, E * H * I // G, "wd_s")
    _ffn_sizes(T, k, E, H, sI, sorted_slots, expert_offsets, slot_out, shared, shared_out)
    _need(y, T * H, "y")
    _check(fname, getattr(_lib, fname)(
        _ptr(x, torch.float16, "x"), _ptr(w_router, torch.float32, "w_router"),
        _ptr(logit_bias, torch.float32, "logit_bias"), T, H, E, k, flags,
        _ptr(topk_ids, torch.int32, "topk_ids"), _ptr(topk_w, torch.float32, "topk_w"),
        _ptr(logits, torch.float32, "logits"),
        _ptr(shared_gate_w, torch.float32, "shared_gate_w"),
        _ptr(shared_gate, torch.float32, "shared_gate"),
        _ptr(expert_counts, torch.int32, "expert_counts"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"),
        _ptr(sorted_slots, torch.int32, "sorted_slots"),
        _ptr(active_experts, torch.int32, "active_experts"),
        _ptr(n_active, torch.int32, "n_active"),
        _ptr(elb_counts, torch.int32, "elb_counts"), L, layer, M,
        _ptr(plan_ids, torch.int32, "plan_ids"), _ptr(plan_counts, torch.int32, "plan_counts"),
        elb_flags, I, group_size,
        _ptr(wg_q, torch.int32, "wg_q"), _ptr(wg_s, torch.float16, "wg_s"),
        _ptr(wu_q, torch.int32, "wu_q"), _ptr(wu_s, torch.float16, "wu_s"),
        _ptr(wd_q, torch.int32, "wd_q"), _ptr(wd_s, torch.float16, "wd_s"),
        sI, sg, su, sd,
        _ptr(workspace, torch.uint8, "workspace"), workspace.numel(),
        _ptr(slot_out, torch.float32, "slot_out"), so, _ptr(y, torch.float16, "y"),
        _stream(stream)))


def smoe_w4a16_expert_ffn_tiled(*args, **kw) -> None:
    """smoe_w4a16_expert_ffn with every weight in the tiled layout."""
    smoe_w4a16_expert_ffn(*args, **kw, _fn="smoe_w4a16_expert_ffn_tiled")


def smoe_fp16_expert_ffn_tiled(*args, **kw) -> None:
    """smoe_fp16_expert_ffn with every weight in the tiled layout."""
    smoe_fp16_expert_ffn(*args, **kw, _fn="smoe_fp16_expert_ffn_tiled")


def smoe_moe_layer_w4a16_tiled(*args, **kw) -> None:
    """smoe_moe_layer_w4a16 with every weight in the tiled layout."""
    smoe_moe_layer_w4a16(*args, **kw, _fn="smoe_moe_layer_w4a16_tiled")


def smoe_tile_weights(w, scales, E: int, N: int, K: int, group_size: int, w_tiled,
                      scales_tiled=None, stream=None) -> None:
    """Tiled copy of one [E][N][K] weight tensor: group_size 0 for fp16 values
    (w, w_tiled float16, scales None), else INT4 codes (int32 [E][N][K/8]) and
    fp16 scales [E][N][K/G]."""
    if group_size:
        wdt, n_w, n_s = torch.int32, E * N * K // 8, E * N * K // group_size
    else:
        wdt, n_w, n_s = torch.float16, E * N * K, 0
    _need(w, n_w, "w")
    _need(w_tiled, n_w, "w_tiled")
    if group_size:
        _need(scales, n_s, "scales")
        _need(scales_tiled, n_s, "scales_tiled")
    _check("smoe_tile_weights", _lib.smoe_tile_weights(
        _ptr(w, wdt, "w"), _ptr(scales, torch.float16, "scales") if group_size else None,
        E, N, K, group_size, _ptr(w_tiled, wdt, "w_tiled"),
        _ptr(scales_tiled, torch.float16, "scales_tiled") if group_size else None,
        _stream(stream)))


# ---------------------------------------------------------------- expert cache
# Host arrays cross the boundary as NumPy arrays (C-contiguous, the stated
# dtype); the cache itself is an opaque handle (an int).

def _np_ptr(a, dtype, name: str):
    import numpy as np
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError(f"{name} must be a C-contiguous numpy {np.dtype(dtype).name} array")
    return a.ctypes.data_as(ctypes.c_void_p)


def _host_ptr(t: Optional[torch.Tensor], name: str) -> Optional[int]:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous host torch.Tensor")
    return t.data_ptr()


def smoe_cache_create(L: int, E: int, M: int, expert_bytes: int, pool=None,
                      host_experts=None) -> int:
    """pool: device tensor of >= L*M*expert_bytes bytes; host_experts: host
    (pinned) tensor of >= L*E*expert_bytes bytes; both None for a cache that
    only takes decisions."""
    if pool is not None and pool.numel() * pool.element_size() < L * M * expert_bytes:
        raise ValueError("pool is smaller than L*M*expert_bytes")
    if host_experts is not None and (host_experts.numel() * host_experts.element_size()
                                     < L * E * expert_bytes):
        raise ValueError("host_experts is smaller than L*E*expert_bytes")
    h = ctypes.c_void_p()
    _check("smoe_cache_create", _lib.smoe_cache_create(
        L, E, M, expert_bytes, _ptr(pool, None, "pool"), _host_ptr(host_experts, "host_experts"),
        ctypes.byref(h)))
    return h.value


def smoe_cache_destroy(cache: int) -> None:
    _check("smoe_cache_destroy", _lib.smoe_cache_destroy(cache))


def smoe_cache_begin_window(cache: int) -> None:
    _check("smoe_cache_begin_window", _lib.smoe_cache_begin_window(cache))


def smoe_cache_state(cache: int, L: int, M: int):
    """(slot_expert int32 [L][M], last_use int64 [L][M], claimed int32 [L][M], clock)."""
    import numpy as np
    se = np.empty((L, M), np.int32)
    lu = np.empty((L, M), np.int64)
    cl = np.empty((L, M), np.int32)
    clock = ctypes.c_int64()
    _check("smoe_cache_state", _lib.smoe_cache_state(
        cache, _np_ptr(se, np.int32, "slot_expert"), _np_ptr(lu, np.int64, "last_use"),
        _np_ptr(cl, np.int32, "claimed"), ctypes.byref(clock)))
    return se, lu, cl, clock.value


def smoe_cache_set_state(cache: int, slot_expert, last_use, clock: int, copy_stream=None) -> None:
    import numpy as np
    _check("smoe_cache_set_state", _lib.smoe_cache_set_state(
        cache, _np_ptr(slot_expert, np.int32, "slot_expert"),
        _np_ptr(last_use, np.int64, "last_use"), clock,
        None if copy_stream is None else _stream(copy_stream)))


def smoe_cache_prefetch(cache: int, plan_ids, plan_counts, L: int, M: int, copy_stream=None):
    """plan_ids / plan_counts: host int32 [L][plan_M]. Returns (loads int32
    [n][4], full)."""
    import numpy as np
    if plan_ids.shape != plan_counts.shape or plan_ids.ndim != 2 or plan_ids.shape[0] != L:
        raise ValueError("plan_ids and plan_counts must both be [L][plan_M]")
    loads = np.empty((max(L * M, 1), 4), np.int32)
    n, full = ctypes.c_int(), ctypes.c_int()
    _check("smoe_cache_prefetch", _lib.smoe_cache_prefetch(
        cache, _np_ptr(plan_ids, np.int32, "plan_ids"),
        _np_ptr(plan_counts, np.int32, "plan_counts"), plan_ids.shape[1],
        _np_ptr(loads, np.int32, "loads"), ctypes.byref(n), ctypes.byref(full),
        None if copy_stream is None else _stream(copy_stream)))
    return loads[:n.value].copy(), bool(full.value)


def smoe_prefetch_next_boundary(b: int, K: int, n_transfer: int, expert_bytes: float,
                                h2d_gb_per_s: float, draft_us_per_token: float) -> int:
    out = ctypes.c_int()
    _check("smoe_prefetch_next_boundary", _lib.smoe_prefetch_next_boundary(
        b, K, n_transfer, float(expert_bytes), float(h2d_gb_per_s), float(draft_us_per_token),
        ctypes.byref(out)))
    return out.value


def smoe_cache_verify_plan(cache: int, layer: int, expert_counts):
    """expert_counts: host int32 [E]. Returns the schedule int32 [n][5]."""
    import numpy as np
    E = expert_counts.shape[0]
    sched = np.empty((max(E, 1), 5), np.int32)
    n = ctypes.c_int()
    _check("smoe_cache_verify_plan", _lib.smoe_cache_verify_plan(
        cache, layer, _np_ptr(expert_counts, np.int32, "expert_counts"),
        _np_ptr(sched, np.int32, "schedule"), ctypes.byref(n)))
    return sched[:n.value].copy()


def smoe_cache_verify_layer(cache: int, layer: int, expert_counts, x, k: int, I: int,
                            sorted_slots, expert_offsets, workspace_shared, workspace_routed,
                            slot_out, shared=None, shared_out=None, tiled: bool = False,
                            compute_stream=None, copy_stream=None):
    """Returns the schedule int32 [n][5] (see smoe_cache_verify_plan)."""
    import numpy as np
    T, H = x.shape
    E = expert_counts.shape[0]
    sI, sg, su, sd, so = _shared_args(shared, shared_out)
    _ffn_sizes(T, k, E, H, sI, sorted_slots, expert_offsets, slot_out, shared, shared_out)
    sched = np.empty((max(E, 1), 5), np.int32)
    n = ctypes.c_int()
    wss = workspace_shared
    _check("smoe_cache_verify_layer", _lib.smoe_cache_verify_layer(
        cache, layer, _np_ptr(expert_counts, np.int32, "expert_counts"),
        _ptr(x, torch.float16, "x"), T, k, H, I, 1 if tiled else 0,
        _ptr(sorted_slots, torch.int32, "sorted_slots"),
        _ptr(expert_offsets, torch.int32, "expert_offsets"), sI, sg, su, sd,
        _ptr(wss, torch.uint8, "workspace_shared"), 0 if wss is None else wss.numel(),
        _ptr(workspace_routed, torch.uint8, "workspace_routed"), workspace_routed.numel(),
        _ptr(slot_out, torch.float32, "slot_out"), so,
        _np_ptr(sched, np.int32, "schedule"), ctypes.byref(n),
        _stream(compute_stream), _stream(copy_stream)))
    return sched[:n.value].copy()


# ---------------------------------------------------------------- SpecFit

def smoe_specfit_select(parent, path_prob, expert_bits, K: int, intercepts, beta: float,
                        resident_bits=None, E: Optional[int] = None):
    """parent int32 [n]; path_prob float64 [n]; expert_bits uint64 [n + 1][L][W]
    (row 0 the root); resident_bits uint64 [L][W] or None; intercepts
    float64 [min(K, n) + 1]. Returns (selected nodes, ratio, legal subtrees
    visited)."""
    import numpy as np
    n = int(parent.shape[0])
    L, W = int(expert_bits.shape[1]), int(expert_bits.shape[2])
    E = 64 * W if E is None else E
    sel = np.empty(max(min(K, n), 1), np.int32)
    ns, ratio, ev = ctypes.c_int(), ctypes.c_double(), ctypes.c_int64()
    _check("smoe_specfit_select", _lib.smoe_specfit_select(
        n, _np_ptr(parent, np.int32, "parent") if n else None,
        _np_ptr(path_prob, np.float64, "path_prob") if n else None, L, E,
        _np_ptr(expert_bits, np.uint64, "expert_bits"),
        None if resident_bits is None else _np_ptr(resident_bits, np.uint64, "resident_bits"),
        K, _np_ptr(intercepts, np.float64, "intercepts"), float(beta),
        _np_ptr(sel, np.int32, "selected"), ctypes.byref(ns), ctypes.byref(ratio),
        ctypes.byref(ev)))
    return sel[:ns.value].tolist(), ratio.value, ev.value
