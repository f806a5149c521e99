"""Plain NumPy reference of the routed-expert MoE layer (test infrastructure).

Sources (cited by page title and paragraph or section):
  * "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step
    Speculative Offloading" (paper body; paragraphs named by topic):
    the Incremental Routing Pattern Analyzer / ELB paragraphs, the fused
    multi-expert draft kernel paragraph, the expert-wise verification
    paragraphs, the hybrid-precision and GPTQ INT4 g128 statements.
  * Specter repository design notes ("Design"), sections "Predictive I/O
    Orchestrator" (pattern_analyzer) and "Streamlined Execution Engine"
    (W4A16 statement: INT4 weight tiles dequantised, FP16 activations).

Readings where the pages are silent (each is also listed with its reason in
the repository's design document):
  * router: softmax over all E logits, experts picked by logit (same set as
    by probability), no renormalisation unless asked;
  * the fp32 router dot product has a fixed summation order (below) so that
    the picked expert IDs are reproducible bit for bit;
  * ties in top-k and top-M go to the lower expert ID;
  * expert MLP = down( SiLU(gate x) * (up x) ), the SiLU-gated form;
  * INT4 value = (code - 8) * scale, groups along the reduction dim.
"""

from __future__ import annotations

from typing import Callable, Dict, Optional, Tuple

import numpy as np

F32 = np.float32
F64 = np.float64

LANES = 64  # width of one partial-sum lane set in the router's stated order


# --------------------------------------------------------------------------
# Routing (Specter paper: the draft router's expert IDs feed the ELB; the
# target router is authoritative in verification)
# --------------------------------------------------------------------------

def router_logits_f32(x16: np.ndarray, w_router: np.ndarray,
                      bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router logits x . W_r^T in float32, in a fixed summation order.

    logit[t, e] is a float32 dot product over h of f32(x[t, h]) * W_r[e, h].
    Because the top-k expert IDs are integers decided by these floats, the
    order of the float32 additions is fixed (a reading; the pages are silent):
      * 64 partial sums p[l], l = 0..63, start at +0.0;
      * for c = 0, 1, ..., H/64 - 1 in turn:
            p[l] = f32( p[l] + f32( x[t, 64c + l] * W_r[e, 64c + l] ) )
        (product and sum each rounded to float32; no fused multiply-add);
      * then for off = 32, 16, 8, 4, 2, 1:  p[l] = f32(p[l] + p[l + off])
        for l < off;
      * logit = p[0]; with a bias, logit = f32(logit + bias[e]).
    NumPy float32 elementwise operations round each op, so this is that
    order written out. Returns float32 [T][E].
    """
    x = np.asarray(x16).astype(F32)
    w = np.asarray(w_router, dtype=F32)
    T, H = x.shape
    E, H2 = w.shape
    if H != H2 or H % LANES:
        raise ValueError("router: H mismatch or H not a multiple of 64")
    p = np.zeros((T, E, LANES), dtype=F32)
    for c in range(H // LANES):
        xs = x[:, None, c * LANES:(c + 1) * LANES]
        ws = w[None, :, c * LANES:(c + 1) * LANES]
        prod = xs * ws                 # float32 multiply, rounded
        p = p + prod                   # float32 add, rounded
    off = LANES // 2
    while off >= 1:
        p[:, :, :off] = p[:, :, :off] + p[:, :, off:2 * off]
        off //= 2
    logits = p[:, :, 0].copy()
    if bias is not None:
        logits = logits + np.asarray(bias, dtype=F32)[None, :]
    return logits.astype(F32)


def topk_experts(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the k expert IDs with the largest logits, in rank order.

    Order: logit descending, then expert ID ascending (lower ID wins a tie;
    -0.0 and +0.0 compare equal). Returns int32 [T][k].
    """
    logits = np.asarray(logits, dtype=F32)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    eidx = np.arange(E)
    for t in range(T):
        # lexsort: last key is primary -> sort by -logit, then by expert ID
        order = np.lexsort((eidx, -logits[t].astype(F64)))
        ids[t] = order[:k]
    return ids


def routing_weights(logits: np.ndarray, ids: np.ndarray,
                    renorm: bool = False) -> np.ndarray:
    """Routing weight of each picked expert: softmax over all E logits.

    p = softmax(logits[t]) in float64 (max subtracted); w[t, j] = p[ids[t, j]].
    With renorm, w[t, :] is divided by its sum over the k picked experts.
    Returns float64 [T][k].
    """
    lg = np.asarray(logits, dtype=F64)
    z = np.exp(lg - lg.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    w = np.take_along_axis(p, np.asarray(ids, dtype=np.int64), axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return w


def shared_gate(x16: np.ndarray, w_sg: np.ndarray) -> np.ndarray:
    """Sigmoid gate of the shared expert: g[t] = 1 / (1 + exp(-x[t] . w_sg)).

    float64 [T]. (Qwen1.5-MoE-shaped configuration; the pages keep shared
    experts in FP16 but do not describe the gate, so this follows the
    configuration's "sigmoid gate".)
    """
    x = np.asarray(x16).astype(F64)
    z = x @ np.asarray(w_sg, dtype=F64)
    return 1.0 / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------
# Alignment (Specter paper: the fused draft kernel first gathers routed
# tokens by expert; design notes: kernels "align token groups")
# --------------------------------------------------------------------------

def align_by_expert(ids: np.ndarray, E: int) -> Dict[str, np.ndarray]:
    """Group the S = T*k routing slots by expert (a stable counting sort).

    Slot s = t*k + j carries expert ids[t, j]. IDs outside [0, E) are dropped.
      counts[e]        number of slots routed to e
      offsets[e]       exclusive prefix sum of counts; offsets[E] = kept slots
      sorted_slots[p]  slot indices ordered by (expert, slot) ascending;
                       entries p >= offsets[E] are -1
      active[i]        experts with counts > 0, ascending, then -1 padding
      n_active         number of such experts
    """
    flat = np.asarray(ids, dtype=np.int64).ravel()
    S = flat.size
    counts = np.zeros(E, dtype=np.int32)
    for s in range(S):
        e = flat[s]
        if 0 <= e < E:
            counts[e] += 1
    offsets = np.zeros(E + 1, dtype=np.int32)
    running = 0
    for e in range(E):
        offsets[e] = running
        running += int(counts[e])
    offsets[E] = running
    cursor = offsets[:E].astype(np.int64).copy()
    sorted_slots = np.full(S, -1, dtype=np.int32)
    for s in range(S):            # walking slots in order keeps the sort stable
        e = flat[s]
        if 0 <= e < E:
            sorted_slots[cursor[e]] = s
            cursor[e] += 1
    active = np.full(E, -1, dtype=np.int32)
    n = 0
    for e in range(E):
        if counts[e] > 0:
            active[n] = e
            n += 1
    return {"counts": counts, "offsets": offsets, "sorted_slots": sorted_slots,
            "active": active, "n_active": np.int32(n)}


# --------------------------------------------------------------------------
# W4A16 weights (Specter paper: GPTQ symmetric INT4, group size 128;
# design notes: kernels dequantize INT4 weight tiles, FP16 activations)
# --------------------------------------------------------------------------

def dequant_int4(codes: np.ndarray, scales: np.ndarray, group: int) -> np.ndarray:
    """Dequantise packed INT4 weights to float64 [N][K].

    codes uint32 [N][K/8]: word w of row n holds k = 8w + j in bits 4j..4j+3.
    scales fp16 [N][K/group]. Value = (code - 8) * scale[n, k // group]
    (exact in float64).
    """
    codes = np.asarray(codes, dtype=np.uint32)
    N, W = codes.shape
    K = 8 * W
    nib = np.empty((N, W, 8), dtype=np.int64)
    for j in range(8):
        nib[:, :, j] = (codes >> np.uint32(4 * j)) & np.uint32(0xF)
    q = nib.reshape(N, K) - 8
    s = np.asarray(scales, dtype=np.float16).astype(F64)
    if s.shape != (N, K // group):
        raise ValueError("scale shape does not match codes and group size")
    return q.astype(F64) * np.repeat(s, group, axis=1)


# --------------------------------------------------------------------------
# Expert MLP
# --------------------------------------------------------------------------

def _silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def swiglu(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
           act_fp16: bool = True) -> np.ndarray:
    """down( SiLU(x Wg^T) * (x Wu^T) ) in float64 for rows of x.

    x [m][H], wg/wu [I][H], wd [H][I] (any float type, used as float64).
    With act_fp16 the intermediate activation h is rounded to fp16 before
    the down projection (W4A16: the projections consume FP16 activations).
    """
    x = np.asarray(x, dtype=F64)
    g = x @ np.asarray(wg, dtype=F64).T
    u = x @ np.asarray(wu, dtype=F64).T
    h = _silu(g) * u
    if act_fp16:
        h = h.astype(np.float16).astype(F64)
    return h @ np.asarray(wd, dtype=F64).T


ExpertLoader = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


def routed_ffn_tokenwise(x16: np.ndarray, ids: np.ndarray, load: ExpertLoader,
                         act_fp16: bool = True) -> np.ndarray:
    """Per-slot expert outputs, token by token (the plain definition).

    slot_out[t*k + j] = FFN_{ids[t, j]}(x[t]); `load(e)` returns float64
    (Wg, Wu, Wd) of expert e. A negative ID is a slot routed to no expert
    (dropped by the alignment): its row is zero. Returns float64 [T*k][H].
    """
    x = np.asarray(x16)
    T, k = ids.shape
    out = np.zeros((T * k, x.shape[1]), dtype=F64)
    cache: Dict[int, Tuple[np.ndarray, np.ndarray, np.ndarray]] = {}
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            if e < 0:
                continue
            if e not in cache:
                cache[e] = load(e)
            out[t * k + j] = swiglu(x[t:t + 1].astype(F64), *cache[e],
                                    act_fp16=act_fp16)[0]
    return out


def routed_ffn_expertwise(x16: np.ndarray, ids: np.ndarray, load: ExpertLoader,
                          act_fp16: bool = True) -> np.ndarray:
    """Per-slot expert outputs computed expert by expert.

    The Specter paper's verification reorder: gather the tokens routed to
    each expert into one sub-batch, run that expert once on the sub-batch,
    scatter each row back to its slot. Each row is the same definition as
    in routed_ffn_tokenwise (negative IDs: zero rows). Returns float64
    [T*k][H].
    """
    x = np.asarray(x16)
    T, k = ids.shape
    flat = np.asarray(ids, dtype=np.int64).ravel()
    out = np.zeros((T * k, x.shape[1]), dtype=F64)
    for e in np.unique(flat[flat >= 0]):
        slots = np.flatnonzero(flat == e)
        tokens = slots // k
        wg, wu, wd = load(int(e))
        out[slots] = swiglu(x[tokens].astype(F64), wg, wu, wd, act_fp16=act_fp16)
    return out


def shared_ffn(x16: np.ndarray, sg16: np.ndarray, su16: np.ndarray, sd16: np.ndarray,
               act_fp16: bool = True) -> np.ndarray:
    """Always-on FP16 shared expert(s) over every token: float64 [T][H].

    Several shared experts concatenated along the intermediate dimension
    give the sum of their outputs.
    """
    return swiglu(np.asarray(x16).astype(F64), sg16, su16, sd16, act_fp16=act_fp16)


# --------------------------------------------------------------------------
# Combine (Specter paper, expert-wise verification paragraph: each expert's
# per-slot outputs return to the token they came from, weighted by the
# router, and are summed there)
# --------------------------------------------------------------------------

def combine(slot_out: np.ndarray, w: np.ndarray,
            shared_out: Optional[np.ndarray] = None,
            gate: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """y[t] = sum_j w[t, j] * slot_out[t*k + j] + gate[t] * shared_out[t].

    gate defaults to 1 when a shared output is given without one.
    Returns (y float64 [T][H], y rounded to fp16).
    """
    w = np.asarray(w, dtype=F64)
    T, k = w.shape
    so = np.asarray(slot_out, dtype=F64).reshape(T, k, -1)
    y = np.zeros((T, so.shape[2]), dtype=F64)
    for j in range(k):
        y += w[:, j:j + 1] * so[:, j, :]
    if shared_out is not None:
        g = np.ones(T) if gate is None else np.asarray(gate, dtype=F64)
        y += g[:, None] * np.asarray(shared_out, dtype=F64)
    return y, y.astype(np.float16)


# --------------------------------------------------------------------------
# ELB activation counter (Specter paper: Incremental Routing Pattern
# Analyzer; design notes: pattern_analyzer accumulates routing counts on
# the GPU and ranks experts at chunk boundaries)
# --------------------------------------------------------------------------

def elb_accumulate(cnt: np.ndarray, ids_layers: np.ndarray,
                   layer_begin: int = 0) -> np.ndarray:
    """cnt[l, e] += number of (token, rank) slots of layer l routed to e.

    cnt int32 [L][E] (returned updated, input not modified); ids_layers
    int [n_layers][T][k] for layers layer_begin .. layer_begin+n_layers-1.
    This is the cumulative activation counter ELB_cnt[j, e]: the count of
    draft tokens whose top-k route set in layer j contains e. IDs outside
    [0, E) are not counted.
    """
    out = np.array(cnt, dtype=np.int64, copy=True)
    L, E = out.shape
    ids_layers = np.asarray(ids_layers, dtype=np.int64)
    for i in range(ids_layers.shape[0]):
        l = layer_begin + i
        for e in ids_layers[i].ravel():
            if 0 <= e < E:
                out[l, e] += 1
    return out.astype(np.int32)


def elb_topm(cnt: np.ndarray, M: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per layer, the M experts with the largest counts (prefetch plan).

    Order: count descending, then expert ID ascending; always M entries
    (zero-count experts included). Returns (plan_ids int32 [L][M],
    plan_counts int32 [L][M]).
    """
    cnt = np.asarray(cnt, dtype=np.int64)
    L, E = cnt.shape
    if not 0 <= M <= E:
        raise ValueError("need 0 <= M <= E")
    ids = np.empty((L, M), dtype=np.int32)
    vals = np.empty((L, M), dtype=np.int32)
    eidx = np.arange(E)
    for l in range(L):
        order = np.lexsort((eidx, -cnt[l]))[:M]
        ids[l] = order
        vals[l] = cnt[l, order]
    return ids, vals


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

def moe_layer(inp, pass_: str = "draft", renorm: bool = False,
              act_fp16: bool = True) -> Dict[str, np.ndarray]:
    """Route, align, routed experts, shared experts and combine for one layer.

    `inp` is a workload.LayerInputs. pass_ = "draft" uses the INT4 routed
    weights, "target" the FP16 routed weights (verification pass). Returns
    every intermediate, keyed by name.
    """
    cfg = inp.cfg
    logits = router_logits_f32(inp.x, inp.w_router, inp.router_bias)
    ids = topk_experts(logits, cfg.k)
    w = routing_weights(logits, ids, renorm=renorm)
    al = align_by_expert(ids, cfg.E)

    if pass_ == "draft":
        def load(e):
            return (dequant_int4(inp.wg_q[e], inp.wg_s[e], cfg.G),
                    dequant_int4(inp.wu_q[e], inp.wu_s[e], cfg.G),
                    dequant_int4(inp.wd_q[e], inp.wd_s[e], cfg.G))
    elif pass_ == "target":
        def load(e):
            return (inp.wg16[e].astype(F64), inp.wu16[e].astype(F64),
                    inp.wd16[e].astype(F64))
    else:
        raise ValueError("pass_ must be 'draft' or 'target'")

    slot_out = routed_ffn_expertwise(inp.x, ids, load, act_fp16=act_fp16)
    shared_out = gate = None
    if inp.sg16 is not None:
        shared_out = shared_ffn(inp.x, inp.sg16, inp.su16, inp.sd16, act_fp16=act_fp16)
        if inp.shared_gate_w is not None:
            gate = shared_gate(inp.x, inp.shared_gate_w)
    y64, y16 = combine(slot_out, w, shared_out, gate)
    return {"logits": logits, "ids": ids, "w": w, **al, "slot_out": slot_out,
            "shared_out": shared_out, "gate": gate, "y64": y64, "y": y16}
