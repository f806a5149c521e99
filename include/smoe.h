/*
 * libsmoe -- routed-expert MoE layer over a window of speculative tokens,
 * hand-written HIP for AMD MI355X (gfx950).
 *
 * Sources the operations follow (cited by page title and paragraph/section):
 *   [P]  "Specter: Fast MoE Inference via Quantization-Enabled Multi-Step
 *        Speculative Offloading" (paper body text).
 *   [D]  Specter repository design notes, page "Design".
 *   [S]  Korean summary page of Specter ("Specter는 양자화 드래프트로 MoE
 *        오프로딩의 PCIe 지연을 숨긴다").
 *
 * Conventions for every call
 *   - Pointers are DEVICE pointers unless stated otherwise, owned by the
 *     caller, 16-byte aligned, and valid for the whole call. The library
 *     never allocates, frees or keeps a pointer after the call returns.
 *     Outputs must not alias inputs.
 *   - `stream` is a hipStream_t (NULL = the null stream). Every call only
 *     enqueues work on it: no host or device synchronisation, no device to
 *     host copies, no memsets, so calls can be captured into a HIP graph.
 *   - Arguments are checked before anything is enqueued; a bad argument
 *     returns SMOE_EINVAL (null / negative / inconsistent) or
 *     SMOE_EUNSUPPORTED (outside the kernels' limits) and touches no memory.
 *     A failed launch returns SMOE_EHIP. smoe_last_error() gives the reason
 *     (thread-local text).
 *   - Limits: 1 <= E <= 256; 1 <= k <= min(8, E) (the expert FFN calls
 *     also take k > E: a call may cover a subset of the experts, e.g. one
 *     expert or one device's share, with the window's k); H and I multiples
 *     of 128; group size G in {32, 64, 128}; T*k < 2^24; M <= E.
 *   - Layouts are row-major. fp16 = IEEE binary16, passed as void*.
 *   - Packed INT4 weights W[N][K]: codes uint32 [N][K/8], word w of row n
 *     holds the codes for k = 8w .. 8w+7, the code for k = 8w+j in bits
 *     4j .. 4j+3; scales fp16 [N][K/G]. A code c stands for (c - 8) * scale.
 *   - Token t of the window owns routing slots s = t*k + j, j = 0..k-1, in
 *     rank order (slot s carries expert topk_ids[t][j]).
 */
#ifndef SMOE_H
#define SMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int smoe_status;
#define SMOE_OK            0
#define SMOE_EINVAL       (-1)
#define SMOE_EUNSUPPORTED (-2)
#define SMOE_EHIP         (-3)

#define SMOE_ROUTE_RENORM    1  /* smoe_route_topk: renormalise the k weights to sum 1 */
#define SMOE_ELB_CLEAR_AFTER 1  /* smoe_elb_accumulate_topm: zero the counter after ranking */

/* Version of this interface (bumped on any signature change). */
int smoe_abi_version(void);

/* Static text for a status code. */
const char* smoe_status_string(smoe_status status);

/* Text describing the last failure on the calling thread ("" if none). */
const char* smoe_last_error(void);

/*
 * Router + top-k.                                     [P] paragraphs on the
 * Incremental Routing Pattern Analyzer (the draft router's top-k expert IDs)
 * and on expert-wise verification (the target router's routing decisions);
 * [D] "Speculative Inference Controller" (routers are shared, FP16/FP32).
 *
 * logits[t][e] = x[t] . w_router[e] (+ logit_bias[e]) in float32, summed in
 * this order: 64 partials p[l] over h = 64c + l for c = 0, 1, ... (each
 * product and each sum rounded separately, no fused multiply-add), then
 * p[l] += p[l + off] for off = 32, 16, 8, 4, 2, 1; the bias is added last.
 * topk_ids[t][0..k-1] = the k experts with the largest logits, by logit
 * descending then expert ID ascending (-0.0 == +0.0).
 * topk_w[t][j] = softmax over all E logits, taken at topk_ids[t][j]
 * (float32); with SMOE_ROUTE_RENORM divided by their sum over j.
 * shared_gate[t] = 1 / (1 + exp(-x[t] . shared_gate_w)) when both pointers
 * are non-NULL (sigmoid gate of a shared expert).
 *
 *   x            fp16 [T][H], 16-byte aligned
 *   w_router     float [E][H]
 *   logit_bias   float [E] or NULL
 *   topk_ids     int32 [T][k]   (out)
 *   topk_w       float [T][k]   (out)
 *   logits       float [T][E]   (out; the top-k is taken from it)
 *   shared_gate_w float [H] or NULL; shared_gate float [T] (out) or NULL
 * T = 0 enqueues nothing. Non-finite logits give an unspecified selection.
 */
smoe_status smoe_route_topk(const void* x, const float* w_router, const float* logit_bias,
                            int T, int H, int E, int k, int flags,
                            int32_t* topk_ids, float* topk_w, float* logits,
                            const float* shared_gate_w, float* shared_gate,
                            void* stream);

/*
 * Align token groups by expert.                       [P] fused multi-expert
 * draft kernel paragraph (gather routed tokens by expert assignment) and
 * expert-wise verification paragraph (pack the tokens of each expert into a
 * contiguous sub-batch); [D] "Streamlined Execution Engine" (kernels align
 * token groups).
 *
 * A stable counting sort of the S = T*k slots by expert:
 *   expert_counts[e]   slots routed to e                       int32 [E]
 *   expert_offsets[e]  exclusive prefix sum; [E] = kept slots  int32 [E+1]
 *   sorted_slots[p]    slots by (expert, slot) ascending; entries from
 *                      expert_offsets[E] on are -1             int32 [S]
 *   active_experts[i]  experts with count > 0 ascending, then -1   int32 [E]
 *   n_active[0]        number of such experts                 int32 [1]
 * IDs outside [0, E) are dropped (neither counted nor written). S = 0 is
 * valid (all outputs describe an empty alignment).
 */
smoe_status smoe_align_by_expert(const int32_t* topk_ids, int T, int k, int E,
                                 int32_t* expert_counts, int32_t* expert_offsets,
                                 int32_t* sorted_slots, int32_t* active_experts,
                                 int32_t* n_active, void* stream);

/*
 * ELB activation counter + top-M prefetch plan.       [P] Incremental Routing
 * Pattern Analyzer paragraphs (GPU-resident layer-indexed counters
 * ELB_cnt[j, e] over the draft route sets; per-layer top-M ranking at each
 * prefetch checkpoint; one compact plan per checkpoint; cleared at the end
 * of the draft stage); [D] "Predictive I/O Orchestrator" (pattern_analyzer);
 * [S] "어떻게 쓰나".
 *
 * If topk_ids != NULL, for i in [0, n_layers):
 *     elb_counts[layer_begin + i][e] += #{(t, j) : topk_ids[i][t][j] == e}
 * (IDs outside [0, E) are not counted). Then if M > 0, for every layer l of
 * the L layers: plan_ids[l][0..M-1] = the M experts with the largest counts,
 * by count descending then expert ID ascending (zero counts included);
 * plan_counts[l][m] = their counts (if plan_counts != NULL). Then, with
 * SMOE_ELB_CLEAR_AFTER, every counter of the L layers is set to 0.
 *
 *   elb_counts   int32 [L][E] (in/out, caller-owned, persists across calls)
 *   topk_ids     int32 [n_layers][T][k] or NULL
 *   plan_ids     int32 [L][M] (out; may be NULL when M = 0)
 *   plan_counts  int32 [L][M] (out) or NULL
 * The plan stays on the device; the caller copies it to the host.
 */
smoe_status smoe_elb_accumulate_topm(int32_t* elb_counts, int L, int E,
                                     const int32_t* topk_ids, int layer_begin, int n_layers,
                                     int T, int k, int M,
                                     int32_t* plan_ids, int32_t* plan_counts,
                                     int flags, void* stream);

/*
 * Routing, alignment and the ELB update of one layer in one call.
 * Computes exactly what these calls made one after the other compute:
 *   smoe_route_topk(x, w_router, logit_bias, T, H, E, k, flags, topk_ids,
 *                   topk_w, logits, shared_gate_w, shared_gate)
 *   smoe_align_by_expert(topk_ids, T, k, E, expert_counts, expert_offsets,
 *                        sorted_slots, active_experts, n_active)
 *   and, when elb_counts is not NULL,
 *   smoe_elb_accumulate_topm(elb_counts, L, E, topk_ids, layer, 1, T, k, M,
 *                            plan_ids, plan_counts, elb_flags)
 * with the same arguments, checks and errors. For windows of at most 512
 * slots (T*k) the top-k, the alignment and the ELB update run in a single
 * workgroup after the router logits, which saves two launches on the
 * layer's critical path; larger windows run the three calls.
 */
smoe_status smoe_route_align_elb(const void* x, const float* w_router, const float* logit_bias,
                                 int T, int H, int E, int k, int flags,
                                 int32_t* topk_ids, float* topk_w, float* logits,
                                 const float* shared_gate_w, float* shared_gate,
                                 int32_t* expert_counts, int32_t* expert_offsets,
                                 int32_t* sorted_slots, int32_t* active_experts,
                                 int32_t* n_active,
                                 int32_t* elb_counts, int L, int layer, int M,
                                 int32_t* plan_ids, int32_t* plan_counts, int elb_flags,
                                 void* stream);

/*
 * Device workspace (bytes) that the expert FFN calls need for a window of
 * T tokens, k slots per token, routed intermediate size I and shared
 * intermediate size shared_I (0 = no shared expert): two fp32 buffers of
 * the gate and up projections of every slot, and a small call counter;
 * windows that take the long-window kernel (1024 to 4096 slots over tiled
 * weights) add their fp16 intermediate rows and the counters the kernel's
 * workgroups claim items from. Returns 0 for invalid sizes.
 *
 * Workspace contract: the caller fills the buffer with zeros
 * (smoe_ffn_workspace_clear, or any fill) before its first use, and again
 * before using it with a different (T, k, I, shared_I). The FFN calls keep
 * it consistent from one call to the next (each call clears what the
 * following call accumulates into), so it must not be written between
 * calls, and two calls that share a workspace must not run concurrently.
 *
 * Misuse is detected on the device: the first call after zeroing stamps
 * the buffer with its (T, k, I, shared_I); a later call of another shape
 * marks the buffer spoiled, and from then on every FFN call on it writes
 * NaN to all of slot_out and shared_out instead of its results, until the
 * buffer is zeroed again.
 */
size_t smoe_ffn_workspace_bytes(int T, int k, int E, int H, int I, int shared_I);

/*
 * Zero a FFN workspace on `stream` with a fill kernel (no memset node, so
 * the call can be captured into a HIP graph). workspace: device, 256-byte
 * aligned; workspace_bytes: a multiple of 16 (smoe_ffn_workspace_bytes
 * values are).
 */
smoe_status smoe_ffn_workspace_clear(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused multi-expert W4A16 expert FFN (draft pass).   [P] fused multi-expert
 * draft kernel paragraph (all active experts' sub-computations in one
 * launch; tokens gathered by expert into dense tiles), paragraph on Marlin
 * and narrow expert matrices (2048x1408, 4096x6400 expert MLPs), GPTQ
 * setup (symmetric INT4, group 128); [D] "Streamlined Execution Engine"
 * (W4A16: INT4 weight tiles dequantised while computing with FP16
 * activations; FP32 reduction).
 *
 * For every kept slot s routed to expert e (from the alignment), with
 * t = s / k:
 *     g = x[t] . Wg_e^T,  u = x[t] . Wu_e^T          (float32 accumulate)
 *     h = fp16( SiLU(g) * u ),  SiLU(g) = g / (1 + exp(-g))
 *     slot_out[s] = h . Wd_e^T                        (float32)
 * with W = (code - 8) * scale. Rows of slot_out for slots that the
 * alignment dropped are zero.
 *
 * With shared_I > 0 the same launches also run the always-on FP16 shared
 * expert (hybrid-precision layout: shared experts stay FP16) over every
 * token: shared_out[t] = fp16(SiLU(x[t] . Sg^T) * (x[t] . Su^T)) . Sd^T.
 * Several shared experts are passed concatenated along shared_I (their
 * outputs add up).
 *
 *   x              fp16 [T][H]
 *   wg_q, wu_q     uint32 [E][I][H/8];  wg_s, wu_s fp16 [E][I][H/G]
 *   wd_q           uint32 [E][H][I/8];  wd_s       fp16 [E][H][I/G]
 *   sorted_slots   int32 [T*k], expert_offsets int32 [E+1]
 *                  (as written by smoe_align_by_expert for these T, k, E)
 *   shared_I       0, or the shared intermediate size (multiple of 128)
 *   shared_wg, shared_wu  fp16 [shared_I][H];  shared_wd fp16 [H][shared_I]
 *                  (NULL when shared_I = 0)
 *   workspace      device buffer of at least
 *                  smoe_ffn_workspace_bytes(T, k, E, H, I, shared_I) bytes,
 *                  256-byte aligned, under the workspace contract above
 *   slot_out       float [T*k][H] (out)
 *   shared_out     float [T][H] (out; NULL when shared_I = 0)
 *
 * Output tiles whose reduction is split between workgroups are summed with
 * float atomics, so where more than two workgroups share a tile the last
 * bits of the result may differ from call to call.
 */
smoe_status smoe_w4a16_expert_ffn(const void* x, int T, int k, int E, int H, int I,
                                  int group_size,
                                  const uint32_t* wg_q, const void* wg_s,
                                  const uint32_t* wu_q, const void* wu_s,
                                  const uint32_t* wd_q, const void* wd_s,
                                  const int32_t* sorted_slots, const int32_t* expert_offsets,
                                  int shared_I, const void* shared_wg, const void* shared_wu,
                                  const void* shared_wd,
                                  void* workspace, size_t workspace_bytes,
                                  float* slot_out, float* shared_out, void* stream);

/*
 * smoe_w4a16_expert_ffn without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation. The call allocates
 * nothing; its workspace is a static device array of the library,
 * SMOE_NOALLOC_SCRATCH_BYTES bytes on each device the library runs on, held
 * until the process ends. Arguments, results, checks and errors are those
 * of smoe_w4a16_expert_ffn (minus workspace and workspace_bytes); the
 * caller still passes every input and output.
 *
 *   - A window whose workspace (smoe_ffn_workspace_bytes(T, k, E, H, I,
 *     shared_I)) exceeds SMOE_NOALLOC_SCRATCH_BYTES is refused with
 *     SMOE_EUNSUPPORTED before anything is enqueued (16 MiB covers windows
 *     of a few hundred slots at I = 1408, e.g. T = 17, k = 6 needs 3 MB).
 *   - Each call first clears the workspace bytes it uses (a fill kernel on
 *     `stream`), so a call never depends on what an earlier call left there,
 *     whatever its shapes.
 *   - Every call on one device shares that device's array: calls that
 *     overlap in time on one device (different streams without ordering
 *     between them, or different host threads) race and give undefined
 *     results. Calls ordered on one stream are safe.
 *   - SMOE_EHIP if the array's device address cannot be obtained.
 */
#define SMOE_NOALLOC_SCRATCH_BYTES (16u << 20)
smoe_status smoe_w4a16_expert_ffn_noalloc(const void* x, int T, int k, int E, int H, int I,
                                          int group_size,
                                          const uint32_t* wg_q, const void* wg_s,
                                          const uint32_t* wu_q, const void* wu_s,
                                          const uint32_t* wd_q, const void* wd_s,
                                          const int32_t* sorted_slots,
                                          const int32_t* expert_offsets,
                                          int shared_I, const void* shared_wg,
                                          const void* shared_wu, const void* shared_wd,
                                          float* slot_out, float* shared_out, void* stream);

/*
 * Expert FFN with FP16 weights (target verification pass and always-on
 * shared experts).                                    [P] expert-wise
 * verification paragraphs (target router decisions; tokens of each expert
 * packed into contiguous sub-batches, GEMVs become GEMMs; routing-weighted
 * outputs scattered back; strict mathematical equivalence) and the
 * hybrid-precision layout (shared experts stay FP16); [D] "Streamlined
 * Execution Engine" (expert_reorder).
 *
 * Same computation, alignment, shared-expert option and workspace contract
 * as smoe_w4a16_expert_ffn with routed weights W = fp16 values:
 *   wg, wu   fp16 [E][I][H];   wd   fp16 [E][H][I]
 * A shared expert can also be run on its own as E = 1, k = 1 with
 * sorted_slots = 0..T-1 and expert_offsets = {0, T}.
 */
smoe_status smoe_fp16_expert_ffn(const void* x, int T, int k, int E, int H, int I,
                                 const void* wg, const void* wu, const void* wd,
                                 const int32_t* sorted_slots, const int32_t* expert_offsets,
                                 int shared_I, const void* shared_wg, const void* shared_wu,
                                 const void* shared_wd,
                                 void* workspace, size_t workspace_bytes,
                                 float* slot_out, float* shared_out, void* stream);

/*
 * smoe_fp16_expert_ffn over weights addressed through a table: the FFN of
 * the verification pass when the routed experts live in a pool of device
 * slots (an expert cache) rather than at their own index.   [P] Verification
 * Expert Cache Residency Manager paragraph (cache-hit experts go to the
 * compute queue first, cache-miss experts join it as their copies land) and
 * cache-aware execution schedule paragraph (compute the resident expert's
 * sub-batch while the missing one is copied); [D] "Predictive I/O
 * Orchestrator" (expert_cache: slot ownership, resident experts first).
 *
 * Same computation, alignment, shared-expert option and workspace contract
 * as smoe_fp16_expert_ffn, except:
 *   - the weights of routed expert e are matrix expert_matrix[e] of each of
 *     wg, wu and wd (address base + expert_matrix[e] * the bytes of one
 *     matrix), which must each hold n_matrices matrices;
 *   - an expert whose entry is negative or >= n_matrices is left out of the
 *     call: its slots are neither computed nor written. Only the rows of
 *     slot_out of the call's experts are written; every other row keeps what
 *     it held, so several calls over disjoint expert sets fill one slot_out
 *     (the rows of slots the alignment dropped are not written either).
 *
 *   expert_matrix  int32 [E], HOST memory, read during the call (the table
 *                  travels in the launch arguments, so a captured graph
 *                  keeps the values it had at capture)
 *   tiled          1: wg, wu, wd in the layout of smoe_tile_weights (each
 *                  matrix tiled on its own), 0: row-major
 * A pool that keeps an expert's three matrices together, [slots][3][matrix],
 * is addressed with wg = pool, wu = pool + one matrix, wd = pool + two
 * matrices, expert_matrix[e] = 3 * slot and n_matrices = 3 * slots - 2.
 */
smoe_status smoe_fp16_expert_ffn_mapped(const void* x, int T, int k, int E, int H, int I,
                                        const void* wg, const void* wu, const void* wd,
                                        int tiled, int n_matrices, const int32_t* expert_matrix,
                                        const int32_t* sorted_slots,
                                        const int32_t* expert_offsets, int shared_I,
                                        const void* shared_wg, const void* shared_wu,
                                        const void* shared_wd, void* workspace,
                                        size_t workspace_bytes, float* slot_out,
                                        float* shared_out, void* stream);

/*
 * Weighted combine back to token order.               [P] expert-wise
 * verification paragraph (per-slot expert outputs go back to their own
 * token, weighted by the router, and add up there); [D] "Streamlined
 * Execution Engine" (kernels reduce expert outputs).
 *
 *   y[t] = fp16( sum_{j=0..k-1} topk_w[t][j] * slot_out[t*k + j]
 *                + gate[t] * shared_out[t] )
 * summed in float32 with j ascending, the shared term last; gate = 1 when
 * shared_gate is NULL; no shared term when shared_out is NULL.
 *
 *   slot_out   float [T*k][H]; topk_w float [T][k]
 *   shared_out float [T][H] or NULL; shared_gate float [T] or NULL
 *   y          fp16 [T][H] (out)
 */
smoe_status smoe_combine(const float* slot_out, const float* topk_w, int T, int k, int H,
                         const float* shared_out, const float* shared_gate,
                         void* y, void* stream);

/*
 * The whole draft layer in one call: routing, alignment and the ELB update
 * (smoe_route_align_elb), the W4A16 expert FFN with the optional FP16 shared
 * experts (smoe_w4a16_expert_ffn) and the weighted combine (smoe_combine),
 * as those calls made one after the other compute them, with the same
 * arguments, checks and errors; every check runs before anything is
 * enqueued. Specter paper: the draft MoE layer of the fused multi-expert
 * draft kernel paragraph, fed by the Incremental Routing Pattern Analyzer.
 *
 * Arguments are those of the three calls (one copy of each shared one):
 * routing and ELB as in smoe_route_align_elb; I, group_size, the routed
 * INT4 weights, the shared FP16 weights, workspace, slot_out and shared_out
 * as in smoe_w4a16_expert_ffn (sorted_slots and expert_offsets are this
 * call's outputs); y [T][H] fp16 as in smoe_combine, whose shared_out is
 * the FFN's when shared_I > 0 and whose gate is shared_gate. All buffers
 * are caller-owned device memory.
 *
 * The layer takes the launches of the three calls: router logits, the
 * top-k / alignment / ELB workgroup, the two FFN launches and the combine.
 * When that workgroup runs alone (T*k <= 512) and the shared weights total
 * at most 40 MB, its launch also holds one workgroup per other CU that only
 * reads the shared weights, so that the FFN finds them in the caches; the
 * results are unchanged. On error nothing is enqueued.
 */
smoe_status smoe_moe_layer_w4a16(const void* x, const float* w_router, const float* logit_bias,
                                 int T, int H, int E, int k, int flags,
                                 int32_t* topk_ids, float* topk_w, float* logits,
                                 const float* shared_gate_w, float* shared_gate,
                                 int32_t* expert_counts, int32_t* expert_offsets,
                                 int32_t* sorted_slots, int32_t* active_experts,
                                 int32_t* n_active,
                                 int32_t* elb_counts, int L, int layer, int M,
                                 int32_t* plan_ids, int32_t* plan_counts, int elb_flags,
                                 int I, int group_size,
                                 const uint32_t* wg_q, const void* wg_s,
                                 const uint32_t* wu_q, const void* wu_s,
                                 const uint32_t* wd_q, const void* wd_s,
                                 int shared_I, const void* shared_wg, const void* shared_wu,
                                 const void* shared_wd, void* workspace, size_t workspace_bytes,
                                 float* slot_out, float* shared_out, void* y, void* stream);

/*
 * Tiled weight layout.  [P] fused multi-expert draft kernel paragraph (INT4
 * weight tiles streamed per expert); [D] "Streamlined Execution Engine"
 * (W4A16 dequantisation of weight tiles). The pages fix no memory layout;
 * this one is the expert FFN's own: the same bytes as the row-major
 * layout, ordered so that every load of the FFN reads one contiguous
 * kilobyte (and the scales of a row slice and block of k one contiguous
 * run). Weights are tiled once, when loaded; the *_tiled calls below then
 * stream them.
 *
 * For one [E][N][K] weight tensor (row n of expert e holds the K
 * reduction values of output n):
 *   group_size 0:   w fp16 [E][N][K], scales ignored (NULL);
 *   group_size G:   w uint32 [E][N][K/8] INT4 codes (the packed format of
 *                   smoe_w4a16_expert_ffn), scales fp16 [E][N][K/G].
 * Output, for each expert e, row slice sl = n / 16 (slices in order) and
 * block b of 64 bytes of a row (blocks in order within a slice): 1 KB
 * where bytes 16 (16 g + r) .. +15 hold four 32-bit words of row
 * 16 sl + r, block b: words 4 g + q (q = 0..3) for FP16 and G = 128;
 * words (q / (G/32)) (G/8) + g (G/32) + q % (G/32) for G = 64 and 32.
 * Scales, for each (e, sl, b): 16 runs (r = 0..15) of 128 / G values, the
 * scales of row 16 sl + r in block b, in k order.
 *
 *   N a multiple of 16, K of 128; w_tiled (and scales_tiled) the sizes of
 *   w (and scales), caller-owned device memory, 16-byte aligned, not
 *   overlapping the inputs.
 * SMOE_EINVAL for null, misaligned or overlapping buffers,
 * SMOE_EUNSUPPORTED for other shapes or group sizes. Asynchronous on
 * `stream`; E = 0 or N = 0 enqueues nothing.
 */
smoe_status smoe_tile_weights(const void* w, const void* scales, int E, int N, int K,
                              int group_size, void* w_tiled, void* scales_tiled, void* stream);

/*
 * smoe_w4a16_expert_ffn, smoe_fp16_expert_ffn and smoe_moe_layer_w4a16
 * with every weight tensor passed (routed codes and scales, and the shared
 * FP16 weights) in the tiled layout of smoe_tile_weights, each tiled as
 * the [E][N][K] tensor its row-major form is. Arguments, results, checks
 * and errors are otherwise those of the row-major calls.
 */
smoe_status smoe_w4a16_expert_ffn_tiled(const void* x, int T, int k, int E, int H, int I,
                                        int group_size,
                                        const uint32_t* wg_q, const void* wg_s,
                                        const uint32_t* wu_q, const void* wu_s,
                                        const uint32_t* wd_q, const void* wd_s,
                                        const int32_t* sorted_slots,
                                        const int32_t* expert_offsets,
                                        int shared_I, const void* shared_wg,
                                        const void* shared_wu, const void* shared_wd,
                                        void* workspace, size_t workspace_bytes,
                                        float* slot_out, float* shared_out, void* stream);
smoe_status smoe_fp16_expert_ffn_tiled(const void* x, int T, int k, int E, int H, int I,
                                       const void* wg, const void* wu, const void* wd,
                                       const int32_t* sorted_slots,
                                       const int32_t* expert_offsets,
                                       int shared_I, const void* shared_wg,
                                       const void* shared_wu, const void* shared_wd,
                                       void* workspace, size_t workspace_bytes,
                                       float* slot_out, float* shared_out, void* stream);
smoe_status smoe_moe_layer_w4a16_tiled(const void* x, const float* w_router,
                                       const float* logit_bias, int T, int H, int E, int k,
                                       int flags, int32_t* topk_ids, float* topk_w,
                                       float* logits, const float* shared_gate_w,
                                       float* shared_gate, int32_t* expert_counts,
                                       int32_t* expert_offsets, int32_t* sorted_slots,
                                       int32_t* active_experts, int32_t* n_active,
                                       int32_t* elb_counts, int L, int layer, int M,
                                       int32_t* plan_ids, int32_t* plan_counts, int elb_flags,
                                       int I, int group_size,
                                       const uint32_t* wg_q, const void* wg_s,
                                       const uint32_t* wu_q, const void* wu_s,
                                       const uint32_t* wd_q, const void* wd_s,
                                       int shared_I, const void* shared_wg,
                                       const void* shared_wu, const void* shared_wd,
                                       void* workspace, size_t workspace_bytes,
                                       float* slot_out, float* shared_out, void* y,
                                       void* stream);

/* ====================================================================
 * Expert cache of the verification pass and the prefetch planner (host
 * runtime).   [P] Layer-Aware Prefetch Planner paragraphs (Cold Start,
 * Prefetch Overlap, Final Cleanup; top-M snapshot at each chunk boundary,
 * the experts not yet cached form the next host-to-device batch, the next
 * boundary chosen so the chunk's draft compute matches the batch's transfer
 * time); Verification Expert Cache Residency Manager paragraph (hits
 * computed first, misses copied and computed as they land, slots protected
 * until their expert's tokens are done); cache-aware execution schedule
 * paragraph; Overlap-Oriented Parallelism Optimizer paragraph (compute and
 * I/O streams, events for readiness and slot reuse, pinned host memory,
 * asynchronous copies); [D] "Predictive I/O Orchestrator" (expert_cache,
 * prefetch_planner; residency is a per-layer slot budget).
 *
 * A cache holds, per layer, M device slots of one expert each (its three
 * FP16 matrices). Its state lives on the host: the expert of each slot (-1
 * empty), the clock value of each slot's last use, and whether the current
 * window's predictions claimed the slot. Decisions:
 *   - replacement: an empty slot first (lowest index), else the least
 *     recently used one (ties to the lower index) among those allowed;
 *   - the clock advances by one for each prefetch call per layer (every slot
 *     it claims or loads gets that value), for the hit group of a
 *     verification, and for each miss's computation.
 * Functions taking a cache are not thread-safe on the same cache. These
 * calls (unlike the kernels above) allocate host memory and HIP events in
 * smoe_cache_create and free them in smoe_cache_destroy.
 * ==================================================================== */
typedef struct smoe_expert_cache smoe_expert_cache;

/*
 * Create a cache of L layers, E experts per layer, M slots per layer.
 *   pool          device [L][M][expert_bytes], caller-owned: slot s of
 *                 layer l at pool + (l*M + s) * expert_bytes
 *   host_experts  host [L][E][expert_bytes] (allocate with hipHostMalloc so
 *                 the copies are asynchronous), caller-owned
 * Both NULL: a cache that only takes decisions (no device, no copies; the
 * verify_layer call is then refused). expert_bytes: a multiple of 16; for
 * verify_layer it must be 3 * I * H * 2 (wg [I][H], wu [I][H], wd [H][I]
 * fp16, in this order, each row-major or each tiled by smoe_tile_weights).
 * Creates two HIP events per slot on the current device.
 */
smoe_status smoe_cache_create(int L, int E, int M, size_t expert_bytes, void* pool,
                              const void* host_experts, smoe_expert_cache** cache);
smoe_status smoe_cache_destroy(smoe_expert_cache* cache);

/* Start a draft window: no slot is claimed. */
smoe_status smoe_cache_begin_window(smoe_expert_cache* cache);

/* Copy the state out (host arrays [L][M]; any may be NULL). */
smoe_status smoe_cache_state(const smoe_expert_cache* cache, int32_t* slot_expert,
                             int64_t* last_use, int32_t* claimed, int64_t* clock);

/*
 * Install a state (host arrays [L][M]: the expert of each slot or -1, each
 * slot's last use in [0, clock]); no slot is claimed. With device memory,
 * every cached expert is copied into its slot on copy_stream.
 */
smoe_status smoe_cache_set_state(smoe_expert_cache* cache, const int32_t* slot_expert,
                                 const int64_t* last_use, int64_t clock, void* copy_stream);

/*
 * Prefetch at a chunk boundary, from the ELB's top-M plan
 * (smoe_elb_accumulate_topm's plan_ids / plan_counts, copied to the host).
 * For each layer l: the selection is the plan's experts with a positive
 * count, in ranking order, at most M of them; the selected experts already
 * cached are claimed first; then each selected expert not cached takes, in
 * ranking order, a slot that is not claimed (replacement rule above) and is
 * claimed, until no unclaimed slot is left. A claimed slot is not taken by
 * another expert until the next window.
 *   plan_ids, plan_counts  host int32 [L][plan_M]
 *   loads     host int32 [L*M][4] (out): (layer, expert, slot, evicted expert
 *             or -1) of every copy, in the order they were decided
 *   n_loads   (out) number of loads; full (out, may be NULL): 1 if no slot
 *             of any layer is left unclaimed (the planner's Final Cleanup)
 * With device memory each load is enqueued on copy_stream (after the last
 * computation that read the slot).
 */
smoe_status smoe_cache_prefetch(smoe_expert_cache* cache, const int32_t* plan_ids,
                                const int32_t* plan_counts, int plan_M, int32_t* loads,
                                int* n_loads, int* full, void* copy_stream);

/*
 * The planner's next chunk boundary after b for a batch of n_transfer
 * experts: b + n with the smallest n >= 1 such that n * draft_us_per_token
 * >= t_io, where t_io = n_transfer * expert_bytes / (h2d_gb_per_s * 1000)
 * microseconds (double precision, in this order); capped at K.
 */
smoe_status smoe_prefetch_next_boundary(int b, int K, int n_transfer, double expert_bytes,
                                        double h2d_gb_per_s, double draft_us_per_token,
                                        int* next_b);

/*
 * Verification decisions for one layer (no device work): expert_counts
 * host int32 [E] (tokens the target router sent to each expert). The
 * required experts (count > 0) split into hits (cached) and misses. The
 * schedule, host int32 [E][5] (out), lists in compute order
 * (expert, slot, kind, evicted, wait):
 *   - first the hits in ascending expert ID: kind 0, evicted = expert,
 *     wait -1; they form one computation (group 0) and their slots are
 *     protected until it ends;
 *   - then the misses in ascending expert ID, each its own computation
 *     (group 1 + j for the j-th miss): kind 1, the slot it is copied into,
 *     the expert it evicts (-1 for an empty slot), and wait = -1 when the
 *     slot was free or unprotected (replacement rule), else the group whose
 *     end releases it: slots come back in the order their computations end
 *     (the hit group's slots in slot order, then each miss's slot).
 * The state is updated (slots, last uses).
 */
smoe_status smoe_cache_verify_plan(smoe_expert_cache* cache, int layer,
                                   const int32_t* expert_counts, int32_t* schedule,
                                   int* n_schedule);

/*
 * The verification FFN of one layer with the cache: the decisions of
 * smoe_cache_verify_plan, then, on compute_stream, the hit group's
 * smoe_fp16_expert_ffn_mapped call (with the FP16 shared experts when
 * shared_I > 0) and, for each miss, its copy on copy_stream followed by its
 * own mapped FFN call on compute_stream. Events order every copy after the
 * slot's last computation and every computation after its slot's copy, so
 * the hits run while the misses are copied; nothing waits on the host.
 *
 *   expert_counts   host int32 [E] (this layer's alignment counts, which the
 *                   caller copied back from the device)
 *   x .. shared_out as in smoe_fp16_expert_ffn (T, k, H, I; sorted_slots and
 *                   expert_offsets from the alignment of the target router's
 *                   IDs; tiled as in smoe_fp16_expert_ffn_mapped)
 *   workspace_shared  FFN workspace for (T, k, I, shared_I) (hit group), or
 *                   NULL when shared_I = 0; workspace_routed a distinct one
 *                   for (T, k, I, 0) (misses). Each follows the workspace
 *                   contract.
 *   schedule, n_schedule  as in smoe_cache_verify_plan (may be NULL)
 * slot_out rows of every required expert's slots are written (the call's
 * experts are all the target router's); shared_out as usual. Checks run
 * before the state changes or anything is enqueued; a HIP failure after
 * that returns SMOE_EHIP with the decisions already taken.
 */
smoe_status smoe_cache_verify_layer(smoe_expert_cache* cache, int layer,
                                    const int32_t* expert_counts, const void* x, int T, int k,
                                    int H, int I, int tiled, const int32_t* sorted_slots,
                                    const int32_t* expert_offsets, int shared_I,
                                    const void* shared_wg, const void* shared_wu,
                                    const void* shared_wd, void* workspace_shared,
                                    size_t workspace_shared_bytes, void* workspace_routed,
                                    size_t workspace_routed_bytes, float* slot_out,
                                    float* shared_out, int32_t* schedule, int* n_schedule,
                                    void* compute_stream, void* copy_stream);

/*
 * SpecFit verification-subtree selection (host): the exact search over the
 * draft pool's legal subtrees.   SpecFit page, sections 3.1 (legal subtree:
 * ancestor-closed, at most K nodes; top-2 expansion, depth <= 5, <= 18
 * nodes, K = min(7, pool size)), 3.2 (reward = 1 + sum of the selected
 * nodes' path probabilities; cycle time = an intercept by node count + beta
 * times the per-layer expert-union feature), 3.3 (the largest reward / time)
 * and appendix A.3 (depth-first enumeration, parent before descendant, with
 * incremental expert bitmaps).
 *
 *   n            pool nodes (0 .. 64); parent int32 [n]: -1 for a child of the
 *                root, else an earlier node (parents precede their children)
 *   path_prob    double [n], the drafter's path probability of each node
 *   expert_bits  uint64 [n + 1][L][W], W = ceil(E / 64): row 0 the root's
 *                experts (the committed token, always verified), row v + 1
 *                node v's; bit e of layer l = expert e activated
 *   resident_bits uint64 [L][W] (experts already in the device cache, which
 *                cost nothing) or NULL (every expert costs)
 *   K            size limit (the search uses min(K, n)); intercepts double
 *                [min(K, n) + 1] > 0, intercept[s] for s selected nodes; beta >= 0
 * Selection: the legal subtree S maximising
 *   (1 + sum_{v in S, ascending v} path_prob[v]) / (intercept[|S|] + beta * F(S)),
 * F(S) = sum over layers of popcount((root | nodes of S) & ~resident), each
 * step one double operation; ties to fewer nodes, then the smaller
 * ascending node list. The empty subtree (root only) is legal.
 *   selected     int32 [min(K, n)] (out), ascending; n_selected (out);
 *   ratio (out, may be NULL); n_evaluated (out, may be NULL): legal subtrees
 *   visited.
 * Drafting goes on after a level only while the selection holds a node of
 * that level (the caller's check).
 */
smoe_status smoe_specfit_select(int n, const int32_t* parent, const double* path_prob, int L,
                                int E, const uint64_t* expert_bits,
                                const uint64_t* resident_bits, int K, const double* intercepts,
                                double beta, int32_t* selected, int* n_selected, double* ratio,
                                int64_t* n_evaluated);

#ifdef __cplusplus
}
#endif

#endif /* SMOE_H */
