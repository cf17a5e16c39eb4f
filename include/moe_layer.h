/*
 * moe_layer.h - C ABI of libmoelayer.so: one GPU's share of an
 * expert-parallel Mixture-of-Experts layer on AMD Instinct MI355X (gfx950).
 *
 * The layer (page "OverlapAdvisor: Modeling and Adapting Computation-
 * Communication Overlap for Distributed MoE Serving", section 2.1: each token
 * activates only its top-k experts; dispatch routes tokens to experts and
 * combine returns the outputs to their origin) is split into the calls
 *
 *   moe_route        top-k softmax gate over router logits
 *   moe_dispatch     expert-major permutation of the local (token, slot)
 *                    pairs plus the gather of their activation rows
 *   moe_grouped_ffn  gated SwiGLU FFN of every local expert over its segment
 *   moe_combine      gate-weighted sum back to token order (+ shared expert)
 *   moe_layer        all of the above in one call
 *   moe_layer_streamed  the layer in invocations over consecutive token
 *                    groups on several streams (streaming FFN), planned by
 *                    moe_stream_threshold / moe_stream_plan
 *
 * plus moe_quantize_fp8 (block-FP8 conversion of bf16 weights at load time and
 * of activations) and the helpers moe_workspace_bytes / moe_status_str.
 *
 * Conventions for every call
 *  - Problem sizes follow the pages' workload tuple (tokens, hidden size H,
 *    experts E, top-k, intermediate size I) plus the local expert range
 *    [expert_begin, expert_begin + num_local) of this rank (moe_problem).
 *  - Every array argument is a DEVICE pointer to caller-owned memory, row
 *    major unless moe_problem.layout says otherwise, 16-byte aligned.  The
 *    library never allocates, keeps no state between calls, is reentrant,
 *    and never synchronises the host: all work
 *    is enqueued on `stream` (a hipStream_t; NULL = the default stream), and
 *    data-dependent sizes (per-expert counts, tile lists) stay on the device.
 *  - Arguments are validated before anything is enqueued.  On any error
 *    nothing is enqueued and outputs are untouched.  A launch failure returns
 *    MOE_ERR_HIP; faults of kernels surface at the caller's next sync.
 *  - num_tokens == 0 is valid: MOE_OK, nothing enqueued.
 *  - Logits must be finite (NaN/Inf logits give unspecified, but in-bounds,
 *    routing).
 *  - Capacity: the permuted buffers hold N_cap rows: T * min(k, E_L) in the
 *    contiguous layout (the number of valid rows is offsets[E_L] on the
 *    device), E_L * capacity in the masked layout (moe_problem.capacity).
 *
 * Supported sizes: 1 <= E <= 1024, 1 <= k <= min(E, 32), 1 <= E_L <= 1024,
 * 0 <= e_lo, e_lo + E_L <= E, 0 <= T <= 2^24, H % 128 == 0, I % 128 == 0
 * (and shared_inter % 128 == 0), H, I <= 65536, and one expert's up
 * projection below 2 GiB in bf16 (4 I H < 2^31, likewise for shared_inter);
 * larger experts return MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 10

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, size out of range, misalignment */
  MOE_ERR_UNSUPPORTED = 2,  /* valid request the library does not implement  */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required     */
  MOE_ERR_HIP = 4           /* a HIP launch or runtime call failed            */
} moe_status;

typedef enum {
  MOE_BF16 = 0,      /* bf16 weights, bf16 GEMM activations                  */
  MOE_FP8_E4M3 = 1,  /* OCP E4M3FN weights with one fp32 scale per 128 x 128
                        block; GEMM activations E4M3 with one fp32 scale per
                        token per 128 consecutive elements                   */
  MOE_MXFP4 = 2      /* MXFP4 weights (OCP MX: E2M1 elements, one E8M0 scale
                        per 32 consecutive K elements of a row); GEMM
                        activations MXFP8 (E4M3, one E8M0 scale per token per
                        32 elements).  Page "CascadeEP ...", section 4.1
                        (MXFP4 routed-expert weights).  Layout 0, SwiGLU.   */
} moe_dtype;

/* MX element formats of moe_quantize_mx. */
#define MOE_MX_E2M1 0
#define MOE_MX_E4M3 1

/* Storage layouts (moe_problem.layout bits; values are never changed by a
 * layout).  bf16: both bits; MOE_MXFP4: MOE_LAYOUT_PANEL_WEIGHTS only;
 * MOE_FP8_E4M3: none.  The panel layout of an [R, K] bf16 matrix
 * cuts its columns into panels of 32 consecutive elements (64 bytes) and
 * stores the panels one after another, each as an [R, 32] row-major block:
 *   element (r, c) lives at index ((c / 32) * R + r) * 32 + c % 32.
 * A GEMM step over 32 columns then reads one contiguous block per operand
 * tile instead of 64 bytes from each of hundreds of rows, which keeps the
 * HBM and L2 traffic of the grouped GEMM in long runs.
 *   MOE_LAYOUT_PANEL_WEIGHTS: each expert's w13 [2I, H] and w2 [H, I] (and
 *     ws13 / ws2) is in panel layout (R = 2I, H, 2 I_s, H); see
 *     moe_pack_panel.
 *   MOE_LAYOUT_PANEL_ACTS: x_perm [N_cap, H] written by moe_dispatch and read
 *     by moe_grouped_ffn, and h [N_cap, I], are in panel layout with
 *     R = N_cap.  moe_layer keeps its own x_perm and h in panel layout
 *     whatever this bit says.
 * MXFP4 panel weights: each matrix's E2M1 codes [R, K/2 bytes] are cut into
 * 64-byte (128-element) panels, [K/128, R, 64 bytes], and its E8M0 scales
 * [R, K/32] into 4-byte pieces, [K/128, R, 4 bytes]: byte j of row r's codes
 * lives at ((j / 64) * R + r) * 64 + j % 64, scale byte j at
 * ((j / 4) * R + r) * 4 + j % 4.  A decode-sized GEMM step then reads each
 * operand tile's weights as one contiguous run.  See moe_pack_panel_mx.     */
#define MOE_LAYOUT_PANEL_WEIGHTS 1
#define MOE_LAYOUT_PANEL_ACTS 2

/* Expert MLP form (moe_problem.activation).  Page "OverlapAdvisor ...",
 * Eq. 8 (m first-layer matrices: 2 for a gated MLP, 1 for a standard one)
 * and Table 6 (the FP8 group runs gated SwiGLU, the BF16 group a standard
 * MLP with GELU).
 *   MOE_ACT_SWIGLU (m = 2): h = silu(x Wg^T) * (x Wu^T), silu(a) = a/(1+e^-a)
 *   MOE_ACT_GELU   (m = 1): h = gelu(x W1^T), gelu(a) = a * Phi(a) (exact,
 *                  Phi the standard normal distribution function); bf16 only */
#define MOE_ACT_SWIGLU 0
#define MOE_ACT_GELU 1

/* The workload tuple of one rank. */
typedef struct {
  int32_t num_tokens;    /* T: tokens in the batch                            */
  int32_t hidden;        /* H: model hidden size                              */
  int32_t num_experts;   /* E: routed experts of the whole layer              */
  int32_t top_k;         /* k: experts per token                              */
  int32_t expert_begin;  /* e_lo: first local expert (global id)              */
  int32_t num_local;     /* E_L: local experts, global ids [e_lo, e_lo+E_L)   */
  int32_t inter;         /* I: expert FFN intermediate size                   */
  int32_t shared_inter;  /* I_s: shared-expert intermediate size, 0 = none    */
  int32_t dtype;         /* moe_dtype                                          */
  int32_t layout;        /* MOE_LAYOUT_* bits, 0 = all row major; must be 0
                            for MOE_FP8_E4M3                                   */
  int32_t activation;    /* MOE_ACT_SWIGLU (0) or MOE_ACT_GELU                 */
  int32_t capacity;      /* 0: contiguous expert segments.  C > 0: masked
                            fixed-capacity layout (see below); C >= T,
                            C <= 2^24, E_L * C < 2^31                         */
} moe_problem;

/* Masked (fixed-capacity) layout, moe_problem.capacity = C > 0.  Page
 * "ExpertPlex": masked grouped-GEMM layout; page "OverlapAdvisor ...",
 * Table 7 and Table 6 note b: the low-latency dispatch used for small batches
 * feeds the GroupGEMM with no permute step.  Local expert e owns the rows
 * [e C, (e + 1) C) of x_perm, h and y_perm, and its counts[e] pairs fill the
 * first counts[e] of them, tokens ascending (the same order as in the
 * contiguous layout, so every per-row result is the same); the other rows
 * are neither read nor written.  Buffers keep one shape for every T <= C.
 * Where a call takes the segment table of the grouped FFN, the masked layout
 * passes counts [E_L] (from moe_dispatch) instead of offsets.              */

/* Expert weights, device pointers, K-contiguous ("[out, in]" row major).
 *   w13  [E_L, m I, H]: SwiGLU (m = 2): rows 0..I-1 gate projection, rows
 *        I..2I-1 up projection; GELU (m = 1): the first-layer matrix W1
 *   w2   [E_L, H, I]:  down projection
 *   ws13 [m I_s, H], ws2 [H, I_s]: shared expert (NULL when I_s == 0), same
 *        form as the routed experts
 * Element type: bf16 for MOE_BF16, E4M3 bytes for MOE_FP8_E4M3; for MOE_MXFP4
 * E2M1 codes two per byte, low nibble first ([E_L, m I, H/2] and
 * [E_L, H, I/2]).
 * fp8 only, fp32 block scales (NULL for bf16):
 *   w13_scale [E_L, 2I/128, H/128], w2_scale [E_L, H/128, I/128],
 *   ws13_scale [2 I_s/128, H/128],  ws2_scale [H/128, I_s/128].
 * MOE_MXFP4: the scale pointers carry E8M0 bytes (uint8, value 2^(e-127)),
 * one per 32 K elements of a row: w13_scale [E_L, 2I, H/32], w2_scale
 * [E_L, H, I/32], ws13_scale [2 I_s, H/32], ws2_scale [H, I_s/32] (see
 * moe_quantize_mx).  The scale pointers are untyped for that reason: fp32
 * (float*) for MOE_FP8_E4M3, bytes (uint8_t*) for MOE_MXFP4.               */
typedef struct {
  const void* w13;
  const void* w2;
  const void* ws13;
  const void* ws2;
  const void* w13_scale;
  const void* w2_scale;
  const void* ws13_scale;
  const void* ws2_scale;
} moe_weights;

/* Top-k gate.  Page "OverlapAdvisor ...", section 2.1 (top-k experts per
 * token); the weights are the softmax of the router logits renormalised over
 * the selected experts.
 *   logits   [T, E] fp32 (input)
 *   topk_ids [T, k] int32 (output): the k experts first in the order
 *            (logit descending, expert id ascending; -0.0 == +0.0)
 *   topk_w   [T, k] fp32 (output): exp(l_s - l_0) / sum_j exp(l_j - l_0)
 * Routing is over all E experts; locality plays no part here.            */
moe_status moe_route(const moe_problem* p, const float* logits,
                     int32_t* topk_ids, float* topk_w, void* stream);

/* Dispatch: permutation plus gather.  Page "CascadeEP: Asynchronous Expert
 * Execution for MoE Prefill under Attention Imbalance", Appendix C, "Grouped
 * FFN invocations" (per-expert row offsets from the selected counts, rows
 * grouped by expert, activations packed with their quantisation metadata, an
 * inverse map to token and routing slot); page "OverlapAdvisor ...", section
 * 4.2.1 (permute groups tokens by expert).
 *   x          [T, H] bf16 (input)
 *   topk_ids   [T, k] int32 (input, e.g. from moe_route).  A slot that repeats
 *              an expert already picked by an earlier slot of the same token
 *              is ignored (treated as non-local).
 *   counts     [E_L] int32: local pairs per local expert
 *   offsets    [E_L + 1] int32: exclusive scan of counts; N = offsets[E_L]
 *              (masked layout: the block starts e C, offsets[E_L] = E_L C)
 *   row_token  [N_cap] int32, row_slot [N_cap] int32: token and slot of row j
 *              (rows holding no pair are left untouched)
 *   token_slot_row [T, k] int32: row of pair (t, s), -1 if not local
 *   x_perm     [N_cap, H]: row j = x[row_token[j]]; bf16, or for
 *              MOE_FP8_E4M3 the E4M3 codes of that row with
 *   x_perm_scale [N_cap, H/128] fp32 (fp8 only; NULL for bf16): scale of each
 *              128-element group, amax/448 (1 for an all-zero group); code =
 *              round-to-nearest-even(v / scale) saturated to +-448.
 *              MOE_MXFP4: x_perm holds MXFP8 (E4M3) codes and x_perm_scale
 *              E8M0 bytes [N_cap, H/32] (moe_quantize_mx's rule).
 * Rows are ordered by local expert, then by token (contiguous segments, or
 * the expert's block in the masked layout).  Bit-exact and deterministic.  x_perm == NULL builds the index only (x_perm_scale is then
 * ignored; see moe_grouped_ffn_gather).
 * Workspace: moe_workspace_bytes(p, MOE_STAGE_DISPATCH).                   */
moe_status moe_dispatch(const moe_problem* p, const void* x,
                        const int32_t* topk_ids, int32_t* counts,
                        int32_t* offsets, int32_t* row_token,
                        int32_t* row_slot, int32_t* token_slot_row,
                        void* x_perm, void* x_perm_scale, void* ws,
                        size_t ws_bytes, void* stream);

/* Grouped expert FFN.  Page "OverlapAdvisor ...", section 4.2.2 and Eq. 8
 * (m first-layer matrices; the up GroupGEMM is 2 m H I FLOPs per row, the
 * down GroupGEMM 2 H I), Table 6 (gated SwiGLU; standard MLP with GELU);
 * page "CascadeEP ...", Appendix C (the two expert GEMMs with the activation
 * and quantisation between them, in stream order).
 * For every local expert e and row j of its segment, [offsets[e],
 * offsets[e+1]) (masked layout: [e C, e C + counts[e]), with `offsets`
 * carrying counts [E_L]):
 *   SwiGLU: h[j] = silu(x_perm[j] . W_gate,e^T) * (x_perm[j] . W_up,e^T) [I]
 *   GELU:   h[j] = gelu(x_perm[j] . W1_e^T)                              [I]
 *   y_perm[j] = h[j] . W2_e^T                                          [H]
 * with fp32 accumulation (see MOE_ACT_*).
 *   x_perm, x_perm_scale, offsets: as produced by moe_dispatch (counts for
 *              the masked layout)
 *   h          [N_cap, I] (optional, NULL = kept in the workspace): bf16,
 *              or E4M3 with h_scale [N_cap, I/128] fp32 for MOE_FP8_E4M3,
 *              or MXFP8 (E4M3) with h_scale E8M0 bytes [N_cap, I/32] for
 *              MOE_MXFP4.  The scale pointers of this call, of moe_dispatch
 *              and of moe_grouped_ffn_gather are untyped: they carry fp32
 *              (block-FP8) or E8M0 bytes (MXFP4) by element type
 *   y_perm     [N_cap, H] bf16 (output)
 * Routing weights are NOT applied here (moe_combine applies them).
 * Only the segments' rows are read or written.  With E_L = 1 and
 * offsets = {0, T} this is a dense SwiGLU FFN (how a shared expert is run).
 * Workspace: moe_workspace_bytes(p, MOE_STAGE_FFN).                        */
moe_status moe_grouped_ffn(const moe_problem* p, const void* x_perm,
                           const void* x_perm_scale, const int32_t* offsets,
                           const moe_weights* w, void* h, void* h_scale,
                           void* y_perm, void* ws, size_t ws_bytes,
                           void* stream);

/* The grouped FFN reading its rows straight from the unpermuted tokens: row
 * j of the permutation is x[row_token[j]] (the page passages are those of
 * moe_grouped_ffn).  Together with moe_dispatch(..., x_perm = NULL, ...)
 * this is the path of moe_layer, kernel for kernel: the permuted
 * activations are never written.
 *   x [T, H] row major: bf16; for MOE_FP8_E4M3 the E4M3 codes of the
 *   tokens with x_scale [T, H/128] fp32 (moe_quantize_fp8 of the bf16
 *   tokens; MOE_MXFP4: the MXFP8 codes with x_scale holding E8M0 bytes
 *   [T, H/32], moe_quantize_mx with MOE_MX_E4M3): a row's codes depend on
 *   that row alone, so the result has the bits of moe_grouped_ffn on
 *   moe_dispatch's x_perm; x_scale NULL for bf16.
 *   row_token [N_cap] (from moe_dispatch), offsets (counts for the masked
 *   layout), w, h and h_scale (optional, as in moe_grouped_ffn; bf16 h in
 *   the layout of MOE_LAYOUT_PANEL_ACTS), y_perm [N_cap, H] bf16 (output).
 * MOE_ERR_UNSUPPORTED for x of 2 GiB or more.
 * Workspace: moe_workspace_bytes(p, MOE_STAGE_FFN).                        */
moe_status moe_grouped_ffn_gather(const moe_problem* p, const void* x,
                                  const void* x_scale,
                                  const int32_t* row_token,
                                  const int32_t* offsets, const moe_weights* w,
                                  void* h, void* h_scale, void* y_perm,
                                  void* ws, size_t ws_bytes, void* stream);

/* Combine.  Page "CascadeEP ...", Appendix C, "Output return and combine"
 * (each routed contribution weighted by its routing coefficient exactly once,
 * accumulated at the origin and added to the shared-expert output); page
 * "OverlapAdvisor ...", section 4.2.1 (unpermute restores token order).
 *   y[t] = sum over slots s with token_slot_row[t,s] >= 0, in slot order, of
 *          topk_w[t,s] * y_perm[token_slot_row[t,s]]  (+ shared_out[t])
 * accumulated in fp32 and rounded to bf16 once; a token with no local slot
 * gets 0 (+ shared_out[t]).  Deterministic (no atomics).
 *   y_perm [N_cap, H] bf16, token_slot_row [T, k] int32, topk_w [T, k] fp32,
 *   shared_out [T, H] bf16 or NULL, y [T, H] bf16 (output).               */
moe_status moe_combine(const moe_problem* p, const void* y_perm,
                       const int32_t* token_slot_row, const float* topk_w,
                       const void* shared_out, void* y, void* stream);

/* The whole layer: route, dispatch, grouped FFN, shared expert (when
 * shared_inter > 0, always on with weight 1) and combine.  Equal to the
 * composed calls (bit-identical routing and permutation).
 *   logits [T, E] fp32, x [T, H] bf16, y [T, H] bf16 (output).
 * Workspace: moe_workspace_bytes(p, MOE_STAGE_LAYER).                      */
moe_status moe_layer(const moe_problem* p, const float* logits, const void* x,
                     const moe_weights* w, void* y, void* ws, size_t ws_bytes,
                     void* stream);

/* moe_layer without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, results and kernels as moe_layer
 * (bit-identical output); the workspace is a static device array of
 * MOE_STATIC_SCRATCH_BYTES (64 MiB) that the library holds on every device it
 * runs on until the process ends.  The call itself allocates nothing; its
 * first call on a device resolves that device's copy of the array
 * (hipGetSymbolAddress), so make one call per device before a graph capture.
 * Every call on a device shares the array and leaves its contents behind
 * (every kernel initialises what it reads), so calls that overlap on one
 * device -- two streams, or two host threads -- race and must be serialised
 * by the caller.
 *   MOE_ERR_WORKSPACE if moe_workspace_bytes(p, MOE_STAGE_LAYER) - 256 exceeds
 *   MOE_STATIC_SCRATCH_BYTES (decode-sized batches fit: the DeepSeek-V3-shaped
 *   shard with 64 tokens needs about 10 MB); other errors as moe_layer.     */
#define MOE_STATIC_SCRATCH_BYTES (64u << 20)
moe_status moe_layer_static(const moe_problem* p, const float* logits, const void* x,
                            const moe_weights* w, void* y, void* stream);

/* Block-FP8 quantisation (page "OverlapAdvisor ...", section 4.4: BF16
 * checkpoints are quantised to block-FP8 at load time; the same rule makes
 * the per-token activation scales).  For each block_rows x 128 block of the
 * [rows, cols] bf16 matrix `src`: scale = amax / 448 in fp32 (1 if the block
 * is all zero), code = round-to-nearest-even(v / scale) (fp32 division),
 * saturated to +-448, as OCP E4M3FN bytes.
 *   block_rows: 1 (activations) or 128 (weights); cols % 128 == 0
 *   codes [rows, cols] uint8, scales [ceil(rows/block_rows), cols/128] fp32
 * A batch of `batch` equally shaped matrices (e.g. all experts' W13) is
 * processed at once: src, codes and scales advance by one matrix each.     */
moe_status moe_quantize_fp8(const void* src, int64_t batch, int64_t rows,
                            int64_t cols, int32_t block_rows, void* codes,
                            float* scales, void* stream);

/* MX conversion (OCP MX): for each block of 32 consecutive elements of a
 * row of the [batch * rows, cols] bf16 matrix src, the E8M0 scale
 * 2^(c - 127) with c = floor(log2 amax) - emax + 127, clamped to [0, 254]
 * (an all-zero block takes 0; emax = 2 for E2M1, 8 for E4M3), and the
 * elements round-to-nearest-even(v / 2^(c - 127)) saturated to the largest
 * normal (6 or 448).  Page "CascadeEP ...", section 4.1 (MXFP4 routed-expert
 * weights, converted at load time); the format is the OCP MX one.
 *   elem MOE_MX_E2M1: codes [.., cols/2] (two per byte, low nibble first)
 *   elem MOE_MX_E4M3: codes [.., cols] (cols % 128 == 0)
 *   scales [.., cols/32] uint8.  cols % 32 == 0, cols <= 2^20.              */
moe_status moe_quantize_mx(const void* src, int64_t batch, int64_t rows,
                           int64_t cols, int32_t elem, void* codes,
                           void* scales, void* stream);

/* Panel packing of bf16 matrices (see MOE_LAYOUT_PANEL_WEIGHTS): for each of
 * `batch` matrices src [rows, cols] (row major), dst receives the same values
 * in panel layout, [cols / 32, rows, 32].  cols % 32 == 0, 0 < cols <= 2^20,
 * batch * rows * cols < 2^40; src and dst must not overlap.  Meant for load
 * time, like moe_quantize_fp8: the weights are packed once.               */
moe_status moe_pack_panel(const void* src, int64_t batch, int64_t rows,
                          int64_t cols, void* dst, void* stream);

/* Panel packing of MXFP4 weights (see MOE_LAYOUT_PANEL_WEIGHTS): for each of
 * `batch` matrices of `rows` rows and K = cols elements, as moe_quantize_mx
 * writes them -- codes [rows, cols/2] bytes, scales [rows, cols/32] E8M0
 * bytes -- codes_dst receives the codes as [cols/128, rows, 64 bytes] and
 * scales_dst the scales as [cols/128, rows, 4 bytes].  cols % 128 == 0,
 * 128 <= cols <= 2^20, batch * rows * cols < 2^40; no two of the four
 * buffers may overlap; all 16-byte aligned.  Load time, like
 * moe_quantize_mx.  MOE_OK, or MOE_ERR_INVALID_ARG (nothing launched).     */
moe_status moe_pack_panel_mx(const void* codes, const void* scales, int64_t batch,
                             int64_t rows, int64_t cols, void* codes_dst,
                             void* scales_dst, void* stream);

/* Streaming FFN, host side (page "CascadeEP ...", section 3.2 "Launch
 * threshold" and Appendix C: ready work accumulates, an invocation is launched
 * once it reaches the threshold, and after the last arrival the rest is
 * flushed; independent invocations run on separate streams).
 *
 * moe_stream_threshold: theta = the smallest profiled expert-token count
 * whose measured FFN throughput reaches rho times the highest throughput
 * observed.  counts [n], throughput [n] are host arrays (the profile, any
 * order), n >= 1, 0 <= rho <= 1, throughputs finite and >= 0.  Returns theta,
 * or -1 for invalid arguments.  No GPU work.                              */
int64_t moe_stream_threshold(const int64_t* counts, const double* throughput,
                             int32_t n, double rho);

/* moe_stream_plan: threshold batching of n arrivals.  ready_rows[i] (host,
 * >= 0) is the number of routed rows that become ready with arrival i; rows
 * accumulate until the ready, unlaunched count reaches theta (>= theta
 * launches), and after the last arrival the remainder is launched whatever
 * its size.  Writes the exclusive end arrival of each invocation to
 * group_end [n] (host) and their number to *n_groups.  theta = 0 launches
 * every arrival on its own; a theta above the total gives one invocation.
 * MOE_ERR_INVALID_ARG for negative counts or theta.  No GPU work.          */
moe_status moe_stream_plan(const int64_t* ready_rows, int32_t n, int64_t theta,
                           int32_t* group_end, int32_t* n_groups);

/* Workspace of moe_layer_streamed for groups of at most max_group_tokens
 * tokens on n_streams streams (1 <= n_streams <= 64); 0 if invalid.        */
size_t moe_workspace_bytes_streamed(const moe_problem* p, int32_t max_group_tokens,
                                    int32_t n_streams);

/* Streamed layer: the tokens are in arrival order (the destination's receive
 * order), and invocation j is moe_layer on tokens [group_tokens[j],
 * group_tokens[j+1]) -- its own route, dispatch, grouped FFN, shared expert
 * and combine, writing rows [group_tokens[j], group_tokens[j+1]) of y -- on
 * streams[j % n_streams] with that stream's own workspace slice.  The output
 * equals moe_layer over all T tokens (each token's result depends on its own
 * row only).
 *   group_tokens [n_groups + 1] host int32: 0 = g_0 <= g_1 <= ... = T
 *   streams [n_streams] hipStream_t handles (NULL entries = default stream)
 *   ws: moe_workspace_bytes_streamed(p, max group length, n_streams) bytes
 * Ordering is the caller's: the inputs must be ready on every stream before
 * the call (e.g. each stream waits on the producer's event), and consumers of
 * y wait on all streams.  All streams at the default priority.             */
moe_status moe_layer_streamed(const moe_problem* p, const float* logits,
                              const void* x, const moe_weights* w, void* y,
                              const int32_t* group_tokens, int32_t n_groups,
                              void* const* streams, int32_t n_streams,
                              void* ws, size_t ws_bytes);

#define MOE_STAGE_LAYER 0
#define MOE_STAGE_DISPATCH 1
#define MOE_STAGE_FFN 2

/* Bytes of workspace a stage needs for problem p (0 if p is invalid). */
size_t moe_workspace_bytes(const moe_problem* p, int32_t stage);

/* Flags of the last grouped FFN run on a workspace (bits, 0 = none).
 *   MOE_FLAG_WAIT_TIMEOUT: in the one-launch decode FFN (the masked-layout
 *   and few-rows-per-expert path, where a down tile waits for the up tiles of
 *   its rows: page "OverlapAdvisor ...", Table 7, fused
 *   GroupGEMM + Act + GroupGEMM), a down tile's bounded wait gave up and the
 *   tile was skipped: y_perm (and so y) of that call is incomplete.  The
 *   ordering of the launch makes every wait end, so this flag reports a
 *   broken assumption (for instance a scheduler that runs a later block
 *   while an earlier one never starts); a test forces it by setting the
 *   environment variable MOE_TEST_FUSED_WAIT_UNREACHABLE=1 before the call.
 * Every moe_grouped_ffn / moe_grouped_ffn_gather / moe_layer call clears its
 * workspace's flags when its FFN starts, so the flags describe the most
 * recent call on that workspace (moe_layer: its routed and shared FFNs).
 * moe_workspace_flags enqueues on `stream` a one-thread kernel that writes
 * the flags of workspace ws (as used with problem p by the calls of `stage`,
 * MOE_STAGE_LAYER or MOE_STAGE_FFN) to *flags (a device int32, 16-byte
 * aligned); read it after the stream has reached that point.  It reports
 * nothing about moe_layer_streamed's per-stream slices.
 * MOE_OK, or MOE_ERR_INVALID_ARG / MOE_ERR_WORKSPACE (nothing enqueued).   */
#define MOE_FLAG_WAIT_TIMEOUT 1
moe_status moe_workspace_flags(const moe_problem* p, int32_t stage, const void* ws,
                               size_t ws_bytes, int32_t* flags, void* stream);

/* Static, human-readable name of a status code. */
const char* moe_status_str(moe_status s);

/* MOE_ABI_VERSION of the built library. */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_LAYER_H */
