/*
 * moe.h - C ABI of the dropless mixture-of-experts (MoE) layer hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow the page "Accelerating dropless MoE training in JAX
 * with NVIDIA Transformer Engine" (cited as TE-MoE):
 *   - a learned router picks the Top-K experts of every token (introduction;
 *     "Optimisation 2": fused router kernels assign tokens to experts);
 *   - tokens are dispatched into expert-contiguous groups of variable length,
 *     two grouped GEMMs run over those groups, and combine restores the
 *     original token order (Figure 3 paragraph of "What specialised
 *     optimisations does dropless MoE need?");
 *   - no token is dropped and nothing is padded ("How is dropless MoE
 *     different from capacity-based MoE?");
 *   - group sizes stay on the device, so no device-to-host copy sits on the
 *     critical path and the whole layer can be captured in a graph
 *     ("What specialised optimisations..." and "Optimisation 1: Grouped GEMM").
 *
 * Notation: T tokens, d model width, E experts, K experts per token, F expert
 * FFN width, M = T*K routed slots; slot s = t*K + k.
 *
 * Conventions shared by every entry point
 *   - Pointers marked DEVICE are device memory (hipMalloc / torch CUDA
 *     tensors) owned by the caller; all tensors are dense row-major
 *     (C-contiguous) and 16-byte aligned.  The library never allocates,
 *     frees, synchronises, copies to the host or prints.
 *   - Every call only enqueues kernels on `stream` (a hipStream_t; NULL is
 *     the default stream) and returns; calls are capturable in a hipGraph.
 *   - Return value: MOE_OK, or MOE_INVALID_ARG / MOE_UNSUPPORTED (and, for the
 *     allocation-free entry point, MOE_SCRATCH_LIMIT) for arguments rejected
 *     on the host before anything is launched, or MOE_HIP_ERROR when a launch
 *     fails.  Values that live on the device
 *     (logits, offsets) are not checked: NaN logits and group offsets that are
 *     not monotone with offsets[G] == M are the caller's error and give
 *     undefined results (never an out-of-bounds access for offsets within
 *     [0, M]).
 *   - dtype: MOE_F32 or MOE_BF16.  bf16 tensors are stored as 16-bit bf16;
 *     arithmetic accumulates in fp32 and rounds results to bf16 to nearest
 *     even.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void* moe_stream_t; /* a hipStream_t */

enum moe_status { MOE_OK = 0, MOE_INVALID_ARG = 1, MOE_UNSUPPORTED = 2, MOE_HIP_ERROR = 3, MOE_SCRATCH_LIMIT = 4 };
enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };
enum moe_score { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 };
enum moe_layout { MOE_LAYOUT_NK = 0, MOE_LAYOUT_KN = 1 };
enum moe_epilogue { MOE_EPI_NONE = 0, MOE_EPI_SWIGLU = 1, MOE_EPI_DSWIGLU = 2, MOE_EPI_SWIGLU_MX = 3 };

#define MOE_ABI_VERSION 10
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 32
#define MOE_MAX_GROUPS 1024

/* Version of this ABI (MOE_ABI_VERSION). */
int32_t moe_abi_version(void);

/* Static string naming a status code; never NULL. */
const char* moe_status_str(int32_t status);

/*
 * Bytes of device workspace moe_route needs for T tokens and E experts.
 * Writes the size to *bytes.  MOE_INVALID_ARG if bytes is NULL, T < 0 or E is
 * outside [1, MOE_MAX_EXPERTS].
 */
int32_t moe_route_workspace_size(int64_t T, int32_t E, size_t* bytes);

/*
 * Router logits (S0; TE-MoE introduction: the learned router scores experts).
 *   logits[t, e] = sum_j x[t, j] * w_router[e, j], fp32 accumulation.
 *   x         DEVICE [T, d]  dtype
 *   w_router  DEVICE [E, d]  dtype (row e scores expert e)
 *   logits    DEVICE [T, E]  fp32 (written)
 * Requires T >= 0, d >= 8 and d % 8 == 0, 1 <= E <= MOE_MAX_EXPERTS.
 */
int32_t moe_router_logits(const void* x, const void* w_router, int64_t T, int64_t d, int32_t E,
                          int32_t dtype, float* logits, moe_stream_t stream);

/*
 * Top-K routing, expert histogram, prefix sum and stable slot positions
 * (S1-S3; TE-MoE introduction and "What are the challenges in MoE training?":
 * every expert gets a data-dependent number of tokens).
 *   key[t, e] = fp32(logits[t, e] + bias[e])   (key = logit when bias is NULL)
 *   topk_idx[t, :]  the K experts with the largest keys, by descending key;
 *                   ties go to the lower expert index; keys compare in the
 *                   total order of fp32 bit patterns (-0.0 < +0.0)
 *   score = SOFTMAX: s_e = softmax over all E keys;  SIGMOID: s_e = 1/(1+exp(-key))
 *   topk_gate[t, k] = s_idx / sum_k' s_idx'  (renorm != 0)  or  s_idx  (renorm == 0)
 *   counts[e]   = number of slots routed to e;  offsets = exclusive scan, offsets[E] = M
 *   slot_pos[s] = row of slot s in expert-contiguous order, rows of an expert
 *                 ordered by ascending slot; row_src[slot_pos[s]] = s
 *   logits   DEVICE [T, E] fp32;   bias DEVICE [E] fp32 or NULL (-inf masks an expert)
 *   topk_idx DEVICE [T, K] int32;  topk_gate DEVICE [T, K] fp32
 *   counts   DEVICE [E] int32;     offsets DEVICE [E+1] int32
 *   slot_pos, row_src DEVICE [T*K] int32
 *   ws       DEVICE scratch of at least moe_route_workspace_size(T, E) bytes
 * Requires 1 <= K <= E <= MOE_MAX_EXPERTS, K <= MOE_MAX_TOPK, T*K < 2^31.
 * Keys must not be NaN and each token needs a finite key among its K chosen.
 */
int32_t moe_route(const float* logits, const float* bias, int64_t T, int32_t E, int32_t K,
                  int32_t score, int32_t renorm, int32_t* topk_idx, float* topk_gate,
                  int32_t* counts, int32_t* offsets, int32_t* slot_pos, int32_t* row_src,
                  void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * Bytes of device workspace moe_router_route needs for T tokens and E experts.
 * MOE_INVALID_ARG if bytes is NULL, T < 0 or E is outside [1, MOE_MAX_EXPERTS].
 */
int32_t moe_router_route_workspace_size(int64_t T, int32_t E, size_t* bytes);

/*
 * Fused router (S0-S3 in three launches; TE-MoE "Optimisation 2": fused router
 * kernels assign tokens to experts): the router product of moe_router_logits,
 * then the routing of moe_route on those logits, with identical results (the
 * same products in the same order, the same keys, choices, gates, counts,
 * offsets and positions).  Each workgroup keeps its tile of logits on chip and
 * routes its own tokens; the histogram scan and the positions follow.
 *   x DEVICE [T, d] bf16;  w_router DEVICE [E, d] bf16;  bias DEVICE [E] fp32 or NULL
 *   logits   DEVICE [T, E] fp32, written when not NULL (the router backward reads them)
 *   topk_idx, topk_gate, counts, offsets, slot_pos, row_src: as moe_route
 *   ws       DEVICE scratch of at least moe_router_route_workspace_size(T, E) bytes
 * Requires dtype == MOE_BF16 (MOE_UNSUPPORTED otherwise: fp32 takes moe_router_logits and
 * moe_route), d >= 8, d % 8 == 0, 1 <= K <= E <= MOE_MAX_EXPERTS, K <= MOE_MAX_TOPK,
 * T*K < 2^31.
 */
int32_t moe_router_route(const void* x, const void* w_router, const float* bias, int64_t T, int64_t d, int32_t E,
                         int32_t K, int32_t dtype, int32_t score, int32_t renorm, float* logits, int32_t* topk_idx,
                         float* topk_gate, int32_t* counts, int32_t* offsets, int32_t* slot_pos, int32_t* row_src,
                         void* ws, size_t ws_bytes, moe_stream_t stream);

/*
 * moe_router_route for callers that cannot allocate device memory: code under
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * kernels and results as moe_router_route, with its workspace (the per-chunk
 * expert histograms) taken from a static device array of
 * MOE_ROUTER_ROUTE_NOALLOC_MAX_BYTES bytes that the library holds on every
 * device it runs on until the process ends.  The caller passes every input and
 * output as for moe_router_route (no ws, ws_bytes).
 *   - The call allocates nothing: no hipMalloc, hipFree or allocating library
 *     routine.  Its first call on a device looks up that device's copy of the
 *     array once (hipGetSymbolAddress) with the device current.
 *   - MOE_SCRATCH_LIMIT (checked on the host, nothing launched) when
 *     moe_router_route_workspace_size(T, E) exceeds MOE_ROUTER_ROUTE_NOALLOC_MAX_BYTES
 *     (for example T > 131072 tokens at E = 256, T > 4194304 at E = 8).
 *   - Every call on a device shares that device's array and leaves its last
 *     contents there; the kernels overwrite every entry they read, so nothing
 *     needs clearing.  Calls that overlap in time on one device (two streams,
 *     two host threads) race on the array and give undefined results: order them
 *     on one stream, or use moe_router_route with separate workspaces.
 * Other arguments, requirements and errors as moe_router_route.
 */
#define MOE_ROUTER_ROUTE_NOALLOC_MAX_BYTES ((size_t)4 << 20)
int32_t moe_router_route_noalloc(const void* x, const void* w_router, const float* bias, int64_t T, int64_t d,
                                 int32_t E, int32_t K, int32_t dtype, int32_t score, int32_t renorm, float* logits,
                                 int32_t* topk_idx, float* topk_gate, int32_t* counts, int32_t* offsets,
                                 int32_t* slot_pos, int32_t* row_src, moe_stream_t stream);

/*
 * Permute / dispatch into expert-contiguous order (S4; TE-MoE Figure 3
 * paragraph), and the combine backward (B1) when the optional arguments are
 * given.  For every slot s = t*K + k of token t, with r = slot_pos[s]:
 *   x_perm[r] = x[t]                                (row_scale == NULL: a bit copy)
 *   x_perm[r] = round(row_scale[s] * x[t])          (row_scale != NULL)
 *   dgate_out[s] = sum_j x[t, j] * y_perm_dot[r, j]  (when y_perm_dot and dgate_out are given)
 * Each token row is read once and written to its K rows.
 *   x          DEVICE [T, d] dtype;   slot_pos DEVICE [T*K] int32 (a permutation of [0, T*K))
 *   row_scale  DEVICE [T*K] fp32 or NULL
 *   y_perm_dot DEVICE [T*K, d] dtype or NULL;  dgate_out DEVICE [T*K] fp32 or NULL (both or neither)
 *   x_perm     DEVICE [T*K, d] dtype (written)
 * Requires d % 8 == 0, 1 <= K <= MOE_MAX_TOPK.
 */
int32_t moe_permute(const void* x, int64_t T, int64_t d, int32_t K, int32_t dtype,
                    const int32_t* slot_pos, const float* row_scale, const void* y_perm_dot,
                    float* dgate_out, void* x_perm, moe_stream_t stream);

/*
 * Grouped GEMM over variable-length row groups in one launch (S5/S6 and
 * backward B2/B4; TE-MoE "Optimisation 1: Grouped GEMM": one kernel call for
 * all experts, each at its actual token count, computing only valid rows).
 * Group g owns rows [group_offsets[g], group_offsets[g+1]) of A and C.
 *   layout NK: B [G, N, Kd],  P = A_g . B_g^T      layout KN: B [G, Kd, N],  P = A_g . B_g
 *   epilogue NONE:    C [M, N]   = P
 *   epilogue SWIGLU:  N = 2F is the width of P = [gate | up];
 *                     C [M, F]   = silu(P[:, :F]) * P[:, F:]
 *                     epi_save [M, 2F] = P (dtype) when not NULL (kept for backward)
 *   epilogue DSWIGLU: P = dH [M, N] with N = F; epi_in = saved pre-activations
 *                     [M, 2F] (G | U);  C [M, 2F] = [dH*U*silu'(G) | dH*silu(G)]
 *   A DEVICE [M, Kd] dtype;  group_offsets DEVICE [G+1] int32 (read on the device only)
 *   workspace DEVICE, NULL or workspace_bytes (moe_grouped_gemm_workspace_size) bytes,
 *     16-byte aligned, caller-owned: lets the last, partly filled round of output tiles be
 *     split along Kd across otherwise idle CUs (fp32 partial tiles summed in a fixed order,
 *     so results are deterministic).  Its first 4096 bytes must be zero before the first
 *     call; every call leaves them zero.  Calls that overlap in time need separate
 *     workspaces.  With NULL no tile is split (results differ only in the fp32 summation
 *     order of those tiles).
 * Requires 0 <= M < 2^31, N >= 8, N % 8 == 0 (SWIGLU: N % 16 == 0 and layout NK),
 * Kd >= 8, Kd % 8 == 0, 1 <= G <= MOE_MAX_GROUPS; epi_in is required for DSWIGLU.
 * Rows of C outside every group are not written.
 */
int32_t moe_grouped_gemm(const void* A, const void* B, int32_t b_layout,
                         const int32_t* group_offsets, int64_t M, int64_t N, int64_t Kd, int32_t G,
                         int32_t dtype, int32_t epilogue, const void* epi_in, void* epi_save,
                         void* C, void* workspace, size_t workspace_bytes, moe_stream_t stream);

/*
 * Bytes of the moe_grouped_gemm workspace for the current device (a 4096-byte counter
 * block, then one fp32 256 x 256 partial tile per compute unit).  Returns
 * MOE_HIP_ERROR when the device cannot be queried.
 */
int32_t moe_grouped_gemm_workspace_size(size_t* bytes);

/*
 * The gate/up grouped GEMM (S5) with the permute (S4) folded into its operand loads:
 * the same product as moe_permute followed by moe_grouped_gemm with layout NK, without
 * writing x_perm (TE-MoE "Optimisation 2": dispatch fused into the expert path rather than
 * run as a separate step whose rows go out to memory and come back; the permutation is a
 * pure row move, so the GEMM fetches each expert's rows from the token matrix itself).
 *   row r of A is x[row_src[r] / K], r in [0, T*K);  M = T*K
 *   x DEVICE [T, Kd] dtype;  row_src DEVICE [T*K] int32 (as moe_route writes it: slot
 *     s = t*K + k sits at row slot_pos[s], and row_src[slot_pos[s]] = s); an entry
 *     outside [0, T*K) reads x[T-1]
 *   B, group_offsets, epilogue, epi_save, C, workspace: as moe_grouped_gemm (layout NK,
 *     epilogue NONE or SWIGLU)
 * Results are bit-identical to moe_permute + moe_grouped_gemm on the same workspace.
 * Requires dtype MOE_BF16, Kd % 64 == 0, (N + 256) * Kd * 2 < 2^32 and T * Kd * 2 < 2^32
 * (MOE_UNSUPPORTED otherwise: use moe_permute + moe_grouped_gemm), 0 <= T*K < 2^31,
 * 1 <= K <= MOE_MAX_TOPK, N % 8 == 0 (SWIGLU: N % 16 == 0), 1 <= G <= MOE_MAX_GROUPS.
 */
int32_t moe_grouped_gemm_gather(const void* x, const int32_t* row_src, int64_t T, int32_t K, const void* B,
                                const int32_t* group_offsets, int64_t N, int64_t Kd, int32_t G, int32_t dtype,
                                int32_t epilogue, void* epi_save, void* C, void* workspace,
                                size_t workspace_bytes, moe_stream_t stream);

/*
 * Unpermute + gate-weighted combine back to token order (S7; TE-MoE Figure 3
 * paragraph: combine restores the original token order), and the permute
 * backward (B6) with gates == NULL.
 *   y[t] = round( sum_{k=0..K-1} g[t, k] * y_perm[slot_pos[t*K + k]] )
 *   accumulated in fp32 in ascending k; g = 1 when gates is NULL.
 *   y_perm DEVICE [T*K, d] dtype;  slot_pos DEVICE [T*K] int32;  gates DEVICE [T, K] fp32 or NULL
 *   y      DEVICE [T, d] dtype (written)
 * Requires d % 8 == 0, 1 <= K <= MOE_MAX_TOPK.
 */
int32_t moe_unpermute_combine(const void* y_perm, const int32_t* slot_pos, const float* gates,
                              int64_t T, int64_t d, int32_t K, int32_t dtype, void* y,
                              moe_stream_t stream);

/*
 * Per-group weight gradient with a ragged reduction length (backward B3/B5 of
 * the grouped GEMMs; the counterpart of "Optimisation 1" for training).
 *   dW[g] = dY_g^T . X_g  over the rows of group g, dW [G, N, Kd] fp32
 *   (the same [out, in] layout as the weights); groups without rows get 0
 *   (accumulate == 0) or are left unchanged (accumulate != 0: dW += ...).
 *   X DEVICE [M, Kd] dtype;  dY DEVICE [M, N] dtype;  group_offsets DEVICE [G+1] int32
 * Deterministic: no atomics, fixed summation order.
 * X and dY may be NULL when M == 0.
 * Requires 0 <= M < 2^31, N >= 8, N % 8 == 0, Kd >= 8, Kd % 8 == 0, 1 <= G <= MOE_MAX_GROUPS.
 */
int32_t moe_grouped_gemm_wgrad(const void* X, const void* dY, const int32_t* group_offsets,
                               int64_t M, int64_t N, int64_t Kd, int32_t G, int32_t dtype,
                               int32_t accumulate, float* dW, moe_stream_t stream);

/*
 * Router backward through the routing scores (the router is learned: TE-MoE
 * introduction).  The top-K choice is held fixed; with key = logit (+ bias),
 *   d_logits[t, e] = sum_k d_gates[t, k] * d topk_gate[t, k] / d key[t, e]
 * for the gates of moe_route (same score and renorm): back through
 * g_k = s_k / S (S = sum of the chosen scores) when renorm != 0, then through
 * the softmax over all E keys (every expert gets a gradient when renorm == 0)
 * or the sigmoid (only the chosen experts do).  Scores are recomputed from the
 * logits in fp32.  The bias is a constant: d bias is not formed (it would be
 * the column sum of d_logits).
 *   logits   DEVICE [T, E] fp32;  bias DEVICE [E] fp32 or NULL
 *   topk_idx DEVICE [T, K] int32 (as written by moe_route);  d_gates DEVICE [T, K] fp32
 *   d_logits DEVICE [T, E] fp32 (written, every element)
 * Requires 1 <= K <= E <= MOE_MAX_EXPERTS, K <= MOE_MAX_TOPK, T*K < 2^31.
 */
int32_t moe_route_backward(const float* logits, const float* bias, const int32_t* topk_idx,
                           const float* d_gates, int64_t T, int32_t E, int32_t K, int32_t score,
                           int32_t renorm, float* d_logits, moe_stream_t stream);

/*
 * Bytes of the moe_router_logits_backward workspace for these sizes (0 for fp32).
 * MOE_INVALID_ARG / MOE_UNSUPPORTED as moe_router_logits_backward would return.
 */
int32_t moe_router_backward_workspace_size(int64_t T, int64_t d, int32_t E, int32_t dtype, size_t* bytes);

/*
 * Backward of the router product logits = x . w_router^T (S0):
 *   d_w_router[e, :] = sum_t d_logits[t, e] * x[t, :]          (when d_w_router != NULL)
 *   dx[t, :] = sum_e d_logits[t, e] * w_router[e, :]            (dx != NULL, accumulate == 0)
 *   dx[t, :] = dx[t, :] + sum_e d_logits[t, e] * w_router[e, :] (accumulate != 0: adds the
 *              router's share to the expert path's dX, rounding once)
 * bf16: d_logits enters the MFMA products as two bf16 parts (high + low, about
 * 16 significant bits); accumulation is fp32.  d_w_router is summed over runs
 * of tokens in a fixed order: deterministic.
 *   d_logits   DEVICE [T, E] fp32;  x DEVICE [T, d] dtype;  w_router DEVICE [E, d] dtype
 *   d_w_router DEVICE [E, d] fp32 or NULL (T == 0 writes zeros);  dx DEVICE [T, d] dtype or NULL
 *   workspace  DEVICE, moe_router_backward_workspace_size bytes, 16-byte aligned, caller-owned;
 *              calls that overlap in time need separate workspaces
 * Requires 0 <= T < 2^31, d >= 8, d % 8 == 0, 1 <= E <= MOE_MAX_EXPERTS.  fp32 inputs
 * take plain per-element kernels meant for small shapes.
 */
int32_t moe_router_logits_backward(const float* d_logits, const void* x, const void* w_router, int64_t T,
                                   int64_t d, int32_t E, int32_t dtype, float* d_w_router, void* dx,
                                   int32_t accumulate, void* workspace, size_t workspace_bytes,
                                   moe_stream_t stream);

/*
 * MXFP8 block quantisation (TE-MoE "Optimisation 1": the grouped GEMM path with
 * MXFP8 block scaling from grouped quantisation).  The format is the OCP
 * Microscaling one: each 32 consecutive values of a row share an E8M0 scale
 * (code c = 2^(c - 127)), each value is an FP8 E4M3 code (bias 7, largest
 * finite 448, subnormals down to 2^-9).  For each block:
 *   shared = floor(log2(max |v|)) - 8 clamped to [-127, 127] (a block of zeros: -127)
 *   scales[r, b] = shared + 127;  codes[r, k] = E4M3(v / 2^shared), nearest even, saturated to +-448
 *   x      DEVICE [R, K] bf16 (rows along the reduction axis: activations or N-by-K weights)
 *   codes  DEVICE [R, K] uint8 (written);  scales DEVICE [R, K / 32] uint8 (written)
 * Requires R >= 0, K >= 32, K % 32 == 0, dtype == MOE_BF16.
 */
int32_t moe_mx_quantize(const void* x, int64_t R, int64_t K, int32_t dtype, uint8_t* codes, uint8_t* scales,
                        moe_stream_t stream);

/*
 * Grouped GEMM on MXFP8 operands (the MX counterpart of moe_grouped_gemm with
 * N-by-K weights): group g owns rows [group_offsets[g], group_offsets[g+1]);
 *   P = A_g . B_g^T on the values the codes and scales represent, fp32 accumulation
 *   epilogue NONE: C [M, N] = P;  SWIGLU: N = 2F, C [M, F] = silu(P[:, :F]) * P[:, F:];  bf16 out
 *   epilogue SWIGLU_MX: H = silu(P[:, :F]) * P[:, F:] rounded to bf16, written as MXFP8 (the
 *     operand of the down GEMM, TE-MoE "Optimisation 1": grouped quantisation): C [M, F]
 *     uint8 codes and C_scales [M, F / 32] uint8, byte for byte what moe_mx_quantize writes for
 *     the bf16 H of the SWIGLU epilogue; needs N % 64 == 0 and C_scales (NULL otherwise: unused)
 *   A DEVICE [M, Kd] codes, A_scales DEVICE [M, Kd / 32];  B DEVICE [G, N, Kd] codes,
 *   B_scales DEVICE [G, N, Kd / 32] (as written by moe_mx_quantize)
 *   workspace DEVICE, NULL or workspace_bytes (moe_grouped_gemm_workspace_size) bytes, 16-byte
 *     aligned, caller-owned, with the same contract as moe_grouped_gemm's: the last, partly
 *     filled round of output tiles is split along Kd across otherwise idle CUs (fp32 partials
 *     summed in a fixed order); its first 4096 bytes must be zero before the first call and
 *     every call leaves them zero; calls that overlap in time need separate workspaces; with
 *     NULL no tile is split (results differ only in the fp32 summation order of those tiles).
 * Requires 0 <= M < 2^31, N >= 8, N % 8 == 0 (SWIGLU: N % 16 == 0), Kd % 128 == 0,
 * (N + 256) * Kd < 2^32, 1 <= G <= MOE_MAX_GROUPS.  Rows of C outside every group are not
 * written.
 */
int32_t moe_grouped_gemm_mx(const uint8_t* A, const uint8_t* A_scales, const uint8_t* B, const uint8_t* B_scales,
                            const int32_t* group_offsets, int64_t M, int64_t N, int64_t Kd, int32_t G,
                            int32_t epilogue, void* C, uint8_t* C_scales, void* workspace,
                            size_t workspace_bytes, moe_stream_t stream);

/*
 * Permute of MXFP8 rows (S4 on quantised tokens): codes_perm[slot_pos[s]] = codes[s / K] and
 * scales_perm[slot_pos[s]] = scales[s / K], bit copies.  Quantising the T tokens once
 * (moe_mx_quantize) and permuting the codes gives the same bytes as quantising the T*K
 * routed rows, with an eighth of the quantisation work at K = 8 and half the permute bytes.
 *   codes DEVICE [T, d] uint8, scales DEVICE [T, d / 32] uint8
 *   codes_perm DEVICE [T*K, d] uint8, scales_perm DEVICE [T*K, d / 32] uint8 (written)
 * Requires d % 512 == 0 (whole 16-byte rows of scales), 1 <= K <= MOE_MAX_TOPK, T*K < 2^31.
 */
int32_t moe_permute_mx(const uint8_t* codes, const uint8_t* scales, int64_t T, int64_t d, int32_t K,
                       const int32_t* slot_pos, uint8_t* codes_perm, uint8_t* scales_perm, moe_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
