// C ABI of the MoE library: host-side argument checks, then kernel launches on
// the caller's stream.  Nothing here allocates, synchronises or reads device
// memory; every rejection happens before the first HIP call.
#include <hip/hip_runtime.h>

#include "../../include/moe.h"
#include "internal.h"

namespace {

constexpr int64_t kMaxGroups = MOE_MAX_GROUPS;

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
inline bool dtype_ok(int32_t dt) { return dt == MOE_F32 || dt == MOE_BF16; }

inline int32_t from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_HIP_ERROR; }

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(int32_t status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_INVALID_ARG: return "invalid argument";
    case MOE_UNSUPPORTED: return "unsupported dtype/layout/epilogue combination";
    case MOE_HIP_ERROR: return "HIP launch error";
    case MOE_SCRATCH_LIMIT: return "input larger than the static scratch of an allocation-free entry point";
    default: return "unknown status";
  }
}

int32_t moe_route_workspace_size(int64_t T, int32_t E, size_t* bytes) {
  if (!bytes || T < 0 || E < 1 || E > MOE_MAX_EXPERTS) return MOE_INVALID_ARG;
  *bytes = moe::route_workspace_bytes(T, E);
  return MOE_OK;
}

int32_t moe_router_logits(const void* x, const void* w_router, int64_t T, int64_t d, int32_t E,
                          int32_t dtype, float* logits, moe_stream_t stream) {
  if (T < 0 || d < 8 || d % 8 != 0 || E < 1 || E > MOE_MAX_EXPERTS) return MOE_INVALID_ARG;
  if (!dtype_ok(dtype)) return MOE_UNSUPPORTED;
  if (T >= ((int64_t)1 << 36)) return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !w_router || !logits) return MOE_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_router) || !aligned4(logits)) return MOE_INVALID_ARG;
  return from_hip(moe::launch_router_logits(x, w_router, T, d, E, dtype, logits, (hipStream_t)stream));
}

int32_t moe_route(const float* logits, const float* bias, int64_t T, int32_t E, int32_t K,
                  int32_t score, int32_t renorm, int32_t* topk_idx, float* topk_gate,
                  int32_t* counts, int32_t* offsets, int32_t* slot_pos, int32_t* row_src,
                  void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || K < 1 || K > E || K > MOE_MAX_TOPK) return MOE_INVALID_ARG;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_UNSUPPORTED;
  if (T * (int64_t)K >= ((int64_t)1 << 31)) return MOE_INVALID_ARG;
  if (!counts || !offsets) return MOE_INVALID_ARG;
  if (T > 0 && (!logits || !topk_idx || !topk_gate || !slot_pos || !row_src)) return MOE_INVALID_ARG;
  const size_t need = moe::route_workspace_bytes(T, E);
  if (ws_bytes < need || (need > 0 && !ws)) return MOE_INVALID_ARG;
  return from_hip(moe::launch_route(logits, bias, T, E, K, score, renorm != 0, topk_idx, topk_gate,
                                    counts, offsets, slot_pos, row_src, ws, (hipStream_t)stream));
}

int32_t moe_permute(const void* x, int64_t T, int64_t d, int32_t K, int32_t dtype,
                    const int32_t* slot_pos, const float* row_scale, const void* y_perm_dot,
                    float* dgate_out, void* x_perm, moe_stream_t stream) {
  if (T < 0 || d < 8 || d % 8 != 0 || K < 1 || K > MOE_MAX_TOPK) return MOE_INVALID_ARG;
  if (!dtype_ok(dtype)) return MOE_UNSUPPORTED;
  if ((y_perm_dot == nullptr) != (dgate_out == nullptr)) return MOE_INVALID_ARG;
  if (T * (int64_t)K >= ((int64_t)1 << 31)) return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !slot_pos || !x_perm) return MOE_INVALID_ARG;
  if (!aligned16(x) || !aligned16(x_perm) || (y_perm_dot && !aligned16(y_perm_dot))) return MOE_INVALID_ARG;
  return from_hip(moe::launch_permute(x, T, d, K, dtype, slot_pos, row_scale, y_perm_dot, dgate_out,
                                      x_perm, (hipStream_t)stream));
}

int32_t moe_grouped_gemm_workspace_size(size_t* bytes) {
  if (!bytes) return MOE_INVALID_ARG;
  *bytes = moe::grouped_gemm_workspace_bytes();
  return *bytes ? MOE_OK : MOE_HIP_ERROR;
}

int32_t moe_grouped_gemm(const void* A, const void* B, int32_t b_layout,
                         const int32_t* group_offsets, int64_t M, int64_t N, int64_t Kd, int32_t G,
                         int32_t dtype, int32_t epilogue, const void* epi_in, void* epi_save,
                         void* C, void* workspace, size_t workspace_bytes, moe_stream_t stream) {
  if (M < 0 || M >= ((int64_t)1 << 31) || N < 8 || N % 8 != 0 || Kd < 8 || Kd % 8 != 0) return MOE_INVALID_ARG;
  if (G < 1 || G > kMaxGroups) return MOE_INVALID_ARG;
  if (!dtype_ok(dtype)) return MOE_UNSUPPORTED;
  if (b_layout != MOE_LAYOUT_NK && b_layout != MOE_LAYOUT_KN) return MOE_UNSUPPORTED;
  if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SWIGLU && epilogue != MOE_EPI_DSWIGLU)
    return MOE_UNSUPPORTED;
  if (epilogue == MOE_EPI_SWIGLU && (b_layout != MOE_LAYOUT_NK || N % 16 != 0)) return MOE_UNSUPPORTED;
  if (epilogue == MOE_EPI_DSWIGLU && !epi_in) return MOE_INVALID_ARG;
  if (!B || !group_offsets) return MOE_INVALID_ARG;
  if (M == 0) return MOE_OK;
  if (!A || !C) return MOE_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B) || !aligned4(group_offsets)) return MOE_INVALID_ARG;
  if ((epi_in && !aligned16(epi_in)) || (epi_save && !aligned16(epi_save)) || !aligned16(C))
    return MOE_INVALID_ARG;
  if (workspace && !aligned16(workspace)) return MOE_INVALID_ARG;
  return from_hip(moe::launch_grouped_gemm(A, B, b_layout, group_offsets, M, N, Kd, G, dtype, epilogue,
                                           epi_in, epilogue == MOE_EPI_SWIGLU ? epi_save : nullptr, C,
                                           workspace, workspace ? workspace_bytes : 0, (hipStream_t)stream));
}

int32_t moe_grouped_gemm_gather(const void* x, const int32_t* row_src, int64_t T, int32_t K, const void* B,
                                const int32_t* group_offsets, int64_t N, int64_t Kd, int32_t G, int32_t dtype,
                                int32_t epilogue, void* epi_save, void* C, void* workspace,
                                size_t workspace_bytes, moe_stream_t stream) {
  if (T < 0 || K < 1 || K > MOE_MAX_TOPK || T * (int64_t)K >= ((int64_t)1 << 31)) return MOE_INVALID_ARG;
  if (N < 8 || N % 8 != 0 || Kd < 8 || Kd % 8 != 0) return MOE_INVALID_ARG;
  if (G < 1 || G > kMaxGroups) return MOE_INVALID_ARG;
  if (!dtype_ok(dtype)) return MOE_UNSUPPORTED;
  if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SWIGLU) return MOE_UNSUPPORTED;
  if (epilogue == MOE_EPI_SWIGLU && N % 16 != 0) return MOE_UNSUPPORTED;
  if (!moe::grouped_gemm_gather_supported(T, N, Kd, dtype, epilogue)) return MOE_UNSUPPORTED;
  if (!B || !group_offsets) return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!x || !row_src || !C) return MOE_INVALID_ARG;
  if (!aligned16(x) || !aligned16(B) || !aligned4(row_src) || !aligned4(group_offsets) || !aligned16(C) ||
      (epi_save && !aligned16(epi_save)) || (workspace && !aligned16(workspace)))
    return MOE_INVALID_ARG;
  return from_hip(moe::launch_grouped_gemm_gather(x, T, row_src, K, B, group_offsets, T * (int64_t)K, N, Kd, G,
                                                  epilogue, epilogue == MOE_EPI_SWIGLU ? epi_save : nullptr, C,
                                                  workspace, workspace ? workspace_bytes : 0,
                                                  (hipStream_t)stream));
}

int32_t moe_unpermute_combine(const void* y_perm, const int32_t* slot_pos, const float* gates,
                              int64_t T, int64_t d, int32_t K, int32_t dtype, void* y,
                              moe_stream_t stream) {
  if (T < 0 || d < 8 || d % 8 != 0 || K < 1 || K > MOE_MAX_TOPK) return MOE_INVALID_ARG;
  if (!dtype_ok(dtype)) return MOE_UNSUPPORTED;
  if (T * (int64_t)K >= ((int64_t)1 << 31)) return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!y_perm || !slot_pos || !y) return MOE_INVALID_ARG;
  if (!aligned16(y_perm) || !aligned16(y)) return MOE_INVALID_ARG;
  return from_hip(moe::launch_combine(y_perm, slot_pos, gates, T, d, K, dtype, y, (hipStream_t)stream));
}

int32_t moe_grouped_gemm_wgrad(const void* X, const void* dY, const int32_t* group_offsets,
                               int64_t M, int64_t N, int64_t Kd, int32_t G, int32_t dtype,
                               int32_t accumulate, float* dW, moe_stream_t stream) {
  if (M < 0 || M >= ((int64_t)1 << 31) || N < 8 || N % 8 != 0 || Kd < 8 || Kd % 8 != 0) return MOE_INVALID_ARG;
  if (G < 1 || G > kMaxGroups) return MOE_INVALID_ARG;
  if (!dtype_ok(dtype)) return MOE_UNSUPPORTED;
  if (!group_offsets || !dW) return MOE_INVALID_ARG;
  if (M > 0 && (!X || !dY)) return MOE_INVALID_ARG;
  if ((X && !aligned16(X)) || (dY && !aligned16(dY)) || !aligned4(dW) || !aligned4(group_offsets))
    return MOE_INVALID_ARG;
  return from_hip(moe::launch_grouped_wgrad(X, dY, group_offsets, M, N, Kd, G, dtype, accumulate != 0, dW,
                                            (hipStream_t)stream));
}

int32_t moe_route_backward(const float* logits, const float* bias, const int32_t* topk_idx,
                           const float* d_gates, int64_t T, int32_t E, int32_t K, int32_t score,
                           int32_t renorm, float* d_logits, moe_stream_t stream) {
  if (T < 0 || E < 1 || E > MOE_MAX_EXPERTS || K < 1 || K > E || K > MOE_MAX_TOPK) return MOE_INVALID_ARG;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_UNSUPPORTED;
  if (T * (int64_t)K >= ((int64_t)1 << 31)) return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !d_gates || !d_logits) return MOE_INVALID_ARG;
  if (!aligned4(logits) || !aligned4(topk_idx) || !aligned4(d_gates) || !aligned4(d_logits) ||
      (bias && !aligned4(bias)))
    return MOE_INVALID_ARG;
  return from_hip(moe::launch_route_backward(logits, bias, topk_idx, d_gates, T, E, K, score, renorm != 0,
                                             d_logits, (hipStream_t)stream));
}

int32_t moe_router_backward_workspace_size(int64_t T, int64_t d, int32_t E, int32_t dtype, size_t* bytes) {
  if (!bytes || T < 0 || T >= ((int64_t)1 << 31) || d < 8 || d % 8 != 0 || E < 1 || E > MOE_MAX_EXPERTS)
    return MOE_INVALID_ARG;
  if (!dtype_ok(dtype)) return MOE_UNSUPPORTED;
  *bytes = moe::router_backward_workspace_bytes(T, d, E, dtype);
  return MOE_OK;
}

int32_t moe_router_logits_backward(const float* d_logits, const void* x, const void* w_router, int64_t T,
                                   int64_t d, int32_t E, int32_t dtype, float* d_w_router, void* dx,
                                   int32_t accumulate, void* workspace, size_t workspace_bytes,
                                   moe_stream_t stream) {
  if (T < 0 || T >= ((int64_t)1 << 31) || d < 8 || d % 8 != 0 || E < 1 || E > MOE_MAX_EXPERTS)
    return MOE_INVALID_ARG;
  if (!dtype_ok(dtype)) return MOE_UNSUPPORTED;
  if (!d_w_router && !dx) return MOE_OK;
  if (d_w_router && (!aligned16(d_w_router) || (T > 0 && (!d_logits || !x)))) return MOE_INVALID_ARG;
  if (dx && T > 0 && (!d_logits || !w_router || !aligned16(dx))) return MOE_INVALID_ARG;
  if ((x && !aligned16(x)) || (w_router && !aligned16(w_router)) || (d_logits && !aligned4(d_logits)))
    return MOE_INVALID_ARG;
  const size_t need = moe::router_backward_workspace_bytes(T, d, E, dtype);
  if (workspace_bytes < need || (need > 0 && (!workspace || !aligned16(workspace)))) return MOE_INVALID_ARG;
  return from_hip(moe::launch_router_logits_backward(d_logits, x, w_router, T, d, E, dtype, d_w_router, dx,
                                                     accumulate != 0, workspace, (hipStream_t)stream));
}

int32_t moe_router_route_workspace_size(int64_t T, int32_t E, size_t* bytes) {
  if (!bytes || T < 0 || E < 1 || E > MOE_MAX_EXPERTS) return MOE_INVALID_ARG;
  *bytes = moe::router_route_workspace_bytes(T, E);
  return MOE_OK;
}

int32_t moe_router_route(const void* x, const void* w_router, const float* bias, int64_t T, int64_t d, int32_t E,
                         int32_t K, int32_t dtype, int32_t score, int32_t renorm, float* logits, int32_t* topk_idx,
                         float* topk_gate, int32_t* counts, int32_t* offsets, int32_t* slot_pos, int32_t* row_src,
                         void* ws, size_t ws_bytes, moe_stream_t stream) {
  if (T < 0 || d < 8 || d % 8 != 0 || E < 1 || E > MOE_MAX_EXPERTS || K < 1 || K > E || K > MOE_MAX_TOPK)
    return MOE_INVALID_ARG;
  if (dtype != MOE_BF16) return MOE_UNSUPPORTED;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_UNSUPPORTED;
  if (T * (int64_t)K >= ((int64_t)1 << 31)) return MOE_INVALID_ARG;
  if (!counts || !offsets) return MOE_INVALID_ARG;
  if (T > 0 && (!x || !w_router || !topk_idx || !topk_gate || !slot_pos || !row_src)) return MOE_INVALID_ARG;
  if ((x && !aligned16(x)) || (w_router && !aligned16(w_router)) || (logits && !aligned4(logits)) ||
      (bias && !aligned4(bias)))
    return MOE_INVALID_ARG;
  const size_t need = moe::router_route_workspace_bytes(T, E);
  if (ws_bytes < need || (need > 0 && !ws)) return MOE_INVALID_ARG;
  return from_hip(moe::launch_router_route(x, w_router, bias, T, d, E, K, score, renorm != 0, logits, topk_idx,
                                           topk_gate, counts, offsets, slot_pos, row_src, ws, (hipStream_t)stream));
}

int32_t moe_router_route_noalloc(const void* x, const void* w_router, const float* bias, int64_t T, int64_t d,
                                 int32_t E, int32_t K, int32_t dtype, int32_t score, int32_t renorm, float* logits,
                                 int32_t* topk_idx, float* topk_gate, int32_t* counts, int32_t* offsets,
                                 int32_t* slot_pos, int32_t* row_src, moe_stream_t stream) {
  if (T < 0 || d < 8 || d % 8 != 0 || E < 1 || E > MOE_MAX_EXPERTS || K < 1 || K > E || K > MOE_MAX_TOPK)
    return MOE_INVALID_ARG;
  if (dtype != MOE_BF16) return MOE_UNSUPPORTED;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_UNSUPPORTED;
  if (T * (int64_t)K >= ((int64_t)1 << 31)) return MOE_INVALID_ARG;
  if (!counts || !offsets) return MOE_INVALID_ARG;
  if (T > 0 && (!x || !w_router || !topk_idx || !topk_gate || !slot_pos || !row_src)) return MOE_INVALID_ARG;
  if ((x && !aligned16(x)) || (w_router && !aligned16(w_router)) || (logits && !aligned4(logits)) ||
      (bias && !aligned4(bias)))
    return MOE_INVALID_ARG;
  if (moe::router_route_workspace_bytes(T, E) > MOE_ROUTER_ROUTE_NOALLOC_MAX_BYTES) return MOE_SCRATCH_LIMIT;
  return from_hip(moe::launch_router_route_noalloc(x, w_router, bias, T, d, E, K, score, renorm != 0, logits,
                                                   topk_idx, topk_gate, counts, offsets, slot_pos, row_src,
                                                   (hipStream_t)stream));
}

int32_t moe_mx_quantize(const void* x, int64_t R, int64_t K, int32_t dtype, uint8_t* codes, uint8_t* scales,
                        moe_stream_t stream) {
  if (R < 0 || K < 32 || K % 32 != 0) return MOE_INVALID_ARG;
  if (dtype != MOE_BF16) return MOE_UNSUPPORTED;
  if (R == 0) return MOE_OK;
  if (!x || !codes || !scales) return MOE_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes)) return MOE_INVALID_ARG;
  return from_hip(moe::launch_mx_quantize(x, R, K, codes, scales, (hipStream_t)stream));
}

int32_t moe_grouped_gemm_mx(const uint8_t* A, const uint8_t* A_scales, const uint8_t* B, const uint8_t* B_scales,
                            const int32_t* group_offsets, int64_t M, int64_t N, int64_t Kd, int32_t G,
                            int32_t epilogue, void* C, uint8_t* C_scales, void* workspace, size_t workspace_bytes,
                            moe_stream_t stream) {
  if (M < 0 || M >= ((int64_t)1 << 31) || N < 8 || N % 8 != 0 || Kd < 128 || Kd % 128 != 0) return MOE_INVALID_ARG;
  if (G < 1 || G > kMaxGroups) return MOE_INVALID_ARG;
  if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SWIGLU && epilogue != MOE_EPI_SWIGLU_MX) return MOE_UNSUPPORTED;
  if (epilogue == MOE_EPI_SWIGLU && N % 16 != 0) return MOE_INVALID_ARG;
  if (epilogue == MOE_EPI_SWIGLU_MX && N % 64 != 0) return MOE_INVALID_ARG;  // whole 32-value blocks of H
  if ((N + 256) * Kd >= ((int64_t)1 << 32)) return MOE_INVALID_ARG;
  if (!group_offsets) return MOE_INVALID_ARG;
  if (M == 0) return MOE_OK;
  if (!A || !A_scales || !B || !B_scales || !C) return MOE_INVALID_ARG;
  if (epilogue == MOE_EPI_SWIGLU_MX && !C_scales) return MOE_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B) || !aligned4(A_scales) || !aligned4(B_scales) || !aligned16(C) ||
      !aligned4(group_offsets) || (workspace && !aligned16(workspace)))
    return MOE_INVALID_ARG;
  return from_hip(moe::launch_grouped_gemm_mx(A, A_scales, B, B_scales, group_offsets, M, N, Kd, G, epilogue, C,
                                              epilogue == MOE_EPI_SWIGLU_MX ? C_scales : nullptr, workspace,
                                              workspace ? workspace_bytes : 0, (hipStream_t)stream));
}

int32_t moe_permute_mx(const uint8_t* codes, const uint8_t* scales, int64_t T, int64_t d, int32_t K,
                       const int32_t* slot_pos, uint8_t* codes_perm, uint8_t* scales_perm, moe_stream_t stream) {
  if (T < 0 || d < 512 || d % 512 != 0 || K < 1 || K > MOE_MAX_TOPK) return MOE_INVALID_ARG;
  if (T * (int64_t)K >= ((int64_t)1 << 31)) return MOE_INVALID_ARG;
  if (T == 0) return MOE_OK;
  if (!codes || !scales || !slot_pos || !codes_perm || !scales_perm) return MOE_INVALID_ARG;
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(codes_perm) || !aligned16(scales_perm))
    return MOE_INVALID_ARG;
  const hipError_t e = moe::launch_permute_rows(codes, T, d, K, slot_pos, codes_perm, (hipStream_t)stream);
  if (e != hipSuccess) return MOE_HIP_ERROR;
  return from_hip(moe::launch_permute_rows(scales, T, d / 32, K, slot_pos, scales_perm, (hipStream_t)stream));
}

}  // extern "C"
