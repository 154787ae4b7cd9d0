// Host-side launchers of the gfx950 kernels; called by the C ABI layer after
// it has validated every argument.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kRouteChunk = 128;  // tokens per workgroup in the routing kernels

size_t route_workspace_bytes(int64_t T, int E);

hipError_t launch_router_logits(const void* x, const void* w, int64_t T, int64_t d, int E, int dtype,
                                float* logits, hipStream_t s);

// fused S0-S3 (bf16): the router product with top-K routing, histogram and positions
size_t router_route_workspace_bytes(int64_t T, int E);
hipError_t launch_router_route(const void* x, const void* w, const float* bias, int64_t T, int64_t d, int E, int K,
                               int score, int renorm, float* logits, int32_t* topk_idx, float* topk_gate,
                               int32_t* counts, int32_t* offsets, int32_t* slot_pos, int32_t* row_src, void* ws,
                               hipStream_t s);

// moe_router_route with the histograms in the library's static device array (no workspace)
hipError_t launch_router_route_noalloc(const void* x, const void* w, const float* bias, int64_t T, int64_t d, int E,
                                       int K, int score, int renorm, float* logits, int32_t* topk_idx,
                                       float* topk_gate, int32_t* counts, int32_t* offsets, int32_t* slot_pos,
                                       int32_t* row_src, hipStream_t s);

hipError_t launch_route(const float* logits, const float* bias, int64_t T, int E, int K, int score,
                        int renorm, int32_t* topk_idx, float* topk_gate, int32_t* counts,
                        int32_t* offsets, int32_t* slot_pos, int32_t* row_src, void* ws,
                        hipStream_t s);

// the histogram scan and slot positions of routing, over nch chunks of `chunk` tokens whose
// per-chunk expert counts are in hist [nch][E] and in-chunk ranks in slot_pos
hipError_t launch_route_scan_finalize(int32_t* hist, int nch, int chunk, int64_t T, int E, int K,
                                      const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                                      int32_t* slot_pos, int32_t* row_src, hipStream_t s);

hipError_t launch_permute(const void* x, int64_t T, int64_t d, int K, int dtype, const int32_t* slot_pos,
                          const float* row_scale, const void* y_perm_dot, float* dgate_out,
                          void* x_perm, hipStream_t s);

hipError_t launch_combine(const void* y_perm, const int32_t* slot_pos, const float* gates, int64_t T,
                          int64_t d, int K, int dtype, void* y, hipStream_t s);

// bytes of the grouped GEMM workspace on the current device (0 if the device cannot be queried)
size_t grouped_gemm_workspace_bytes();

hipError_t launch_grouped_gemm(const void* A, const void* B, int b_layout, const int32_t* offs,
                               int64_t M, int64_t N, int64_t Kd, int G, int dtype, int epilogue,
                               const void* epi_in, void* epi_save, void* C, void* ws, size_t ws_bytes,
                               hipStream_t s);
// The gate/up GEMM with the permute folded into its A loads: row m of A is row
// a_rows[m] / a_div of X [T, Kd] (bf16, N-by-K weights, plain or SwiGLU epilogue).  It runs
// on the ring kernel only: whole 128-byte K stages of a row, and the per-lane DMA offsets of
// token rows and of weight rows within 32 bits.
constexpr int64_t kGatherStageBytes = 128;
inline bool grouped_gemm_gather_supported(int64_t T, int64_t N, int64_t Kd, int dtype, int epilogue) {
  const int64_t kbytes = Kd * 2;
  return dtype == 1 && (epilogue == 0 || epilogue == 1) && kbytes % kGatherStageBytes == 0 &&
         (N + 256) * kbytes < ((int64_t)1 << 32) && T * kbytes < ((int64_t)1 << 32);
}
hipError_t launch_grouped_gemm_gather(const void* X, int64_t T, const int32_t* a_rows, int a_div, const void* B,
                                      const int32_t* offs, int64_t M, int64_t N, int64_t Kd, int G, int epilogue,
                                      void* epi_save, void* C, void* ws, size_t ws_bytes, hipStream_t s);

hipError_t launch_grouped_wgrad(const void* X, const void* dY, const int32_t* offs, int64_t M,
                                int64_t N, int64_t Kd, int G, int dtype, int accumulate, float* dW,
                                hipStream_t s);

hipError_t launch_route_backward(const float* logits, const float* bias, const int32_t* idx,
                                 const float* d_gates, int64_t T, int E, int K, int score, int renorm,
                                 float* d_logits, hipStream_t s);

// bytes of the moe_router_logits_backward workspace (0 for fp32 inputs)
size_t router_backward_workspace_bytes(int64_t T, int64_t d, int E, int dtype);

hipError_t launch_router_logits_backward(const float* d_logits, const void* x, const void* w, int64_t T,
                                         int64_t d, int E, int dtype, float* d_w, void* dx, int accumulate,
                                         void* ws, hipStream_t s);

// row copy of the permute over rows of row_bytes bytes (a multiple of 16): MXFP8 codes and scales
hipError_t launch_permute_rows(const void* x, int64_t T, int64_t row_bytes, int K, const int32_t* slot_pos,
                               void* x_perm, hipStream_t s);

// MXFP8: block quantisation (bf16 rows, 32-value blocks) and the grouped GEMM on MX operands
hipError_t launch_mx_quantize(const void* x, int64_t R, int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_grouped_gemm_mx(const uint8_t* A, const uint8_t* SA, const uint8_t* B, const uint8_t* SB,
                                  const int32_t* offs, int64_t M, int64_t N, int64_t Kd, int G, int epilogue,
                                  void* C, uint8_t* CS, void* ws, size_t ws_bytes, hipStream_t s);

}  // namespace moe
