// Router logits: logits[t, e] = x[t, :] . w_router[e, :] with fp32 accumulation.
//
// The learned router scores every expert for every token (page "Accelerating
// dropless MoE training in JAX with NVIDIA Transformer Engine", introduction).
// With E <= 256 this product is a skinny GEMM whose cost is reading x once, so
// it is shaped for HBM bandwidth: a workgroup owns 32 tokens, its 4 waves split
// the d axis, and each wave runs 32x32 MFMA tiles (one per 32 experts) fed
// straight from global memory with several 16-byte loads per lane in flight.
// The 4 partial tiles are summed through LDS.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

template <typename T> struct RMma;
template <> struct RMma<bf16_t> {
  __device__ __forceinline__ static void run(const uint4& a, const uint4& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct RMma<float> {
  __device__ __forceinline__ static void run(const uint4& a, const uint4& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

// NF = expert tiles of 32; U = K-steps whose loads are issued together.
template <typename T, int NF, int U>
__global__ __launch_bounds__(256) void router_logits_kernel(const char* __restrict__ x,
                                                            const char* __restrict__ w, int64_t T_,
                                                            int64_t d, int E, float* __restrict__ logits) {
  constexpr int VE = Elem<T>::kVec;
  constexpr int ES = Elem<T>::kBytes;
  constexpr int KC = 8 * VE;  // K elements per step: 2 half-waves x 4 vectors
  __shared__ float red[3][NF][16][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  const int64_t row = min(t0 + l32, T_ - 1);
  const char* xr = x + row * d * ES;
  const char* wr[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) wr[f] = w + (int64_t)min(f * 32 + l32, E - 1) * d * ES;

  f32x16 acc[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[f][r] = 0.f;

  const int64_t nkc = (d + KC - 1) / KC;
  const int64_t kc0 = nkc * wave / 4, kc1 = nkc * (wave + 1) / 4;
  for (int64_t kc = kc0; kc < kc1; kc += U) {
    uint4 a[U][4], b[U][NF][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t kb = (kc + u) * KC + hi * (KC / 2);
      const bool step_ok = kc + u < kc1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t k = kb + j * VE;
        const bool ok = step_ok && k < d;
        a[u][j] = ok ? *(const uint4*)(xr + k * ES) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int f = 0; f < NF; ++f)
          b[u][f][j] = ok ? *(const uint4*)(wr[f] + k * ES) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int f = 0; f < NF; ++f) RMma<T>::run(a[u][j], b[u][f][j], acc[f]);
  }

  if (wave > 0) {
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[wave - 1][f][r][lane] = acc[f][r];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int e = f * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = acc[f][r] + red[0][f][r][lane] + red[1][f][r][lane] + red[2][f][r][lane];
        const int64_t t = t0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (t < T_ && e < E) logits[t * E + e] = v;
      }
    }
  }
}

template <typename T>
hipError_t router_t(const void* x, const void* w, int64_t T_, int64_t d, int E, float* logits,
                    hipStream_t s) {
  const dim3 grid((unsigned)((T_ + 31) / 32));
  const int nf = (E + 31) / 32;
  const char* xc = (const char*)x;
  const char* wc = (const char*)w;
  switch (nf) {
    case 1: hipLaunchKernelGGL((router_logits_kernel<T, 1, 4>), grid, dim3(256), 0, s, xc, wc, T_, d, E, logits); break;
    case 2: hipLaunchKernelGGL((router_logits_kernel<T, 2, 2>), grid, dim3(256), 0, s, xc, wc, T_, d, E, logits); break;
    case 3: hipLaunchKernelGGL((router_logits_kernel<T, 3, 1>), grid, dim3(256), 0, s, xc, wc, T_, d, E, logits); break;
    case 4: hipLaunchKernelGGL((router_logits_kernel<T, 4, 1>), grid, dim3(256), 0, s, xc, wc, T_, d, E, logits); break;
    case 5: case 6: hipLaunchKernelGGL((router_logits_kernel<T, 6, 1>), grid, dim3(256), 0, s, xc, wc, T_, d, E, logits); break;
    default: hipLaunchKernelGGL((router_logits_kernel<T, 8, 1>), grid, dim3(256), 0, s, xc, wc, T_, d, E, logits); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_router_logits(const void* x, const void* w, int64_t T, int64_t d, int E, int dtype,
                                float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 1) return router_t<bf16_t>(x, w, T, d, E, logits, s);
  return router_t<float>(x, w, T, d, E, logits, s);
}

}  // namespace moe
