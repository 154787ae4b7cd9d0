// MXFP8 block quantisation of the expert matmul operands (page "Accelerating
// dropless MoE training in JAX with NVIDIA Transformer Engine", "Optimisation
// 1": the grouped GEMM path with MXFP8 block scaling from grouped quantisation).
//
// The pages name the format only; its definition is the OCP Microscaling (MX)
// one: every 32 consecutive values of a row share a power-of-two scale stored
// as E8M0 (code c = 2^(c - 127)); the values are FP8 E4M3 (bias 7, largest
// finite 448, subnormals down to 2^-9).  Shared exponent = floor(log2(max |v|))
// - 8, clamped to [-127, 127]; a block of zeros takes code 0; each value is
// v / 2^shared rounded to nearest even and saturated to +-448.  The encoding
// is done in exact float steps (scaling by powers of two, rint), not by the
// hardware conversion, so that it is this rule bit for bit.
//
// One thread per block: 64 bytes of bf16 in, 32 code bytes and 1 scale byte out.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

// floor(log2(a)) of a finite a > 0 (normal or subnormal fp32)
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t u = __float_as_uint(a);
  const int e = (int)((u >> 23) & 0xff);
  if (e != 0) return e - 127;
  return -149 + (31 - __clz(u & 0x7fffffu));
}

// nearest E4M3 code of a finite q, ties to the even mantissa, saturating to +-448
__device__ __forceinline__ uint32_t e4m3_rne_sat(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  const float a = fabsf(q);
  if (a >= 448.f) return sign | 0x7Eu;
  if (a < 0.015625f) {                        // below 2^-6: the subnormal grid of 2^-9
    const float m = rintf(a * 512.f);         // 0 .. 8; 8 is the smallest normal, code 0x08
    return sign | (uint32_t)m;
  }
  int e = floor_log2(a);                      // -6 .. 8
  const float m = rintf((ldexpf(a, -e) - 1.f) * 8.f);  // exact steps; 0 .. 8
  uint32_t mi = (uint32_t)m;
  if (mi == 8u) {
    ++e;
    mi = 0u;
  }
  return sign | ((uint32_t)(e + 7) << 3) | mi;
}

__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t K,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t nb = K / 32;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= R * nb) return;
  const int64_t r = i / nb, b = i % nb;
  const uint4* src = (const uint4*)(x + r * K + b * 32);
  float v[32];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    float f[8];
    Elem<bf16_t>::to_f32(src[u], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[u * 8 + e] = f[e];
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) amax = fmaxf(amax, fabsf(v[e]));
  int shared = -127;
  if (amax > 0.f) shared = min(127, max(-127, floor_log2(amax) - 8));
  scales[r * nb + b] = (uint8_t)(shared + 127);
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) word |= e4m3_rne_sat(ldexpf(v[k * 4 + e], -shared)) << (8 * e);
    w[k] = word;
  }
  uint4* dst = (uint4*)(codes + r * K + b * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

}  // namespace

hipError_t launch_mx_quantize(const void* x, int64_t R, int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  const int64_t n = R * (K / 32);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (const uint16_t*)x, R,
                     K, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
