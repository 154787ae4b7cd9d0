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
// is done in exact steps (scaling by powers of two, integer rounding of the
// fp32 mantissa), not by the hardware conversion, so that it is this rule bit
// for bit.
//
// Four threads per block: 64 bytes of bf16 in, 32 code bytes and 1 scale byte out.
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

// nearest E4M3 code of a finite q, ties to the even mantissa, saturating to +-448 (|q| >= 448
// gives 0x7e).  For 2^-6 <= |q| < 448 the fp32 mantissa is rounded to 3 bits, to nearest even,
// by adding 0x7ffff plus the lowest kept bit and shifting (a carry moves into the exponent),
// then the exponent bias 127 becomes 7; below 2^-6, |q| 2^9 rounded to an integer (0 .. 8, and
// 8 is the smallest normal's code) is the subnormal code.  Both are computed and one selected,
// so a wave never diverges.  (Equal, for every finite fp32 q, to rounding the exact mantissa
// (|q| / 2^floor(log2 |q|) - 1) 8 with rintf and carrying 8 into the exponent.)
__device__ __forceinline__ uint32_t e4m3_rne_sat_bits(float q) {
  const uint32_t u = __float_as_uint(q);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  const uint32_t nrm = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
  const uint32_t sub = (uint32_t)rintf(__uint_as_float(a) * 512.f);
  const uint32_t c = a >= 0x43e00000u ? 0x7eu : a < 0x3c800000u ? sub : nrm;  // 448, 2^-6
  return sign | c;
}

// Four lanes a block: lane k of a group holds values 8 k .. 8 k + 7 (16 bytes of bf16), so a
// wave reads and writes whole contiguous kilobytes; the block maximum is reduced over the four.
__global__ __launch_bounds__(256) void mx_quantize_kernel(const uint16_t* __restrict__ x, int64_t nblk,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = t >> 2;
  const int sub = (int)(t & 3);
  const bool live = blk < nblk;
  float v[8];
  {
    const uint4 w = live ? ((const uint4*)x)[t] : make_uint4(0u, 0u, 0u, 0u);
    Elem<bf16_t>::to_f32(w, v);
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  if (!live) return;
  int shared = -127;
  if (amax > 0.f) shared = min(127, max(-127, floor_log2(amax) - 8));
  if (sub == 0) scales[blk] = (uint8_t)(shared + 127);
  uint32_t w[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) word |= e4m3_rne_sat_bits(ldexpf(v[k * 4 + e], -shared)) << (8 * e);
    w[k] = word;
  }
  ((uint2*)codes)[t] = make_uint2(w[0], w[1]);
}

}  // namespace

hipError_t launch_mx_quantize(const void* x, int64_t R, int64_t K, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  // rows are contiguous and K % 32 == 0, so the blocks of x are one contiguous sequence: block b
  // of row r is block r K / 32 + b, its codes and its scale at the same index
  const int64_t n = R * (K / 32);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)((4 * n + 255) / 256)), dim3(256), 0, s, (const uint16_t*)x,
                     n, codes, scales);
  return hipGetLastError();
}

}  // namespace moe
