// MXFP8 block quantisation of the expert matmul operands (page "Accelerating
// dropless MoE training in JAX with NVIDIA Transformer Engine", "Optimisation
// 1": the grouped GEMM path with MXFP8 block scaling from grouped quantisation).
//
// The pages name the format only; its definition is the OCP Microscaling (MX)
// one: every 32 consecutive values of a row share a power-of-two scale stored
// as E8M0 (code c = 2^(c - 127)); the values are FP8 E4M3 (bias 7, largest
// finite 448, subnormals down to 2^-9).  Shared exponent = floor(log2(max |v|))
// - 8, clamped to [-127, 127]; a block of zeros takes code 0; each value is
// v / 2^shared rounded to nearest even and saturated to +-448.  The scaling is
// exact (powers of two); the rounding is the hardware conversion of the value
// clamped to +-448, which is this rule bit for bit (mx_encode.h).
//
// Four threads per block: 64 bytes of bf16 in, 32 code bytes and 1 scale byte out.
#include "common.h"
#include "internal.h"
#include "mx_encode.h"

namespace moe {

namespace {

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
  const int shared = mx_shared_exponent(amax);
  if (sub == 0) scales[blk] = (uint8_t)(shared + 127);
  uint32_t w[2];
#pragma unroll
  for (int k = 0; k < 2; ++k)
    w[k] = e4m3_pack4(ldexpf(v[4 * k], -shared), ldexpf(v[4 * k + 1], -shared), ldexpf(v[4 * k + 2], -shared),
                      ldexpf(v[4 * k + 3], -shared));
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
