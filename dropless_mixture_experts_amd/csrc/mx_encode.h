// MXFP8 encoding helpers shared by the quantisation kernel and the grouped GEMM's quantising
// epilogue (OCP Microscaling: E8M0 block scales, E4M3 values; the rule is stated in
// mxfp8.hip).
#pragma once
#include <cstdint>

namespace moe {

// floor(log2(a)) of a finite a > 0 (normal or subnormal fp32)
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t u = __float_as_uint(a);
  const int e = (int)((u >> 23) & 0xff);
  if (e != 0) return e - 127;
  return -149 + (31 - __clz(u & 0x7fffffu));
}

// the block's shared exponent from its largest magnitude: floor(log2(amax)) - 8 clamped to
// [-127, 127], -127 for a block of zeros (scale byte = shared + 127)
__device__ __forceinline__ int mx_shared_exponent(float amax) {
  return amax > 0.f ? min(127, max(-127, floor_log2(amax) - 8)) : -127;
}

// Four E4M3 codes, byte k = q_k: each value rounded to the nearest E4M3 value, ties to the even
// mantissa, and saturated to +-448 (|q| >= 448 gives 0x7e, or 0xfe when negative).  The hardware
// conversion rounds to nearest even and the clamp to +-448 before it is the saturation; for
// every finite fp32 q the pair gives the code of that rule (checked over all 2^32 fp32 bit
// patterns on gfx950 against the rule computed in integer steps: no difference, signed zeros
// and subnormals included).
__device__ __forceinline__ uint32_t e4m3_pack4(float q0, float q1, float q2, float q3) {
  const float c0 = fmaxf(fminf(q0, 448.f), -448.f), c1 = fmaxf(fminf(q1, 448.f), -448.f);
  const float c2 = fmaxf(fminf(q2, 448.f), -448.f), c3 = fmaxf(fminf(q3, 448.f), -448.f);
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, lo, true);
}

}  // namespace moe
