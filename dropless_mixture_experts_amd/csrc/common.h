// Device helpers shared by the gfx950 kernels of the MoE library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits, round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// two fp32 -> packed bf16 (lo in the low half), one v_cvt_pk_bf16_f32 for the pair; converting
// them one at a time and shifting the halves together took three VALU ops per pair
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2v v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Element traits: a 16-byte vector holds kVec elements.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kVec = 4;
  static constexpr int kBytes = 4;
  __device__ static void to_f32(const uint4& v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static uint4 from_f32(const float (&f)[4]) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
  __device__ static float load1(const void* p, int64_t i) { return ((const float*)p)[i]; }
  __device__ static void store1(void* p, int64_t i, float v) { ((float*)p)[i] = v; }
  // elements i..i+3 (i a multiple of 4: one 16-byte access)
  __device__ static void load4(const void* p, int64_t i, float (&f)[4]) {
    const f32x4 v = *(const f32x4*)((const float*)p + i);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
  __device__ static void store4(void* p, int64_t i, const float (&f)[4]) {
    const f32x4 v = {f[0], f[1], f[2], f[3]};
    *(f32x4*)((float*)p + i) = v;
  }
};
struct bf16_t {};
template <> struct Elem<bf16_t> {
  static constexpr int kVec = 8;
  static constexpr int kBytes = 2;
  __device__ static void to_f32(const uint4& v, float (&f)[8]) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ static uint4 from_f32(const float (&f)[8]) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
  __device__ static float load1(const void* p, int64_t i) {
    return bf16_bits_to_f32(((const uint16_t*)p)[i]);
  }
  __device__ static void store1(void* p, int64_t i, float v) { ((uint16_t*)p)[i] = f32_to_bf16_bits(v); }
  // elements i..i+3 (i a multiple of 4: one 8-byte access)
  __device__ static void load4(const void* p, int64_t i, float (&f)[4]) {
    const uint2 v = *(const uint2*)((const uint16_t*)p + i);
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
  }
  __device__ static void store4(void* p, int64_t i, const float (&f)[4]) {
    *(uint2*)((uint16_t*)p + i) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
  }
};

// streaming (non-temporal) 16-byte global accesses
__device__ __forceinline__ uint4 ld_nt(const uint4* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt(uint4* p, const uint4& v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (u32x4*)p);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace moe
