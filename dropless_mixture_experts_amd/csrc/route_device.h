// Device side of top-K routing, shared by the routing kernel (keys read from the
// logits in global memory) and the fused router (keys read from the logits tile
// it has just computed in LDS).
//
// The learned router picks the Top-K experts of every token and every expert
// then owns a data-dependent, ragged number of slots (page "Accelerating
// dropless MoE training in JAX with NVIDIA Transformer Engine": introduction
// and "What are the challenges in MoE training?").
#pragma once
#include "common.h"

namespace moe {
namespace rdev {

constexpr int kMaxTopK = 32;
constexpr int kMaxExperts = 256;

// rank in the total order of fp32 bit patterns: -inf < ... < -0 < +0 < ... < +inf
__device__ __forceinline__ uint32_t f32_order(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float order_to_f32(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, m, 64);
  hi = __shfl_xor(hi, m, 64);
  return ((uint64_t)hi << 32) | lo;
}

// v of the lane that DPP control CTRL names (within a row of 16 lanes; every lane of a group
// reads a lane of the same group, all of whose lanes are active together)
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

// Maximum of v over an aligned group of G lanes (G a power of two), in every lane of it: swaps
// within quads, then the mirror of each half row and of each row (the two halves being equal
// by then, any pairing across them completes the maximum); shuffles past 16 lanes.
template <int G>
__device__ __forceinline__ uint64_t group_max_u64(uint64_t v) {
  if constexpr (G >= 2) { const uint64_t o = dpp_u64<0xB1>(v); v = o > v ? o : v; }   // quad_perm 1,0,3,2
  if constexpr (G >= 4) { const uint64_t o = dpp_u64<0x4E>(v); v = o > v ? o : v; }   // quad_perm 2,3,0,1
  if constexpr (G >= 8) { const uint64_t o = dpp_u64<0x141>(v); v = o > v ? o : v; }  // row_half_mirror
  if constexpr (G >= 16) { const uint64_t o = dpp_u64<0x140>(v); v = o > v ? o : v; } // row_mirror
#pragma unroll
  for (int m = 16; m < G; m <<= 1) {
    const uint64_t o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < G; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Top-K of one token held by a group of G lanes; lane lig holds the keys of experts
// e_lo .. e_lo + KPL - 1 in kf (-inf past E).  A key packs the fp32 order of the key above
// the complemented expert index, so one unsigned maximum picks the largest key and, among
// equal keys, the smallest expert; a cleared or absent key is 0, below every real key.
// Each of the K rounds takes the lane-local maximum (a tree of independent compares), then
// the maximum over the group.  Round k is kept by lane k mod G of the group (s_sel / s_score at slot tl*K + k),
// which also writes it out: topk_idx[t*K + k] and topk_gate[t*K + k].
template <int G, int KPL>
__device__ __forceinline__ void select_token(float (&kf)[KPL], int e_lo, int E, int K, int score, int renorm,
                                             int lig, int64_t t, int tl, uint8_t* s_sel, float* s_score,
                                             int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate) {
  uint64_t comp[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int e = e_lo + j;
    if (e < E) {
      comp[j] = ((uint64_t)f32_order(kf[j]) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e);
    } else {
      kf[j] = -INFINITY;
      comp[j] = 0;
    }
  }
  float top_key = 0.f, denom = 0.f;
  for (int k = 0; k < K; ++k) {
    uint64_t m[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) m[j] = comp[j];
#pragma unroll
    for (int w = 1; w < KPL; w *= 2)
#pragma unroll
      for (int j = 0; j + w < KPL; j += 2 * w) m[j] = m[j + w] > m[j] ? m[j + w] : m[j];
    const uint64_t best = group_max_u64<G>(m[0]);
    const int e = (int)(0xffffffffu - (uint32_t)best);
#pragma unroll
    for (int j = 0; j < KPL; ++j)
      if (e_lo + j == e) comp[j] = 0;
    const float key = order_to_f32((uint32_t)(best >> 32));
    if (k == 0) top_key = key;
    const float s = (score == 1) ? 1.f / (1.f + expf(-key)) : expf(key - top_key);
    denom += s;
    if (lig == (k & (G - 1))) {
      s_sel[tl * K + k] = (uint8_t)e;
      s_score[tl * K + k] = s;
    }
  }
  if (!renorm) {
    if (score == 0) {
      float z = 0.f;
#pragma unroll
      for (int j = 0; j < KPL; ++j) z += expf(kf[j] - top_key);
      denom = group_sum<G>(z);
    } else {
      denom = 1.f;
    }
  }
  for (int k = lig; k < K; k += G) {
    topk_idx[t * K + k] = s_sel[tl * K + k];
    topk_gate[t * K + k] = s_score[tl * K + k] / denom;
  }
}

// Stable per-expert ranks of a chunk's n slots (slot order = t*K + k), by NW waves of the
// workgroup: each wave ranks a contiguous segment with 8 ballots per 64 slots; the
// per-wave counts become per-wave bases.  Writes the chunk's histogram (hist_row[e]) and
// each slot's rank inside the chunk (local_rank[s]).  Every thread of the workgroup calls it.
template <int NW>
__device__ __forceinline__ void rank_chunk(int n, int E, const uint8_t* s_sel, uint16_t* s_rank,
                                           int (*s_cnt)[kMaxExperts], int32_t* __restrict__ hist_row,
                                           int32_t* __restrict__ local_rank) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int e = lane; e < E; e += 64) s_cnt[wave][e] = 0;
  __syncthreads();
  // slots per wave, a multiple of 64
  const int seg = ((n + 64 * NW - 1) / (64 * NW)) * 64;
  const int beg = wave * seg;
  const int end = min(n, beg + seg);
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b = beg; b < end; b += 64) {
    const int s = b + lane;
    const bool valid = s < end;
    const int e = valid ? (int)s_sel[s] : 0;
    uint64_t eq = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t m = __ballot(valid && ((e >> bit) & 1));
      eq &= ((e >> bit) & 1) ? m : ~m;
    }
    int c = 0;
    if (valid) {
      c = s_cnt[wave][e];
      s_rank[s] = (uint16_t)(c + __popcll(eq & lt_mask));
    }
    // the highest lane of each equal-expert set advances that expert's counter
    if (valid && (eq >> lane) == 1ull) s_cnt[wave][e] = c + __popcll(eq);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 64 * NW) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int v = s_cnt[w][e];
      s_cnt[w][e] = run;
      run += v;
    }
    hist_row[e] = run;
  }
  __syncthreads();
  for (int s = tid; s < n; s += 64 * NW) {
    const int w = s / seg;
    local_rank[s] = s_cnt[w][s_sel[s]] + s_rank[s];
  }
}

}  // namespace rdev
}  // namespace moe
