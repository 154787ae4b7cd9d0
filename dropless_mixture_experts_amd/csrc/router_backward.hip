// Router backward: the router is learned (page "Accelerating dropless MoE
// training in JAX with NVIDIA Transformer Engine", introduction), so training
// takes the gate gradients back to the router's weights and inputs.  The top-K
// choice is a discrete decision and is held fixed.
//
//   route_backward_kernel  d_gates -> d_logits: back through the renormalisation
//                          g_k = s_k / S (S = sum of the chosen scores) and the
//                          score function (softmax over all E keys, or a
//                          sigmoid per key).  G lanes share one token as in the
//                          forward top-K; group sums use butterfly shuffles.
//   router_prep_*          d_logits split into bf16 high and low parts (their
//                          sum carries about 16 significant bits), transposed
//                          for dWr and row-major for dx; Wr transposed.
//   router_dwr_kernel      dWr = d_logits^T x, an MFMA reduction over tokens:
//                          a workgroup owns 256 columns of d and one run of
//                          tokens; x tiles go through LDS and are read
//                          transposed with ds_read_b64_tr_b16; runs are summed
//                          in a fixed order by router_dwr_reduce_kernel.
//   router_dx_kernel       dx (+)= d_logits Wr, MFMA with a reduction over the
//                          E experts; results leave through LDS as whole rows.
//   fp32 inputs take plain per-element kernels (small shapes only).
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kRbThreads = 256;
constexpr int kRbMaxE = 256;

template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = 1; o < G; o <<= 1) v += __shfl_xor(v, o, 64);
  return v;
}
template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = 1; o < G; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// G lanes per token (G = next power of two >= E, at most 64); lane l holds experts
// l, l + G, ... (KPL of them).  Lane k < K holds the k-th chosen expert.
template <int G>
__global__ __launch_bounds__(kRbThreads) void route_backward_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, const int32_t* __restrict__ idx,
    const float* __restrict__ d_gates, int64_t T, int E, int K, int score, int renorm,
    float* __restrict__ d_logits) {
  constexpr int KPL = (G == 64) ? kRbMaxE / 64 : 1;
  constexpr int TPB = kRbThreads / G;  // tokens per workgroup
  __shared__ float s_ds[kRbThreads * KPL];
  const int tid = threadIdx.x;
  const int lig = tid & (G - 1);
  const int tl = tid / G;
  const int64_t t = (int64_t)blockIdx.x * TPB + tl;
  const bool live = t < T;
  float* ds_row = s_ds + tl * (G * KPL);  // d loss / d score of every expert of the token
#pragma unroll
  for (int j = 0; j < KPL; ++j) ds_row[lig + j * G] = 0.f;

  float kv[KPL];
#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int e = lig + j * G;
    float v = -INFINITY;
    if (live && e < E) {
      v = logits[t * E + e];
      if (bias) v = v + bias[e];
    }
    kv[j] = v;
  }
  float m = kv[0];
#pragma unroll
  for (int j = 1; j < KPL; ++j) m = fmaxf(m, kv[j]);
  m = group_max<G>(m);
  float z = 0.f;
  if (score == 0) {
#pragma unroll
    for (int j = 0; j < KPL; ++j) z += expf(kv[j] - m);  // exp(-inf) = 0 past E
    z = group_sum<G>(z);
  }

  // the chosen experts: score s_k and d loss / d s_k
  const bool mine = live && lig < K;
  int ek = -1;
  float dgk = 0.f, sk = 0.f;
  if (mine) {
    ek = idx[t * K + lig];
    dgk = d_gates[t * K + lig];
    if (ek >= 0 && ek < E) {
      float kk = logits[t * E + ek];
      if (bias) kk = kk + bias[ek];
      sk = (score == 1) ? 1.f / (1.f + expf(-kk)) : expf(kk - m) / z;
    }
  }
  float dsk = dgk;
  if (renorm) {
    // g_k = s_k / S:  d loss / d s_k = (dg_k - sum_j g_j dg_j) / S
    const float S = group_sum<G>(mine ? sk : 0.f);
    const float c = group_sum<G>(mine ? sk * dgk : 0.f) / S;
    dsk = (dgk - c) / S;
  }
  if (mine && ek >= 0 && ek < E) ds_row[ek] = dsk;
  // softmax: d key_e = s_e (ds_e - sum_j s_j ds_j); with renormalisation that sum is 0 exactly
  float c2 = 0.f;
  if (score == 0 && !renorm) c2 = group_sum<G>(mine ? sk * dsk : 0.f);
  __builtin_amdgcn_wave_barrier();  // the group's LDS row is written before it is read back

#pragma unroll
  for (int j = 0; j < KPL; ++j) {
    const int e = lig + j * G;
    if (live && e < E) {
      float dk;
      if (score == 1) {
        const float sg = 1.f / (1.f + expf(-kv[j]));
        dk = ds_row[e] * sg * (1.f - sg);
      } else {
        dk = (expf(kv[j] - m) / z) * (ds_row[e] - c2);
      }
      d_logits[t * E + e] = dk;
    }
  }
}

// ---------------------------------------------------------------------------
// split of d_logits into bf16 high + low parts

__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16_bits(v);
  lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}

// dlT_hi / dlT_lo [E32][Tp]: element (e, t) = part of d_logits[t][e], 0 for e >= E or t >= T.
// Thread (e, run of 8 tokens), e fastest.
__global__ __launch_bounds__(256) void router_prep_t_kernel(const float* __restrict__ dl, int64_t T, int E,
                                                            int E32, int64_t Tp, uint16_t* __restrict__ hi_out,
                                                            uint16_t* __restrict__ lo_out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t n8 = Tp / 8;
  if (i >= (int64_t)E32 * n8) return;
  const int e = (int)(i % E32);
  const int64_t t0 = (i / E32) * 8;
  uint16_t h[8], l[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t t = t0 + u;
    const float v = (e < E && t < T) ? dl[t * E + e] : 0.f;
    split_bf16(v, h[u], l[u]);
  }
  uint4 vh, vl;
  vh.x = h[0] | ((uint32_t)h[1] << 16); vh.y = h[2] | ((uint32_t)h[3] << 16);
  vh.z = h[4] | ((uint32_t)h[5] << 16); vh.w = h[6] | ((uint32_t)h[7] << 16);
  vl.x = l[0] | ((uint32_t)l[1] << 16); vl.y = l[2] | ((uint32_t)l[3] << 16);
  vl.z = l[4] | ((uint32_t)l[5] << 16); vl.w = l[6] | ((uint32_t)l[7] << 16);
  *(uint4*)(hi_out + (int64_t)e * Tp + t0) = vh;
  *(uint4*)(lo_out + (int64_t)e * Tp + t0) = vl;
}

// dl_hi / dl_lo [T][E16] (row-major, experts past E are 0), and WrT [d][E16] = Wr^T.
// Thread (row, run of 8 experts).
__global__ __launch_bounds__(256) void router_prep_rows_kernel(const float* __restrict__ dl, int64_t T, int E,
                                                               int E16, uint16_t* __restrict__ hi_out,
                                                               uint16_t* __restrict__ lo_out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n8 = E16 / 8;
  if (i >= T * n8) return;
  const int64_t t = i / n8;
  const int e0 = (int)(i % n8) * 8;
  uint16_t h[8], l[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e = e0 + u;
    split_bf16(e < E ? dl[t * E + e] : 0.f, h[u], l[u]);
  }
  uint4 vh, vl;
  vh.x = h[0] | ((uint32_t)h[1] << 16); vh.y = h[2] | ((uint32_t)h[3] << 16);
  vh.z = h[4] | ((uint32_t)h[5] << 16); vh.w = h[6] | ((uint32_t)h[7] << 16);
  vl.x = l[0] | ((uint32_t)l[1] << 16); vl.y = l[2] | ((uint32_t)l[3] << 16);
  vl.z = l[4] | ((uint32_t)l[5] << 16); vl.w = l[6] | ((uint32_t)l[7] << 16);
  *(uint4*)(hi_out + t * E16 + e0) = vh;
  *(uint4*)(lo_out + t * E16 + e0) = vl;
}

__global__ __launch_bounds__(256) void router_prep_wt_kernel(const uint16_t* __restrict__ w, int64_t d, int E,
                                                             int E16, uint16_t* __restrict__ wt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int n8 = E16 / 8;
  if (i >= d * n8) return;
  const int64_t j = i % d;  // column of Wr: consecutive threads read consecutive columns
  const int e0 = (int)(i / d) * 8;
  uint16_t h[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int e = e0 + u;
    h[u] = e < E ? w[(int64_t)e * d + j] : (uint16_t)0;
  }
  uint4 v;
  v.x = h[0] | ((uint32_t)h[1] << 16); v.y = h[2] | ((uint32_t)h[3] << 16);
  v.z = h[4] | ((uint32_t)h[5] << 16); v.w = h[6] | ((uint32_t)h[7] << 16);
  *(uint4*)(wt + j * E16 + e0) = v;
}

__device__ __forceinline__ f32x16 mfma_bf16(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// dWr = d_logits^T x
//
// Workgroup (column block of 256, run of tokens); stages of 64 tokens.  The x
// tile of a stage ([64 tokens][256 columns] bf16, 512-byte LDS rows whose
// 32-byte segments are XORed with (token & 3)) is loaded one stage ahead into
// registers and written to the other of two LDS buffers.  The MFMA A operand
// (lane = expert, 8 consecutive tokens) comes straight from the transposed
// high/low parts; the B operand (lane = column, 8 consecutive tokens) is read
// from LDS with two ds_read_b64_tr_b16: within each 16 lanes, lane 4 e + q
// points at token row k0 + e, columns 4 q .. 4 q + 3, and lane i receives
// column i at rows k0 .. k0 + 3.
// Waves: WE groups over the NF expert tiles x WJ groups over the 8 column tiles.
namespace rdw {
constexpr int kCols = 256;
constexpr int kRowBytes = kCols * 2;
constexpr int kStageTok = 64;
constexpr int kStageBytes = kStageTok * kRowBytes;      // 32 KB
constexpr int kChunksPerLane = kStageBytes / 16 / 256;  // 8
}  // namespace rdw

template <int NF>
__global__ __launch_bounds__(256) void router_dwr_kernel(const uint16_t* __restrict__ dlt_hi,
                                                         const uint16_t* __restrict__ dlt_lo,
                                                         const uint16_t* __restrict__ x, int64_t T, int64_t d,
                                                         int E, int64_t Tp, int64_t tps, float* __restrict__ out) {
  using namespace rdw;
  constexpr int WE = NF < 4 ? NF : 4;
  constexpr int WJ = 4 / WE;
  constexpr int NFW = NF / WE;
  constexpr int NJW = 8 / WJ;
  static_assert(WE * WJ == 4 && WE * NFW == NF && WJ * NJW == 8, "wave split");
  __shared__ uint4 smem[2 * kStageBytes / 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int we = wave % WE, wj = wave / WE;
  const int64_t j0 = (int64_t)blockIdx.x * kCols;
  const int64_t ta = (int64_t)blockIdx.y * tps;
  const int64_t tb = min(T, ta + tps);
  const int ns = (int)((tb - ta + kStageTok - 1) / kStageTok);

  // x chunks of this lane: chunk c = it * 256 + tid -> token row c / 32, logical chunk c % 32
  int64_t xcol[kChunksPerLane];
  uint32_t xlds[kChunksPerLane];
  int xrow[kChunksPerLane];
#pragma unroll
  for (int it = 0; it < kChunksPerLane; ++it) {
    const int c = it * 256 + tid;
    const int r = c >> 5, lc = c & 31;
    int64_t col = j0 + lc * 8;
    xcol[it] = col < d ? col : d - 8;
    xrow[it] = r;
    const int pc = (((lc >> 1) ^ (r & 3)) << 1) | (lc & 1);
    xlds[it] = (uint32_t)(r * kRowBytes + pc * 16);
  }
  auto load_x = [&](int s, uint4 (&v)[kChunksPerLane]) {
#pragma unroll
    for (int it = 0; it < kChunksPerLane; ++it) {
      int64_t row = ta + (int64_t)s * kStageTok + xrow[it];
      row = row < T ? row : T - 1;
      v[it] = *(const uint4*)(x + row * d + xcol[it]);
    }
  };
  auto store_x = [&](int buf, const uint4 (&v)[kChunksPerLane]) {
    char* base = (char*)smem + buf * kStageBytes;
#pragma unroll
    for (int it = 0; it < kChunksPerLane; ++it) *(uint4*)(base + xlds[it]) = v[it];
  };
  // A fragments: rows e = (we NFW + f) 32 + l32 of the transposed parts, tokens + 8 hi
  const uint16_t* arow_hi[NFW];
  const uint16_t* arow_lo[NFW];
#pragma unroll
  for (int f = 0; f < NFW; ++f) {
    const int e = (we * NFW + f) * 32 + l32;
    arow_hi[f] = dlt_hi + (int64_t)e * Tp + ta + hi * 8;
    arow_lo[f] = dlt_lo + (int64_t)e * Tp + ta + hi * 8;
  }
  auto load_a = [&](int s, uint4 (&ah)[4][NFW], uint4 (&al)[4][NFW]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int f = 0; f < NFW; ++f) {
        const int64_t o = (int64_t)s * kStageTok + kk * 16;
        ah[kk][f] = *(const uint4*)(arow_hi[f] + o);
        al[kk][f] = *(const uint4*)(arow_lo[f] + o);
      }
  };
  // transposed reads: lane (g, e4, q) of each 16; row kk 16 + 8 hi + 4 t + e4
  const int g = (lane >> 4) & 1, e4 = (lane >> 2) & 3, q = lane & 3;
  uint32_t boff[NJW];
#pragma unroll
  for (int jt = 0; jt < NJW; ++jt) {
    const int seg = (wj * NJW + jt) * 2 + g;
    boff[jt] = (uint32_t)((hi * 8 + e4) * kRowBytes + ((seg ^ e4) * 32) + q * 8);
  }

  f32x16 acc[NFW][NJW];
#pragma unroll
  for (int f = 0; f < NFW; ++f)
#pragma unroll
    for (int jt = 0; jt < NJW; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[f][jt][r] = 0.f;

  uint4 xv[kChunksPerLane];
  uint4 ah[4][NFW], al[4][NFW];
  if (ns > 0) {
    load_x(0, xv);
    load_a(0, ah, al);
    store_x(0, xv);
  }
  for (int s = 0; s < ns; ++s) {
    const int buf = s & 1;
    uint4 ah2[4][NFW], al2[4][NFW];
    if (s + 1 < ns) {
      load_x(s + 1, xv);
      load_a(s + 1, ah2, al2);
    }
    __syncthreads();  // buffer buf holds stage s; buffer buf ^ 1 is read by no wave
    const char* L = (const char*)smem + buf * kStageBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      uint4 b[NJW];
#pragma unroll
      for (int jt = 0; jt < NJW; ++jt) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          typedef short s16x4 __attribute__((ext_vector_type(4)));
          typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
          const char* addr = L + boff[jt] + (kk * 16 + 4 * t2) * kRowBytes;
          const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)addr);
          const uint32_t w0 = (uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
          const uint32_t w1 = (uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
          if (t2 == 0) {
            b[jt].x = w0;
            b[jt].y = w1;
          } else {
            b[jt].z = w0;
            b[jt].w = w1;
          }
        }
      }
#pragma unroll
      for (int f = 0; f < NFW; ++f)
#pragma unroll
        for (int jt = 0; jt < NJW; ++jt) {
          acc[f][jt] = mfma_bf16(ah[kk][f], b[jt], acc[f][jt]);
          acc[f][jt] = mfma_bf16(al[kk][f], b[jt], acc[f][jt]);
        }
    }
    if (s + 1 < ns) {
      store_x(buf ^ 1, xv);
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int f = 0; f < NFW; ++f) {
          ah[kk][f] = ah2[kk][f];
          al[kk][f] = al2[kk][f];
        }
    }
  }

  // out[e][j]: lane l32 = column, rows e = 8 (r >> 2) + 4 hi + (r & 3) of each 32 x 32 tile
  float* o = out + (int64_t)blockIdx.y * E * d;
#pragma unroll
  for (int f = 0; f < NFW; ++f)
#pragma unroll
    for (int jt = 0; jt < NJW; ++jt) {
      const int64_t col = j0 + (wj * NJW + jt) * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = (we * NFW + f) * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (e < E && col < d) o[(int64_t)e * d + col] = acc[f][jt][r];
      }
    }
}

// dWr[i] = sum over runs p = 0 .. P-1 of part[p][i], in that order (float4 per thread)
__global__ __launch_bounds__(256) void router_dwr_reduce_kernel(const float* __restrict__ part, int P,
                                                                int64_t n4, float* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const f32x4* p4 = (const f32x4*)part;
  f32x4 s = p4[i];
  int p = 1;
  for (; p + 8 <= P; p += 8) {  // eight loads in flight, added in order
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p4[(int64_t)(p + u) * n4 + i];
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; p < P; ++p) s += p4[(int64_t)p * n4 + i];
  ((f32x4*)dw)[i] = s;
}

// ---------------------------------------------------------------------------
// dx (+)= d_logits Wr, computed as its transpose per tile: C^T[j][t] = sum_e WrT[j][e] dl[t][e]
// (MFMA A = WrT rows, B = d_logits rows; both 16-byte loads of 8 consecutive experts).
// Workgroup: 64 tokens x 256 columns (one-dimensional grid, column blocks fastest); wave
// (wt, wj): 32 tokens x 128 columns (4 tiles).
// Each lane ends with 4 consecutive columns of its token per register group: they go
// to the wave's LDS region in fp32, then out as 16-byte chunks of 8 bf16 (with the old
// dx added in fp32 first when accumulating: one rounding).
__global__ __launch_bounds__(256) void router_dx_kernel(const uint16_t* __restrict__ dl_hi,
                                                        const uint16_t* __restrict__ dl_lo,
                                                        const uint16_t* __restrict__ wt, int64_t T, int64_t d,
                                                        int E16, int accumulate, uint16_t* __restrict__ dx) {
  __shared__ uint4 smem[4 * 32 * 256 / 16];  // 4 waves x [32][64] fp32
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int wt_ = wave & 1, wj = wave >> 1;
  const int64_t ncb = (d + 255) / 256;  // blocks: column block fastest, then 64-token block
  const int64_t t0 = ((int64_t)blockIdx.x / ncb) * 64 + wt_ * 32;
  const int64_t c0 = ((int64_t)blockIdx.x % ncb) * 256 + wj * 128;
  int64_t tr = t0 + l32;
  tr = tr < T ? tr : T - 1;
  const uint16_t* ah_p = dl_hi + tr * E16 + hi * 8;
  const uint16_t* al_p = dl_lo + tr * E16 + hi * 8;
  const uint16_t* b_p[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t col = c0 + j * 32 + l32;
    col = col < d ? col : d - 1;
    b_p[j] = wt + col * E16 + hi * 8;
  }
  f32x16 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
#pragma unroll 2
  for (int k0 = 0; k0 < E16; k0 += 16) {
    const uint4 bh = *(const uint4*)(ah_p + k0);
    const uint4 bl = *(const uint4*)(al_p + k0);
    uint4 a[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = *(const uint4*)(b_p[j] + k0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[j] = mfma_bf16(a[j], bh, acc[j]);
      acc[j] = mfma_bf16(a[j], bl, acc[j]);
    }
  }
  // two rounds of 64 columns: lane (token l32) writes 4 consecutive fp32 columns per register
  // group to the wave's [32][64] region (16-byte chunks XORed with the token), then 32 rows x
  // 8 groups of 8 columns leave as bf16, the old values added first when accumulating
  char* wl = (char*)smem + wave * (32 * 256);
  const int c = lane & 7;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int64_t col = c0 + half * 64 + c * 8;
    uint4 old[4];
    if (accumulate) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int64_t t = t0 + it * 8 + (lane >> 3);
        old[it] = (t < T && col < d) ? *(const uint4*)(dx + t * d + col) : make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (half) __builtin_amdgcn_wave_barrier();  // the first round's reads are done
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int j = half * 2 + jj;
        const int ch = (jj * 8 + 2 * rg + hi) ^ (l32 & 15);
        *(f32x4*)(wl + l32 * 256 + ch * 16) =
            f32x4{acc[j][4 * rg], acc[j][4 * rg + 1], acc[j][4 * rg + 2], acc[j][4 * rg + 3]};
      }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int r = it * 8 + (lane >> 3);
      const int64_t t = t0 + r;
      const f32x4 v0 = *(const f32x4*)(wl + r * 256 + (((2 * c) ^ (r & 15)) * 16));
      const f32x4 v1 = *(const f32x4*)(wl + r * 256 + (((2 * c + 1) ^ (r & 15)) * 16));
      float a[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      if (accumulate) {
        float b[8];
        Elem<bf16_t>::to_f32(old[it], b);
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] += b[u];
      }
      if (t < T && col < d) *(uint4*)(dx + t * d + col) = Elem<bf16_t>::from_f32(a);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs: one thread per output element

__global__ __launch_bounds__(256) void router_dwr_f32_kernel(const float* __restrict__ dl, const float* __restrict__ x,
                                                             int64_t T, int64_t d, int E, float* __restrict__ dw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)E * d) return;
  const int e = (int)(i / d);
  const int64_t j = i % d;
  float s = 0.f;
  for (int64_t t = 0; t < T; ++t) s = fmaf(dl[t * E + e], x[t * d + j], s);
  dw[i] = s;
}

__global__ __launch_bounds__(256) void router_dx_f32_kernel(const float* __restrict__ dl, const float* __restrict__ w,
                                                            int64_t T, int64_t d, int E, int accumulate,
                                                            float* __restrict__ dx) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * d) return;
  const int64_t t = i / d, j = i % d;
  float s = accumulate ? dx[i] : 0.f;
  for (int e = 0; e < E; ++e) s = fmaf(dl[t * E + e], w[(int64_t)e * d + j], s);
  dx[i] = s;
}

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
// expert tiles of 32 the dWr kernel is launched with: 1, 2, 4 or 8
inline int dwr_tiles(int E) {
  const int nf = (E + 31) / 32;
  return nf <= 1 ? 1 : nf <= 2 ? 2 : nf <= 4 ? 4 : 8;
}
inline size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// runs of tokens of the dWr reduction: enough workgroups for two per CU, while the fp32
// partial sums stay below about a quarter of the bytes of x
struct DwrPlan {
  int64_t ncb, P, tps;
};
DwrPlan dwr_plan(int64_t T, int64_t d, int E) {
  DwrPlan p;
  p.ncb = (d + rdw::kCols - 1) / rdw::kCols;
  const int64_t nstg = std::max<int64_t>(1, (T + rdw::kStageTok - 1) / rdw::kStageTok);
  int64_t P = (512 + p.ncb - 1) / p.ncb;
  P = std::min(P, std::max<int64_t>(1, T / (4 * (int64_t)E)));
  P = std::max<int64_t>(1, std::min(P, nstg));
  p.tps = (nstg + P - 1) / P * rdw::kStageTok;
  p.P = std::max<int64_t>(1, (T + p.tps - 1) / p.tps);
  return p;
}

struct RbLayout {
  size_t dlt, dl, wt, part, total;
  int64_t Tp;
  int E32, E16;
};
RbLayout rb_layout(int64_t T, int64_t d, int E) {
  RbLayout L;
  L.E32 = 32 * dwr_tiles(E);
  L.E16 = (int)round_up(E, 16);
  L.Tp = round_up(std::max<int64_t>(T, 1), rdw::kStageTok);
  size_t off = 0;
  L.dlt = off;
  off = align256(off + 2 * (size_t)L.E32 * L.Tp * 2);
  L.dl = off;
  off = align256(off + 2 * (size_t)T * L.E16 * 2);
  L.wt = off;
  off = align256(off + (size_t)d * L.E16 * 2);
  L.part = off;
  const DwrPlan p = dwr_plan(T, d, E);
  if (p.P > 1) off = align256(off + (size_t)p.P * E * d * 4);
  L.total = off;
  return L;
}

}  // namespace

hipError_t launch_route_backward(const float* logits, const float* bias, const int32_t* idx,
                                 const float* d_gates, int64_t T, int E, int K, int score, int renorm,
                                 float* d_logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  int G = 1;
  while (G < E && G < 64) G <<= 1;
#define MOE_RB_CASE(g)                                                                              \
  case g:                                                                                           \
    hipLaunchKernelGGL(route_backward_kernel<g>, dim3((unsigned)((T + kRbThreads / g - 1) / (kRbThreads / g))), \
                       dim3(kRbThreads), 0, s, logits, bias, idx, d_gates, T, E, K, score, renorm, d_logits); \
    break;
  switch (G) {
    MOE_RB_CASE(1)
    MOE_RB_CASE(2)
    MOE_RB_CASE(4)
    MOE_RB_CASE(8)
    MOE_RB_CASE(16)
    MOE_RB_CASE(32)
    MOE_RB_CASE(64)
    default:
      return hipErrorInvalidValue;
  }
#undef MOE_RB_CASE
  return hipGetLastError();
}

size_t router_backward_workspace_bytes(int64_t T, int64_t d, int E, int dtype) {
  if (dtype != 1) return 0;
  return rb_layout(T, d, E).total;
}

hipError_t launch_router_logits_backward(const float* d_logits, const void* x, const void* w, int64_t T,
                                         int64_t d, int E, int dtype, float* d_w, void* dx, int accumulate,
                                         void* ws, hipStream_t s) {
  if (dtype != 1) {
    if (d_w) {
      const int64_t n = (int64_t)E * d;
      hipLaunchKernelGGL(router_dwr_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, d_logits,
                         (const float*)x, T, d, E, d_w);
    }
    if (dx && T > 0) {
      const int64_t n = T * d;
      hipLaunchKernelGGL(router_dx_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, d_logits,
                         (const float*)w, T, d, E, accumulate, (float*)dx);
    }
    return hipGetLastError();
  }
  const RbLayout L = rb_layout(T, d, E);
  char* wsb = (char*)ws;
  if (d_w) {
    if (T == 0) {
      // no tokens: dWr = 0 (a fill kernel, so that the call stays capturable in a graph)
      const int64_t n = (int64_t)E * d;
      hipLaunchKernelGGL(router_dwr_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, d_logits,
                         (const float*)x, T, d, E, d_w);
    } else {
      uint16_t* th = (uint16_t*)(wsb + L.dlt);
      uint16_t* tl = th + (size_t)L.E32 * L.Tp;
      const int64_t n = (int64_t)L.E32 * (L.Tp / 8);
      hipLaunchKernelGGL(router_prep_t_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, d_logits, T,
                         E, L.E32, L.Tp, th, tl);
      const DwrPlan p = dwr_plan(T, d, E);
      float* out = p.P > 1 ? (float*)(wsb + L.part) : d_w;
      const dim3 grid((unsigned)p.ncb, (unsigned)p.P);
      const uint16_t* xb = (const uint16_t*)x;
      switch (L.E32 / 32) {
        case 1: hipLaunchKernelGGL(router_dwr_kernel<1>, grid, dim3(256), 0, s, th, tl, xb, T, d, E, L.Tp, p.tps, out); break;
        case 2: hipLaunchKernelGGL(router_dwr_kernel<2>, grid, dim3(256), 0, s, th, tl, xb, T, d, E, L.Tp, p.tps, out); break;
        case 4: hipLaunchKernelGGL(router_dwr_kernel<4>, grid, dim3(256), 0, s, th, tl, xb, T, d, E, L.Tp, p.tps, out); break;
        default: hipLaunchKernelGGL(router_dwr_kernel<8>, grid, dim3(256), 0, s, th, tl, xb, T, d, E, L.Tp, p.tps, out); break;
      }
      if (p.P > 1) {
        const int64_t n4 = (int64_t)E * d / 4;
        hipLaunchKernelGGL(router_dwr_reduce_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, out,
                           (int)p.P, n4, d_w);
      }
    }
  }
  if (dx && T > 0) {
    uint16_t* rh = (uint16_t*)(wsb + L.dl);
    uint16_t* rl = rh + (size_t)T * L.E16;
    uint16_t* wt = (uint16_t*)(wsb + L.wt);
    const int64_t n = T * (L.E16 / 8);
    hipLaunchKernelGGL(router_prep_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, d_logits, T, E,
                       L.E16, rh, rl);
    const int64_t nw = d * (L.E16 / 8);
    hipLaunchKernelGGL(router_prep_wt_kernel, dim3((unsigned)((nw + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)w, d, E, L.E16, wt);
    const dim3 grid((unsigned)(((d + 255) / 256) * ((T + 63) / 64)));
    hipLaunchKernelGGL(router_dx_kernel, grid, dim3(256), 0, s, rh, rl, wt, T, d, L.E16, accumulate,
                       (uint16_t*)dx);
  }
  return hipGetLastError();
}

}  // namespace moe
