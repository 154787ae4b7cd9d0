// Top-K routing, expert histogram, prefix sum and stable slot positions.
//
// The learned router picks the Top-K experts of every token, and every expert
// then owns a data-dependent, ragged number of slots (page "Accelerating
// dropless MoE training in JAX with NVIDIA Transformer Engine": introduction
// and "What are the challenges in MoE training?").  The counts never leave
// the device ("What specialised optimisations does dropless MoE need?").
//
// Three launches, all with shapes fixed on the host:
//   R1 route_topk_kernel     one workgroup per chunk of 128 tokens.  A group of
//                            G lanes shares one token, each lane holding up to
//                            16 of its keys in registers (G = ceil(E/16) rounded
//                            to a power of two); every one of the K rounds takes
//                            the lane-local maximum, then a butterfly maximum
//                            over the group.  Scores and gates follow.  The
//                            chunk's slots are then ranked stably per expert
//                            with wave ballots, giving a per-chunk histogram
//                            and each slot's rank inside its chunk.
//   R2 route_scan_kernel     one workgroup: per expert, an exclusive scan of
//                            the chunk histograms; counts and offsets.
//   R3 route_finalize_kernel slot_pos = offsets[e] + chunk base + rank; row_src.
#include "common.h"
#include "internal.h"
#include "route_device.h"

namespace moe {

namespace {

using namespace rdev;

constexpr int kTopkThreads = 512;
constexpr int kTopkWaves = kTopkThreads / 64;

// G lanes per token; lane l of a group holds experts l*KPL .. l*KPL + KPL - 1.
// vec4: the rows may be read as float4 (E % 4 == 0, 16-byte aligned base).
template <int G, int KPL>
__global__ __launch_bounds__(kTopkThreads) void route_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int K,
    int score, int renorm, int vec4, int32_t* __restrict__ topk_idx,
    float* __restrict__ topk_gate, int32_t* __restrict__ local_rank, int32_t* __restrict__ hist) {
  constexpr int TPP = kTopkThreads / G;  // tokens per pass
  __shared__ uint8_t s_sel[kRouteChunk * kMaxTopK];
  __shared__ uint16_t s_rank[kRouteChunk * kMaxTopK];
  __shared__ float s_score[kRouteChunk * kMaxTopK];
  __shared__ float s_bias[kMaxExperts];
  __shared__ int s_cnt[kTopkWaves][kMaxExperts];

  const int tid = threadIdx.x;
  const int lig = tid & (G - 1);
  const int e_lo = lig * KPL;
  const int64_t t0 = (int64_t)blockIdx.x * kRouteChunk;
  const int ntok = (int)min((int64_t)kRouteChunk, (int64_t)T - t0);

  if (bias)
    for (int e = tid; e < E; e += kTopkThreads) s_bias[e] = bias[e];
  __syncthreads();

  for (int tl = tid / G; tl < ntok; tl += TPP) {
    const int64_t t = t0 + tl;
    const float* row = logits + t * E;
    float kf[KPL];
    if constexpr (KPL % 4 == 0) {
      if (vec4) {
#pragma unroll
        for (int q = 0; q < KPL / 4; ++q) {
          const int e = e_lo + 4 * q;
          float4 v = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
          if (e < E) v = *reinterpret_cast<const float4*>(row + e);
          kf[4 * q] = v.x;
          kf[4 * q + 1] = v.y;
          kf[4 * q + 2] = v.z;
          kf[4 * q + 3] = v.w;
        }
      } else {
#pragma unroll
        for (int j = 0; j < KPL; ++j) kf[j] = (e_lo + j < E) ? row[e_lo + j] : -INFINITY;
      }
    } else {
#pragma unroll
      for (int j = 0; j < KPL; ++j) kf[j] = (e_lo + j < E) ? row[e_lo + j] : -INFINITY;
    }
    if (bias) {
#pragma unroll
      for (int j = 0; j < KPL; ++j)
        if (e_lo + j < E) kf[j] = kf[j] + s_bias[e_lo + j];
    }
    select_token<G, KPL>(kf, e_lo, E, K, score, renorm, lig, t, tl, s_sel, s_score, topk_idx, topk_gate);
  }
  __syncthreads();
  rank_chunk<kTopkWaves>(ntok * K, E, s_sel, s_rank, s_cnt, hist + (int64_t)blockIdx.x * E, local_rank + t0 * K);
}

constexpr int kScanThreads = 1024;
constexpr int kScanParts = 64;  // at most this many threads share one expert's column

// One workgroup.  hist[c][e] (chunk counts) becomes the exclusive prefix of
// expert e's counts over chunks 0..c-1.  Thread (part p, expert e) owns a run
// of consecutive chunks of column e: it loads them all at once, adds the run
// totals of parts 0..p-1 from LDS and writes its prefixes back.
// RUN: chunk counts a thread holds in registers (16, or 32 when a thread owns more than 16 chunks)
template <int RUN>
__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(int32_t* __restrict__ hist,
                                                                  int nch, int E,
                                                                  int32_t* __restrict__ counts,
                                                                  int32_t* __restrict__ offsets) {
  __shared__ int s_part[kScanThreads];
  __shared__ int s_tot[kMaxExperts];
  const int tid = threadIdx.x;
  const int nparts = min(kScanParts, kScanThreads / E);
  const int e = tid % E;
  const int part = tid / E;
  const bool active = part < nparts;
  const int per = (nch + nparts - 1) / nparts;
  const int c_beg = active ? part * per : 0;
  const int c_end = active ? min(nch, c_beg + per) : 0;

  int v[RUN];
  int sum = 0;
#pragma unroll
  for (int u = 0; u < RUN; ++u) {
    const int c = c_beg + u;
    v[u] = (c < c_end) ? hist[(int64_t)c * E + e] : 0;
    sum += v[u];
  }
  for (int c0 = c_beg + RUN; c0 < c_end; c0 += RUN) {
#pragma unroll
    for (int u = 0; u < RUN; ++u) {
      const int c = c0 + u;
      if (c < c_end) sum += hist[(int64_t)c * E + e];
    }
  }
  if (active) s_part[part * E + e] = sum;
  __syncthreads();
  int run = 0;
  if (active) {
    for (int q = 0; q < part; ++q) run += s_part[q * E + e];
    if (part == nparts - 1) s_tot[e] = run + sum;
  }
#pragma unroll
  for (int u = 0; u < RUN; ++u) {
    const int c = c_beg + u;
    if (c < c_end) {
      hist[(int64_t)c * E + e] = run;
      run += v[u];
    }
  }
  for (int c0 = c_beg + RUN; c0 < c_end; c0 += RUN) {
    int w[RUN];
#pragma unroll
    for (int u = 0; u < RUN; ++u) {
      const int c = c0 + u;
      w[u] = (c < c_end) ? hist[(int64_t)c * E + e] : 0;
    }
#pragma unroll
    for (int u = 0; u < RUN; ++u) {
      const int c = c0 + u;
      if (c < c_end) {
        hist[(int64_t)c * E + e] = run;
        run += w[u];
      }
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    int v4[4];
    int loc = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int x = lane * 4 + j;
      v4[j] = (x < E) ? s_tot[x] : 0;
      loc += v4[j];
    }
    int inc = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(inc, o, 64);
      if (lane >= o) inc += u;
    }
    int r = inc - loc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int x = lane * 4 + j;
      if (x < E) {
        counts[x] = v4[j];
        offsets[x] = r;
      }
      r += v4[j];
    }
    if (lane == 63) offsets[E] = inc;
  }
}

// chunk = tokens per histogram chunk
__global__ __launch_bounds__(256) void route_finalize_kernel(const int32_t* __restrict__ topk_idx,
                                                             const int32_t* __restrict__ hist,
                                                             const int32_t* __restrict__ offsets,
                                                             int64_t M, int K, int E, int chunk,
                                                             int32_t* __restrict__ slot_pos,
                                                             int32_t* __restrict__ row_src) {
  const int64_t s = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (s >= M) return;
  const int64_t c = (s / K) / chunk;
  const int e = topk_idx[s];
  const int pos = offsets[e] + hist[c * E + e] + slot_pos[s];
  slot_pos[s] = pos;
  if ((uint64_t)pos < (uint64_t)M) row_src[pos] = (int32_t)s;
}

}  // namespace

size_t route_workspace_bytes(int64_t T, int E) {
  const int64_t nch = (T + kRouteChunk - 1) / kRouteChunk;
  return (size_t)(((nch * E * 4) + 255) / 256 * 256);
}

hipError_t launch_route(const float* logits, const float* bias, int64_t T, int E, int K, int score,
                        int renorm, int32_t* topk_idx, float* topk_gate, int32_t* counts,
                        int32_t* offsets, int32_t* slot_pos, int32_t* row_src, void* ws,
                        hipStream_t s) {
  const int nch = (int)((T + kRouteChunk - 1) / kRouteChunk);
  int32_t* hist = (int32_t*)ws;
  if (nch > 0) {
    int P = 1;
    while (P < E) P <<= 1;
    const int vec4 = (E % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0);
#define MOE_TOPK_CASE(p, g, kpl)                                                                 \
  case p:                                                                                        \
    hipLaunchKernelGGL((route_topk_kernel<g, kpl>), dim3(nch), dim3(kTopkThreads), 0, s, logits, \
                       bias, (int)T, E, K, score, renorm, vec4, topk_idx, topk_gate, slot_pos,   \
                       hist);                                                                    \
    break;
    switch (P) {
      MOE_TOPK_CASE(1, 1, 1)
      MOE_TOPK_CASE(2, 1, 2)
      MOE_TOPK_CASE(4, 1, 4)
      MOE_TOPK_CASE(8, 1, 8)
      MOE_TOPK_CASE(16, 1, 16)
      MOE_TOPK_CASE(32, 2, 16)
      MOE_TOPK_CASE(64, 4, 16)
      MOE_TOPK_CASE(128, 8, 16)
      MOE_TOPK_CASE(256, 16, 16)
      default:
        return hipErrorInvalidValue;
    }
#undef MOE_TOPK_CASE
  }
  return launch_route_scan_finalize(hist, nch, kRouteChunk, T, E, K, topk_idx, counts, offsets, slot_pos, row_src,
                                    s);
}

hipError_t launch_route_scan_finalize(int32_t* hist, int nch, int chunk, int64_t T, int E, int K,
                                      const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                                      int32_t* slot_pos, int32_t* row_src, hipStream_t s) {
  // chunks a thread scans (as the kernel splits them): more than 16 take the deeper register run
  const int nparts = std::min(kScanParts, kScanThreads / E);
  if ((nch + nparts - 1) / nparts > 16)
    hipLaunchKernelGGL(route_scan_kernel<32>, dim3(1), dim3(kScanThreads), 0, s, hist, nch, E, counts, offsets);
  else
    hipLaunchKernelGGL(route_scan_kernel<16>, dim3(1), dim3(kScanThreads), 0, s, hist, nch, E, counts, offsets);
  const int64_t M = T * K;
  if (M > 0) {
    hipLaunchKernelGGL(route_finalize_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s,
                       topk_idx, hist, offsets, M, K, E, chunk, slot_pos, row_src);
  }
  return hipGetLastError();
}

}  // namespace moe
