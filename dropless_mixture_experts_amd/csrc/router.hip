// Router logits: logits[t, e] = x[t, :] . w_router[e, :] with fp32 accumulation.
//
// The learned router scores every expert for every token (page "Accelerating
// dropless MoE training in JAX with NVIDIA Transformer Engine", introduction).
// With E <= 256 this product is a skinny GEMM whose cost is reading x once, so
// it is shaped for HBM bandwidth.
//
// bf16 (router_ring_kernel): a workgroup owns 64 tokens and all experts.  Stages
// of 64 d-elements of its x rows and of every W row go straight from global
// memory into an LDS ring with global_load_lds_dwordx4 (whole 128-byte row
// pieces, no registers spent), as many stages deep as LDS holds, so that enough
// of x is in flight to cover HBM latency; W (at most 0.5 MB) is re-read from L2
// once per 64 tokens.  The 4 waves split the experts when there are 128 or more
// and otherwise also the d axis of each stage, summing their partial tiles
// through LDS at the end.  32x32x16 MFMA tiles; d past the last whole stage is
// read as zeros.
//
// fp32 (router_logits_kernel): a workgroup owns 32 tokens, its 4 waves split
// the d axis, and each wave runs 32x32 MFMA tiles (one per 32 experts) fed
// straight from global memory; the 4 partial tiles are summed through LDS.
#include <mutex>

#include "../../include/moe.h"
#include "common.h"
#include "internal.h"
#include "route_device.h"

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

namespace rring {

constexpr int kThreads = 256;
constexpr int kRowBytes = 128;    // bytes of one row in one stage (64 bf16)
constexpr int kLdsBytes = 160 * 1024;

// 16-byte chunk XOR of a 128-byte LDS row: 16 consecutive rows at one logical
// chunk land in 16 distinct 16-byte bank groups
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// 16 bytes per lane from a per-lane global address into LDS at M0 + 16 * lane
__device__ __forceinline__ void dma(const void* gptr, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_byte), "v"(gptr) : "memory", "m0");
}

// wait until at most N of this wave's vector memory operations are outstanding,
// and for every LDS access
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" :: "n"(N) : "memory");
}
template <int NQ, int A>
__device__ __forceinline__ void wait_ahead(int ahead) {
  if constexpr (A <= 0) {
    wait_vm_lgkm0<0>();
  } else {
    if (ahead >= A) {
      wait_vm_lgkm0<A * NQ>();
      return;
    }
    wait_ahead<NQ, A - 1>(ahead);
  }
}

__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ const uint4 kZeroChunk = {0u, 0u, 0u, 0u};  // source of the d tail past the row end

// TT = token tiles of 32 (the workgroup's tokens), NF = expert tiles of 32
// (E <= 32 NF), D = ring stages, SPB = stages per barrier (D >= 2 SPB).  Waves: NE groups
// over the expert tiles (NFW each) x NKS over the four 16-element k steps of a stage.
// A barrier publishes SPB landed stages at once and frees the SPB slots read before it, which
// are refilled right after it; the ring then holds D - 2 SPB stages in flight beyond them.
// FUSE: after the product, the tile's logits stay in LDS and the same workgroup routes its
// tokens there (top-K, scores, gates, the tile's expert histogram and in-tile ranks; G lanes
// of KPL keys per token), so that the logits need not return from HBM (they are still written
// when `logits` is given).
template <int TT, int NF, int D, int SPB, bool FUSE = false, int G = 1, int KPL = 1>
__global__ __launch_bounds__(kThreads) void router_ring_kernel(const bf16_t* __restrict__ x,
                                                               const bf16_t* __restrict__ w,
                                                               int64_t T_, int64_t d, int E,
                                                               float* __restrict__ logits,
                                                               const float* __restrict__ bias = nullptr,
                                                               int K = 0, int score = 0, int renorm = 0,
                                                               int32_t* __restrict__ topk_idx = nullptr,
                                                               float* __restrict__ topk_gate = nullptr,
                                                               int32_t* __restrict__ local_rank = nullptr,
                                                               int32_t* __restrict__ hist = nullptr) {
  constexpr int EP = NF * 32;
  constexpr int NE = NF < 4 ? NF : 4;
  constexpr int NKS = 4 / NE;
  constexpr int NFW = NF / NE;
  constexpr int kBT = 32 * TT;
  constexpr int NQ = TT + NF;  // DMA instructions of a wave per stage: TT of x, NF of W
  constexpr int kSlotBytes = (kBT + EP) * kRowBytes;
  static_assert(NE * NKS == 4 && NE * NFW == NF, "wave split");
  static_assert(D >= 2 && D * kSlotBytes <= kLdsBytes, "ring size");
  static_assert(SPB >= 1 && D >= 2 * SPB, "a barrier's stages and the ones refilled after it");
  __shared__ uint4 smem[D * kSlotBytes / 16];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l32 = lane & 31, hi = lane >> 5;
  const int eg = wave % NE, ks = wave / NE;
  const int64_t t0 = (int64_t)blockIdx.x * kBT;
  const int64_t dbytes = d * 2;
  const int nk = (int)((dbytes + kRowBytes - 1) / kRowBytes);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)smem);

  // this wave's DMA instructions: x rows 8 (TT wave + q) .. +7, W rows 8 (NF wave + q) .. +7;
  // lane L fills row L / 8, physical chunk L % 8, which holds logical chunk c
  const char* src[NQ];
  uint32_t cbyte[NQ];
  uint32_t ldsoff[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const bool isx = q < TT;
    const int row = (isx ? (TT * wave + q) : (NF * wave + (q - TT))) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(row);
    int64_t grow;
    if (isx) {
      grow = t0 + row;
      grow = grow < T_ ? grow : T_ - 1;
      src[q] = (const char*)x + grow * dbytes + c * 16;
    } else {
      grow = row < E ? row : E - 1;
      src[q] = (const char*)w + grow * dbytes + c * 16;
    }
    cbyte[q] = (uint32_t)(c * 16);
    ldsoff[q] = (uint32_t)((isx ? 0 : kBT * kRowBytes) + (row & ~7) * kRowBytes);
  }
  auto issue = [&](int s) {
    const uint32_t slot = lds0 + (uint32_t)((s % D) * kSlotBytes);
    const int64_t kb = (int64_t)s * kRowBytes;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const void* g = (kb + cbyte[q] < dbytes) ? (const void*)(src[q] + kb) : (const void*)&kZeroChunk;
      dma(g, __builtin_amdgcn_readfirstlane(slot + ldsoff[q]));
    }
  };

  // fragment offsets inside a slot: x rows tt * 32 + l32, W rows (eg NFW + f) * 32 + l32
  uint32_t aoff[TT], boff[NFW];
  int aswz[TT], bswz[NFW];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int r = tt * 32 + l32;
    aoff[tt] = (uint32_t)(r * kRowBytes);
    aswz[tt] = swz(r);
  }
#pragma unroll
  for (int f = 0; f < NFW; ++f) {
    const int r = (eg * NFW + f) * 32 + l32;
    boff[f] = (uint32_t)(kBT * kRowBytes + r * kRowBytes);
    bswz[f] = swz(r);
  }

  f32x16 acc[TT][NFW];
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int f = 0; f < NFW; ++f)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[tt][f][r] = 0.f;

#pragma unroll
  for (int s = 0; s < D - SPB; ++s)
    if (s < nk) issue(s);
  const char* lbase = (const char*)smem;
  for (int s = 0; s < nk; s += SPB) {
    // stages s .. s + SPB - 1 landed (at most D - 2 SPB later stages still in flight)
    wait_ahead<NQ, D - 2 * SPB>(max(0, min(nk - s - SPB, D - 2 * SPB)));
    barrier();  // ... for every wave; the slots of stages s - SPB .. s - 1 are read by none
#pragma unroll
    for (int u = 0; u < SPB; ++u)
      if (s + D - SPB + u < nk) issue(s + D - SPB + u);
#pragma unroll
    for (int u = 0; u < SPB; ++u) {
      if (s + u >= nk) break;
      const char* slot = lbase + ((s + u) % D) * kSlotBytes;
#pragma unroll
      for (int j = 0; j < 4 / NKS; ++j) {
        const int c = 2 * (ks + j * NKS) + hi;  // logical chunk of this lane's 8 k values
        uint4 a[TT], b[NFW];
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) a[tt] = *(const uint4*)(slot + aoff[tt] + ((c ^ aswz[tt]) << 4));
#pragma unroll
        for (int f = 0; f < NFW; ++f) b[f] = *(const uint4*)(slot + boff[f] + ((c ^ bswz[f]) << 4));
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
#pragma unroll
          for (int f = 0; f < NFW; ++f)
            acc[tt][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[tt]),
                                                                __builtin_bit_cast(bf16x8, b[f]),
                                                                acc[tt][f], 0, 0, 0);
      }
    }
  }

  if constexpr (NKS > 1) {
    // partial tiles of k groups 1 .. NKS-1 through the (now idle) ring
    __syncthreads();
    float* red = (float*)smem;
    if (ks > 0) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int f = 0; f < NFW; ++f)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            red[((((ks - 1) * NE + eg) * TT + tt) * NFW + f) * 1024 + r * 64 + lane] = acc[tt][f][r];
    }
    __syncthreads();
    if constexpr (!FUSE) {
      if (ks > 0) return;
    }
#pragma unroll
    for (int k2 = 1; k2 < NKS; ++k2)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int f = 0; f < NFW; ++f)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[tt][f][r] += red[((((k2 - 1) * NE + eg) * TT + tt) * NFW + f) * 1024 + r * 64 + lane];
  }
  if constexpr (!FUSE) {
#pragma unroll
    for (int tt = 0; tt < TT; ++tt)
#pragma unroll
      for (int f = 0; f < NFW; ++f) {
        const int e = (eg * NFW + f) * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t t = t0 + tt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (t < T_ && e < E) logits[t * E + e] = acc[tt][f][r];
        }
      }
  } else {
    using namespace rdev;
    // LDS of the idle ring: logits [kBT][EP] fp32, then the routing scratch
    constexpr int kLogBytes = kBT * EP * 4;
    constexpr int kSelOff = kLogBytes;
    constexpr int kRankOff = kSelOff + kBT * kMaxTopK;
    constexpr int kScoreOff = kRankOff + kBT * kMaxTopK * 2;
    constexpr int kBiasOff = kScoreOff + kBT * kMaxTopK * 4;
    constexpr int kCntOff = kBiasOff + kMaxExperts * 4;
    static_assert(kCntOff + 4 * kMaxExperts * 4 <= D * kSlotBytes, "routing scratch fits the ring");
    static_assert(G * KPL >= EP || G * KPL >= 8, "a token's lanes hold its keys");
    char* lds = (char*)smem;
    float* s_log = (float*)lds;
    uint8_t* s_sel = (uint8_t*)(lds + kSelOff);
    uint16_t* s_rank = (uint16_t*)(lds + kRankOff);
    float* s_score = (float*)(lds + kScoreOff);
    float* s_bias = (float*)(lds + kBiasOff);
    int(*s_cnt)[kMaxExperts] = (int(*)[kMaxExperts])(lds + kCntOff);
    __syncthreads();  // every wave is done with the ring and with the partial tiles
    if (ks == 0) {
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
#pragma unroll
        for (int f = 0; f < NFW; ++f) {
          const int e = (eg * NFW + f) * 32 + l32;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int tl = tt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            s_log[tl * EP + e] = acc[tt][f][r];
            const int64_t t = t0 + tl;
            if (logits && t < T_ && e < E) logits[t * E + e] = acc[tt][f][r];
          }
        }
    }
    if (bias)
      for (int e = threadIdx.x; e < E; e += kThreads) s_bias[e] = bias[e];
    __syncthreads();
    const int tid = threadIdx.x;
    const int lig = tid & (G - 1);
    const int e_lo = lig * KPL;
    const int ntok = (int)min((int64_t)kBT, T_ - t0);
    for (int tl = tid / G; tl < ntok; tl += kThreads / G) {
      float kf[KPL];
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int e = e_lo + j;
        float v = -INFINITY;
        if (e < E) {
          v = s_log[tl * EP + e];
          if (bias) v = v + s_bias[e];
        }
        kf[j] = v;
      }
      select_token<G, KPL>(kf, e_lo, E, K, score, renorm, lig, t0 + tl, tl, s_sel, s_score, topk_idx, topk_gate);
    }
    __syncthreads();
    rank_chunk<kThreads / 64>(ntok * K, E, s_sel, s_rank, s_cnt, hist + (int64_t)blockIdx.x * E,
                              local_rank + t0 * K);
  }
}

}  // namespace rring

// Stages per barrier of each ring shape (tokens x experts x depth): 1x32x16, 2x32x8, 1x64x13,
// 2x64x10, 2x128x6, 2x256x4.  Measured with the caches flushed: four stages a barrier make the
// 32-token, 8-expert ring (the Mixtral shape) 4% faster; two stages left the 64-token rings
// unchanged (32 experts) or 2% slower (128 experts), so those keep one.
#define SPB_A 4
#define SPB_B 1
#define SPB_C 1
#define SPB_D 1
#define SPB_E 1
#define SPB_F 1

// 32-token workgroups when few experts leave fewer than about 1.5 workgroups of
// 64 tokens per CU, so that every CU streams x; deeper rings where stages are small.
hipError_t router_ring(const void* x, const void* w, int64_t T_, int64_t d, int E, float* logits,
                       hipStream_t s) {
  using namespace rring;
  const bf16_t* xb = (const bf16_t*)x;
  const bf16_t* wb = (const bf16_t*)w;
  const int nf = (E + 31) / 32;
  const bool small_t = (T_ + 63) / 64 < 384;
#define MOE_ROUTER_RING(tt, nfe, depth, spb)                                                    \
  hipLaunchKernelGGL((router_ring_kernel<tt, nfe, depth, spb>), dim3((unsigned)((T_ + 32 * tt - 1) / (32 * tt))), \
                     dim3(kThreads), 0, s, xb, wb, T_, d, E, logits)
  if (nf <= 1) {
    if (small_t) MOE_ROUTER_RING(1, 1, 16, SPB_A);
    else MOE_ROUTER_RING(2, 1, 8, SPB_B);
  } else if (nf <= 2) {
    if (small_t) MOE_ROUTER_RING(1, 2, 13, SPB_C);
    else MOE_ROUTER_RING(2, 2, 10, SPB_D);
  } else if (nf <= 4) {
    MOE_ROUTER_RING(2, 4, 6, SPB_E);
  } else {
    MOE_ROUTER_RING(2, 8, 4, SPB_F);
  }
#undef MOE_ROUTER_RING
  return hipGetLastError();
}

// Tokens per workgroup of the fused router: the same choice as the router product's.
int router_route_chunk(int64_t T_, int E) {
  const int nf = (E + 31) / 32;
  return (nf <= 2 && (T_ + 63) / 64 < 384) ? 32 : 64;
}

hipError_t router_route(const void* x, const void* w, const float* bias, int64_t T_, int64_t d, int E, int K,
                        int score, int renorm, float* logits, int32_t* topk_idx, float* topk_gate,
                        int32_t* counts, int32_t* offsets, int32_t* slot_pos, int32_t* row_src, void* ws,
                        hipStream_t s) {
  using namespace rring;
  const bf16_t* xb = (const bf16_t*)x;
  const bf16_t* wb = (const bf16_t*)w;
  const int nf = (E + 31) / 32;
  const int chunk = router_route_chunk(T_, E);
  const int nch = (int)((T_ + chunk - 1) / chunk);
  int32_t* hist = (int32_t*)ws;
  if (nch > 0) {
    const dim3 grid((unsigned)nch);
#define MOE_ROUTER_FUSED(tt, nfe, depth, spb, g, kpl)                                                   \
  hipLaunchKernelGGL((router_ring_kernel<tt, nfe, depth, spb, true, g, kpl>), grid, dim3(kThreads), 0, s, xb, wb, \
                     T_, d, E, logits, bias, K, score, renorm, topk_idx, topk_gate, slot_pos, hist)
    if (nf <= 1) {
      if (chunk == 32) {
        if (E <= 8) MOE_ROUTER_FUSED(1, 1, 16, SPB_A, 1, 8);
        else if (E <= 16) MOE_ROUTER_FUSED(1, 1, 16, SPB_A, 1, 16);
        else MOE_ROUTER_FUSED(1, 1, 16, SPB_A, 2, 16);
      } else {
        if (E <= 8) MOE_ROUTER_FUSED(2, 1, 8, SPB_B, 1, 8);
        else if (E <= 16) MOE_ROUTER_FUSED(2, 1, 8, SPB_B, 1, 16);
        else MOE_ROUTER_FUSED(2, 1, 8, SPB_B, 2, 16);
      }
    } else if (nf <= 2) {
      if (chunk == 32) MOE_ROUTER_FUSED(1, 2, 13, SPB_C, 4, 16);
      else MOE_ROUTER_FUSED(2, 2, 10, SPB_D, 4, 16);
    } else if (nf <= 4) {
      MOE_ROUTER_FUSED(2, 4, 6, SPB_E, 8, 16);
    } else {
      MOE_ROUTER_FUSED(2, 8, 4, SPB_F, 16, 16);
    }
#undef MOE_ROUTER_FUSED
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_route_scan_finalize(hist, nch, chunk, T_, E, K, topk_idx, counts, offsets, slot_pos, row_src, s);
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

size_t router_route_workspace_bytes(int64_t T, int E) {
  const int64_t nch = (T + 31) / 32;  // the smallest chunk the fused router uses
  return (size_t)(((nch * E * 4) + 255) / 256 * 256);
}

hipError_t launch_router_route(const void* x, const void* w, const float* bias, int64_t T, int64_t d, int E, int K,
                               int score, int renorm, float* logits, int32_t* topk_idx, float* topk_gate,
                               int32_t* counts, int32_t* offsets, int32_t* slot_pos, int32_t* row_src, void* ws,
                               hipStream_t s) {
  return router_route(x, w, bias, T, d, E, K, score, renorm, logits, topk_idx, topk_gate, counts, offsets, slot_pos,
                      row_src, ws, s);
}

// The allocation-free fused router's workspace: one static device array per device (each
// device that loads the library holds its own copy at its own address until the process
// ends).  In host code `scratch` names a host-side stand-in, not device memory: its device
// address is looked up once per device with hipGetSymbolAddress, and only that address is
// ever handed to a kernel.
static __device__ __align__(256) int32_t scratch[MOE_ROUTER_ROUTE_NOALLOC_MAX_BYTES / sizeof(int32_t)];

namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
}  // namespace

hipError_t launch_router_route_noalloc(const void* x, const void* w, const float* bias, int64_t T, int64_t d, int E,
                                       int K, int score, int renorm, float* logits, int32_t* topk_idx,
                                       float* topk_gate, int32_t* counts, int32_t* offsets, int32_t* slot_pos,
                                       int32_t* row_src, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  if (g_scratch_ptr[dev] == nullptr) return hipErrorInvalidSymbol;
  return router_route(x, w, bias, T, d, E, K, score, renorm, logits, topk_idx, topk_gate, counts, offsets, slot_pos,
                      row_src, g_scratch_ptr[dev], s);
}

hipError_t launch_router_logits(const void* x, const void* w, int64_t T, int64_t d, int E, int dtype,
                                float* logits, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (dtype == 1) return router_ring(x, w, T, d, E, logits, s);
  return router_t<float>(x, w, T, d, E, logits, s);
}

}  // namespace moe
