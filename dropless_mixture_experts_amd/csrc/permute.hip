// Dispatch (permute) and combine (unpermute + gate-weighted sum) on one GPU.
//
// Tokens move into expert-contiguous order before the grouped MLP and come
// back to their original order afterwards (page "Accelerating dropless MoE
// training in JAX with NVIDIA Transformer Engine", Figure 3 paragraph of
// "What specialised optimisations does dropless MoE need?").  Both are pure
// HBM streams over token rows: one wave per token (two, each with half the row, when rows
// hold 512 or more 16-byte vectors and no dot product is formed) moves whole rows with
// 16-byte lanes, so every row is read once and written once as full 64-byte segments.
// Measured with the caches flushed before each launch, on the three workload shapes:
// non-temporal stores cost 5-25% everywhere, so every output is written with ordinary
// stores; combine reads its gathered rows non-temporally (2-4% faster than ordinary
// loads except on one shape); a 4096-wide bf16 row moves in passes of 4 vectors per lane
// (3% faster than 8), shorter rows in one pass of 8; two waves a wide token were 1-4%
// faster than one for combine and for the 7168-wide permute, the same for the 4096-wide
// permute (eleven variants of lanes, waves and rows in flight per token were all within
// 3% of each other).
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kRowsPerBlock = 4;  // one wave per row
constexpr int kCUnroll = 8;  // 16-byte vectors per lane per gathered row (combine)

// x_perm[slot_pos[s]] = (scale_s *) x[t] for the K slots s = t K + k of token t; optional
// dgate_s = <x[t], ydot[slot_pos[s]]>.  One wave per token, so each token row is read from
// HBM once and written to its K rows.  Without the dot, every loaded piece of the row goes
// straight to all K rows; with it, the slots are taken one by one (the row comes back from
// the cache) so that each slot's dot product is a single wave reduction.
// UN: 16-byte vectors in flight per lane per pass over the row.  SPLIT (without the dot):
// waves a token, each moving a contiguous 1/SPLIT of the row.
template <typename T, bool SCALE, bool DOT, int UN = 8, int SPLIT = 1>
__global__ __launch_bounds__(256) void permute_kernel(const uint4* __restrict__ x, int64_t nvec, int K,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ row_scale,
                                                      const uint4* __restrict__ ydot,
                                                      float* __restrict__ dgate,
                                                      uint4* __restrict__ xp, int64_t ntok) {
  static_assert(SPLIT == 1 || !DOT, "the dot product needs the whole row in one wave");
  using E = Elem<T>;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int64_t t = w / SPLIT;
  if (t >= ntok) return;
  const int64_t seg = (nvec + SPLIT - 1) / SPLIT;
  const int64_t beg = (w % SPLIT) * seg, end = beg + seg < nvec ? beg + seg : nvec;
  const int64_t M = ntok * K;
  // lane k holds slot k's destination row and scale (K <= 32)
  int pos = 0;
  float sk = 1.f;
  if (lane < K) {
    pos = slot_pos[t * K + lane];
    pos = pos < 0 ? 0 : (pos >= M ? (int)(M - 1) : pos);  // never leave the buffers
    if (SCALE) sk = row_scale[t * K + lane];
  }
  const uint4* src = x + t * nvec;
  if constexpr (!DOT) {
    for (int64_t i0 = beg; i0 < end; i0 += 64 * UN) {
      uint4 v[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int64_t i = i0 + u * 64 + lane;
        if (i < end) v[u] = src[i];
      }
      for (int k = 0; k < K; ++k) {
        const int64_t p = __shfl(pos, k, 64);
        const float sc = __shfl(sk, k, 64);
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const int64_t i = i0 + u * 64 + lane;
          if (i < end) {
            uint4 o = v[u];
            if (SCALE) {
              float f[E::kVec];
              E::to_f32(v[u], f);
#pragma unroll
              for (int q = 0; q < E::kVec; ++q) f[q] *= sc;
              o = E::from_f32(f);
            }
            xp[p * nvec + i] = o;
          }
        }
      }
    }
  } else {
    for (int k = 0; k < K; ++k) {
      const int64_t p = __shfl(pos, k, 64);
      const float sc = __shfl(sk, k, 64);
      const uint4* yd = ydot + p * nvec;
      float dot = 0.f;
      for (int64_t i0 = 0; i0 < nvec; i0 += 64 * UN) {
        uint4 v[UN], w[UN];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const int64_t i = i0 + u * 64 + lane;
          if (i < nvec) {
            v[u] = src[i];  // read once from HBM, again from the cache for the other slots
            w[u] = ld_nt(yd + i);
          }
        }
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const int64_t i = i0 + u * 64 + lane;
          if (i < nvec) {
            float f[E::kVec], g[E::kVec];
            E::to_f32(v[u], f);
            E::to_f32(w[u], g);
#pragma unroll
            for (int q = 0; q < E::kVec; ++q) dot += f[q] * g[q];
            uint4 o = v[u];
            if (SCALE) {
#pragma unroll
              for (int q = 0; q < E::kVec; ++q) f[q] *= sc;
              o = E::from_f32(f);
            }
            xp[p * nvec + i] = o;
          }
        }
      }
      dot = wave_sum(dot);
      if (lane == 0) dgate[t * K + k] = dot;
    }
  }
}

// y[t] = sum_k g_tk * y_perm[slot_pos[t*K + k]], fp32 in ascending k, rounded once.
// SPLIT waves share a token, each taking a contiguous 1/SPLIT of the row; UN: 16-byte vectors
// in flight per lane per gathered row.
template <typename T, bool GATES, int SPLIT = 1, int UN = kCUnroll>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ yp,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ gates, int64_t ntok,
                                                      int64_t nvec, int K, uint4* __restrict__ y) {
  using E = Elem<T>;
  const int lane = threadIdx.x & 63;
  const int64_t w = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  const int64_t t = w / SPLIT;
  if (t >= ntok) return;
  const int64_t seg = (nvec + SPLIT - 1) / SPLIT;
  const int64_t beg = (w % SPLIT) * seg, end = beg + seg < nvec ? beg + seg : nvec;
  // lane k holds slot k's row and gate (K <= 32)
  int pos = 0;
  float gk = 1.f;
  const int64_t M = ntok * K;
  if (lane < K) {
    pos = slot_pos[t * K + lane];
    pos = pos < 0 ? 0 : (pos >= M ? (int)(M - 1) : pos);
    if (GATES) gk = gates[t * K + lane];
  }
  for (int64_t i0 = beg; i0 < end; i0 += 64 * UN) {
    float acc[UN][E::kVec];
#pragma unroll
    for (int u = 0; u < UN; ++u)
#pragma unroll
      for (int q = 0; q < E::kVec; ++q) acc[u][q] = 0.f;
    // two gathered rows per step: their loads are in flight together
    for (int k = 0; k < K; k += 2) {
      const bool two = k + 1 < K;
      const int64_t p0 = __shfl(pos, k, 64), p1 = __shfl(pos, two ? k + 1 : k, 64);
      const float g0 = __shfl(gk, k, 64), g1 = __shfl(gk, two ? k + 1 : k, 64);
      uint4 v0[UN], v1[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int64_t i = i0 + u * 64 + lane;
        if (i < end) {
          v0[u] = ld_nt(yp + p0 * nvec + i);
          if (two) v1[u] = ld_nt(yp + p1 * nvec + i);
        }
      }
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int64_t i = i0 + u * 64 + lane;
        if (i < end) {
          float f[E::kVec];
          E::to_f32(v0[u], f);
#pragma unroll
          for (int q = 0; q < E::kVec; ++q) acc[u][q] = fmaf(g0, f[q], acc[u][q]);
          if (two) {
            E::to_f32(v1[u], f);
#pragma unroll
            for (int q = 0; q < E::kVec; ++q) acc[u][q] = fmaf(g1, f[q], acc[u][q]);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int64_t i = i0 + u * 64 + lane;
      if (i < end) y[t * nvec + i] = E::from_f32(acc[u]);
    }
  }
}

template <typename T>
hipError_t permute_t(const void* x, int64_t T_, int64_t d, int K, const int32_t* slot_pos,
                     const float* row_scale, const void* ydot, float* dgate, void* xp, hipStream_t s) {
  if (T_ == 0) return hipSuccess;
  const int64_t nvec = d / Elem<T>::kVec;
  const dim3 grid((unsigned)((T_ + kRowsPerBlock - 1) / kRowsPerBlock));
  const uint4* xv = (const uint4*)x;
  const uint4* yv = (const uint4*)ydot;
  uint4* o = (uint4*)xp;
  const bool dot = ydot != nullptr && dgate != nullptr;
  if (row_scale && dot)
    hipLaunchKernelGGL((permute_kernel<T, true, true>), grid, dim3(256), 0, s, xv, nvec, K, slot_pos,
                       row_scale, yv, dgate, o, T_);
  else if (row_scale)
    hipLaunchKernelGGL((permute_kernel<T, true, false>), grid, dim3(256), 0, s, xv, nvec, K, slot_pos,
                       row_scale, yv, dgate, o, T_);
  else if (dot)
    hipLaunchKernelGGL((permute_kernel<T, false, true>), grid, dim3(256), 0, s, xv, nvec, K, slot_pos,
                       row_scale, yv, dgate, o, T_);
  else if (nvec > 512)
    hipLaunchKernelGGL((permute_kernel<T, false, false, 8, 2>), dim3((unsigned)((2 * T_ + kRowsPerBlock - 1) / kRowsPerBlock)),
                       dim3(256), 0, s, xv, nvec, K, slot_pos, row_scale, yv, dgate, o, T_);
  else if (nvec == 512)
    hipLaunchKernelGGL((permute_kernel<T, false, false, 4, 2>), dim3((unsigned)((2 * T_ + kRowsPerBlock - 1) / kRowsPerBlock)),
                       dim3(256), 0, s, xv, nvec, K, slot_pos, row_scale, yv, dgate, o, T_);
  else
    hipLaunchKernelGGL((permute_kernel<T, false, false>), grid, dim3(256), 0, s, xv, nvec, K, slot_pos,
                       row_scale, yv, dgate, o, T_);
  return hipGetLastError();
}

template <typename T>
hipError_t combine_t(const void* yp, const int32_t* slot_pos, const float* gates, int64_t T_, int64_t d,
                     int K, void* y, hipStream_t s) {
  if (T_ == 0) return hipSuccess;
  const int64_t nvec = d / Elem<T>::kVec;
  // rows of 512 or more 16-byte vectors: two waves a token (more waves in flight for the same
  // bytes), each with up to 8 vectors a lane per gathered row
  const bool wide = nvec >= 512;
  const int64_t waves = wide ? 2 * T_ : T_;
  const dim3 grid((unsigned)((waves + kRowsPerBlock - 1) / kRowsPerBlock));
#define MOE_COMBINE(G_, S_, U_)                                                                             \
  hipLaunchKernelGGL((combine_kernel<T, G_, S_, U_>), grid, dim3(256), 0, s, (const uint4*)yp, slot_pos, gates, \
                     T_, nvec, K, (uint4*)y)
  if (gates) {
    if (wide && nvec <= 512) MOE_COMBINE(true, 2, 4);
    else if (wide) MOE_COMBINE(true, 2, 8);
    else MOE_COMBINE(true, 1, kCUnroll);
  } else {
    if (wide && nvec <= 512) MOE_COMBINE(false, 2, 4);
    else if (wide) MOE_COMBINE(false, 2, 8);
    else MOE_COMBINE(false, 1, kCUnroll);
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace

hipError_t launch_permute(const void* x, int64_t T, int64_t d, int K, int dtype, const int32_t* slot_pos,
                          const float* row_scale, const void* y_perm_dot, float* dgate_out,
                          void* x_perm, hipStream_t s) {
  if (dtype == 1)
    return permute_t<bf16_t>(x, T, d, K, slot_pos, row_scale, y_perm_dot, dgate_out, x_perm, s);
  return permute_t<float>(x, T, d, K, slot_pos, row_scale, y_perm_dot, dgate_out, x_perm, s);
}

// Permute of MXFP8 rows: the same row copy as the plain permute, over rows of `row_bytes`
// bytes (a multiple of 16) of codes, then of scales.
hipError_t launch_permute_rows(const void* x, int64_t T, int64_t row_bytes, int K, const int32_t* slot_pos,
                               void* x_perm, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((T + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL((permute_kernel<bf16_t, false, false>), grid, dim3(256), 0, s, (const uint4*)x, row_bytes / 16,
                     K, slot_pos, nullptr, nullptr, nullptr, (uint4*)x_perm, T);
  return hipGetLastError();
}

hipError_t launch_combine(const void* y_perm, const int32_t* slot_pos, const float* gates, int64_t T,
                          int64_t d, int K, int dtype, void* y, hipStream_t s) {
  if (dtype == 1) return combine_t<bf16_t>(y_perm, slot_pos, gates, T, d, K, y, s);
  return combine_t<float>(y_perm, slot_pos, gates, T, d, K, y, s);
}

}  // namespace moe
