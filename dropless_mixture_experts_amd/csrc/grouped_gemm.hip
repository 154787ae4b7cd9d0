// Grouped GEMM over variable-length expert groups, and its weight gradient.
//
// Page "Accelerating dropless MoE training in JAX with NVIDIA Transformer
// Engine", "Optimisation 1: Grouped GEMM": all expert matmuls run in one
// kernel call, each at its actual token count, computing only the regions
// that hold valid tokens; the group sizes are never copied to the host, so
// the launch shape is fixed and the call can be captured in a graph.
//
// gfx950 design
//   * 256x256 output tile per workgroup of 4 waves (2x2), 128x128 per wave,
//     accumulated in 16 v_mfma_f32_32x32x16_bf16 tiles (v_mfma_f32_32x32x2_f32
//     for fp32 inputs).
//   * K is staged through LDS 128 bytes per row at a time, two stages
//     (2 x 64 KB); rows are 8 chunks of 16 bytes with the chunk index XORed by
//     (row & 7), so both the 16-byte LDS writes and the MFMA operand reads hit
//     distinct banks.  The next stage's global loads are in flight while the
//     current stage is multiplied.
//   * Operands stored K-contiguous are copied chunk for chunk; operands stored
//     with K as the row index (the K-by-N weight layout of the data-gradient
//     GEMMs, and both operands of the weight gradient) are read as 8x8 (bf16)
//     or 4x4 (fp32) blocks and transposed in registers before the LDS write.
//   * Each workgroup finds its (group, row tile, column tile) from the group
//     offsets in device memory.  The grid is an upper bound computed on the
//     host; surplus workgroups exit.  Consecutive tiles go to one XCD in
//     contiguous runs and, within a run, 8 row tiles share each column tile,
//     so concurrently running tiles share operands in that XCD's L2.
//   * Epilogues: plain store; SwiGLU (gate and up columns of one output column
//     live in the same lane); SwiGLU backward using the saved pre-activations.
#include "common.h"
#include "internal.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 256;                 // BM = BN
constexpr int kRowBytes = 128;             // K bytes per LDS row per stage
constexpr int kCPR = kRowBytes / 16;       // 16-byte chunks per LDS row
constexpr int kTileChunks = kTile * kCPR;  // chunks per operand stage (32 KB)
constexpr int kXcd = 8;                    // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kGroupM = 8;                 // row tiles that share a column tile

enum { EPI_NONE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2 };
enum { LAYOUT_NK = 0, LAYOUT_KN = 1 };

__device__ __forceinline__ int swz(int row, int c) { return row * kCPR + (c ^ (row & 7)); }

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  __device__ __forceinline__ static void run(const uint4& a, const uint4& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  __device__ __forceinline__ static void run(const uint4& a, const uint4& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
  }
};

// ---------------------------------------------------------------------------
// Loader of an operand whose rows are K-contiguous: LDS row r <- global row ptr_r.
// Thread tid moves chunk (tid & 7) of rows (tid >> 3) + 32 i, i < 8.
struct RowLoader {
  const char* ptr[8];  // start of each row (K offset 0)
  int64_t kbytes;  // K extent in bytes
  int c;
  uint4 reg[8];

  __device__ __forceinline__ void load(int stage) {
    const int64_t off = (int64_t)stage * kRowBytes + c * 16;
    const bool ok = off < kbytes;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      reg[i] = ok ? *(const uint4*)(ptr[i] + off) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void store(uint4* lds) const {
    const int r0 = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) lds[swz(r0 + 32 * i, c)] = reg[i];
  }
};

// Loader of an operand stored [k][n] (n contiguous) whose LDS tile is [n][k]:
// blocks of VE x VE elements are read as VE 16-byte rows and transposed.
template <typename T>
struct ColLoader {
  static constexpr int VE = Elem<T>::kVec;      // elements per 16 bytes
  static constexpr int NB = kTile / VE;         // blocks along n
  static constexpr int PB = NB * 8 / kThreads;  // blocks per thread (8 blocks along k)
  const char* base;   // element (k = 0, n = 0) of this operand
  int64_t ld;         // row pitch in bytes
  int64_t n0;         // first column (LDS row) of the tile
  int64_t k_begin, k_end;
  int n_valid[PB];    // n-block in range
  int nb[PB], kb[PB];
  uint4 reg[PB][VE];

  __device__ __forceinline__ void init(const void* b, int64_t ld_elems, int64_t n_first, int64_t ncols,
                                       int64_t kbeg, int64_t kend) {
    base = (const char*)b;
    ld = ld_elems * Elem<T>::kBytes;
    n0 = n_first;
    k_begin = kbeg;
    k_end = kend;
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int q = threadIdx.x + kThreads * p;
      nb[p] = q % NB;
      kb[p] = q / NB;
      n_valid[p] = n0 + (int64_t)nb[p] * VE < ncols;
    }
  }

  __device__ __forceinline__ void load(int stage) {
    constexpr int BK = kRowBytes / Elem<T>::kBytes;
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int64_t n = n0 + (int64_t)nb[p] * VE;
#pragma unroll
      for (int v = 0; v < VE; ++v) {
        const int64_t k = k_begin + (int64_t)stage * BK + kb[p] * VE + v;
        reg[p][v] = (n_valid[p] && k < k_end)
                        ? *(const uint4*)(base + k * ld + n * Elem<T>::kBytes)
                        : make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(uint4* lds) const;
};

template <>
__device__ __forceinline__ void ColLoader<bf16_t>::store(uint4* lds) const {
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    uint32_t w[8][4];
#pragma unroll
    for (int v = 0; v < 8; ++v) {
      w[v][0] = reg[p][v].x; w[v][1] = reg[p][v].y; w[v][2] = reg[p][v].z; w[v][3] = reg[p][v].w;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = w[2 * q][j >> 1], hi = w[2 * q + 1][j >> 1];
        o[q] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      lds[swz(nb[p] * 8 + j, kb[p])] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

template <>
__device__ __forceinline__ void ColLoader<float>::store(uint4* lds) const {
#pragma unroll
  for (int p = 0; p < PB; ++p) {
    const uint4* r = reg[p];
    lds[swz(nb[p] * 4 + 0, kb[p])] = make_uint4(r[0].x, r[1].x, r[2].x, r[3].x);
    lds[swz(nb[p] * 4 + 1, kb[p])] = make_uint4(r[0].y, r[1].y, r[2].y, r[3].y);
    lds[swz(nb[p] * 4 + 2, kb[p])] = make_uint4(r[0].z, r[1].z, r[2].z, r[3].z);
    lds[swz(nb[p] * 4 + 3, kb[p])] = make_uint4(r[0].w, r[1].w, r[2].w, r[3].w);
  }
}

// ---------------------------------------------------------------------------
// Double-buffered main loop: acc[i][j] += A-tile rows x B-tile rows over nk stages.
// BROW(wn, j) gives the first LDS row of B fragment j of wave column wn.
template <typename T, int EPI, typename LA, typename LB>
__device__ __forceinline__ void mainloop(LA& la, LB& lb, int nk, uint4* smem, f32x16 (&acc)[4][4]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  if (nk <= 0) return;

  int arow[4], brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) arow[i] = wm * 128 + i * 32 + l32;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    brow[j] = (EPI == EPI_SWIGLU ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32) : (wn * 128 + j * 32)) + l32;

  la.load(0);
  lb.load(0);
  la.store(smem);
  lb.store(smem + kTileChunks);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const uint4* As = smem + (s & 1) * 2 * kTileChunks;
    const uint4* Bs = As + kTileChunks;
    const bool more = s + 1 < nk;
    if (more) {
      la.load(s + 1);
      lb.load(s + 1);
    }
#pragma unroll
    for (int kk = 0; kk < kCPR / 2; ++kk) {
      const int c = 2 * kk + hi;
      uint4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[swz(arow[i], c)];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[swz(brow[j], c)];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) Mma<T>::run(a[i], b[j], acc[i][j]);
    }
    if (more) {
      uint4* An = smem + ((s + 1) & 1) * 2 * kTileChunks;
      la.store(An);
      lb.store(An + kTileChunks);
    }
    __syncthreads();
  }
}

// XCD-aware bijection of [0, total): XCD x (blocks b = x mod 8) gets a contiguous run.
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t total) {
  const int64_t xcd = b % kXcd, local = b / kXcd;
  const int64_t q = total / kXcd, r = total % kXcd;
  return xcd * q + (xcd < r ? xcd : r) + local;
}

__device__ __forceinline__ void group_rows(const int32_t* offs, int g, int64_t M, int64_t& rs, int64_t& re) {
  int64_t a = offs[g], b = offs[g + 1];
  a = a < 0 ? 0 : (a > M ? M : a);
  b = b < a ? a : (b > M ? M : b);
  rs = a;
  re = b;
}

struct GemmParams {
  const void* A;
  const void* B;
  const int32_t* offs;
  const void* epi_in;
  void* epi_save;
  void* C;
  int64_t M, N, Kd;
  int G;
  int NT;  // column tiles
};

template <typename T, int BL, int EPI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_kernel(GemmParams p) {
  __shared__ uint4 smem[4 * kTileChunks];
  __shared__ int s_wtot[4];
  __shared__ int s_res[2];
  using E = Elem<T>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- row tiles per group and their prefix sum (group counts stay on the device)
  const int gpt = (p.G + kThreads - 1) / kThreads;
  const int g0 = tid * gpt;
  int local = 0;
  for (int g = g0; g < g0 + gpt && g < p.G; ++g) {
    int64_t rs, re;
    group_rows(p.offs, g, p.M, rs, re);
    local += (int)((re - rs + kTile - 1) / kTile);
  }
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) s_wtot[wave] = incl;
  if (tid == 0) {
    s_res[0] = 0;
    s_res[1] = 0;
  }
  __syncthreads();
  int total_mt = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int v = s_wtot[w];
    if (w < wave) incl += v;
    total_mt += v;
  }
  const int excl = incl - local;
  const int64_t total = (int64_t)total_mt * p.NT;
  if ((int64_t)blockIdx.x >= total) return;  // uniform over the workgroup

  const int64_t L = xcd_remap(blockIdx.x, total);
  const int64_t per = (int64_t)kGroupM * p.NT;
  const int64_t grp = L / per;
  const int first = (int)(grp * kGroupM);
  const int gm = min(total_mt - first, kGroupM);
  const int rem = (int)(L - grp * per);
  const int mt = first + rem % gm;
  const int nt = rem / gm;
  if (excl <= mt && mt < incl) {
    int run = excl;
    for (int g = g0; g < g0 + gpt && g < p.G; ++g) {
      int64_t rs, re;
      group_rows(p.offs, g, p.M, rs, re);
      const int c = (int)((re - rs + kTile - 1) / kTile);
      if (mt < run + c) {
        s_res[0] = g;
        s_res[1] = mt - run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
  const int g = min(max(s_res[0], 0), p.G - 1);
  int64_t rs, re;
  group_rows(p.offs, g, p.M, rs, re);
  const int64_t m0 = rs + (int64_t)s_res[1] * kTile;

  // ---- operand loaders
  const int64_t esz = E::kBytes;
  RowLoader la;
  la.c = tid & 7;
  la.kbytes = p.Kd * esz;
  {
    const char* A = (const char*)p.A;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      int64_t row = m0 + (tid >> 3) + 32 * i;
      row = row < p.M ? row : p.M - 1;
      la.ptr[i] = A + row * p.Kd * esz;
    }
  }
  f32x16 acc[4][4];
  const int nk = (int)((p.Kd * esz + kRowBytes - 1) / kRowBytes);
  if constexpr (BL == LAYOUT_NK) {
    RowLoader lb;
    lb.c = tid & 7;
    lb.kbytes = p.Kd * esz;
    const char* Bg = (const char*)p.B + (int64_t)g * p.N * p.Kd * esz;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = (tid >> 3) + 32 * i;
      int64_t n;
      if (EPI == EPI_SWIGLU) {
        const int64_t F = p.N / 2;
        const int64_t c = (int64_t)nt * 128 + (r & 127);
        n = (r < 128 ? 0 : F) + (c < F ? c : F - 1);
      } else {
        n = (int64_t)nt * kTile + r;
        n = n < p.N ? n : p.N - 1;
      }
      lb.ptr[i] = Bg + n * p.Kd * esz;
    }
    mainloop<T, EPI>(la, lb, nk, smem, acc);
  } else {
    ColLoader<T> lb;
    lb.init((const char*)p.B + (int64_t)g * p.Kd * p.N * esz, p.N, (int64_t)nt * kTile, p.N, 0, p.Kd);
    mainloop<T, EPI>(la, lb, nk, smem, acc);
  }

  // ---- epilogue: lane holds column (lane & 31) and rows 8*(r/4) + 4*(lane/32) + r%4 of each 32x32 tile
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  if constexpr (EPI == EPI_SWIGLU) {
    const int64_t F = p.N / 2;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int64_t col = (int64_t)nt * 128 + wn * 64 + j * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (row < re && col < F) {
            const float gt = acc[i][j][r], up = acc[i][j + 2][r];
            E::store1(p.C, row * F + col, gt / (1.f + __expf(-gt)) * up);
            if (p.epi_save) {
              E::store1(p.epi_save, row * p.N + col, gt);
              E::store1(p.epi_save, row * p.N + F + col, up);
            }
          }
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = (int64_t)nt * kTile + wn * 128 + j * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (row < re && col < p.N) {
            const float v = acc[i][j][r];
            if (EPI == EPI_NONE) {
              E::store1(p.C, row * p.N + col, v);
            } else {  // DSWIGLU: v = dH; saved pre-activations [G | U] of width 2N
              const float gt = E::load1(p.epi_in, row * 2 * p.N + col);
              const float up = E::load1(p.epi_in, row * 2 * p.N + p.N + col);
              const float sg = 1.f / (1.f + __expf(-gt));
              E::store1(p.C, row * 2 * p.N + col, v * up * sg * (1.f + gt * (1.f - sg)));
              E::store1(p.C, row * 2 * p.N + p.N + col, v * gt * sg);
            }
          }
        }
      }
  }
}

// ---------------------------------------------------------------------------
// dW[g] = dY_g^T X_g: output tile (n, kd) of group g, reduction over the group's rows.
struct WgradParams {
  const void* X;
  const void* dY;
  const int32_t* offs;
  float* dW;
  int64_t M, N, Kd;
  int G;
  int TN, TK;
  int accumulate;
};

template <typename T>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_wgrad_kernel(WgradParams p) {
  __shared__ uint4 smem[4 * kTileChunks];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t tpg = (int64_t)p.TN * p.TK;
  const int64_t total = tpg * p.G;
  const int64_t L = xcd_remap(blockIdx.x, total);
  const int g = (int)(L / tpg);
  const int rem = (int)(L - (int64_t)g * tpg);
  const int tk = rem / p.TN;  // neighbouring tiles share the same X columns
  const int tn = rem % p.TN;
  int64_t rs, re;
  group_rows(p.offs, g, p.M, rs, re);
  const int64_t n0 = (int64_t)tn * kTile, k0 = (int64_t)tk * kTile;
  float* out = p.dW + (int64_t)g * p.N * p.Kd;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;

  f32x16 acc[4][4];
  constexpr int BK = kRowBytes / Elem<T>::kBytes;
  const int nk = (int)((re - rs + BK - 1) / BK);
  ColLoader<T> la, lb;
  la.init(p.dY, p.N, n0, p.N, rs, re);
  lb.init(p.X, p.Kd, k0, p.Kd, rs, re);
  mainloop<T, EPI_NONE>(la, lb, nk, smem, acc);  // zeros when the group is empty

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = k0 + wn * 128 + j * 32 + l32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = n0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (row < p.N && col < p.Kd) {
          float* q = out + row * p.Kd + col;
          if (p.accumulate) {
            if (nk > 0) *q += acc[i][j][r];
          } else {
            *q = acc[i][j][r];
          }
        }
      }
    }
}

template <typename T>
hipError_t gemm_dispatch(const GemmParams& prm, int b_layout, int epi, dim3 grid, hipStream_t s) {
#define MOE_GG(BL, EP) hipLaunchKernelGGL((grouped_gemm_kernel<T, BL, EP>), grid, dim3(kThreads), 0, s, prm)
  if (b_layout == LAYOUT_NK) {
    if (epi == EPI_NONE) MOE_GG(LAYOUT_NK, EPI_NONE);
    else if (epi == EPI_SWIGLU) MOE_GG(LAYOUT_NK, EPI_SWIGLU);
    else MOE_GG(LAYOUT_NK, EPI_DSWIGLU);
  } else {
    if (epi == EPI_NONE) MOE_GG(LAYOUT_KN, EPI_NONE);
    else if (epi == EPI_DSWIGLU) MOE_GG(LAYOUT_KN, EPI_DSWIGLU);
    else return hipErrorInvalidValue;
  }
#undef MOE_GG
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm(const void* A, const void* B, int b_layout, const int32_t* offs,
                               int64_t M, int64_t N, int64_t Kd, int G, int dtype, int epilogue,
                               const void* epi_in, void* epi_save, void* C, hipStream_t s) {
  if (M == 0) return hipSuccess;
  GemmParams prm{A, B, offs, epi_in, epi_save, C, M, N, Kd, G, 0};
  prm.NT = (epilogue == EPI_SWIGLU) ? (int)((N / 2 + 127) / 128) : (int)((N + kTile - 1) / kTile);
  const int64_t max_mt = (M + kTile - 1) / kTile + G;
  const dim3 grid((unsigned)(max_mt * prm.NT));
  if (dtype == 1) return gemm_dispatch<bf16_t>(prm, b_layout, epilogue, grid, s);
  return gemm_dispatch<float>(prm, b_layout, epilogue, grid, s);
}

hipError_t launch_grouped_wgrad(const void* X, const void* dY, const int32_t* offs, int64_t M,
                                int64_t N, int64_t Kd, int G, int dtype, int accumulate, float* dW,
                                hipStream_t s) {
  WgradParams prm{X, dY, offs, dW, M, N, Kd, G, 0, 0, accumulate};
  prm.TN = (int)((N + kTile - 1) / kTile);
  prm.TK = (int)((Kd + kTile - 1) / kTile);
  const dim3 grid((unsigned)((int64_t)prm.TN * prm.TK * G));
  if (dtype == 1)
    hipLaunchKernelGGL((grouped_wgrad_kernel<bf16_t>), grid, dim3(kThreads), 0, s, prm);
  else
    hipLaunchKernelGGL((grouped_wgrad_kernel<float>), grid, dim3(kThreads), 0, s, prm);
  return hipGetLastError();
}

}  // namespace moe
