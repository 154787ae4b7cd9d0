// Grouped GEMM over variable-length expert groups, and its weight gradient.
//
// Page "Accelerating dropless MoE training in JAX with NVIDIA Transformer
// Engine", "Optimisation 1: Grouped GEMM": all expert matmuls run in one
// kernel call, each at its actual token count, computing only the regions
// that hold valid tokens; the group sizes are never copied to the host, so
// the launch shape is fixed and the call can be captured in a graph.
//
// gfx950 design: three engines share the tile lookup and the epilogues.
//   * Ring kernel (bf16, weights N-by-K, K a multiple of 64: the forward GEMMs).
//     256x256 output tile per workgroup of 4 waves (one per SIMD), 128x128 per
//     wave in 16 v_mfma_f32_32x32x16_bf16 tiles.  K advances 64 elements at a
//     time; each 32 KB half-stage (A or B) is copied global->LDS by DMA into a
//     five-slot ring that fills the 160 KB LDS, two stages ahead of the MFMAs.
//     Operand fragments are read from LDS two sub-steps ahead, one read between
//     consecutive MFMAs.  An optional workspace splits the last, partly filled
//     round of tiles along K (see the split-tail notes at the kernel).
//   * Eight-wave DMA kernel (bf16 data gradient with K-by-N weights, the weight
//     gradient, and the N-by-K cases the ring does not take).  Two waves per
//     SIMD, 128x64 per wave; K-contiguous operands are copied chunk for chunk,
//     K-row operands are read with transposing LDS reads.
//   * Register-staged kernel (fp32, and K not a multiple of 32 elements).  Operands
//     with K as the row index are read as 8x8 (bf16) or 4x4 (fp32) blocks and
//     transposed in registers before the LDS write.
//   * LDS rows are 16-byte chunks with the chunk index XORed by a function of the
//     row, so DMA writes and MFMA operand reads hit distinct banks.
//   * Each workgroup finds its (group, row tile, column tile) from the group
//     offsets in device memory.  The grid is an upper bound computed on the
//     host; surplus workgroups exit.  Each round of 256 blocks covers 256
//     consecutive tiles, dealt to the XCDs in runs of 32 in which 8 row tiles
//     share each column tile, so concurrently running tiles share operands in
//     their XCD's L2 and the XCDs share panels through the Infinity Cache.
//   * Epilogues: plain store; SwiGLU (gate and up columns of one output column
//     live in the same lane); SwiGLU backward using the saved pre-activations.
#include <algorithm>
#include <cstdint>
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "moe.h"
#include "mx_encode.h"

namespace moe {

namespace {

constexpr int kThreads = 256;
constexpr int kTile = 256;                 // BM = BN
constexpr int kRowBytes = 128;             // K bytes per LDS row per stage
constexpr int kCPR = kRowBytes / 16;       // 16-byte chunks per LDS row
constexpr int kTileChunks = kTile * kCPR;  // chunks per operand stage (32 KB)
constexpr int kXcd = 8;                    // MI355X: 8 XCDs, workgroups dealt round-robin
constexpr int kGroupM = 8;                 // row tiles that share a column tile
constexpr int kWindow = 256;               // blocks per XCD-remap window (one round: one per CU)
constexpr int kSwigluSkipRows = 1536;      // mean group rows below which SwiGLU skips empty fragments

enum { EPI_NONE = 0, EPI_SWIGLU = 1, EPI_DSWIGLU = 2, EPI_SWIGLU_MX = 3 };  // MX: SwiGLU, MXFP8 out
enum { LAYOUT_NK = 0, LAYOUT_KN = 1 };
constexpr int LAYOUT_WG = 2;  // ring pipeline of the weight gradient: both operands K-row

// LDS chunk index of (row, 16-byte chunk c).  The XOR pattern g(row) = (row & 7) ^ ((row >> 3) & 1)
// makes the 16 lanes that one LDS cycle serves (16 consecutive rows, one logical chunk:
// the MFMA operand reads) and the row-major writes (2 rows x 8 chunks) hit 16 distinct
// 16-byte bank groups of a 256-byte-wide LDS, and any 8 consecutive rows distinct ones too.
__device__ __forceinline__ int swz_x(int row) { return (row & 7) ^ ((row >> 3) & 1); }
__device__ __forceinline__ int swz(int row, int c) { return row * kCPR + (c ^ swz_x(row)); }

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

// acc += (A B^T)^T for a 32 x 32 tile: the MFMA is fed B as its first operand, so
// a lane ends up holding row (lane & 31) of the output at the 16 columns
// 8 (r / 4) + 4 (lane / 32) + r % 4: runs of 4 consecutive columns, which the
// epilogues store as one 8-byte (bf16) or 16-byte (fp32) access each.
template <typename T>
__device__ __forceinline__ void mma_rows(const uint4& a, const uint4& b, f32x16& acc) {
  Mma<T>::run(b, a, acc);
}

// ---------------------------------------------------------------------------
// Loader of an operand whose rows are K-contiguous: LDS row r <- global row ptr_r.
// Thread tid moves chunk (tid & 7) of rows (tid >> 3) + 32 i, i < 8.
struct RowLoader {
  const char* ptr[8];  // start of each row (K offset 0)
  int64_t kbytes;  // K extent in bytes
  int c;
  uint4 reg[8];

  // branch-free: a chunk past the K extent reads an in-row address and is replaced by zeros
  __device__ __forceinline__ void load(int stage) {
    int64_t off = (int64_t)stage * kRowBytes + c * 16;
    const bool ok = off < kbytes;
    off = ok ? off : kbytes - 16;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 v = *(const uint4*)(ptr[i] + off);
      reg[i] = ok ? v : make_uint4(0, 0, 0, 0);
    }
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

  // branch-free: rows past k_end and column blocks past ncols read an in-range
  // address of the same operand and are replaced by zeros
  __device__ __forceinline__ void load(int stage) {
    constexpr int BK = kRowBytes / Elem<T>::kBytes;
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int64_t n = n_valid[p] ? n0 + (int64_t)nb[p] * VE : n0;
#pragma unroll
      for (int v = 0; v < VE; ++v) {
        const int64_t k = k_begin + (int64_t)stage * BK + kb[p] * VE + v;
        const bool ok = n_valid[p] && k < k_end;
        const uint4 val = *(const uint4*)(base + (ok ? k : k_begin) * ld + n * Elem<T>::kBytes);
        reg[p][v] = ok ? val : make_uint4(0, 0, 0, 0);
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

// Instruction order of one main-loop stage (scheduler groups, in order):
// operand reads of sub-step 0, the next stage's global loads, operand reads of
// sub-step 1, then each sub-step's MFMAs with the following sub-step's operand
// reads behind them; the next stage's LDS writes are spread through the MFMAs
// of sub-steps 2 and 3.
enum { SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100, SG_DS_WRITE = 0x200 };
template <typename T>
__device__ __forceinline__ void schedule_stage() {
  constexpr int kMfmaPerSub = 16 * (Elem<T>::kVec == 8 ? 1 : 4);
  __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 8, 0);
  __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 16, 0);
  __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 8, 0);
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, kMfmaPerSub, 0);
  __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 8, 0);
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, kMfmaPerSub, 0);
  __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 8, 0);
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, kMfmaPerSub / 8, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 1, 0);
  }
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, kMfmaPerSub / 8, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_WRITE, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, kMfmaPerSub, 0);
}

// ---------------------------------------------------------------------------
// Main loop: acc[i][j] += A-tile rows x B-tile rows over nk stages of 128 K-bytes.
// LDS holds two stages.  Within a stage the four 16-byte K sub-steps use two
// register sets of MFMA operands, so the LDS reads of sub-step kk+1 are in
// flight while sub-step kk multiplies; the global loads of the next stage are
// issued at the top of the stage and written to the other LDS buffer during
// the last sub-step.  The loop body has no branches.
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

  // every operand row a lane reads is l32 plus a multiple of 32: one XOR for all fragments
  const int x = swz_x(l32);
  const int a_row8 = (wm * 128 + l32) * kCPR;
  int b_row8[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    b_row8[j] = ((EPI == EPI_SWIGLU ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32) : (wn * 128 + j * 32)) + l32) * kCPR;

  auto read = [&](const uint4* As, const uint4* Bs, int kk, uint4 (&a)[4], uint4 (&b)[4]) {
    const int cc = (2 * kk + hi) ^ x;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = As[a_row8 + i * 32 * kCPR + cc];
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = Bs[b_row8[j] + cc];
  };
  auto mma16 = [&](const uint4 (&a)[4], const uint4 (&b)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) mma_rows<T>(a[i], b[j], acc[i][j]);
  };

  la.load(0);
  lb.load(0);
  la.store(smem);
  lb.store(smem + kTileChunks);
  __syncthreads();
  uint4 fa0[4], fb0[4], fa1[4], fb1[4];
  for (int s = 0; s < nk; ++s) {
    const uint4* As = smem + (s & 1) * 2 * kTileChunks;
    const uint4* Bs = As + kTileChunks;
    uint4* An = smem + ((s + 1) & 1) * 2 * kTileChunks;
    const int sn = s + 1 < nk ? s + 1 : s;  // the last stage reloads itself into the idle buffer
    read(As, Bs, 0, fa0, fb0);
    la.load(sn);
    lb.load(sn);
    read(As, Bs, 1, fa1, fb1);
    mma16(fa0, fb0);
    read(As, Bs, 2, fa0, fb0);
    mma16(fa1, fb1);
    read(As, Bs, 3, fa1, fb1);
    mma16(fa0, fb0);
    la.store(An);
    lb.store(An + kTileChunks);
    mma16(fa1, fb1);
    schedule_stage<T>();
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// LDS-DMA pipeline.  global_load_lds_dwordx4 moves 16 bytes per lane from
// global memory straight into LDS (lane L lands at M0 + 16 L), so no VGPRs or
// LDS write instructions are spent on staging and several stages can be in
// flight: 4 LDS stages, each stage's loads issued three stages before it is
// consumed.  The DMA is issued through inline assembly so that the compiler
// does not serialise every LDS read behind it; completion is tracked with
// explicit vmcnt waits and one workgroup barrier per stage.
constexpr int kDmaUnits = 8192;                   // LDS of the pipelines: 128 KB in 16-byte units

__device__ __forceinline__ void lds_dma16(const void* gptr, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_byte), "v"(gptr) : "memory", "m0");
}
__device__ __forceinline__ void wait_vmcnt_8() { asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); }
__device__ __forceinline__ void wait_vmcnt_6() { asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); }
__device__ __forceinline__ void wait_vmcnt_4() { asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); }
__device__ __forceinline__ void wait_vmcnt_0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_all_0() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// Eight-wave LDS-DMA main loops.  Two waves per SIMD, each owning a 128 x 64
// block of the 256 x 256 tile (4 x 2 MFMA tiles, 128 accumulators): a single
// wave per SIMD cannot pull LDS operands fast enough to keep its MFMA pipe busy;
// two waves per SIMD double the LDS read rate, and each wave's MFMAs cover the
// other's LDS, barrier and memory waits.
//
// A stage holds 16 NQ K values of both operands (8 NQ KB each); each wave issues
// NQ DMA instructions of 1 KB per operand per stage.  NQ = 4 (64-element stages
// for bf16, two 64 KB buffers) makes every row request a whole 128-byte cache
// line, which halves the requests the address unit and L1 must process compared
// with NQ = 2 (32-element stages, four 32 KB buffers, 64-byte half lines); NQ = 2
// serves K that is a multiple of 64 bytes but not of 128.
//
// Operand modes:
//   OpRow: the tile's rows are K-contiguous global rows (the forward operands and
//          the data-gradient A).  An LDS row holds 32 NQ K-bytes = 2 NQ chunks of
//          16 bytes, the chunk index XORed with a function of the row chosen so
//          that the 16 lanes of one LDS cycle (16 consecutive rows, one chunk) hit
//          distinct bank groups.  One ds_read_b128 gives a lane its 8 K values.
//   OpCol: the global row index is K and the tile's rows are columns (the K-by-N
//          weights of the data gradient; both operands of the weight gradient).
//          LDS row = one K value x 256 columns (512 bytes, whole cache lines from
//          global memory), 32-byte segments XORed with (k & 3) << 1.  Operands are
//          read with ds_read_b64_tr_b16: within each group of 16 lanes, lane i
//          receives halfword (i & 3) of the 8 bytes addressed by lane 4e + (i >> 2)
//          as its element e; lanes 4e + q point at K row k0 + e, columns 4q..4q+3,
//          so lane i gets column i at K rows k0..k0+3, and two reads give the 8
//          consecutive K values of an MFMA operand.  K rows past the valid range
//          are read from a zero block, so ragged reductions need no LDS clearing.
constexpr int kThreads8 = 512;
constexpr int kColRowBytes = kTile * 2;             // 512 bytes (bf16)

__device__ const uint4 kZero16 = {0u, 0u, 0u, 0u};  // DMA source of rows outside the reduction

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int NQ>
struct Stage {
  static constexpr int kRowBytes = 32 * NQ;           // OpRow K bytes per row
  static constexpr int kCPR = kRowBytes / 16;         // 16-byte chunks per OpRow row
  static constexpr int kColRows = 16 * NQ;            // OpCol K rows
  static constexpr int kOpUnits = kTile * kCPR;       // per operand (8 NQ KB)
  static constexpr int kUnits = 2 * kOpUnits;         // A then B
  static constexpr int kBuffers = kDmaUnits / kUnits; // 4 (NQ = 2) or 2 (NQ = 4)
};

template <int NQ>
struct OpRow {
  using S = Stage<NQ>;
  const char* src[NQ];  // per DMA instruction q: global address at K offset 0
  __device__ __forceinline__ static int swz(int row) { return (row >> (NQ == 2 ? 2 : 1)) & (S::kCPR - 1); }
  // LDS row filled by this lane in DMA instruction q, and the logical chunk it fetches
  __device__ __forceinline__ static int dma_row(int q) {
    return ((threadIdx.x >> 6) * NQ + q) * (64 / S::kCPR) + (threadIdx.x & 63) / S::kCPR;
  }
  __device__ __forceinline__ static int dma_chunk(int row) { return ((threadIdx.x & 63) % S::kCPR) ^ swz(row); }
  __device__ __forceinline__ const char* at(int q, int st) const { return src[q] + (int64_t)st * S::kRowBytes; }
  // operand of the 32 x 16 MFMA tile whose rows start at LDS row rb (a multiple of 32)
  __device__ __forceinline__ static uint4 frag(const uint4* L, int rb, int kk) {
    const int lane = threadIdx.x & 63;
    const int l32 = lane & 31, hi = lane >> 5;
    return L[(rb + l32) * S::kCPR + ((2 * kk + hi) ^ swz(l32))];
  }
};

template <int NQ>
struct OpCol {
  using S = Stage<NQ>;
  // global address of K row 0 at this lane's columns for DMA instruction q: the column
  // swizzle depends on kr[q] & 3 = (2 q + lane / 32) & 3, so base[q & 1] serves every q
  const char* base[2];
  const char* zero;      // this lane's bytes when its K row is out of range
  int64_t ld;            // row pitch in bytes
  int64_t k0, kend;      // first and end K row of the reduction
  int kr[NQ];            // per DMA instruction q: K row within the stage
  __device__ __forceinline__ const char* at(int q, int st) const {
    const int64_t k = k0 + (int64_t)st * S::kColRows + kr[q];
    return k < kend ? base[q & 1] + k * ld : zero;
  }
  __device__ __forceinline__ static uint4 frag(const uint4* L, int cb, int kk) {
    const int lane = threadIdx.x & 63;
    const int hi = lane >> 5, g = (lane >> 4) & 1, e = (lane >> 2) & 3, q = lane & 3;
    const char* Lb = (const char*)L;
    const int seg = ((cb >> 4) + g) ^ (e << 1);
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int row = 16 * kk + 8 * hi + 4 * t + e;
      const char* addr = Lb + row * kColRowBytes + seg * 32 + q * 8;
      const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)addr);
      w[2 * t] = (uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
      w[2 * t + 1] = (uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
  // set up DMA sources for an operand stored [K rows][ncols] (ld elements per row) whose tile
  // covers columns [c0, c0 + 256); lanes of DMA instruction q fill LDS K row (wave*NQ+q)*2 + lane/32
  __device__ __forceinline__ void init(const void* g, int64_t ld_elems, int64_t c0, int64_t ncols, int64_t kbeg,
                                       int64_t kfin) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    ld = ld_elems * 2;
    k0 = kbeg;
    kend = kfin;
    zero = (const char*)&kZero16;
#pragma unroll
    for (int q = 0; q < NQ; ++q) kr[q] = (wave * NQ + q) * 2 + (lane >> 5);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int u = lane & 31;                                          // physical 16-byte unit in the LDS row
      const int lu = (((u >> 1) ^ ((kr[q] & 3) << 1)) << 1) | (u & 1);  // logical unit (8 columns)
      int64_t col = c0 + (int64_t)lu * 8;
      col = col < ncols ? col : ncols - 8;                             // clamped: only unstored outputs use it
      base[q] = (const char*)g + col * 2;
    }
  }
};

template <typename O> struct OpTraits;
template <int NQ> struct OpTraits<OpRow<NQ>> { static constexpr int kReads = 1; static constexpr int kNQ = NQ; };
template <int NQ> struct OpTraits<OpCol<NQ>> { static constexpr int kReads = 2; static constexpr int kNQ = NQ; };

// Workgroup barrier without the LDS-drain wait that __syncthreads() implies: the
// only LDS writes here are DMA, completed by the explicit vmcnt waits, and the
// callers wait for their own LDS reads where a buffer is refilled right after.
// The memory clobber keeps the compiler from moving LDS reads across it.
__device__ __forceinline__ void dma_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Shared pieces of both main loops: DMA issue, fragment reads and MFMA ranges.
template <typename T, int EPI, typename OA, typename OB>
struct Pipe8 {
  static constexpr int NQ = OpTraits<OA>::kNQ;
  using S = Stage<NQ>;
  // LDS read instructions per sub-step (a transposed fragment takes two)
  static constexpr int kReads = 4 * OpTraits<OA>::kReads + 2 * OpTraits<OB>::kReads;
  static constexpr int kMfmaPer = Elem<T>::kVec == 8 ? 1 : 4;  // MFMA instructions per 32 x 32 x 16 step
  const OA& oa;
  const OB& ob;
  uint4* smem;
  f32x16 (&acc)[4][2];
  uint32_t wbase;
  int arow, b_rb[2];
  __device__ __forceinline__ Pipe8(const OA& a, const OB& b, uint4* sm, f32x16 (&c)[4][2]) : oa(a), ob(b), smem(sm), acc(c) {
    const int wave = threadIdx.x >> 6;
    const int wm = wave >> 2, wn = wave & 3;
    wbase = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)smem + wave * NQ * 1024);
    arow = wm * 128;
#pragma unroll
    for (int j = 0; j < 2; ++j) b_rb[j] = EPI == EPI_SWIGLU ? (j * 128 + wn * 32) : (wn * 64 + j * 32);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }
  __device__ __forceinline__ uint32_t lbase(int st) const {
    return wbase + (uint32_t)(st % S::kBuffers) * (S::kUnits * 16);
  }
  __device__ __forceinline__ void issue_a(int st, int q) const { lds_dma16(oa.at(q, st), lbase(st) + q * 1024); }
  __device__ __forceinline__ void issue_b(int st, int q) const {
    lds_dma16(ob.at(q, st), lbase(st) + S::kOpUnits * 16 + q * 1024);
  }
  __device__ __forceinline__ void read(int st, int kk, uint4 (&a)[4], uint4 (&b)[2]) const {
    const uint4* L = smem + (st % S::kBuffers) * S::kUnits;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = OA::frag(L, arow + i * 32, kk);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = OB::frag(L + S::kOpUnits, b_rb[j], kk);
  }
  // MFMAs t0 .. t1-1 of a sub-step (t = 2 i + j)
  __device__ __forceinline__ void mma(const uint4 (&a)[4], const uint4 (&b)[2], int t0, int t1) const {
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (t >= t0 && t < t1) mma_rows<T>(a[t >> 1], b[t & 1], acc[t >> 1][t & 1]);
  }
  // a sub-step's reads (issued first), then its MFMAs with DMA instructions between them
  template <typename F>
  __device__ __forceinline__ void step_with_dma(const uint4 (&a)[4], const uint4 (&b)[2], F&& dma) const {
    mma(a, b, 0, 1);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, kReads, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, kMfmaPer, 0);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      __builtin_amdgcn_sched_barrier(0);
      dma(q);
      __builtin_amdgcn_sched_barrier(0);
      mma(a, b, 1 + q * 7 / NQ, 1 + (q + 1) * 7 / NQ);
    }
  }
  __device__ __forceinline__ void step(const uint4 (&a)[4], const uint4 (&b)[2]) const {
    mma(a, b, 0, 8);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, kReads, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 8 * kMfmaPer, 0);
  }
};

// 32-element stages (NQ = 2), four buffers.  Stage st is issued in two halves: its A
// rows one iteration before its B rows.  In every state below, the DMAs issued after
// the last one of stage st+1 are exactly the 4 of stage st+2, so vmcnt(4) (vmcnt(0)
// at the end) means stage st+1 has landed.
template <typename T, int EPI, typename OA, typename OB>
__device__ __forceinline__ void mainloop8(const OA& oa, const OB& ob, int nk, uint4* smem, f32x16 (&acc)[4][2]) {
  Pipe8<T, EPI, OA, OB> P(oa, ob, smem, acc);
  static_assert(Pipe8<T, EPI, OA, OB>::NQ == 2, "four-buffer loop takes 32-element stages");
  if (nk <= 0) return;
  P.issue_a(0, 0); P.issue_a(0, 1); P.issue_b(0, 0); P.issue_b(0, 1);
  if (nk > 1) { P.issue_a(1, 0); P.issue_a(1, 1); P.issue_b(1, 0); P.issue_b(1, 1); }
  if (nk > 2) { P.issue_a(2, 0); P.issue_a(2, 1); }
  if (nk > 2) wait_vmcnt_6();
  else if (nk > 1) wait_vmcnt_4();
  else wait_vmcnt_0();
  dma_barrier();
  uint4 fa0[4], fb0[2], fa1[4], fb1[2];
  P.read(0, 0, fa0, fb0);
  int s = 0;
  // steady state, straight-line so that LDS read counts stay exact.  The DMAs are spread
  // between MFMAs so that the 8 waves do not hand the address unit a burst at once.
  // The B half of stage s+2 reuses the buffer of stage s-2 and the A half of stage s+3
  // that of stage s-1: every wave consumed its reads of those before the previous barrier.
  for (; s + 3 < nk; ++s) {
    // region 1: operand reads of sub-step 1, the MFMAs of sub-step 0, B half of stage s+2
    P.read(s, 1, fa1, fb1);
    P.step_with_dma(fa0, fb0, [&](int q) { P.issue_b(s + 2, q); });
    __builtin_amdgcn_sched_barrier(0);  // keep those MFMAs ahead of the workgroup barrier
    wait_vmcnt_4();
    dma_barrier();
    // region 2: sub-step-0 reads of stage s+1, the MFMAs of sub-step 1, A half of stage s+3
    P.read(s + 1, 0, fa0, fb0);
    P.step_with_dma(fa1, fb1, [&](int q) { P.issue_a(s + 3, q); });
  }
  // drain the last (up to three) stages
  for (; s < nk; ++s) {
    P.read(s, 1, fa1, fb1);
    if (s + 2 < nk) { P.issue_b(s + 2, 0); P.issue_b(s + 2, 1); }
    P.mma(fa0, fb0, 0, 8);
    if (s + 1 < nk) {
      if (s + 2 < nk) wait_vmcnt_4();
      else wait_vmcnt_0();
      dma_barrier();
      P.read(s + 1, 0, fa0, fb0);
    }
    P.mma(fa1, fb1, 0, 8);
  }
}

// 64-element stages (NQ = 4), two buffers, four MFMA sub-steps per stage.  Stage s+1's
// A half is issued after the barrier of stage s-1 and its B half during the first
// sub-step of stage s; the barrier of stage s sits before its last sub-step and
// certifies that stage s+1 has landed (vmcnt(0): nothing is issued after it by then)
// and that every wave's reads of stage s are complete (lgkmcnt(0)), so stage s+2 may
// refill that buffer right after it.
template <typename T, int EPI, typename OA, typename OB>
__device__ __forceinline__ void mainloop8w(const OA& oa, const OB& ob, int nk, uint4* smem, f32x16 (&acc)[4][2]) {
  Pipe8<T, EPI, OA, OB> P(oa, ob, smem, acc);
  static_assert(Pipe8<T, EPI, OA, OB>::NQ == 4, "two-buffer loop takes 64-element stages");
  if (nk <= 0) return;
#pragma unroll
  for (int q = 0; q < 4; ++q) P.issue_a(0, q);
#pragma unroll
  for (int q = 0; q < 4; ++q) P.issue_b(0, q);
  if (nk > 1) {
#pragma unroll
    for (int q = 0; q < 4; ++q) P.issue_a(1, q);
    wait_vmcnt_4();
  } else {
    wait_vmcnt_0();
  }
  dma_barrier();
  uint4 fa0[4], fb0[2], fa1[4], fb1[2];
  P.read(0, 0, fa0, fb0);
  int s = 0;
  for (; s + 2 < nk; ++s) {
    P.read(s, 1, fa1, fb1);
    P.step_with_dma(fa0, fb0, [&](int q) { P.issue_b(s + 1, q); });
    P.read(s, 2, fa0, fb0);
    P.step(fa1, fb1);
    P.read(s, 3, fa1, fb1);
    P.step(fa0, fb0);
    __builtin_amdgcn_sched_barrier(0);
    wait_all_0();
    dma_barrier();
    P.read(s + 1, 0, fa0, fb0);
    P.step_with_dma(fa1, fb1, [&](int q) { P.issue_a(s + 2, q); });
  }
  for (; s < nk; ++s) {
    P.read(s, 1, fa1, fb1);
    if (s + 1 < nk) {
#pragma unroll
      for (int q = 0; q < 4; ++q) P.issue_b(s + 1, q);
    }
    P.mma(fa0, fb0, 0, 8);
    P.read(s, 2, fa0, fb0);
    P.mma(fa1, fb1, 0, 8);
    P.read(s, 3, fa1, fb1);
    P.mma(fa0, fb0, 0, 8);
    if (s + 1 < nk) {
      wait_all_0();
      dma_barrier();
      P.read(s + 1, 0, fa0, fb0);
    }
    P.mma(fa1, fb1, 0, 8);
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
  // split tail of the ring kernel: per-(split tile, wave) counters, then fp32 partial
  // tiles (kSplitSlotFloats each); ws_slots == 0 disables the split
  int* ws_count;
  float* ws_part;
  int ws_slots;
  int P;   // CUs the split tail spreads over
  int nk;  // K stages of a tile (ring kernel)
  // MXFP8 operands: E8M0 block scales of A [M][Kd/32] and B [G*N][Kd/32]
  const uint8_t* sa = nullptr;
  const uint8_t* sb = nullptr;
  // gathered A (ring kernel, N-by-K weights): row m of A is row a_rows[m] / a_div of the
  // matrix at A (the permute fused into the GEMM's loads), clamped to a_last
  const int32_t* a_rows = nullptr;
  uint32_t a_div = 1;
  uint32_t a_last = 0;
  // EPI_SWIGLU_MX: C holds the E4M3 codes of H [M][N/2] and cs its E8M0 scales [M][N/64]
  uint8_t* cs = nullptr;
};
constexpr int kSplitCountBytes = 4096;             // counters: up to 1024 (tile, wave) pairs
constexpr int kSplitSlotFloats = 256 * 256;        // one fp32 256 x 256 partial tile

// Logistic sigmoid for the SwiGLU epilogues: the hardware exponential and reciprocal
// (about 1 ulp each) instead of an IEEE division, far below the bf16 rounding of the
// outputs and within the fp32 tolerance.
__device__ __forceinline__ float sigmoid_fast(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }

// Epilogue of one wave: acc[i][j] is the 32 x 32 tile at rows row0 + 32 i and
// columns col[j]; a lane holds row (lane & 31) at columns 8 q + 4 (lane / 32) + 0..3
// in acc[i][j][4 q .. 4 q + 3].  Widths are multiples of 8 elements, so a run of 4
// columns is either wholly inside the output or wholly past its end.
// SwiGLU: fragments j < NJ/2 are gate columns and j + NJ/2 the matching up columns.
template <typename T, int EPI, int NI, int NJ>
__device__ __forceinline__ void store_tile(const GemmParams& p, const f32x16 (&acc)[NI][NJ], int64_t row0,
                                           int64_t re, const int64_t (&col)[NJ]) {
  using E = Elem<T>;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int64_t row = row0 + i * 32 + l32;
    if (EPI == EPI_DSWIGLU) {
      // SwiGLU backward: acc = dH; saved pre-activations [G | U] of width 2N.  The loads
      // of JB fragments go first (clamped into range) so that they are in flight together.
      constexpr int JB = NJ < 2 ? NJ : 2;
      const int64_t rc = row < re ? row : re - 1;
#pragma unroll
      for (int j0 = 0; j0 < NJ; j0 += JB) {
        float gt[JB][4][4], up[JB][4][4];
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            int64_t c = col[j0 + jj] + 8 * q + 4 * hi;
            c = c < p.N ? c : p.N - 4;
            E::load4(p.epi_in, rc * 2 * p.N + c, gt[jj][q]);
            E::load4(p.epi_in, rc * 2 * p.N + p.N + c, up[jj][q]);
          }
        if (row >= re) continue;
#pragma unroll
        for (int jj = 0; jj < JB; ++jj)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t c = col[j0 + jj] + 8 * q + 4 * hi;
            if (c >= p.N) continue;
            float da[4], du[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float v = acc[i][j0 + jj][4 * q + e], g = gt[jj][q][e], u = up[jj][q][e];
              const float sg = sigmoid_fast(g);
              da[e] = v * u * sg * (1.f + g * (1.f - sg));
              du[e] = v * g * sg;
            }
            E::store4(p.C, row * 2 * p.N + c, da);
            E::store4(p.C, row * 2 * p.N + p.N + c, du);
          }
      }
      continue;
    }
    if (row >= re) continue;
    if constexpr (EPI == EPI_SWIGLU) {
      const int64_t F = p.N / 2;
      char* hrow = (char*)p.C + row * F * E::kBytes;
      char* srow = p.epi_save ? (char*)p.epi_save + row * p.N * E::kBytes : nullptr;
#pragma unroll
      for (int j = 0; j < NJ / 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t c = col[j] + 8 * q + 4 * hi;
          if (c >= F) continue;
          float h[4], g[4], u[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            g[e] = acc[i][j][4 * q + e];
            u[e] = acc[i][j + NJ / 2][4 * q + e];
            h[e] = g[e] * sigmoid_fast(g[e]) * u[e];
          }
          E::store4(hrow, c, h);
          if (srow) {
            E::store4(srow, c, g);
            E::store4(srow, F + c, u);
          }
        }
    } else {
      char* crow = (char*)p.C + row * p.N * E::kBytes;
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t c = col[j] + 8 * q + 4 * hi;
          if (c >= p.N) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          E::store4(crow, c, v);
        }
    }
  }
}

// Block -> (group, first row, column tile) from the group offsets in device
// memory; false when this workgroup has no tile.  Uniform over the workgroup.
// Split tail of the ring kernel.  With dynamic dispatch the last R tiles (R = total mod P)
// would run alone on R CUs, so, given a workspace, the grid ends in R f piece blocks
// instead: each of those tiles is cut along K into f pieces (f <= P / R, at least two
// stages each) that run at once.  Every piece stores its fp32 partial tile, then counts
// itself in a per-(tile, wave) counter; the piece that counts last sums all f partials in
// piece order (so the result does not depend on which piece finished last), writes the
// epilogue and resets the counter.  No workgroup waits for another.
struct Piece {
  int part = -1;  // piece of a split tile, -1 for a whole tile
  int f = 1;      // pieces per split tile
  int R = 0;      // split tiles
  int slot = 0;   // partial-tile slot of this piece (part R + tile)
};

template <int NTHR>
__device__ __forceinline__ bool find_tile(const GemmParams& p, int& g_out, int64_t& m0_out, int64_t& re_out,
                                          int& nt_out, int* scratch, Piece* piece = nullptr) {
  constexpr int NW = NTHR / 64;
  int* s_wtot = scratch;       // NW ints
  int* s_res = scratch + NW;   // 5 ints: group, row tile in the group, first and end row, column tile
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  // row tiles per group and their prefix sum
  const int gpt = (p.G + NTHR - 1) / NTHR;
  const int g0 = tid * gpt;
  int local = 0;
  int64_t rs0 = 0, re0 = 0;  // rows of group g0 (the only group of a thread when G <= NTHR)
  for (int g = g0; g < g0 + gpt && g < p.G; ++g) {
    int64_t rs, re;
    group_rows(p.offs, g, p.M, rs, re);
    if (g == g0) {
      rs0 = rs;
      re0 = re;
    }
    local += (int)((re - rs + kTile - 1) / kTile);
  }
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) s_wtot[wave] = incl;
  if (tid < 5) s_res[tid] = 0;
  __syncthreads();
  int total_mt = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int v = s_wtot[w];
    if (w < wave) incl += v;
    total_mt += v;
  }
  const int excl = incl - local;
  const int64_t total = (int64_t)total_mt * p.NT;
  int64_t full = total, L;
  const int64_t b = blockIdx.x;
  if (piece && p.ws_slots > 0 && p.P > 0) {
    const int R = (int)(total % p.P);
    int f = 1;
    if (R > 0 && 4 * R <= kSplitCountBytes / 4) f = min(min(p.P / R, p.nk / 2), p.ws_slots / R);
    if (f > 1) {
      full = total - R;
      piece->f = f;
      piece->R = R;
    }
  }
  if (b < full) {
    // round-major: each window of 256 blocks (one round on 256 CUs) covers 256 consecutive
    // tiles of the order, and XCD x takes the x-th run of 32 of them.  All XCDs then work on
    // neighbouring tiles at once, so the operand panels they share are fetched from HBM once
    // and served to the others from the Infinity Cache (a run per XCD over the whole grid
    // made each XCD re-read its own panels every round: 1-7% slower, more HBM traffic).
    const int64_t win = b / kWindow * kWindow;
    L = win + xcd_remap(b - win, min((int64_t)kWindow, full - win));
  } else if (piece && piece->f > 1 && b < full + (int64_t)piece->R * piece->f) {
    const int pi = (int)(b - full);
    L = full + pi % piece->R;
    piece->part = pi / piece->R;
    piece->slot = pi;
  } else {
    return false;
  }
  // Tile order: group by group (a group's r row tiles give r NT consecutive tiles, so group g
  // starts at tile excl_g NT); a group's row tiles are cut into ceil(r / kGroupM) balanced
  // chunks, and a chunk's tiles run column by column, its row tiles innermost.  Neighbouring
  // tiles then share one group's weight rows, and no chunk mixes two groups.
  const int u = (int)(L / p.NT);  // a row-tile index inside the group that holds tile L
  if (excl <= u && u < incl) {
    int run = excl;
    for (int g = g0; g < g0 + gpt && g < p.G; ++g) {
      int64_t rs = rs0, re = re0;
      if (g != g0) group_rows(p.offs, g, p.M, rs, re);
      const int r = (int)((re - rs + kTile - 1) / kTile);
      if (u < run + r) {
        const int64_t local = L - (int64_t)run * p.NT;
        const int c = (r + kGroupM - 1) / kGroupM, sz = r / c, extra = r % c;
        const int ul = u - run;  // row tile of the chunk's first column
        const int k = ul < extra * (sz + 1) ? ul / (sz + 1) : extra + (ul - extra * (sz + 1)) / sz;
        const int start = k * sz + min(k, extra), size = sz + (k < extra ? 1 : 0);
        const int64_t in_chunk = local - (int64_t)start * p.NT;
        // the owner passes the group's rows on, so no thread reads the offsets again (M < 2^31)
        s_res[0] = g;
        s_res[1] = start + (int)(in_chunk % size);
        s_res[2] = (int)rs;
        s_res[3] = (int)re;
        s_res[4] = (int)(in_chunk / size);
        break;
      }
      run += r;
    }
  }
  __syncthreads();
  g_out = min(max(s_res[0], 0), p.G - 1);
  m0_out = (int64_t)s_res[2] + (int64_t)s_res[1] * kTile;
  re_out = s_res[3];
  nt_out = s_res[4];
  return true;
}

template <typename T, int BL, int EPI>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_kernel(GemmParams p) {
  __shared__ uint4 smem[4 * kTileChunks];
  using E = Elem<T>;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  int g, nt;
  int64_t m0, re;
  __shared__ int s_find[kThreads / 64 + 5];
  if (!find_tile<kThreads>(p, g, m0, re, nt, s_find)) return;

  // ---- operands
  const int64_t esz = E::kBytes;
  f32x16 acc[4][4];
  const char* A = (const char*)p.A;
  // global row of B (weights of group g) that LDS row r of the tile holds
  auto b_row = [&](int r) -> int64_t {
    if (EPI == EPI_SWIGLU) {
      const int64_t F = p.N / 2;
      const int64_t c = (int64_t)nt * 128 + (r & 127);
      return (r < 128 ? 0 : F) + (c < F ? c : F - 1);
    }
    const int64_t n = (int64_t)nt * kTile + r;
    return n < p.N ? n : p.N - 1;
  };
  auto a_row = [&](int r) -> int64_t {
    const int64_t row = m0 + r;
    return row < p.M ? row : p.M - 1;
  };
  RowLoader la;
  la.c = tid & 7;
  la.kbytes = p.Kd * esz;
#pragma unroll
  for (int i = 0; i < 8; ++i) la.ptr[i] = A + a_row((tid >> 3) + 32 * i) * p.Kd * esz;
  const int nk = (int)((p.Kd * esz + kRowBytes - 1) / kRowBytes);
  if constexpr (BL == LAYOUT_NK) {
    RowLoader lb;
    lb.c = tid & 7;
    lb.kbytes = p.Kd * esz;
    const char* Bg = (const char*)p.B + (int64_t)g * p.N * p.Kd * esz;
#pragma unroll
    for (int i = 0; i < 8; ++i) lb.ptr[i] = Bg + b_row((tid >> 3) + 32 * i) * p.Kd * esz;
    mainloop<T, EPI>(la, lb, nk, smem, acc);
  } else {
    ColLoader<T> lb;
    lb.init((const char*)p.B + (int64_t)g * p.Kd * p.N * esz, p.N, (int64_t)nt * kTile, p.N, 0, p.Kd);
    mainloop<T, EPI>(la, lb, nk, smem, acc);
  }

  // ---- epilogue
  const int wm = wave >> 1, wn = wave & 1;
  int64_t col[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    col[j] = EPI == EPI_SWIGLU ? (int64_t)nt * 128 + wn * 64 + (j & 1) * 32 : (int64_t)nt * kTile + wn * 128 + j * 32;
  store_tile<T, EPI, 4, 4>(p, acc, m0 + wm * 128, re, col);
}

// Eight-wave grouped GEMM with whole K stages of 16 NQ elements (bf16; 8 NQ for
// fp32).  A (activations) is always K-contiguous; B is the N-by-K weight layout
// (OpRow) or the K-by-N one (OpCol, bf16 only).
template <int NQ, typename T, int EPI, typename OA, typename OB>
__device__ __forceinline__ void run_mainloop(const OA& oa, const OB& ob, int nk, uint4* smem, f32x16 (&acc)[4][2]) {
  if constexpr (NQ == 4) mainloop8w<T, EPI>(oa, ob, nk, smem, acc);
  else mainloop8<T, EPI>(oa, ob, nk, smem, acc);
}

template <typename T, int EPI, int BL, int NQ>
__global__ __launch_bounds__(kThreads8) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_gemm8_kernel(GemmParams p) {
  __shared__ uint4 smem[kDmaUnits];
  using E = Elem<T>;
  int g, nt;
  int64_t m0, re;
  __shared__ int s_find[kThreads8 / 64 + 5];
  if (!find_tile<kThreads8>(p, g, m0, re, nt, s_find)) return;
  const int64_t esz = E::kBytes;
  const char* A = (const char*)p.A;
  const char* Bg = (const char*)p.B + (int64_t)g * p.N * p.Kd * esz;
  OpRow<NQ> oa;
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int r = OpRow<NQ>::dma_row(q);
    int64_t ar = m0 + r;
    ar = ar < p.M ? ar : p.M - 1;
    oa.src[q] = A + ar * p.Kd * esz + OpRow<NQ>::dma_chunk(r) * 16;
  }
  const int nk = (int)(p.Kd * esz / Stage<NQ>::kRowBytes);
  f32x16 acc[4][2];
  if constexpr (BL == LAYOUT_NK) {
    OpRow<NQ> ob;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int r = OpRow<NQ>::dma_row(q);
      int64_t br;
      if (EPI == EPI_SWIGLU) {
        const int64_t F = p.N / 2;
        const int64_t cc = (int64_t)nt * 128 + (r & 127);
        br = (r < 128 ? 0 : F) + (cc < F ? cc : F - 1);
      } else {
        br = (int64_t)nt * kTile + r;
        br = br < p.N ? br : p.N - 1;
      }
      ob.src[q] = Bg + br * p.Kd * esz + OpRow<NQ>::dma_chunk(r) * 16;
    }
    run_mainloop<NQ, T, EPI>(oa, ob, nk, smem, acc);
  } else {
    OpCol<NQ> ob;
    ob.init(Bg, p.N, (int64_t)nt * kTile, p.N, 0, p.Kd);
    run_mainloop<NQ, T, EPI>(oa, ob, nk, smem, acc);
  }
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  int64_t col[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    col[j] = EPI == EPI_SWIGLU ? (int64_t)nt * 128 + wn * 32 : (int64_t)nt * kTile + wn * 64 + j * 32;
  store_tile<T, EPI, 4, 2>(p, acc, m0 + wm * 128, re, col);
}

// ---------------------------------------------------------------------------
// Four-wave grouped GEMM on a five-slot LDS ring (bf16, N-by-K weights).
//
// One wave per SIMD owns a 128 x 128 block of the 256 x 256 tile (4 x 4 MFMA
// tiles, 256 accumulators): per 16-element K step a wave reads 8 operand
// fragments for 16 MFMAs, a third fewer LDS reads per flop than two waves of
// 128 x 64 per SIMD.  Stages are 64 K elements, so every DMA row request is a
// whole 128-byte line.  LDS is a ring of five 32 KB slots, each holding one
// operand of one stage (half-stage h: A of stage h/2 when h is even, B when odd,
// in slot h mod 5).  The two slots of stage s are released together by the
// barrier that follows the last operand reads of stage s; the ring then holds
// stage s+1 (landed), the A half of stage s+2 (in flight) and two free slots, so
// the loads run up to a stage and a half ahead of the MFMAs instead of one.
//
// Per stage s the wave issues: the A half of stage s+2 spread over the MFMAs of
// sub-steps 0..2, then, right after the barrier, the B half of stage s+2 within
// sub-step 3.  The barrier waits for stage s+1 only (vmcnt(8): the 8 DMAs of the
// A half of stage s+2 may still be in flight).
namespace ring4 {

constexpr int kThreads = 256;
constexpr int kSlotUnits = 256 * 8;       // one operand of one stage: 256 rows x 8 chunks of 16 B
constexpr int kSlotBytes = kSlotUnits * 16;
constexpr int kSlots = 5;                 // 160 KB: all of a CU's LDS
constexpr int kQ = 8;                     // DMA instructions per wave per half-stage (8 rows x 128 B each)
constexpr int kStageBytes = 128;          // K bytes per row per stage

// 16-byte chunk XOR of an LDS row (8 chunks): the 16 lanes served by one LDS cycle
// (16 consecutive rows, one logical chunk) hit 16 distinct 16-byte bank groups
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// global_load_lds_dwordx4 with a uniform 64-bit base and a 32-bit per-lane offset;
// lane L lands at M0 + 16 L
__device__ __forceinline__ void dma(const char* sbase, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:0"
               :: "v"(voff), "s"(sbase), "s"(lds_byte) : "memory", "m0");
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ const char* uniform_ptr(const char* p) { return (const char*)uniform64((int64_t)p); }

// BL = LAYOUT_NK: B rows are K-contiguous like A (a B half-stage is 256 rows of 128 bytes).
// BL = LAYOUT_KN (the data gradient's weights, [K rows][N]): a B half-stage is 64 K rows of the
// tile's 256 columns (512 bytes each); 32-byte segments of an LDS row are XORed with
// (k & 3) << 1 and fragments are read with ds_read_b64_tr_b16, two reads per fragment: within
// each 16 lanes, lane i gets halfword (i & 3) of the 8 bytes at lane 4 e + (i >> 2) as element
// e, so lanes pointed at K rows k0 + e, columns 4 q .. 4 q + 3, leave lane i with column i at
// K rows k0 .. k0 + 3.
// BL = LAYOUT_WG (the weight gradient, dW = dY^T X over a group's rows): both operands are
// K-row like the KN B operand, and both are read with ds_read_b64_tr_b16.
template <int EPI, int BL = LAYOUT_NK, bool SK = false>
struct Pipe {
  const char* a_base;   // uniform: A at (first tile row, K = 0)
  const char* b_base;   // uniform: B at (first tile row, K = 0); KN: at (K row 0, column 0)
  uint32_t va[kQ], vb[kQ];
  uint32_t lds_w;       // uniform: LDS byte address of slot 0 + this wave's DMA block
  uint32_t a_off, b_off[4];  // per lane: byte offset of fragment row l32 within a slot
                             // (KN: b_off[j] = 32-byte segment and 8-byte part of fragment j)
  uint32_t ch[4];            // per lane: byte offset of the 16-byte chunk of sub-step kk
  uint32_t b_row = 0;        // KN, per lane: byte offset of K row 8 hi + e within a slot
  uint32_t a_seg[4];         // WG, per lane: segment and 8-byte part of A fragment i
                             // (WG: a_seg and b_off also hold the LDS base and b_row)
  int64_t b_stage = kStageBytes;  // uniform: global bytes of B per stage
  int64_t a_stage = kStageBytes;  // uniform: global bytes of A per stage (WG)
  int kvalid = 1 << 30;      // WG: rows of the reduction; DMAs of rows past them write zeros
  // LDS byte offsets of the slots of half-stages 2 s .. 2 s + 4 for the main loop's current
  // stage s, rotated by two halves from stage to stage.  Every half-stage the loop touches is
  // 0..6 halves past 2 s, a distance known at compile time (H below), so its offset is one of
  // these registers (computing (2 st + OP) mod 5 took 6 scalar instructions a slot).
  uint32_t so0 = 0, so1 = kSlotBytes, so2 = 2 * kSlotBytes, so3 = 3 * kSlotBytes, so4 = 4 * kSlotBytes;
  const char* L;
  f32x16 (&acc)[4][4];
  static constexpr int kBL = BL;
  // the plain N-by-K form (and the SwiGLU form with SK): wave row wm takes the tile's 32-row
  // fragments wm, wm + 2, wm + 4, wm + 6 (LDS bytes kAStr apart), so that a partly filled tile
  // leaves both wave rows the same number of live fragments; the other forms take 128
  // contiguous rows a wave row
  static constexpr bool kIL = BL == LAYOUT_NK && (EPI == EPI_NONE || (EPI == EPI_SWIGLU && SK));
  static constexpr int kAStr = kIL ? 8192 : 4096;

  __device__ __forceinline__ Pipe(f32x16 (&c)[4][4], uint4* smem) : acc(c) {
    L = (const char*)smem;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int l32 = lane & 31, hi = lane >> 5;
    lds_w = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)smem + wave * kQ * 1024);
    a_off = ((kIL ? wm * 32 : wm * 128) + l32) * 128;
    if constexpr (BL == LAYOUT_KN || BL == LAYOUT_WG) {
      const int g = (lane >> 4) & 1, e = (lane >> 2) & 3, q = lane & 3;
      b_row = (8 * hi + e) * 512;
#pragma unroll
      for (int j = 0; j < 4; ++j) b_off[j] = (((wn * 8 + 2 * j + g) ^ (e << 1)) * 32) + q * 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) a_seg[i] = (((wm * 8 + 2 * i + g) ^ (e << 1)) * 32) + q * 8;
      if constexpr (BL == LAYOUT_WG) {
        // full per-lane LDS byte offsets of each fragment column at K row 0 of slot 0
        const uint32_t base = (uint32_t)(size_t)L + b_row;
#pragma unroll
        for (int i = 0; i < 4; ++i) a_seg[i] += base;
#pragma unroll
        for (int j = 0; j < 4; ++j) b_off[j] += base;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b_off[j] = ((EPI == EPI_SWIGLU ? ((j >> 1) * 128 + wn * 64 + (j & 1) * 32) : (wn * 128 + j * 32)) + l32) * 128;
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) ch[kk] = ((2 * kk + hi) ^ swz(l32)) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  }
  template <int H>
  __device__ __forceinline__ uint32_t sob() const {
    constexpr int h = H % kSlots;
    if constexpr (h == 0) return so0;
    else if constexpr (h == 1) return so1;
    else if constexpr (h == 2) return so2;
    else if constexpr (h == 3) return so3;
    else return so4;
  }
  // the slot offset of half-stage h = 2 s + H (H >= 0: from the carried offsets)
  template <int H>
  __device__ __forceinline__ uint32_t slot_bytes(int h) const {
    if constexpr (H >= 0) return sob<H>();
    else return (uint32_t)(h % kSlots) * kSlotBytes;
  }
  __device__ __forceinline__ void rotate() {
    const uint32_t t0 = so0, t1 = so1;
    so0 = so2;
    so1 = so3;
    so2 = so4;
    so3 = t0;
    so4 = t1;
  }
  // DMA q of operand OP (0: A, 1: B) of stage st, i.e. of half-stage 2 st + OP
  // CHK (WG only): the stage may be the reduction's last, partly filled one
  // H: that half-stage's distance from the current stage's first half (-1: unknown)
  template <int OP, bool CHK = true, int H = -1>
  __device__ __forceinline__ void issue(int st, int q) const {
    const uint32_t lb = lds_w + slot_bytes<H>(2 * st + OP) + q * 1024;
    const char* src = OP ? b_base + (int64_t)st * (BL != LAYOUT_NK ? b_stage : (int64_t)kStageBytes)
                         : a_base + (int64_t)st * (BL == LAYOUT_WG ? a_stage : (int64_t)kStageBytes);
    const uint32_t vo = OP ? vb[q] : va[q];
    if constexpr (BL == LAYOUT_WG && CHK) {
      if (st * 64 + 64 > kvalid) {
        // the reduction's last stage: lanes whose row lies past its end write zeros instead
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        const int kr = (wave * kQ + q) * 2 + (lane >> 5);
        if (st * 64 + kr < kvalid) {
          dma(src, vo, lb);
        } else {
          *(uint4*)(L + slot_bytes<H>(2 * st + OP) + (wave * kQ + q) * 1024 + lane * 16) = make_uint4(0u, 0u, 0u, 0u);
        }
        return;
      }
    }
    dma(src, vo, lb);
  }
  // KN: half t (K rows 4 t .. 4 t + 3 of each lane's 8) of B fragment j of sub-step kk
  __device__ __forceinline__ void read_tr(uint32_t sb, int kk, int j, int t, uint4& b) const {
    read_tr_at(sb, kk, b_off[j], t, b);
  }
  __device__ __forceinline__ void read_tr_at(uint32_t sb, int kk, uint32_t seg, int t, uint4& b) const {
    const char* addr = L + sb + (16 * kk + 4 * t) * 512 + b_row + seg;
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)addr);
    const uint32_t w0 = (uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
    const uint32_t w1 = (uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
    if (t == 0) {
      b.x = w0;
      b.y = w1;
    } else {
      b.z = w0;
      b.w = w1;
    }
  }
  // WG: the LDS byte addresses of the 8 fragment columns of stage s at K row 0 (A: ab, B: bb),
  // one VALU add each; every read is then one of them plus an immediate offset.  (With the slot
  // offset computed as (2 s) mod 5, the compiler re-derived every read's address with VALU adds
  // in the MFMA stream unless these went through an empty asm, which cost 16 register copies a
  // stage; with the carried slot offsets neither is needed.)
  template <int H = -1>
  __device__ __forceinline__ void wg_bases(int s, uint32_t (&ab)[4], uint32_t (&bb)[4]) const {
    const uint32_t sa = __builtin_amdgcn_readfirstlane(slot_bytes<H>(2 * s));
    const uint32_t sb = __builtin_amdgcn_readfirstlane(slot_bytes<H < 0 ? -1 : H + 1>(2 * s + 1));
#pragma unroll
    for (int i = 0; i < 4; ++i) ab[i] = a_seg[i] + sa;
#pragma unroll
    for (int j = 0; j < 4; ++j) bb[j] = b_off[j] + sb;
  }
  // WG: read r of sub-step kk: r < 8 half r & 1 of A fragment r >> 1, else half (r - 8) & 1 of
  // B fragment (r - 8) >> 1 (K rows 16 kk + 4 t .. + 3 of each lane's 8, as in read_tr_at)
  __device__ __forceinline__ void wg_read(const uint32_t (&ab)[4], const uint32_t (&bb)[4], int kk, int r,
                                          uint4 (&a)[4], uint4 (&b)[4]) const {
    const int t = r & 1;
    const uint32_t base = r < 8 ? ab[r >> 1] : bb[(r - 8) >> 1];
    uint4& d = r < 8 ? a[r >> 1] : b[(r - 8) >> 1];
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)(base + (16 * kk + 4 * t) * 512));
    const uint32_t w0 = (uint16_t)v[0] | ((uint32_t)(uint16_t)v[1] << 16);
    const uint32_t w1 = (uint16_t)v[2] | ((uint32_t)(uint16_t)v[3] << 16);
    if (t == 0) {
      d.x = w0;
      d.y = w1;
    } else {
      d.z = w0;
      d.w = w1;
    }
  }
  template <int H = -1>
  __device__ __forceinline__ void read(int s, int kk, uint4 (&a)[4], uint4 (&b)[4]) const {
    const uint32_t sa = slot_bytes<H>(2 * s);
    const uint32_t sb = slot_bytes<H < 0 ? -1 : H + 1>(2 * s + 1);
    if constexpr (BL == LAYOUT_WG) {
      uint32_t ab[4], bb[4];
      wg_bases<H>(s, ab, bb);
#pragma unroll
      for (int r = 0; r < 16; ++r) wg_read(ab, bb, kk, r, a, b);
      return;
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const uint4*)(L + sa + a_off + i * kAStr + ch[kk]);
    }
    if constexpr (BL == LAYOUT_KN) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        read_tr(sb, kk, j, 0, b[j]);
        read_tr(sb, kk, j, 1, b[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *(const uint4*)(L + sb + b_off[j] + ch[kk]);
    }
  }
  // fragment r of sub-step kk of stage s: r < 4 the A fragment of rows 32 r, else B fragment r - 4
  // (KN: r < 4 as above, else half (r - 4) & 1 of B fragment (r - 4) >> 1; 12 reads a set;
  // WG reads go through wg_read)
  template <int H = -1>
  __device__ __forceinline__ void read1(int s, int kk, int r, uint4 (&a)[4], uint4 (&b)[4]) const {
    constexpr int HB = H < 0 ? -1 : H + 1;
    if (r < 4) {
      a[r] = *(const uint4*)(L + slot_bytes<H>(2 * s) + a_off + r * kAStr + ch[kk]);
    } else if constexpr (BL == LAYOUT_KN) {
      read_tr(slot_bytes<HB>(2 * s + 1), kk, (r - 4) >> 1, (r - 4) & 1, b[(r - 4) >> 1]);
    } else {
      b[r - 4] = *(const uint4*)(L + slot_bytes<HB>(2 * s + 1) + b_off[r - 4] + ch[kk]);
    }
  }
  __device__ __forceinline__ void mma(const uint4 (&a)[4], const uint4 (&b)[4], int t0, int t1) const {
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (t >= t0 && t < t1) mma_rows<bf16_t>(a[t >> 2], b[t & 3], acc[t >> 2][t & 3]);
  }
  // one sub-step's 16 MFMAs with DMAs Q0 .. Q1-1 of operand OP of stage st spread between them
  template <int OP, int Q0, int Q1>
  __device__ __forceinline__ void step_dma(const uint4 (&a)[4], const uint4 (&b)[4], int st) const {
    constexpr int n = Q1 - Q0;
#pragma unroll
    for (int q = 0; q < n; ++q) {
      mma(a, b, q * 16 / n, (q + 1) * 16 / n);
      __builtin_amdgcn_sched_barrier(0);
      issue<OP>(st, Q0 + q);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  __device__ __forceinline__ void step(const uint4 (&a)[4], const uint4 (&b)[4]) const { mma(a, b, 0, 16); }
};

// The main loop of a wave whose last fragments lie past the end of its group (NF < 4 live
// fragments of the four): their MFMAs are left out, the reads, DMAs and barriers kept, so
// every wave of the tile still runs the same ring.  NF is a compile-time count, so each such
// loop is scheduled like the full one, only shorter.
template <typename PP, int NF>
struct SkipView {
  PP& P;
  f32x16 (&acc)[4][4];
  static constexpr int kBL = PP::kBL;
  template <int OP, bool CHK = true, int H = -1>
  __device__ __forceinline__ void issue(int st, int q) const { P.template issue<OP, CHK, H>(st, q); }
  template <int H = -1>
  __device__ __forceinline__ void read1(int s, int kk, int r, uint4 (&a)[4], uint4 (&b)[4]) const {
    P.template read1<H>(s, kk, r, a, b);
  }
  template <int H = -1>
  __device__ __forceinline__ void read(int s, int kk, uint4 (&a)[4], uint4 (&b)[4]) const {
    P.template read<H>(s, kk, a, b);
  }
  __device__ __forceinline__ void rotate() { P.rotate(); }
  __device__ __forceinline__ void mma(const uint4 (&a)[4], const uint4 (&b)[4], int t0, int t1) const {
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (t >= t0 && t < t1 && (t >> 2) < NF) mma_rows<bf16_t>(a[t >> 2], b[t & 3], P.acc[t >> 2][t & 3]);
  }
};

__device__ __forceinline__ void wait_vm8_lgkm0() { asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_vm18() { asm volatile("s_waitcnt vmcnt(18)" ::: "memory"); }
__device__ __forceinline__ void wait_vm16() { asm volatile("s_waitcnt vmcnt(16)" ::: "memory"); }

// Operand fragments of the four sub-steps of a stage: set u holds sub-step u.
struct Frags {
  uint4 a[4][4], b[4][4];
};

// One sub-step: the 16 MFMAs of set CUR, one LDS read after each of them when RD (the
// fragments of sub-steps R0 and R0 + 1 of stage rs, into their sets), and DMAs Q0 .. Q1-1
// of operand OP of stage st spread between them.  HR, HD: the first half-stages of stages rs
// and st, counted from the current stage's (compile-time slot distances).
template <typename PP, int CUR, bool RD, int R0, int OP, int Q0, int Q1, bool CHK, int HR, int HD>
__device__ __forceinline__ void substep(const PP& P, Frags& f, int rs, int st) {
  constexpr int n = Q1 - Q0;
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    P.mma(f.a[CUR], f.b[CUR], t, t + 1);
    if (RD) {
      if (t < 8) P.template read1<HR>(rs, R0, t, f.a[R0], f.b[R0]);
      else P.template read1<HR>(rs, R0 + 1, t - 8, f.a[R0 + 1], f.b[R0 + 1]);
    }
#pragma unroll
    for (int q = 0; q < n; ++q)
      if (t == (2 * q + 1) * 16 / (2 * (n > 0 ? n : 1))) P.template issue<OP, CHK, HD + OP>(st, Q0 + q);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// KN form of a sub-step: the reads of one fragment set (set R0 of stage rs: 12 for KN, 16 for
// WG), one after each of the first MFMAs.
template <typename PP, int CUR, bool RD, int R0, int OP, int Q0, int Q1, bool CHK, int HR, int HD>
__device__ __forceinline__ void substep_kn(const PP& P, Frags& f, int rs, int st) {
  constexpr int n = Q1 - Q0;
  constexpr bool WG = PP::kBL == LAYOUT_WG;
  constexpr int NR = WG ? 16 : 12;
  uint32_t ab[4], bb[4];
  if constexpr (WG)
    if (RD) P.template wg_bases<HR>(rs, ab, bb);
#pragma unroll
  for (int t = 0; t < 16; ++t) {
    P.mma(f.a[CUR], f.b[CUR], t, t + 1);
    if constexpr (WG) {
      if (RD) P.wg_read(ab, bb, R0, t, f.a[R0], f.b[R0]);
    } else if (RD && t < NR) {
      P.template read1<HR>(rs, R0, t, f.a[R0], f.b[R0]);
    }
#pragma unroll
    for (int q = 0; q < n; ++q)
      if (t == (2 * q + 1) * 16 / (2 * (n > 0 ? n : 1))) P.template issue<OP, CHK, HD + OP>(st, Q0 + q);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One stage.  Sub-step 0 reads the fragments of sub-steps 2 and 3, sub-step 2 those of
// sub-steps 0 and 1 of the next stage, so every read has at least a sub-step of MFMAs
// to land; the barrier sits between sub-steps 1 and 2, after the last reads of the
// stage.  Loads: the A half of stage s+2 (DMAs 2..7) in sub-steps 0 and 1, the B half of
// stage s+2 in sub-step 2 and DMAs 0..1 of the A half of stage s+3 in sub-step 3.
// LOADS = 2: all of those; 1: no A half of stage s+3; 0: none.  VMC: the vmcnt the
// barrier waits for (the DMAs issued after the B half of stage s+1).
// The KN form reads one set per sub-step instead (sets 2 and 3 of stage s in sub-steps 0 and
// 1, sets 0 and 1 of stage s+1 in sub-steps 2 and 3): the same slots are read before the same
// barrier, and every read still has a sub-step of MFMAs to land.
template <typename PP, int LOADS, bool NEXT, int VMC, bool CHK = true>
__device__ __forceinline__ void stage(const PP& P, int s, Frags& f) {
  constexpr int L1 = LOADS ? 1 : 0, L2 = LOADS == 2 ? 1 : 0;
  constexpr bool KN = PP::kBL == LAYOUT_KN || PP::kBL == LAYOUT_WG;
  if constexpr (KN) {
    substep_kn<PP, 0, true, 2, 0, 2, 2 + 3 * L1, CHK, 0, 4>(P, f, s, s + 2);
    substep_kn<PP, 1, true, 3, 0, 5, 5 + 3 * L1, CHK, 0, 4>(P, f, s, s + 2);
  } else {
    substep<PP, 0, true, 2, 0, 2, 2 + 3 * L1, true, 0, 4>(P, f, s, s + 2);
    substep<PP, 1, false, 0, 0, 5, 5 + 3 * L1, true, 0, 4>(P, f, s, s + 2);
  }
  if (NEXT) {
    if (VMC == 8) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    dma_barrier();  // stage s+1 landed and visible; every read of stage s done
  }
  if constexpr (KN) {
    substep_kn<PP, 2, NEXT, 0, 1, 0, 8 * L1, CHK, 2, 4>(P, f, s + 1, s + 2);
    substep_kn<PP, 3, NEXT, 1, 0, 0, 2 * L2, CHK, 2, 6>(P, f, s + 1, s + 3);
  } else {
    substep<PP, 2, NEXT, 0, 1, 0, 8 * L1, true, 2, 4>(P, f, s + 1, s + 2);
    substep<PP, 3, false, 0, 0, 0, 2 * L2, true, 2, 6>(P, f, s + 1, s + 3);
  }
}

template <typename PP>
__device__ __forceinline__ void mainloop(PP& P, int nk) {
  if (nk <= 0) return;
  // prologue: stages 0 and 1, and DMAs 0..1 of the A half of stage 2
#pragma unroll
  for (int q = 0; q < kQ; ++q) P.template issue<0, true, 0>(0, q);
#pragma unroll
  for (int q = 0; q < kQ; ++q) P.template issue<1, true, 1>(0, q);
  if (nk > 1) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) P.template issue<0, true, 2>(1, q);
#pragma unroll
    for (int q = 0; q < kQ; ++q) P.template issue<1, true, 3>(1, q);
  }
  // the accumulators are zeroed here, while the first stages are in flight (left to itself
  // the compiler zeroed them after the first wait, 256 writes on the tile's critical path)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(P.acc[i][j]));
  // The weight gradient's last stage may be partly filled: a wave whose DMA of it covers no row
  // before the reduction's end writes zeros with LDS stores and issues no DMA at all, so a wait
  // that counts DMAs still outstanding must not count on that stage's.  There it waits for all.
  constexpr bool WG = PP::kBL == LAYOUT_WG;
  if (nk > 2) {
    P.template issue<0, true, 4>(2, 0);
    P.template issue<0, true, 4>(2, 1);
    if (WG && nk == 3) wait_all_0();
    else wait_vm18();
  } else if (nk > 1 && !WG) {
    wait_vm16();
  } else {
    wait_all_0();
  }
  dma_barrier();
  Frags f;
  P.template read<0>(0, 0, f.a[0], f.b[0]);
  P.template read<0>(0, 1, f.a[1], f.b[1]);
  __builtin_amdgcn_sched_barrier(0);
  int s = 0;
  if constexpr (PP::kBL == LAYOUT_WG) {
    // stages up to nk - 5 load nothing of the last stage: no zero-fill checks there
    for (; s + 4 < nk; ++s, P.rotate()) stage<PP, 2, true, 8, false>(P, s, f);
  }
  for (; s + 3 < nk; ++s, P.rotate()) stage<PP, 2, true, 8>(P, s, f);
  if (s + 2 < nk) {
    // its mid-stage wait would count the DMAs of stage s + 2, the last one
    stage<PP, 1, true, WG ? 0 : 8>(P, s++, f);
    P.rotate();
  }
  if (s + 1 < nk) {
    stage<PP, 0, true, 0>(P, s++, f);
    P.rotate();
  }
  stage<PP, 0, false, 0>(P, s, f);
}

}  // namespace ring4


// Partial tiles of the split tail: a wave's 128 x 128 block is 64 float4 per lane,
// coalesced per register group.  The pieces of a tile run on any XCD, and each XCD has its
// own L2, so the partials travel through memory.  They are written with system-scope buffer
// stores (sc0 sc1: written through L1 and L2), whose vmcnt completes once they are visible
// there, so a piece only waits for vmcnt(0) before counting itself.  The last piece reads
// them with ordinary loads after its count returned: a slot is written once and read once
// per launch, so no L1 or L2 holds an older copy of it (the caches are invalidated at launch).
// Device-scope fences here wrote back and invalidated the whole L2, full of the GEMM's
// output, twice a piece: 45-50 us of the tail.  (System-scope loads as well made the
// compiler spill around the main loop: gate/up 4-8% slower.)  The store descriptor covers
// the one slot, so a store outside it writes nothing.
namespace ring4 {

typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr int kSysScope = 1 | 16;  // cache-policy bits sc0 | sc1 of a buffer access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const GemmParams& p, int slot) {
  return __builtin_amdgcn_make_buffer_rsrc(p.ws_part + (size_t)slot * kSplitSlotFloats, (short)0,
                                           kSplitSlotFloats * (int)sizeof(float), 0x00020000);
}
// byte offset in the slot of this lane's float4 r (0..63) of the wave's block
__device__ __forceinline__ int part_off(int r) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  return (wave * 4096 + lane + r * 64) * 16;
}

__device__ __forceinline__ void store_partial(const GemmParams& p, int slot, const f32x16 (&acc)[4][4]) {
  const __amdgpu_buffer_rsrc_t rs = part_rsrc(p, slot);
#pragma unroll
  for (int t = 0; t < 16; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x16& a = acc[t >> 2][t & 3];
      const i32x4 w = {__float_as_int(a[4 * e]), __float_as_int(a[4 * e + 1]), __float_as_int(a[4 * e + 2]),
                       __float_as_int(a[4 * e + 3])};
      __builtin_amdgcn_raw_buffer_store_b128(w, rs, part_off(t * 4 + e), 0, kSysScope);
    }
}

// Epilogue through LDS.  A wave's results leave the MFMAs with 4 consecutive columns per
// lane (row lane & 31 of fragment i, columns 8 q + 4 (lane >> 5) + 0..3), so direct stores
// would write 16 bytes to each of 32 rows per instruction.  Instead the wave converts its
// 128-row block to bf16 in its own 32 KB of LDS (16-byte chunks XORed with the row, as in
// the ring) and reads it back a row segment at a time: each store then writes whole rows
// of CW columns (CW = 128: 4 rows of 256 bytes, CW = 64: 8 rows of 128 bytes).
template <int CW>
struct Out {
  static constexpr int kCPR = CW / 8;         // 16-byte chunks per row
  static constexpr int kRowBytes = CW * 2;
  static constexpr int kRPI = 64 / kCPR;      // rows per store instruction
  // columns 8 q + 4 hi + 0..3 of fragment jc at local row r
  __device__ static void put(char* wl, int r, int jc, int q, int hi, const float (&v)[4]) {
    const int chunk = (jc * 4 + q) ^ (r % kCPR);
    *(uint2*)(wl + r * kRowBytes + chunk * 16 + hi * 8) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
  // local rows 0 .. NR-1 = rows row0 .. row0 + NR - 1 (those below re) of columns col0 ..
  // col0 + CW - 1 (those below ncols, a multiple of 8) to base + row * ld + col * 2; the stores
  // are non-temporal: the kernel never reads its output back
  // IL: local row r is row row0 + 64 (r / 32) + r % 32 (a wave's interleaved fragments)
  template <int NR = 128, bool IL = false>
  __device__ static void flush(const char* wl, char* base, int64_t ld, int64_t row0, int64_t re, int64_t col0,
                               int64_t ncols) {
    const int lane = threadIdx.x & 63;
    const int c = lane % kCPR, rr = lane / kCPR;
    const int64_t col = col0 + c * 8;
    const bool cok = col < ncols;
    // in batches of 8 rows: the 8 LDS reads are in flight together before the 8 stores (one
    // read, wait, store at a time left each store waiting for its own read)
    constexpr int kIt = NR / kRPI, kB = kIt < 8 ? kIt : 8;
#pragma unroll
    for (int i0 = 0; i0 < kIt; i0 += kB) {
      uint4 v[kB];
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int r = (i0 + u) * kRPI + rr;
        v[u] = *(const uint4*)(wl + r * kRowBytes + ((c ^ (r % kCPR)) * 16));
      }
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int r = (i0 + u) * kRPI + rr;
        const int64_t row = row0 + (IL ? ((r >> 5) << 6) + (r & 31) : r);
        if (cok && row < re) st_nt((uint4*)(base + row * ld + col * 2), v[u]);
      }
    }
  }
};

// The ring kernel's epilogue (bf16 outputs; EPI_NONE or EPI_SWIGLU) for the wave's 128-row
// block at row0; wl = this wave's 32 KB of LDS, free of every other wave's accesses.
template <int EPI, bool IL = false>
__device__ __forceinline__ void store_tile_lds(const GemmParams& p, const f32x16 (&acc)[4][4], char* wl,
                                               int64_t row0, int64_t re, int64_t col0) {
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  if constexpr (EPI == EPI_SWIGLU) {
    // h (and, when saved, the gate half) in phase 1, the up half in phase 2
    const int64_t F = p.N / 2;
    char* wl2 = wl + 16384;
    const bool save = p.epi_save != nullptr;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float h[4], g[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            g[e] = acc[i][j][4 * q + e];
            h[e] = g[e] * sigmoid_fast(g[e]) * acc[i][j + 2][4 * q + e];
          }
          Out<64>::put(wl, i * 32 + l32, j, q, hi, h);
          if (save) Out<64>::put(wl2, i * 32 + l32, j, q, hi, g);
        }
    Out<64>::flush<128, IL>(wl, (char*)p.C, F * 2, row0, re, col0, F);
    if (save) {
      Out<64>::flush<128, IL>(wl2, (char*)p.epi_save, p.N * 2, row0, re, col0, F);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float u[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) u[e] = acc[i][j + 2][4 * q + e];
            Out<64>::put(wl, i * 32 + l32, j, q, hi, u);
          }
      // the up half sits F columns to the right of the gate half of the saved row
      Out<64>::flush<128, IL>(wl, (char*)p.epi_save + F * 2, p.N * 2, row0, re, col0, F);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
          Out<128>::put(wl, i * 32 + l32, j, q, hi, v);
        }
    Out<128>::flush<128, IL>(wl, (char*)p.C, p.N * 2, row0, re, col0, p.N);
  }
}

// SwiGLU backward through LDS: acc = dH for the wave's 128 rows x 128 columns at (row0, col0);
// epi_in = saved [G | U] of width 2F (F = N); C [M, 2F] = [dH U silu'(G) | dH silu(G)].  In
// rounds of 32 rows, double-buffered in the wave's 32 KB of LDS: round i + 1's rows of G and U
// go global -> LDS by DMA (in the row swizzle of Out<128>) while round i is computed in place,
// and round i leaves as whole row segments after a wait that covers round i + 1's loads and
// round i - 1's stores, both issued before round i's arithmetic.  (Loading each round only after
// the previous round's stores left a memory round trip a round: 24 of a tile's 115 µs.)
__device__ __forceinline__ void store_tile_dswiglu_lds(const GemmParams& p, const f32x16 (&acc)[4][4], char* wl,
                                                       int64_t row0, int64_t re, int64_t col0) {
  using O = Out<128>;
  const int64_t F = p.N;
  const int64_t ld = 4 * F;  // bytes per row of epi_in and of C
  const char* pre = (const char*)p.epi_in;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)wl);
  // round i's G and U rows into buffer b: DMA j of 8 fills rows 4 j .. 4 j + 3, lane L landing at
  // 16-byte position L % 16 of row 4 j + L / 16, which holds logical chunk (L % 16) ^ (row % 16).
  // Rows are clamped to M - 1 and columns to F - 8 (in bounds; such rows and columns are never
  // stored).
  auto issue = [&](int i, int b) {
    const int64_t rb = min(row0 + i * 32, p.M - 1);
    const char* base = uniform_ptr(pre + rb * ld);
    const uint32_t lb = lds0 + b * 16384;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + (lane >> 4);
      const int64_t row = min(row0 + i * 32 + r, p.M - 1);
      const int c = (lane & 15) ^ (r % O::kCPR);
      const int64_t col = min(col0 + c * 8, F - 8);
      const uint32_t off = (uint32_t)((row - rb) * ld + col * 2);
      dma(base, off, lb + j * 1024);
      dma(base, off + (uint32_t)(F * 2), lb + 8192 + j * 1024);
    }
  };
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    char* wg = wl + (i & 1) * 16384;
    char* wu = wg + 32 * O::kRowBytes;
    if (i < 3) issue(i + 1, (i + 1) & 1);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int off = l32 * O::kRowBytes + (((j * 4 + q) ^ (l32 % O::kCPR)) * 16) + hi * 8;
        const uint2 gv = *(const uint2*)(wg + off), uv = *(const uint2*)(wu + off);
        const float gs[4] = {__uint_as_float(gv.x << 16), __uint_as_float(gv.x & 0xffff0000u),
                             __uint_as_float(gv.y << 16), __uint_as_float(gv.y & 0xffff0000u)};
        const float us[4] = {__uint_as_float(uv.x << 16), __uint_as_float(uv.x & 0xffff0000u),
                             __uint_as_float(uv.y << 16), __uint_as_float(uv.y & 0xffff0000u)};
        float da[4], du[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[i][j][4 * q + e], gg = gs[e], sg = sigmoid_fast(gg);
          da[e] = v * us[e] * sg * (1.f + gg * (1.f - sg));
          du[e] = v * gg * sg;
        }
        *(uint2*)(wg + off) = make_uint2(pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3]));
        *(uint2*)(wu + off) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
      }
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");  // round i + 1 in LDS, round i - 1 out
    O::template flush<32>(wg, (char*)p.C, ld, row0 + i * 32, re, col0, F);
    O::template flush<32>(wu, (char*)p.C + F * 2, ld, row0 + i * 32, re, col0, F);
  }
}

// In batches of 16 float4 (four accumulator tiles): the loads of a batch are in flight together
// (one load, wait, add at a time made the reduction of a split tile latency-bound).
__device__ __forceinline__ void load_partial(const GemmParams& p, int slot, f32x16 (&acc)[4][4], bool add) {
  const float4* src = (const float4*)(p.ws_part + (size_t)slot * kSplitSlotFloats) + (threadIdx.x >> 6) * 4096 +
                      (threadIdx.x & 63);
#pragma unroll
  for (int t0 = 0; t0 < 16; t0 += 4) {
    float4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = src[(t0 * 4 + u) * 64];
    __builtin_amdgcn_sched_barrier(0);  // keep the batch's loads ahead of its adds
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int t = t0 + u / 4, e = u % 4;
      f32x16& a = acc[t >> 2][t & 3];
      if (add) {
        a[4 * e] += v[u].x; a[4 * e + 1] += v[u].y; a[4 * e + 2] += v[u].z; a[4 * e + 3] += v[u].w;
      } else {
        a[4 * e] = v[u].x; a[4 * e + 1] = v[u].y; a[4 * e + 2] = v[u].z; a[4 * e + 3] = v[u].w;
      }
    }
  }
}

}  // namespace ring4

// GA: gathered A rows (GemmParams::a_rows), N-by-K weights only
// SK (SwiGLU only): interleaved fragments and the MFMAs of fragments past the group's end left out
template <int EPI, int BL, bool GA = false, bool SK = false>
__global__ __launch_bounds__(ring4::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_ring4_kernel(GemmParams p) {
  static_assert(!GA || BL == LAYOUT_NK, "rows are gathered for N-by-K weights only");
  using namespace ring4;
  __shared__ uint4 smem[kSlots * kSlotUnits];
  int g, nt;
  int64_t m0, re;
  Piece pc;
  if (!find_tile<ring4::kThreads>(p, g, m0, re, nt, (int*)smem, &pc)) return;
  __syncthreads();  // every thread has read the tile from the scratch that the loads overwrite
  g = __builtin_amdgcn_readfirstlane(g);
  nt = __builtin_amdgcn_readfirstlane(nt);
  m0 = uniform64(m0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ldb = p.Kd * 2;
  // stages of this block: the whole K extent, or one piece of it
  const int nk = (int)(ldb / kStageBytes);
  const int k0 = pc.part >= 0 ? pc.part * nk / pc.f : 0;
  const int len = pc.part >= 0 ? (pc.part + 1) * nk / pc.f - k0 : nk;

  f32x16 acc[4][4];
  Pipe<EPI, BL, SK> P(acc, smem);
  P.a_base = uniform_ptr((const char*)p.A + (GA ? 0 : m0 * ldb) + (int64_t)k0 * kStageBytes);
  const int64_t b0row = EPI == EPI_SWIGLU ? (int64_t)nt * 128 : (int64_t)nt * 256;
  if constexpr (BL == LAYOUT_KN) {
    // B = [Kd rows][N] per group; a stage is 64 K rows; lanes of DMA q fill K row
    // 2 (wave * 8 + q) + lane / 32, 16 bytes each of the tile's 256 columns (clamped past N:
    // those columns are never stored)
    const int64_t ldn = p.N * 2;
    P.b_stage = 64 * ldn;
    P.b_base = uniform_ptr((const char*)p.B + (int64_t)g * p.Kd * ldn + (int64_t)k0 * 64 * ldn);
  } else {
    P.b_base = uniform_ptr((const char*)p.B + ((int64_t)g * p.N + b0row) * ldb + (int64_t)k0 * kStageBytes);
  }
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int r = (wave * kQ + q) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    int64_t ar = m0 + r;
    ar = ar < p.M ? ar : p.M - 1;
    P.va[q] = GA ? (uint32_t)((int64_t)min((uint32_t)p.a_rows[ar] / p.a_div, p.a_last) * ldb + c * 16)
                     : (uint32_t)((ar - m0) * ldb + c * 16);
    int64_t br;
    if constexpr (BL == LAYOUT_KN) {
      const int kr = (wave * kQ + q) * 2 + (lane >> 5);
      const int u = lane & 31;                                      // 16-byte unit of the LDS row
      const int lu = (((u >> 1) ^ ((kr & 3) << 1)) << 1) | (u & 1);  // the 8 columns it holds
      int64_t col = (int64_t)nt * 256 + lu * 8;
      col = col < p.N ? col : p.N - 8;
      P.vb[q] = (uint32_t)(kr * p.N * 2 + col * 2);
      continue;
    } else if (EPI == EPI_SWIGLU) {
      const int64_t F = p.N / 2;
      int64_t cc = (int64_t)nt * 128 + (r & 127);
      cc = cc < F ? cc : F - 1;
      br = (r < 128 ? 0 : F) + cc;
    } else {
      br = (int64_t)nt * 256 + r;
      br = br < p.N ? br : p.N - 1;
    }
    P.vb[q] = (uint32_t)((br - b0row) * ldb + c * 16);
  }
  if constexpr (decltype(P)::kIL) {
    // live fragments of this wave: its rows m0 + 32 wm + 64 i below the group's end
    const int64_t live = re - m0 - 32 * (wave >> 1);
    const int nf = live <= 0 ? 0 : live >= 256 ? 4 : (int)((live + 63) / 64);
    using PT = decltype(P);
    switch (__builtin_amdgcn_readfirstlane(nf)) {
      case 4: mainloop(P, len); break;
      case 3: { SkipView<PT, 3> sv{P, P.acc}; mainloop(sv, len); break; }
      case 2: { SkipView<PT, 2> sv{P, P.acc}; mainloop(sv, len); break; }
      case 1: { SkipView<PT, 1> sv{P, P.acc}; mainloop(sv, len); break; }
      default: { SkipView<PT, 0> sv{P, P.acc}; mainloop(sv, len); break; }
    }
  } else {
    mainloop(P, len);
  }
  __syncthreads();  // every wave is done with the ring: its LDS now holds the epilogue staging

  const int wm = wave >> 1, wn = wave & 1;
  if (pc.part >= 0) {
    // a piece of a split tile: publish the partial; the last piece of the tile reduces
    const int r = pc.slot % pc.R;
    store_partial(p, pc.slot, acc);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the partial is visible in memory
    int old = 0;
    if (lane == 0) old = atomicAdd(p.ws_count + r * 4 + wave, 1);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != pc.f - 1) return;
    asm volatile("" ::: "memory");  // the loads stay after the count that allowed them
    load_partial(p, r, acc, false);
    for (int j = 1; j < pc.f; ++j) load_partial(p, j * pc.R + r, acc, true);
    if (lane == 0) p.ws_count[r * 4 + wave] = 0;
  }
  if constexpr (EPI == EPI_DSWIGLU) {
    store_tile_dswiglu_lds(p, acc, (char*)smem + wave * 32768, m0 + wm * 128, re, (int64_t)nt * 256 + wn * 128);
  } else {
    const int64_t col0 = EPI == EPI_SWIGLU ? (int64_t)nt * 128 + wn * 64 : (int64_t)nt * 256 + wn * 128;
    constexpr bool IL = decltype(P)::kIL;
    store_tile_lds<EPI, IL>(p, acc, (char*)smem + wave * 32768, IL ? m0 + wm * 32 : m0 + wm * 128, re, col0);
  }
}

// ---------------------------------------------------------------------------
// dW[g] = dY_g^T X_g: output tile (n, kd) of group g, reduction over the group's rows.
constexpr int kMaxGroupsWg = 1024;  // group sizes the ring weight-gradient kernel sorts in LDS
constexpr int kWgBand = 4;          // column tiles of X in a band of the weight-gradient tile order

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

// dW epilogue of one wave: acc[i][j] covers rows row0 + 32 i and columns col0 + 32 j of
// one group's [N, Kd] fp32 gradient (lane layout as in store_tile).  Accumulate mode
// loads the previous values of a row first, all together, then adds and stores.
template <int NI, int NJ>
__device__ __forceinline__ void store_wgrad(float* out, const f32x16 (&acc)[NI][NJ], int64_t row0, int64_t col0,
                                            int64_t N, int64_t Kd, int accumulate) {
  using E = Elem<float>;
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int64_t row = row0 + i * 32 + l32;
    if (row >= N) continue;
    float prev[NJ][4][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (accumulate) {
          int64_t c = col0 + j * 32 + 8 * q + 4 * hi;
          c = c < Kd ? c : Kd - 4;
          E::load4(out, row * Kd + c, prev[j][q]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) prev[j][q][e] = 0.f;
        }
      }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t c = col0 + j * 32 + 8 * q + 4 * hi;
        if (c >= Kd) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = prev[j][q][e] + acc[i][j][4 * q + e];
        E::store4(out, row * Kd + c, v);
      }
  }
}

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
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[4][4];
  constexpr int BK = kRowBytes / Elem<T>::kBytes;
  const int nk = (int)((re - rs + BK - 1) / BK);
  ColLoader<T> la, lb;
  la.init(p.dY, p.N, n0, p.N, rs, re);
  lb.init(p.X, p.Kd, k0, p.Kd, rs, re);
  mainloop<T, EPI_NONE>(la, lb, nk, smem, acc);  // zeros when the group is empty
  if (p.accumulate && nk == 0) return;  // accumulate mode leaves an empty group's dW as it is
  store_wgrad<4, 4>(p.dW + (int64_t)g * p.N * p.Kd, acc, n0 + wm * 128, k0 + wn * 128, p.N, p.Kd, p.accumulate);
}

// Eight-wave weight gradient (bf16): both operands are read along the group's
// rows (OpCol); rows past the group end come from the zero block.
//
// Every group has the same number of output tiles but a tile's cost grows with
// the group's row count, so tiles are handed out longest group first (groups
// ranked by row count, ties by index): the short tiles of small groups then
// fill the machine at the end instead of a few long ones trailing.  The XCD
// remap is applied per window of 256 blocks, which keeps that order in time
// while each XCD still runs contiguous tiles of a window.
template <int NQ>
__global__ __launch_bounds__(kThreads8) __attribute__((amdgpu_waves_per_eu(2, 2)))
void grouped_wgrad8_kernel(WgradParams p) {
  __shared__ uint4 smem[kDmaUnits];
  __shared__ int s_rows[kThreads8];
  __shared__ int s_group;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t tpg = (int64_t)p.TN * p.TK;
  const int64_t total = tpg * p.G;
  const int64_t win = (int64_t)blockIdx.x / kWindow * kWindow;
  const int64_t L = win + xcd_remap((int64_t)blockIdx.x - win, min((int64_t)kWindow, total - win));
  const int rank = (int)(L / tpg);
  int g = rank;
  if (p.G <= kThreads8) {
    int64_t rs, re;
    int rows = 0;
    if (tid < p.G) {
      group_rows(p.offs, tid, p.M, rs, re);
      rows = (int)(re - rs);
      s_rows[tid] = rows;
    }
    if (tid == 0) s_group = 0;
    __syncthreads();
    if (tid < p.G) {
      int r = 0;
      for (int h = 0; h < p.G; ++h) {
        const int o = s_rows[h];
        r += (o > rows) | ((o == rows) & (h < tid));
      }
      if (r == rank) s_group = tid;
    }
    __syncthreads();
    g = s_group;
  }
  const int rem = (int)(L - (int64_t)rank * tpg);
  const int tk = rem / p.TN;  // neighbouring tiles share the same X columns
  const int tn = rem % p.TN;
  int64_t rs, re;
  group_rows(p.offs, g, p.M, rs, re);
  const int64_t n0 = (int64_t)tn * kTile, k0 = (int64_t)tk * kTile;
  const int nk = (int)((re - rs + Stage<NQ>::kColRows - 1) / Stage<NQ>::kColRows);
  OpCol<NQ> oa, ob;
  oa.init(p.dY, p.N, n0, p.N, rs, re);
  ob.init(p.X, p.Kd, k0, p.Kd, rs, re);
  f32x16 acc[4][2];
  run_mainloop<NQ, bf16_t, EPI_NONE>(oa, ob, nk, smem, acc);  // zeros when the group is empty

  const int wm = wave >> 2, wn = wave & 3;
  if (p.accumulate && nk == 0) return;  // accumulate mode leaves an empty group's dW as it is
  store_wgrad<4, 2>(p.dW + (int64_t)g * p.N * p.Kd, acc, n0 + wm * 128, k0 + wn * 64, p.N, p.Kd, p.accumulate);
}

// Weight-gradient epilogue of a ring wave: acc[i][j] = rows row0 + 32 i (N index) and columns
// col0 + 32 j (Kd index) of one group's [N, Kd] fp32 dW, a lane holding 4 consecutive columns.
// Through the wave's 32 KB of LDS in two rounds of 64 rows (16-byte chunks XORed with the
// row), so each store (or accumulate) covers two whole rows of 512 bytes.
__device__ __forceinline__ void store_wgrad_lds(float* out, const f32x16 (&acc)[4][4], char* wl, int64_t row0,
                                                int64_t col0, int64_t N, int64_t Kd, int accumulate) {
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int c = lane & 31, rr = lane >> 5;
  const int64_t col = col0 + c * 4;
  const bool cok = col < Kd;  // Kd is a multiple of 8: a chunk of 4 columns is all in or all out
#pragma unroll
  for (int i0 = 0; i0 < 4; i0 += 2) {
#pragma unroll
    for (int di = 0; di < 2; ++di)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = di * 32 + l32;
          const int chunk = (j * 8 + 2 * q + hi) ^ (r & 31);
          const f32x16& a = acc[i0 + di][j];
          *(float4*)(wl + r * 512 + chunk * 16) = make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
        }
    // in batches of 8 rows: a batch's LDS reads (and, accumulating, its dW loads) are all in
    // flight before its first store, not one read, wait and store at a time
#pragma unroll
    for (int i1 = 0; i1 < 32; i1 += 8) {
      float4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = (i1 + u) * 2 + rr;
        v[u] = *(const float4*)(wl + r * 512 + ((c ^ (r & 31)) * 16));
      }
      if (accumulate) {
        float4 o[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t row = row0 + i0 * 32 + (i1 + u) * 2 + rr;
          o[u] = cok && row < N ? *(const float4*)(out + row * Kd + col) : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        __builtin_amdgcn_sched_barrier(0);  // keeps the 8 loads ahead of the first add
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          v[u].x += o[u].x; v[u].y += o[u].y; v[u].z += o[u].z; v[u].w += o[u].w;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t row = row0 + i0 * 32 + (i1 + u) * 2 + rr;
        if (cok && row < N) *(float4*)(out + row * Kd + col) = v[u];
      }
    }
  }
}

// Weight gradient on the ring pipeline: dW_g[n0:n0+256, k0:k0+256] = dY_g^T X_g over the
// group's rows, 64 rows a stage (the last one zero-filled past the group's end).  Groups are
// taken by decreasing size; within a group the tiles go in bands of column tiles of X.
__global__ __launch_bounds__(ring4::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_wgrad_ring_kernel(WgradParams p) {
  using namespace ring4;
  __shared__ uint4 smem[kSlots * kSlotUnits];
  int* s_rows = (int*)smem;  // group sizes, before any load targets the LDS
  int* s_group = s_rows + kMaxGroupsWg;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t tpg = (int64_t)p.TN * p.TK;
  const int64_t total = tpg * p.G;
  const int64_t win = (int64_t)blockIdx.x / kWindow * kWindow;
  const int64_t L = win + xcd_remap((int64_t)blockIdx.x - win, min((int64_t)kWindow, total - win));
  const int rank = (int)(L / tpg);
  for (int h = tid; h < p.G; h += ring4::kThreads) {
    int64_t a, b;
    group_rows(p.offs, h, p.M, a, b);
    s_rows[h] = (int)(b - a);
  }
  if (tid == 0) s_group[0] = 0;
  __syncthreads();
  for (int h = tid; h < p.G; h += ring4::kThreads) {
    const int rows = s_rows[h];
    int r = 0;
    for (int u = 0; u < p.G; ++u) {
      const int o = s_rows[u];
      r += (o > rows) | ((o == rows) & (u < h));
    }
    if (r == rank) s_group[0] = h;
  }
  __syncthreads();
  const int g = __builtin_amdgcn_readfirstlane(s_group[0]);
  __syncthreads();  // every thread has read the scratch before the loads overwrite it
  // Bands of kWgBand column tiles of X, the tiles of a band in column-major order: the 32
  // consecutive tiles one XCD runs together cover 4 column tiles of X by 8 of dY, so its L2
  // streams 12 operand panels a stage instead of 33 with a row of 32 dY tiles.
  const int rem = (int)(L - (int64_t)rank * tpg);
  const int band = rem / (kWgBand * p.TN);
  const int h = min(kWgBand, p.TK - band * kWgBand);
  const int w = rem - band * kWgBand * p.TN;
  const int tk = band * kWgBand + w % h;
  const int tn = w / h;
  int64_t rs, re;
  group_rows(p.offs, g, p.M, rs, re);
  rs = uniform64(rs);
  const int rows = (int)(re - rs);
  const int64_t n0 = (int64_t)tn * kTile, k0 = (int64_t)tk * kTile;
  const int nk = (rows + 63) / 64;

  f32x16 acc[4][4];
  Pipe<EPI_NONE, LAYOUT_WG> P(acc, smem);
  const int64_t lda = p.N * 2, ldb = p.Kd * 2;
  P.a_stage = 64 * lda;
  P.b_stage = 64 * ldb;
  P.kvalid = rows;
  P.a_base = uniform_ptr((const char*)p.dY + rs * lda);
  P.b_base = uniform_ptr((const char*)p.X + rs * ldb);
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    // lanes of DMA q fill row 2 (wave * 8 + q) + lane / 32 of the stage, 16 bytes each of the
    // tile's 256 columns (clamped past the width: those outputs are never stored)
    const int kr = (wave * kQ + q) * 2 + (lane >> 5);
    const int u = lane & 31;
    const int lu = (((u >> 1) ^ ((kr & 3) << 1)) << 1) | (u & 1);
    int64_t ca = n0 + lu * 8, cb = k0 + lu * 8;
    ca = ca < p.N ? ca : p.N - 8;
    cb = cb < p.Kd ? cb : p.Kd - 8;
    P.va[q] = (uint32_t)(kr * lda + ca * 2);
    P.vb[q] = (uint32_t)(kr * ldb + cb * 2);
  }
  mainloop(P, nk);  // zeros when the group is empty
  __syncthreads();  // every wave is done with the ring: its LDS now holds the epilogue staging
  if (p.accumulate && nk == 0) return;  // accumulate mode leaves an empty group's dW as it is
  const int wm = wave >> 1, wn = wave & 1;
  store_wgrad_lds(p.dW + (int64_t)g * p.N * p.Kd, acc, (char*)smem + wave * 32768, n0 + wm * 128, k0 + wn * 128,
                  p.N, p.Kd, p.accumulate);
}

// nq: DMA instructions per wave per operand per stage (4: 64-element stages, 2: 32-element
// stages), 0 for the register-staged kernel
template <typename T>
hipError_t gemm_dispatch(const GemmParams& prm, int b_layout, int epi, int nq, dim3 grid, hipStream_t s) {
#define MOE_GG(BL, EP) hipLaunchKernelGGL((grouped_gemm_kernel<T, BL, EP>), grid, dim3(kThreads), 0, s, prm)
#define MOE_GG8(EP, BL)                                                                                   \
  do {                                                                                                    \
    if (nq == 4) hipLaunchKernelGGL((grouped_gemm8_kernel<T, EP, BL, 4>), grid, dim3(kThreads8), 0, s, prm); \
    else hipLaunchKernelGGL((grouped_gemm8_kernel<T, EP, BL, 2>), grid, dim3(kThreads8), 0, s, prm);        \
  } while (0)
  if (b_layout == LAYOUT_NK) {
    if (nq) {
      if (epi == EPI_NONE) MOE_GG8(EPI_NONE, LAYOUT_NK);
      else if (epi == EPI_SWIGLU) MOE_GG8(EPI_SWIGLU, LAYOUT_NK);
      else MOE_GG8(EPI_DSWIGLU, LAYOUT_NK);
    } else {
      if (epi == EPI_NONE) MOE_GG(LAYOUT_NK, EPI_NONE);
      else if (epi == EPI_SWIGLU) MOE_GG(LAYOUT_NK, EPI_SWIGLU);
      else MOE_GG(LAYOUT_NK, EPI_DSWIGLU);
    }
  } else {
    if (epi == EPI_SWIGLU) return hipErrorInvalidValue;
    if constexpr (std::is_same<T, bf16_t>::value) {
      if (nq) {
        if (epi == EPI_NONE) MOE_GG8(EPI_NONE, LAYOUT_KN);
        else MOE_GG8(EPI_DSWIGLU, LAYOUT_KN);
        return hipGetLastError();
      }
    }
    if (epi == EPI_NONE) MOE_GG(LAYOUT_KN, EPI_NONE);
    else MOE_GG(LAYOUT_KN, EPI_DSWIGLU);
  }
#undef MOE_GG
#undef MOE_GG8
  return hipGetLastError();
}

}  // namespace

size_t grouped_gemm_workspace_bytes() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return kSplitCountBytes + (size_t)cus * kSplitSlotFloats * sizeof(float);
}

// ---------------------------------------------------------------------------
// MXFP8 grouped GEMM (N-by-K weights): A [M][Kd] and B [G][N][Kd] are FP8 E4M3 codes with
// one E8M0 scale per 32 consecutive Kd values of a row; C = A_g . B_g^T in fp32, bf16 out
// (plain or SwiGLU epilogue).  256 x 256 tiles in the grouped order of find_tile, 4 waves of
// 128 x 128.  A stage is 128 Kd values (128 bytes a row) of both operands plus their 4 scale
// bytes a row, moved by LDS DMA into one of two 66 KB slots while the other is read (one
// barrier a stage: it publishes the stage and frees the slot the next one loads into).  The
// MFMA v_mfma_scale_f32_32x32x64_f8f6f4 takes 32 bytes a lane for 64 Kd values of a row
// split over two lanes (hi = 0, 1); the hardware applies lane hi's scale byte to bytes
// 16 hi .. 16 hi + 15 of both lanes.  So lane hi holds Kd values 64 j + 16 hi .. + 15 (block
// 2 j) then 64 j + 32 + 16 hi .. + 15 (block 2 j + 1) of sub-step j, and the scale of block
// 2 j + hi.
namespace mxg {
constexpr int kMxRow = 128;                     // Kd values of a row per stage
constexpr int kOpBytes = 256 * kMxRow;          // 32 KB: one operand's rows of a stage
constexpr int kScaleOff = 2 * kOpBytes;            // then 256 scale words of A, 256 of B
constexpr int kSlotBytes = 2 * kOpBytes + 2 * 1024;
constexpr int kQ = 8;                              // row DMAs of one operand per wave per stage

__device__ __forceinline__ void dma4(const char* sbase, uint32_t voff, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1 offset:0"
               :: "v"(voff), "s"(sbase), "s"(lds_byte) : "memory", "m0");
}
__device__ __forceinline__ void wait_none() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory"); }

typedef int i32x8 __attribute__((ext_vector_type(8)));

// The SwiGLU epilogue with MXFP8 output: h = silu(g) u for the wave's 128 rows x 64 columns,
// fragment i at rows row0 + 64 i .. + 31 (a wave row's interleaved fragments), columns col0 ..,
// rounded to bf16 (so the bytes equal quantising the bf16 H afterwards), then quantised in
// 32-column blocks: fragment j of a row is one block, its 32 values held by lanes l32 (columns
// 8 q + 0..3) and l32 + 32 (8 q + 4..7), which exchange their maxima.  The codes go through the
// wave's LDS (wl: 64 bytes a row, two rows to a 128-byte line, 16-byte pieces XOR-swizzled by
// the line) and leave as whole 16-byte pieces; lane l32 writes the row's two scale bytes.
// A piece holds columns 16 p .. 16 p + 15 as the words (q even, hi 0), (q odd, hi 0), (q even,
// hi 1), (q odd, hi 1); the flush puts the words back in column order.
// Requires F = N / 2 with F % 32 == 0.
__device__ __forceinline__ uint32_t mxq_lds_off(int lr, int piece) {
  return (uint32_t)((lr >> 1) * 128 + ((((lr & 1) << 2) | piece) ^ ((lr >> 1) & 7)) * 16);
}
__device__ __forceinline__ void store_tile_mxq(const GemmParams& p, const f32x16 (&acc)[4][4], char* wl,
                                               int64_t row0, int64_t re, int64_t col0) {
  const int lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t F = p.N / 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int lr = i * 32 + l32;  // local row
    const int64_t row = row0 + i * 64 + l32;
    uint32_t sc = 0;  // the row's two scale bytes (blocks j = 0, 1)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float h[16];
      float amax = 0.f;
#pragma unroll
      for (int t = 0; t < 16; ++t) {
        const float g = acc[i][j][t], u = acc[i][j + 2][t];
        h[t] = (float)(__bf16)(g * sigmoid_fast(g) * u);
        amax = fmaxf(amax, fabsf(h[t]));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
      const int shared = mx_shared_exponent(amax);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *(uint32_t*)(wl + mxq_lds_off(lr, 2 * j + (q >> 1)) + 8 * hi + 4 * (q & 1)) =
            e4m3_pack4(ldexpf(h[4 * q], -shared), ldexpf(h[4 * q + 1], -shared), ldexpf(h[4 * q + 2], -shared),
                       ldexpf(h[4 * q + 3], -shared));
      sc |= (uint32_t)(shared + 127) << (8 * j);
    }
    if (hi == 0 && row < re && col0 < F) {
      p.cs[row * (F / 32) + col0 / 32] = (uint8_t)sc;
      if (col0 + 32 < F) p.cs[row * (F / 32) + col0 / 32 + 1] = (uint8_t)(sc >> 8);
    }
  }
  // each lane reads and stores one 16-byte piece: 4 pieces a row, 16 rows an instruction
  const int c = lane & 3, rr = lane >> 2;
  const int64_t col = col0 + c * 16;
  uint8_t* codes = (uint8_t*)p.C;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int lr = k * 16 + rr;
    const uint4 v = *(const uint4*)(wl + mxq_lds_off(lr, c));
    const int64_t row = row0 + ((lr >> 5) << 6) + (lr & 31);
    if (row < re && col < F) st_nt((uint4*)(codes + row * F + col), make_uint4(v.x, v.z, v.y, v.w));
  }
}
}  // namespace mxg

template <int EPI>
__global__ __launch_bounds__(ring4::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void grouped_gemm_mx_kernel(GemmParams p) {
  using namespace mxg;
  __shared__ uint4 smem[2 * kSlotBytes / 16];
  int g, nt;
  int64_t m0, re;
  Piece pc;
  if (!find_tile<ring4::kThreads>(p, g, m0, re, nt, (int*)smem, &pc)) return;
  __syncthreads();  // every thread has read the tile from the scratch that the loads overwrite
  g = __builtin_amdgcn_readfirstlane(g);
  nt = __builtin_amdgcn_readfirstlane(nt);
  m0 = ring4::uniform64(m0);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, hi = lane >> 5;
  const int64_t ld = p.Kd;           // bytes per row of codes
  const int64_t lds_ = p.Kd / 32;    // bytes per row of scales
  // stages of this block: the whole Kd extent, or one piece of it (a split tile of the tail)
  const int nkt = (int)(p.Kd / kMxRow);
  const int k0 = pc.part >= 0 ? pc.part * nkt / pc.f : 0;
  const int nk = pc.part >= 0 ? (pc.part + 1) * nkt / pc.f - k0 : nkt;
  constexpr bool SW = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_MX;  // gate|up B rows
  const int64_t b0row = SW ? (int64_t)nt * 128 : (int64_t)nt * 256;
  const int64_t F = p.N / 2;
  // the tile's B row of local row r (SwiGLU: gate rows, then the matching up rows)
  auto brow = [&](int r) -> int64_t {
    int64_t br;
    if (SW) {
      int64_t cc = (int64_t)nt * 128 + (r & 127);
      cc = cc < F ? cc : F - 1;
      br = (r < 128 ? 0 : F) + cc;
    } else {
      br = (int64_t)nt * 256 + r;
      br = br < p.N ? br : p.N - 1;
    }
    return (int64_t)g * p.N + br;
  };
  auto arow = [&](int r) -> int64_t {
    const int64_t ar = m0 + r;
    return ar < p.M ? ar : p.M - 1;
  };
  // uniform bases at the tile's first rows; per-lane 32-bit offsets of rows relative to them
  // (within (N + 256) Kd bytes, checked on the host)
  const int64_t b_first = (int64_t)g * p.N + b0row;
  const char* a_base = ring4::uniform_ptr((const char*)p.A + m0 * ld + (int64_t)k0 * kMxRow);
  const char* b_base = ring4::uniform_ptr((const char*)p.B + b_first * ld + (int64_t)k0 * kMxRow);
  const char* sa_base = ring4::uniform_ptr((const char*)p.sa + m0 * lds_ + k0 * 4);
  const char* sb_base = ring4::uniform_ptr((const char*)p.sb + b_first * lds_ + k0 * 4);
  uint32_t va[kQ], vb[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int r = (wave * kQ + q) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ring4::swz(r);
    va[q] = (uint32_t)((arow(r) - m0) * ld + c * 16);
    vb[q] = (uint32_t)((brow(r) - b_first) * ld + c * 16);
  }
  const int sr = wave * 64 + lane;  // scale DMA: this lane's row
  const uint32_t vsa = (uint32_t)((arow(sr) - m0) * lds_), vsb = (uint32_t)((brow(sr) - b_first) * lds_);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)smem);
  // this wave's LDS destinations, uniform: its 8 KB blocks of the A and B rows, its 256 bytes of each scale
  const uint32_t lw = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(wave * kQ * 1024));
  const uint32_t lws = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(kScaleOff + wave * 256));
  auto issue = [&](int st) {
    const uint32_t slot = (uint32_t)((st & 1) * kSlotBytes);
    const char* ab = a_base + (int64_t)st * kMxRow;
    const char* bb = b_base + (int64_t)st * kMxRow;
#pragma unroll
    for (int q = 0; q < kQ; ++q) ring4::dma(ab, va[q], lw + slot + (uint32_t)(q * 1024));
#pragma unroll
    for (int q = 0; q < kQ; ++q) ring4::dma(bb, vb[q], lw + slot + (uint32_t)(kOpBytes + q * 1024));
    dma4(sa_base + st * 4, vsa, lws + slot);
    dma4(sb_base + st * 4, vsb, lws + slot + 1024u);
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // LDS row of B fragment jj of this wave: plain, 32-column tiles of its 128 columns; SwiGLU,
  // gate fragments (jj = 0, 1) and the matching up fragments (jj = 2, 3) of its 64 columns
  auto bfrag_row = [&](int jj) -> int {
    return SW ? (jj >> 1) * 128 + wn * 64 + (jj & 1) * 32 + l32 : wn * 128 + jj * 32 + l32;
  };
  const char* L = (const char*)smem;
  // Wave row wm takes the tile's 32-row fragments wm, wm + 2, wm + 4, wm + 6, so a partly filled
  // tile leaves both wave rows the same number NF of live fragments; each wave runs the loop
  // compiled for its NF, the reads and MFMAs of dead fragments left out (the DMAs and barriers,
  // which every wave shares, kept).
  auto arow_frag = [&](int i) -> int { return wm * 32 + i * 64 + l32; };
  auto mainloop = [&](auto nfc) {
  constexpr int NF = decltype(nfc)::value;
  issue(0);
  for (int st = 0; st < nk; ++st) {
    wait_none();    // stage st has landed for this wave
    dma_barrier();  // ... and for every wave, which are all done with stage st - 1
    if (st + 1 < nk) issue(st + 1);  // into the slot stage st - 1 used
    const char* slot = L + (st & 1) * kSlotBytes;
    uint32_t wsa[4], wsb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < NF) wsa[i] = *(const uint32_t*)(slot + kScaleOff + arow_frag(i) * 4);
      wsb[i] = *(const uint32_t*)(slot + kScaleOff + 1024 + bfrag_row(i) * 4);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // this lane's 16-byte chunks: 4 j + hi (Kd 64 j + 16 hi ..) then 4 j + 2 + hi (64 j + 32 + 16 hi ..).
      // The MFMA forms an MX block from the same 16-byte half of the two lanes of a row, with the
      // scale of lane 0 for the first halves and of lane 1 for the second.
      const int c0 = 4 * j + hi, c1 = 4 * j + 2 + hi;
      i32x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rb = bfrag_row(i);
        if (i < NF) {
          const int ra = arow_frag(i);
          const uint4 a0 = *(const uint4*)(slot + ra * kMxRow + ((c0 ^ ring4::swz(ra)) << 4));
          const uint4 a1 = *(const uint4*)(slot + ra * kMxRow + ((c1 ^ ring4::swz(ra)) << 4));
          a[i] = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        }
        const uint4 b0 = *(const uint4*)(slot + kOpBytes + rb * kMxRow + ((c0 ^ ring4::swz(rb)) << 4));
        const uint4 b1 = *(const uint4*)(slot + kOpBytes + rb * kMxRow + ((c1 ^ ring4::swz(rb)) << 4));
        b[i] = i32x8{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
      }
      const int sh = 8 * (2 * j + hi);
#pragma unroll
      for (int i = 0; i < NF; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          // B first, as mma_rows: each lane ends with one A row and 4 consecutive columns a register
          // group, the layout the epilogues store
          acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              b[jj], a[i], acc[i][jj], 0, 0, 0, (int)((wsb[jj] >> sh) & 0xffu), 0, (int)((wsa[i] >> sh) & 0xffu));
    }
  }
  };
  {
    const int64_t live = re - m0 - 32 * wm;
    const int nf = live <= 0 ? 0 : live >= 256 ? 4 : (int)((live + 63) / 64);
    switch (__builtin_amdgcn_readfirstlane(nf)) {
      case 4: mainloop(std::integral_constant<int, 4>{}); break;
      case 3: mainloop(std::integral_constant<int, 3>{}); break;
      case 2: mainloop(std::integral_constant<int, 2>{}); break;
      case 1: mainloop(std::integral_constant<int, 1>{}); break;
      default: mainloop(std::integral_constant<int, 0>{}); break;
    }
  }
  __syncthreads();  // every wave is done with the slots: they hold the epilogue staging now
  if (pc.part >= 0) {
    // a piece of a split tile: publish the partial; the last piece of the tile reduces (as the
    // ring kernel does)
    const int r = pc.slot % pc.R;
    ring4::store_partial(p, pc.slot, acc);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the partial is visible in memory
    int old = 0;
    if (lane == 0) old = atomicAdd(p.ws_count + r * 4 + wave, 1);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != pc.f - 1) return;
    asm volatile("" ::: "memory");  // the loads stay after the count that allowed them
    ring4::load_partial(p, r, acc, false);
    for (int j = 1; j < pc.f; ++j) ring4::load_partial(p, j * pc.R + r, acc, true);
    if (lane == 0) p.ws_count[r * 4 + wave] = 0;
  }
  // the ring kernel's epilogue: LDS staging (32 KB a wave of the idle slots), bf16 out
  const int64_t col0 = SW ? (int64_t)nt * 128 + wn * 64 : (int64_t)nt * 256 + wn * 128;
  // (fragment i of wave row wm: rows m0 + 32 wm + 64 i ..)
  if constexpr (EPI == EPI_SWIGLU_MX)
    mxg::store_tile_mxq(p, acc, (char*)smem + wave * 32768, m0 + wm * 32, re, col0);
  else
    ring4::store_tile_lds<EPI, true>(p, acc, (char*)smem + wave * 32768, m0 + wm * 32, re, col0);
}

hipError_t launch_grouped_gemm_mx(const uint8_t* A, const uint8_t* SA, const uint8_t* B, const uint8_t* SB,
                                  const int32_t* offs, int64_t M, int64_t N, int64_t Kd, int G, int epilogue,
                                  void* C, uint8_t* CS, void* ws, size_t ws_bytes, hipStream_t s) {
  if (M == 0) return hipSuccess;
  if ((N + 256) * Kd >= ((int64_t)1 << 32)) return hipErrorInvalidValue;  // per-lane DMA offsets
  GemmParams prm{A, B, offs, nullptr, nullptr, C, M, N, Kd, G, 0, nullptr, nullptr, 0, 0, 0};
  prm.sa = SA;
  prm.sb = SB;
  prm.cs = CS;
  const bool sw = epilogue == EPI_SWIGLU || epilogue == EPI_SWIGLU_MX;
  prm.NT = sw ? (int)((N / 2 + 127) / 128) : (int)((N + kTile - 1) / kTile);
  prm.nk = (int)(Kd / mxg::kMxRow);
  // with a workspace the grid ends in up to P piece blocks of a split tail (as the ring kernel)
  if (ws && ws_bytes >= kSplitCountBytes + kSplitSlotFloats * sizeof(float)) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipGetLastError();
    prm.ws_count = (int*)ws;
    prm.ws_part = (float*)((char*)ws + kSplitCountBytes);
    prm.ws_slots = (int)std::min<size_t>((ws_bytes - kSplitCountBytes) / (kSplitSlotFloats * sizeof(float)), 1 << 20);
    prm.P = cus;
  }
  const int64_t max_mt = (M + kTile - 1) / kTile + G;
  const dim3 grid((unsigned)(max_mt * prm.NT + prm.P));
  if (epilogue == EPI_SWIGLU_MX)
    hipLaunchKernelGGL((grouped_gemm_mx_kernel<EPI_SWIGLU_MX>), grid, dim3(ring4::kThreads), 0, s, prm);
  else if (epilogue == EPI_SWIGLU)
    hipLaunchKernelGGL((grouped_gemm_mx_kernel<EPI_SWIGLU>), grid, dim3(ring4::kThreads), 0, s, prm);
  else
    hipLaunchKernelGGL((grouped_gemm_mx_kernel<EPI_NONE>), grid, dim3(ring4::kThreads), 0, s, prm);
  return hipGetLastError();
}

namespace {
hipError_t grouped_gemm_impl(const void* A, const void* B, int b_layout, const int32_t* offs, int64_t M, int64_t N,
                             int64_t Kd, int G, int dtype, int epilogue, const void* epi_in, void* epi_save, void* C,
                             void* ws, size_t ws_bytes, const int32_t* a_rows, int a_div, int64_t a_rows_total,
                             hipStream_t s) {
  if (M == 0) return hipSuccess;
  GemmParams prm{A, B, offs, epi_in, epi_save, C, M, N, Kd, G, 0, nullptr, nullptr, 0, 0, 0};
  prm.a_rows = a_rows;
  prm.a_div = (uint32_t)a_div;
  prm.a_last = a_rows ? (uint32_t)(a_rows_total - 1) : 0;
  if (ws && ws_bytes >= kSplitCountBytes + kSplitSlotFloats * sizeof(float)) {
    prm.ws_count = (int*)ws;
    prm.ws_part = (float*)((char*)ws + kSplitCountBytes);
    prm.ws_slots = (int)std::min<size_t>((ws_bytes - kSplitCountBytes) / (kSplitSlotFloats * sizeof(float)), 1 << 20);
  }
  prm.NT = (epilogue == EPI_SWIGLU) ? (int)((N / 2 + 127) / 128) : (int)((N + kTile - 1) / kTile);
  const int64_t max_mt = (M + kTile - 1) / kTile + G;
  const dim3 grid((unsigned)(max_mt * prm.NT));
  // the LDS-DMA pipelines need whole K stages of A (128 or 64 bytes per row), 16-byte
  // aligned rows of B in the K-by-N layout, and 16-byte aligned operands
  const int64_t kbytes = Kd * (dtype == 1 ? 2 : 4);
  const bool aligned = ((uintptr_t)A | (uintptr_t)B) % 16 == 0 && (b_layout == LAYOUT_NK || N % 8 == 0);
  const int nq = !aligned ? 0 : kbytes % Stage<4>::kRowBytes == 0 ? 4 : kbytes % Stage<2>::kRowBytes == 0 ? 2 : 0;
  // the ring kernel: bf16, whole 128-byte K stages, per-lane DMA offsets within 32 bits; N-by-K
  // weights with the plain or SwiGLU epilogue, K-by-N weights with the plain or SwiGLU-backward one
  const bool ring_nk = b_layout == LAYOUT_NK && epilogue != EPI_DSWIGLU && (N + 256) * kbytes < ((int64_t)1 << 32);
  const bool ring_kn = b_layout == LAYOUT_KN && epilogue != EPI_SWIGLU && 64 * N * 2 < ((int64_t)1 << 32) &&
                       (int64_t)256 * kbytes < ((int64_t)1 << 32);
  if (dtype == 1 && nq == 4 && (ring_nk || ring_kn)) {
    // with a workspace the grid ends in up to P piece blocks of a split tail
    int dev = 0, cus = 0;
    if (prm.ws_slots > 0) {
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipGetLastError();
    }
    prm.P = cus;
    prm.nk = (int)(kbytes / ring4::kStageBytes);
    const dim3 rgrid((unsigned)(grid.x + cus));
    if (ring_kn) {
      if (epilogue == EPI_DSWIGLU)
        hipLaunchKernelGGL((grouped_gemm_ring4_kernel<EPI_DSWIGLU, LAYOUT_KN>), rgrid, dim3(ring4::kThreads), 0, s, prm);
      else
        hipLaunchKernelGGL((grouped_gemm_ring4_kernel<EPI_NONE, LAYOUT_KN>), rgrid, dim3(ring4::kThreads), 0, s, prm);
    } else if (epilogue == EPI_SWIGLU) {
      // groups of under 1536 rows on average: each group's partly filled last row tile is a large
      // share of the work, so the form that leaves out the MFMAs of its empty fragments is taken
      // (its epilogue spills a little; with larger groups that cost outweighs the skipped MFMAs)
      const bool skip = M < (int64_t)kSwigluSkipRows * G;
      if (a_rows && skip)
        hipLaunchKernelGGL((grouped_gemm_ring4_kernel<EPI_SWIGLU, LAYOUT_NK, true, true>), rgrid,
                           dim3(ring4::kThreads), 0, s, prm);
      else if (a_rows)
        hipLaunchKernelGGL((grouped_gemm_ring4_kernel<EPI_SWIGLU, LAYOUT_NK, true>), rgrid, dim3(ring4::kThreads), 0,
                           s, prm);
      else if (skip)
        hipLaunchKernelGGL((grouped_gemm_ring4_kernel<EPI_SWIGLU, LAYOUT_NK, false, true>), rgrid,
                           dim3(ring4::kThreads), 0, s, prm);
      else
        hipLaunchKernelGGL((grouped_gemm_ring4_kernel<EPI_SWIGLU, LAYOUT_NK>), rgrid, dim3(ring4::kThreads), 0, s, prm);
    } else if (a_rows) {
      hipLaunchKernelGGL((grouped_gemm_ring4_kernel<EPI_NONE, LAYOUT_NK, true>), rgrid, dim3(ring4::kThreads), 0, s,
                         prm);
    } else {
      hipLaunchKernelGGL((grouped_gemm_ring4_kernel<EPI_NONE, LAYOUT_NK>), rgrid, dim3(ring4::kThreads), 0, s, prm);
    }
    return hipGetLastError();
  }
  if (a_rows) return hipErrorInvalidValue;  // only the ring kernel gathers A rows
  if (dtype == 1) return gemm_dispatch<bf16_t>(prm, b_layout, epilogue, nq, grid, s);
  return gemm_dispatch<float>(prm, b_layout, epilogue, nq, grid, s);
}
}  // namespace

hipError_t launch_grouped_gemm(const void* A, const void* B, int b_layout, const int32_t* offs,
                               int64_t M, int64_t N, int64_t Kd, int G, int dtype, int epilogue,
                               const void* epi_in, void* epi_save, void* C, void* ws, size_t ws_bytes,
                               hipStream_t s) {
  return grouped_gemm_impl(A, B, b_layout, offs, M, N, Kd, G, dtype, epilogue, epi_in, epi_save, C, ws, ws_bytes,
                           nullptr, 1, 0, s);
}

static_assert(ring4::kStageBytes == kGatherStageBytes && EPI_NONE == 0 && EPI_SWIGLU == 1,
              "the gathered form's shape test assumes the ring kernel's stage and epilogue codes");
static_assert(EPI_NONE == MOE_EPI_NONE && EPI_SWIGLU == MOE_EPI_SWIGLU && EPI_DSWIGLU == MOE_EPI_DSWIGLU &&
                  EPI_SWIGLU_MX == MOE_EPI_SWIGLU_MX,
              "the ABI's epilogue codes reach the launchers unchanged");

hipError_t launch_grouped_gemm_gather(const void* X, int64_t T, const int32_t* a_rows, int a_div, const void* B,
                                      const int32_t* offs, int64_t M, int64_t N, int64_t Kd, int G, int epilogue,
                                      void* epi_save, void* C, void* ws, size_t ws_bytes, hipStream_t s) {
  return grouped_gemm_impl(X, B, LAYOUT_NK, offs, M, N, Kd, G, 1, epilogue, nullptr, epi_save, C, ws, ws_bytes,
                           a_rows, a_div, T, s);
}

hipError_t launch_grouped_wgrad(const void* X, const void* dY, const int32_t* offs, int64_t M,
                                int64_t N, int64_t Kd, int G, int dtype, int accumulate, float* dW,
                                hipStream_t s) {
  WgradParams prm{X, dY, offs, dW, M, N, Kd, G, 0, 0, accumulate};
  prm.TN = (int)((N + kTile - 1) / kTile);
  prm.TK = (int)((Kd + kTile - 1) / kTile);
  const dim3 grid((unsigned)((int64_t)prm.TN * prm.TK * G));
  // the LDS-DMA pipeline moves 16-byte pieces of rows: bf16 widths that are multiples of 8
  const bool dma = dtype == 1 && N % 8 == 0 && Kd % 8 == 0 && ((uintptr_t)X | (uintptr_t)dY) % 16 == 0;
  // the ring form: per-lane DMA offsets of 64 rows within 32 bits
  const bool ring = dma && G <= kMaxGroupsWg && 64 * std::max(N, Kd) * 2 < ((int64_t)1 << 32);
  if (ring)
    hipLaunchKernelGGL(grouped_wgrad_ring_kernel, grid, dim3(ring4::kThreads), 0, s, prm);
  else if (dma)
    hipLaunchKernelGGL(grouped_wgrad8_kernel<4>, grid, dim3(kThreads8), 0, s, prm);
  else if (dtype == 1)
    hipLaunchKernelGGL((grouped_wgrad_kernel<bf16_t>), grid, dim3(kThreads), 0, s, prm);
  else
    hipLaunchKernelGGL((grouped_wgrad_kernel<float>), grid, dim3(kThreads), 0, s, prm);
  return hipGetLastError();
}

}  // namespace moe
