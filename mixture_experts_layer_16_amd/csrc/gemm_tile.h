// Persistent grouped "NT" GEMM for gfx950: C[r, n] = sum_k A[r, k] * B_g[n, k]
// for every row r of group g (ragged row segments, each with its own B), with
// an epilogue chosen at compile time.  One template serves the router GEMM
// (one group, float32 logits plus bias), the expert gate/up GEMM (two B
// matrices with a fused SwiGLU epilogue) and the expert down GEMM.
//
// Design (CDNA4):
//  * a workgroup of WM x WN waves owns a BM x BN output tile; each wave owns
//    BM/WM rows (the 32-row blocks wm, wm + WM, wm + 2 WM, ...) and BN/WN
//    columns, as 32x32 MFMA blocks whose float32 accumulators stay in registers
//    for the whole K loop.  Interleaving the row blocks keeps a ragged tile's
//    live rows spread evenly over the SIMDs (waves w and w + 4 share a SIMD);
//  * A and B k-slices travel global -> LDS with the gfx950 16-byte direct-to-LDS
//    load (no register staging), STAGES deep; each LDS row holds BK elements
//    (64 or 128 bytes) with its 16-byte chunks XOR-swizzled by row so that the
//    MFMA operand reads (ds_read_b128, 16 rows per LDS cycle) hit distinct banks;
//  * the kernel is persistent: the grid is sized to the machine and each
//    workgroup walks tiles blockIdx.x, blockIdx.x + gridDim.x, ...  The tile
//    list is built on the device from the group offsets (a prefix over groups
//    of ceil(rows/BM) * column tiles), so ragged and empty groups need no host
//    round trip; an empty group owns no tile and its weights are never read.
#pragma once

#include <type_traits>

#include "common.h"
#include "tile_walk.h"

namespace moe {

enum GemmFeature { kFeatGroups = 1, kFeatStrides = 2, kFeatBKN = 4 };

enum Epilogue {
  EPI_STORE = 0,
  EPI_SWIGLU = 1,
  EPI_F32_BIAS = 2,
  EPI_AXPBY = 3,
  EPI_SWIGLU_BWD = 4,
  EPI_F32 = 5,
  EPI_SWIGLU_SAVE = 6,   // EPI_SWIGLU that also stores G | U (rounded to T) for the backward
  EPI_DH_SWIGLU = 7      // accumulators are dH; G | U read back: dG | dU and H, as EPI_SWIGLU_BWD
};
// float32 output: the accumulators plus an optional per-column bias (EPI_F32_BIAS),
// or as they are (EPI_F32)
constexpr bool f32_epilogue(int epi) { return epi == EPI_F32_BIAS || epi == EPI_F32; }
// Epilogues whose B tile holds gate rows and the matching up rows.
constexpr bool paired_epilogue(int epi) { return epi == EPI_SWIGLU || epi == EPI_SWIGLU_BWD || epi == EPI_SWIGLU_SAVE; }
// Epilogues that store dG | dU (C, row stride ldc) and H (C2) from G, U and dH.
constexpr bool swiglu_grad_epilogue(int epi) { return epi == EPI_SWIGLU_BWD || epi == EPI_DH_SWIGLU; }

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time.
template <int N, int I = 0, typename F> __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

template <typename X> struct TypeTag { typedef X type; };

constexpr int kMaxGroups = 1024;
constexpr int kXcds = 8;   // accelerator complex dies of an MI355X, one L2 each
// A recycled stage's copies are threaded between the MFMAs of the kDmaSpread
// sub-steps that follow the barrier (0: all issued at the barrier).  Issued as one
// burst, the copies of eight waves queue up in the vector-memory path and hold up
// the MFMAs behind them in every wave; two sub-steps measured 1-2% faster than one
// (and 4% faster than none) on the page-shape grouped FFN and its backward.
#ifndef MOE_DMA_SPREAD
#define MOE_DMA_SPREAD 2
#endif
constexpr int kDmaSpread = MOE_DMA_SPREAD;

struct GemmArgs {
  const void* A;          // [rows, K]; group g owns rows seg[g] .. seg[g+1]-1
  const int32_t* a_rows;  // nullptr, or a gather map: logical row r is row a_rows[r] of A
                          // (A's byte size must then stay below 4 GiB)
  int64_t a_rows_n;       // a_rows != nullptr: rows of A; map entries are clamped to
                          // [0, a_rows_n) (they come from device memory)
  const void* B0;         // group g: B0 + g * b_stride elements, [N, K]
  const void* B1;         // EPI_SWIGLU: the "up" matrix, same layout as B0
  int64_t b_stride;       // elements between two groups' B matrices
  const int32_t* seg;     // [G+1] device row offsets; nullptr: see group_rows
  int32_t G;
  int64_t M;
  int64_t group_rows;     // seg == nullptr: G groups of group_rows rows each (> 0), or one
                          // group of M rows (0)
  int32_t N;              // output columns
  int32_t K;              // contraction length, a multiple of BK
  void* C;                // [rows, N] output (row stride N)
  const float* bias;      // EPI_F32_BIAS: [N] or nullptr
  int32_t n_group;        // tile order: column tiles per group (<= 0: all columns of a row tile)
  int32_t m_chunk;        // tile order: row tiles per chunk (<= 0: all row tiles of a group)
  float alpha, beta;      // EPI_AXPBY: C = alpha * (A B^T) + beta * D
  const void* D;          // EPI_AXPBY: [rows, N], same layout and type as C
                          // EPI_SWIGLU_BWD: dH [rows, N] float32
                          // EPI_DH_SWIGLU: G | U [rows, 2N], type T (G in columns
                          // [0, N), U in [N, 2N))
  int64_t lda, ldb;       // row strides of A and B in elements (0: K)
  const int32_t* kseg;    // [G+1] device k offsets (multiples of BK): group g contracts
                          // over k in [kseg[g], kseg[g+1]) (nullptr: [0, K) for all)
  int32_t a_shared;       // 1: every group reads the same A rows (row r of a group's
                          // tile block is A row r, not the group's first row + r)
  void* C2;               // EPI_SWIGLU_BWD, EPI_DH_SWIGLU: H = silu(G) * U, [rows, N]
                          // EPI_SWIGLU_SAVE: G | U [rows, 2N] (G in columns [0, N))
  int64_t ldc;            // row stride of C in elements (0: N)
  int64_t ksa, ksb;       // elements from one BK-deep k-slice of A (B) to the next
                          // (0: BK).  With lda = BK and ksa = rows * BK, A is stored
                          // k-blocked: slice j is a contiguous [rows, BK] block, so a
                          // tile's k-step reads one contiguous piece of memory
  int32_t k_split;        // kFeatBKN: k-slices at k >= k_split come from B1 (its rows
                          // k - k_split); 0: every k-slice comes from B0
};

// Per element type: how one wave multiplies a 32x32 block over 16 k values.
// Each lane supplies 8 consecutive (in LDS) k values of one A row and of one B
// row; lanes 0-31 and 32-63 take the two halves of the 16.  Any assignment of
// k values to (lane, element) is fine as long as A and B agree on it.
template <typename T> struct Mma;

template <> struct Mma<bf16> {
  typedef bf16x8 Frag;
  static constexpr int kReads = 1;  // ds_read_b128 per fragment
  __device__ __forceinline__ static void load(Frag& f, const char* p) {
    f = *reinterpret_cast<const bf16x8*>(p);
  }
  __device__ __forceinline__ static void mma(const Frag& a, const Frag& b, f32x16& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  struct Frag { f32x4 lo, hi; };
  static constexpr int kReads = 2;
  __device__ __forceinline__ static void load(Frag& f, const char* p0, const char* p1) {
    f.lo = *reinterpret_cast<const f32x4*>(p0);
    f.hi = *reinterpret_cast<const f32x4*>(p1);
  }
  __device__ __forceinline__ static void mma(const Frag& a, const Frag& b, f32x16& c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo[i], b.lo[i], c, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi[i], b.hi[i], c, 0, 0, 0);
  }
};

// 16-byte global -> LDS copy per lane (gfx950 LDS DMA).  Lane i of the wave
// writes LDS bytes [lds + 16 i, lds + 16 i + 16).  Issued as inline assembly so
// the compiler neither waits on it before unrelated LDS reads nor reorders
// memory accesses across it; completion is tracked explicitly with vmcnt.
// M0 (which holds the LDS destination) is saved and restored around the copy, so
// the compiler's own view of M0 stays valid.
__device__ __forceinline__ void lds_dma16(const char* gbase, uint32_t voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(gbase), "s"(lds_addr)
      : "memory");
}
// gfx950 transposing LDS read (ds_read_b64_tr_b16), twice.  Within each 16-lane
// group, lane i receives element i % 4 of the 8-byte pieces that lanes i / 4,
// 4 + i / 4, 8 + i / 4 and 12 + i / 4 of the group point at: with lane 4 j + m
// pointing at row j, columns 4 m .. 4 m + 3 of a row-major 16-bit tile, lane i
// gets column i of rows 0 .. 3.  The second read starts `stride` bytes further;
// its 4 values follow the first read's in the result.
__device__ __forceinline__ bf16x8 read_tr16x2(const char* p, int stride) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS s16x4*)const_cast<char*>(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MOE_LDS s16x4*)const_cast<char*>(p + stride));
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait for every outstanding LDS (and scalar-memory) access of this wave.  Issued
// through the builtin, which the compiler's own wait insertion accounts for (an
// inline-asm wait is opaque to it, and it would then wait again later for reads
// that have already landed); the empty asm keeps memory accesses from moving
// across.  Encoding (gfx9): vmcnt 63, expcnt 7, lgkmcnt 0.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
}
// Workgroup barrier without the memory fence of __syncthreads (which would
// also drain every outstanding prefetch).
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const MOE_LDS char*)p);
}

// Load 4 consecutive values (8 bytes of bf16 or 16 bytes of float) as floats.
__device__ __forceinline__ void load4(const bf16* p, float* v) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  const bf16x4 q = *reinterpret_cast<const bf16x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = static_cast<float>(q[i]);
}
__device__ __forceinline__ void load4(const float* p, float* v) {
  const f32x4 q = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = q[i];
}

// Store 4 consecutive outputs (8 bytes of bf16 or 16 bytes of float).
__device__ __forceinline__ void store4(bf16* p, const float* v) {
  typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
  bf16x4 q;
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = static_cast<bf16>(v[i]);
  *reinterpret_cast<bf16x4*>(p) = q;
}
__device__ __forceinline__ void store4(float* p, const float* v) {
  f32x4 q;
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = v[i];
  *reinterpret_cast<f32x4*>(p) = q;
}

// Direct epilogue stores of 16-bit outputs, 16 bytes per lane.  For two consecutive
// 8-column groups of one row, lane l holds columns 0-3 of each (a: the first group,
// b: the second) and lane l + 32 columns 4-7; one exchange across the halves gives
// lane l the first group's 8 values and lane l + 32 the second group's.  Returns
// this lane's 8 values (as bf16 bit patterns) to store at group (lane < 32 ? 0 : 1).
__device__ __forceinline__ u32x4 pair_groups16(const float* a, const float* b, int lane) {
  auto pack = [](float x, float y) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
    bf16x2 v;
    v[0] = static_cast<bf16>(x);
    v[1] = static_cast<bf16>(y);
    return __builtin_bit_cast(uint32_t, v);
  };
  const uint32_t a0 = pack(a[0], a[1]), a1 = pack(a[2], a[3]);
  const uint32_t b0 = pack(b[0], b[1]), b1 = pack(b[2], b[3]);
  const bool lo = lane < 32;
  const uint32_t r0 = (uint32_t)__shfl_xor((int)(lo ? b0 : a0), 32, 64);
  const uint32_t r1 = (uint32_t)__shfl_xor((int)(lo ? b1 : a1), 32, 64);
  u32x4 out;
  out[0] = lo ? a0 : r0;
  out[1] = lo ? a1 : r1;
  out[2] = lo ? r0 : b0;
  out[3] = lo ? r1 : b1;
  return out;
}

template <typename T, int BM, int BN, int BK, int WM, int WN, int STAGES, int EPI>
struct GemmTile {
  static constexpr int kThreads = WM * WN * 64;
  static constexpr int RB = BK * (int)sizeof(T);      // bytes per LDS row
  static constexpr int CPR = RB / 16;                 // 16-byte chunks per row
  static constexpr int RP = 256 / RB;                 // rows per 256-byte LDS bank window
  static constexpr int kStageBytes = (BM + BN) * RB;
  static constexpr int kChunks = kStageBytes / 16;
  static constexpr int CPT = kChunks / kThreads;      // direct-to-LDS loads per thread per stage
  static constexpr int kRowsPerStep = kThreads * 16 / RB;  // LDS rows one load step covers
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int MI = WTM / 32, NI = WTN / 32;
  static constexpr int kSub = BK / 16;                // 16-k MFMA sub-steps per k-tile
  static constexpr int CPL = 8 * (int)sizeof(T) / 16; // chunks per lane per fragment
  static constexpr int NOUT = paired_epilogue(EPI) ? BN / 2 : BN;
  static constexpr int kLdsBytes = STAGES * kStageBytes;

  static_assert(RB == 64 || RB == 128, "LDS row must be 64 or 128 bytes");
  static_assert(kChunks % kThreads == 0, "stage must split evenly over threads");
  static_assert(BM % kRowsPerStep == 0 && BN % kRowsPerStep == 0, "load steps must not straddle A and B");
  static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be made of 32x32 blocks");
  static_assert(!paired_epilogue(EPI) || (NI % 2 == 0 && (BN / 2) % kRowsPerStep == 0), "SwiGLU needs paired blocks");
  static_assert(STAGES >= 2, "need at least double buffering");

  // gfx950 serves a ds_read_b128 16 lanes at a time across 64 four-byte banks (a
  // 256-byte window).  The 16 lanes of a group read 16 consecutive rows at the
  // same logical chunk; XOR-ing the chunk with (row / RP) % CPR puts them in 16
  // distinct 16-byte slots of the window.
  __device__ __forceinline__ static int swz(int row, int lc) { return lc ^ ((row / RP) % CPR); }

  // LDS row (within the B region) that MFMA column block ni of wave column wn reads.
  __device__ __forceinline__ static int b_row(int wn, int ni) {
    if (paired_epilogue(EPI)) {
      constexpr int H = NI / 2;
      return ni < H ? wn * (WTN / 2) + ni * 32 : BN / 2 + wn * (WTN / 2) + (ni - H) * 32;
    }
    return wn * WTN + ni * 32;
  }
};

// With offsets (seg != nullptr): the segment bounds of tile_walk.h into
// gbound[0..G] (the running maximum of seg clamped to [0, M]).  Then the exclusive
// prefix over groups of the tiles each owns into tstart[0..G], saturated at
// INT32_MAX.  One wavefront does the work; the barriers publish it.
template <int BM, int NTHREADS>
__device__ void build_tile_prefix(const int32_t* seg, int G, int64_t M, int64_t group_rows, int ntn, int* tstart,
                                  int* gbound) {
  const int tid = threadIdx.x;
  if (seg) {
    if (tid < 64) {
      const int lane = tid;
      const int nb = G + 1;                         // bounds 0 .. G
      const int per = (nb + 63) / 64;
      const int lo = min(nb, lane * per), hi = min(nb, lo + per);
      int64_t m = INT64_MIN;
      for (int i = lo; i < hi; ++i) m = max(m, (int64_t)seg[i]);
      int64_t incl = m;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int64_t v = __shfl_up(incl, o, 64);
        if (lane >= o) incl = max(incl, v);
      }
      int64_t run = __shfl_up(incl, 1, 64);         // maximum of the raw offsets before lo
      if (lane == 0) run = INT64_MIN;
      for (int i = lo; i < hi; ++i) {
        const int64_t raw = seg[i];
        gbound[i] = (int)segment_bound(run, raw, M);
        run = max(run, raw);
      }
    }
    __syncthreads();
  }
  if (tid < 64) {
    const int lane = tid;
    const int per = (G + 63) / 64;
    const int lo = min(G, lane * per), hi = min(G, lo + per);
    auto rows_of = [&](int g) -> int64_t {
      return seg ? (int64_t)gbound[g + 1] - gbound[g] : (group_rows > 0 ? group_rows : M);
    };
    int64_t sum = 0;
    for (int g = lo; g < hi; ++g) sum += group_tiles(rows_of(g), BM, ntn);
    int64_t incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int64_t v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    int64_t run = incl - sum;
    for (int g = lo; g < hi; ++g) {
      tstart[g] = saturate_tiles(run);
      run += group_tiles(rows_of(g), BM, ntn);
    }
    if (lane == 63) tstart[G] = saturate_tiles(incl);
  }
  __syncthreads();
}

// PD: how many 16-k sub-steps ahead the MFMA operand fragments are read from LDS
// FEAT (compile-time, so that kernels without them compile as if absent):
//   kFeatGroups:  equal groups without offsets (seg == nullptr, group_rows > 0);
//   kFeatStrides: lda, ldb, ksa, ksb, kseg and a_shared;
//   kFeatBKN:     16-bit B stored along N: group g's B is [K, N] (row stride N), so
//                 C = A B instead of A B^T (k_split: see GemmArgs).  A B k-slice goes
//                 to LDS as it lies in memory (BK rows of BN columns) and the MFMA
//                 operand fragments come out of gfx950's transposing LDS read;
// otherwise those fields are ignored: operands are [rows, K] with one K for every
// group, and the groups come from seg (or are one group of M rows).
template <typename T, int BM, int BN, int BK, int WM, int WN, int STAGES, int EPI, int PD = 1, int FEAT = 0>
__global__ __launch_bounds__(WM * WN * 64, 1) void grouped_gemm_kernel(GemmArgs p) {
  typedef GemmTile<T, BM, BN, BK, WM, WN, STAGES, EPI> Cfg;
  typedef Mma<T> Op;
  constexpr int NT = Cfg::kThreads;
  constexpr int RB = Cfg::RB;
  constexpr int CPT = Cfg::CPT;
  constexpr int MI = Cfg::MI, NI = Cfg::NI;
  constexpr int NOUT = Cfg::NOUT;
  constexpr int EPC = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  constexpr int KSUB = Cfg::kSub;
  static_assert(PD >= 1 && PD < KSUB, "prefetch distance must be 1 .. sub-steps - 1");
  constexpr bool GRP = (FEAT & kFeatGroups) != 0, STR = (FEAT & kFeatStrides) != 0;
  // only the SwiGLU epilogues' GEMMs (the expert FFN's first product, forward and
  // backward recompute) read A through a gather map; the others ignore a_rows
  constexpr bool kMayGather = paired_epilogue(EPI);
  constexpr bool BKN = (FEAT & kFeatBKN) != 0;
  static_assert(!BKN || (sizeof(T) == 2 && !paired_epilogue(EPI) && !STR && Cfg::kSub * 16 == BK && BN % 128 == 0),
                "B along N: 16-bit elements, one B per output column block, BN a multiple of 128");
  // B along N: each LDS row of the B region is one k value, BN columns (RBN bytes,
  // 16-byte chunks).  Chunk c of row k sits at chunk c ^ (4 (k % 4)): the
  // transposing read takes 4 consecutive k rows at once, and the XOR moves them to
  // four distinct 64-byte bank groups.
  constexpr int RBN = BN * 2;

  constexpr int kEpiRowBytes = 144;                 // staging row stride of the epilogue (bytes)
  constexpr int kEpiWaveBytes = 32 * kEpiRowBytes;  // one wave's staging buffer: 32 rows
  __shared__ __attribute__((aligned(1024))) char smem[Cfg::kLdsBytes];
  __shared__ int tstart[kMaxGroups + 1];
  __shared__ int gbound[kMaxGroups + 1];   // segment bounds (with offsets)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  const int G = (p.seg || (GRP && p.group_rows > 0)) ? p.G : 1;
  const int ntn = (p.N + NOUT - 1) / NOUT;
  // equal groups (a batch of matrices): group g owns tiles [g * per_g, (g+1) * per_g)
  const bool uniform = GRP && p.seg == nullptr;
  const int per_g = uniform ? (int)((p.group_rows > 0 ? p.group_rows : p.M) + BM - 1) / BM * ntn : 0;
  if (!uniform) build_tile_prefix<BM, NT>(p.seg, G, p.M, GRP ? p.group_rows : 0, ntn, tstart, gbound);
  const int total = uniform ? G * per_g : __builtin_amdgcn_readfirstlane(tstart[G]);
  const int K = p.K;
  const int64_t lda = (STR && p.lda) ? p.lda : K, ldb = (STR && p.ldb) ? p.ldb : K;
  const T* __restrict__ Abase = static_cast<const T*>(p.A);
  // B along N: bytes from one k-slice to the next; the first k-slice read from B1
  // and the byte jump from B0's rows to B1's there
  const uint32_t bkn_step = BKN ? (uint32_t)BK * (uint32_t)p.N * (uint32_t)sizeof(T) : 0u;
  const int bkn_split = (BKN && p.k_split > 0) ? p.k_split / BK : 0x7fffffff;
  const int64_t bkn_jump = (BKN && p.k_split > 0)
                               ? (int64_t)((uintptr_t)p.B1 - (uintptr_t)p.B0) - (int64_t)bkn_split * bkn_step
                               : 0;

  // ---- tile bookkeeping (all wave-uniform) ------------------------------------
  struct TileInfo {
    int g, n0, rows_valid, nk;
    int64_t m0, mrel, k0;   // first output row, its offset in the group, first k
  };
  auto locate = [&](int tile) -> TileInfo {
    TileInfo t;
    int local;
    if (uniform) {
      t.g = tile / per_g;
      local = tile - t.g * per_g;
    } else {
      t.g = __builtin_amdgcn_readfirstlane(find_group(tstart, G, tile));
      local = tile - __builtin_amdgcn_readfirstlane(tstart[t.g]);
    }
    const int64_t grows = GRP ? p.group_rows : 0;
    // offsets: the clamped segment bounds built with the tile prefix
    const int64_t seg_lo = p.seg ? (int64_t)gbound[t.g] : (int64_t)t.g * grows;
    const int64_t seg_hi = p.seg ? (int64_t)gbound[t.g + 1] : (grows > 0 ? seg_lo + grows : p.M);
    // Within a group the tiles run in chunks of m_chunk row tiles; inside a chunk,
    // in column groups of n_group column tiles; inside a column group, row tile by
    // row tile.  Consecutive tiles then share A rows (same row tile) and B columns
    // (same column group), and a chunk's A rows stay hot while its column groups
    // go by.
    const int mtc = (int)((seg_hi - seg_lo + BM - 1) / BM);
    const TileSpot spot = tile_spot(local, mtc, ntn, p.m_chunk, p.n_group);
    const int mt = spot.mt, nt = spot.nt;
    t.m0 = seg_lo + (int64_t)mt * BM;
    t.mrel = (int64_t)mt * BM;
    t.n0 = nt * NOUT;
    t.rows_valid = (int)min<int64_t>(BM, seg_hi - t.m0);
    t.k0 = (STR && p.kseg) ? (int64_t)p.kseg[t.g] : 0;
    t.nk = (STR && p.kseg) ? (int)(((int64_t)p.kseg[t.g + 1] - t.k0) / BK) : K / BK;
    return t;
  };

  // A rows this lane copies for a tile: load step i (< CPA) covers LDS rows
  // [i*kRowsPerStep, (i+1)*kRowsPerStep) of the A region.  With a gather map the
  // row numbers are fetched from it (early, so the fetch hides under a K loop).
  constexpr int CPA = BM / Cfg::kRowsPerStep;
  auto fetch_rows = [&](const TileInfo& t, int* arow) {
#pragma unroll
    for (int i = 0; i < CPA; ++i) {
      const int row = (i * NT + tid) * 16 / RB;
      const int r = min(row, t.rows_valid - 1);              // rows past the segment: any valid row
      arow[i] = (kMayGather && p.a_rows) ? p.a_rows[t.m0 + r] : r;   // clamped where used (setup), so the
                                                   // loads' wait lands there, not here
    }
  };

  // Uniform (SGPR) tile bases plus a fixed 32-bit byte offset per lane and load
  // step, so the direct-to-LDS loads use the scalar-base + vector-offset form.
  const char* Ab = nullptr;
  const char* Bgb = nullptr;
  const char* Bub = nullptr;
  uint32_t soff[CPT];
  auto setup = [&](const TileInfo& t, const int* arow) {
    const int64_t k0 = STR ? t.k0 : 0;
    const int64_t ka0 = (STR && p.ksa) ? k0 / BK * p.ksa : k0, kb0 = (STR && p.ksb) ? k0 / BK * p.ksb : k0;
    Ab = reinterpret_cast<const char*>(Abase + ka0 +
                                       ((kMayGather && p.a_rows) ? 0 : ((STR && p.a_shared) ? t.mrel : t.m0) * lda));
    if constexpr (BKN) {
      // [K, N]: the tile's columns start n0 elements into every k row
      Bgb = reinterpret_cast<const char*>(static_cast<const T*>(p.B0) + (int64_t)t.g * p.b_stride + t.n0);
    } else {
      Bgb = reinterpret_cast<const char*>(static_cast<const T*>(p.B0) + (int64_t)t.g * p.b_stride +
                                          (int64_t)t.n0 * ldb + kb0);
      if (paired_epilogue(EPI))
        Bub = reinterpret_cast<const char*>(static_cast<const T*>(p.B1) + (int64_t)t.g * p.b_stride +
                                            (int64_t)t.n0 * ldb + kb0);
    }
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      // whether load step i reads A, gate or up is known at compile time
      const int byte = (i * NT + tid) * 16;
      if constexpr (BKN) {
        if (i >= CPA) {
          // B along N: LDS chunk pc of k row kr holds columns 8 (pc ^ 4 (kr % 4)) .. + 7
          const int ob = byte - BM * RB;
          const int kr = ob / RBN;
          const int col = min((((ob % RBN) / 16) ^ (4 * (kr % 4))) * 8, p.N - t.n0 - 8);  // past N: any valid
          soff[i] = ((uint32_t)kr * (uint32_t)p.N + (uint32_t)col) * (uint32_t)sizeof(T);
          continue;
        }
      }
      const int row = byte / RB;
      const int lc = Cfg::swz(row, (byte % RB) / 16);
      int r;
      if (i < CPA) {
        r = (kMayGather && p.a_rows) ? clamp_row(arow[i], p.a_rows_n) : arow[i];
      } else {
        const int br = row - BM;
        const int half = paired_epilogue(EPI) ? BN / 2 : BN;
        const int n = (br < half) ? br : br - half;
        r = min(n, p.N - t.n0 - 1);                            // columns past N: any valid column
      }
      soff[i] = ((uint32_t)r * (uint32_t)(i < CPA ? lda : ldb) + (uint32_t)(lc * EPC)) * (uint32_t)sizeof(T);
    }
  };
  // copy i (of CPT) of k-tile kt into `stage`
  auto load_one = [&](int stage, int kt, int i) {
    const uint32_t lbase = lds_addr_of(smem) + stage * Cfg::kStageBytes + wave * 64 * 16;
    const int row0 = i * Cfg::kRowsPerStep;
    int64_t kstep = BK;
    if constexpr (STR) {
      const int64_t ks = row0 < BM ? p.ksa : p.ksb;
      if (ks) kstep = ks;
    }
    if constexpr (BKN) {
      if (row0 >= BM) {
        // k-slice kt is BK rows of B0, or of B1 past k_split (one base pointer
        // and a fixed jump, so that only one pointer stays live)
        lds_dma16(Bgb + (int64_t)kt * bkn_step + (kt >= bkn_split ? bkn_jump : 0), soff[i], lbase + i * NT * 16);
        return;
      }
    }
    const int64_t kb = (int64_t)kt * kstep * (int64_t)sizeof(T);
    const char* base;
    if (row0 < BM) base = Ab;
    else if (paired_epilogue(EPI) && row0 - BM >= BN / 2) base = Bub;
    else base = Bgb;
    lds_dma16(base + kb, soff[i], lbase + i * NT * 16);
  };
  auto load_stage = [&](int stage, int kt) {
#pragma unroll
    for (int i = 0; i < CPT; ++i) load_one(stage, kt, i);
  };
  auto prologue = [&](int nkt) {
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nkt) load_stage(s, s);
  };

  // Row blocks past the end of a ragged row tile carry no output: their MFMAs and
  // A-fragment reads are skipped (mi_live is wave-uniform).  With this wave's
  // blocks wm + WM mi, a tile with r live blocks leaves each SIMD at most
  // ceil(r / 2) of them (contiguous blocks per wave: up to 4 for r = 6).
  int mi_live = MI;

  // ---- MFMA operand fragments: one buffer per sub-step of a k-tile, read PD
  //      sub-steps ahead of the MFMAs that use them -------------------------------
  // Sub-step s reads buffer s % NBUF and fills buffer (s + PD) % NBUF: PD + 1
  // buffers are all that is ever live (KSUB is a multiple of NBUF), and the smaller
  // register footprint keeps the K loop free of spills.
  constexpr int NBUF = PD + 1;
  static_assert(KSUB % NBUF == 0, "the fragment ring wraps at k-tile boundaries");
  typename Op::Frag fa[NBUF][MI], fb[NBUF][NI];
  // full: every row block of this wave is live (no per-block checks)
  auto read_frags = [&](bool full, int buf, int stage, int sub) {
    const char* sA = smem + stage * Cfg::kStageBytes;
    const char* sB = sA + BM * RB;
    const int lc0 = sub * 2 * Cfg::CPL + (lane >> 5) * Cfg::CPL;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (!full && mi >= mi_live) continue;
      const int r = (wm + WM * mi) * 32 + (lane & 31);
      if constexpr (Op::kReads == 1)
        Op::load(fa[buf % NBUF][mi], sA + r * RB + Cfg::swz(r, lc0) * 16);
      else
        Op::load(fa[buf % NBUF][mi], sA + r * RB + Cfg::swz(r, lc0) * 16, sA + r * RB + Cfg::swz(r, lc0 + 1) * 16);
    }
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      if constexpr (BKN) {
        // lane 4 j + m of each 16-lane group q points at k row kr + j, columns
        // col .. col + 3; each lane then holds 4 consecutive k of one column, and the
        // second read (4 rows further) completes the lane's 8 k values
        const int q = lane >> 4, j = (lane >> 2) & 3;
        const int kr = sub * 16 + 8 * (q >> 1) + j;
        const int col = wn * Cfg::WTN + ni * 32 + 16 * (q & 1) + 4 * (lane & 3);
        fb[buf % NBUF][ni] = read_tr16x2(sB + kr * RBN + (((col >> 3) ^ (4 * j)) << 4) + (col & 7) * 2, 4 * RBN);
        continue;
      }
      const int r = Cfg::b_row(wn, ni) + (lane & 31);
      if constexpr (Op::kReads == 1)
        Op::load(fb[buf % NBUF][ni], sB + r * RB + Cfg::swz(r, lc0) * 16);
      else
        Op::load(fb[buf % NBUF][ni], sB + r * RB + Cfg::swz(r, lc0) * 16, sB + r * RB + Cfg::swz(r, lc0 + 1) * 16);
    }
  };
  f32x16 acc[MI][NI];
  // B (weights) is the MFMA's first operand: each block comes out transposed, so a
  // lane ends up holding 4 consecutive output columns of one row.
  auto mma_all = [&](bool full, int buf) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      if (full || mi < mi_live) {
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) Op::mma(fb[buf % NBUF][ni], fa[buf % NBUF][mi], acc[mi][ni]);
      }
  };
  // the same MFMAs with copies J0 .. J1-1 of k-tile kt into `stage` (if copy)
  // threaded between them
  auto mma_all_copy = [&](auto j0c, auto j1c, bool full, int buf, int stage, int kt, bool copy) {
    constexpr int J0 = decltype(j0c)::value, J1 = decltype(j1c)::value;
    constexpr int NM = MI * NI, NJ = J1 - J0;
    // the copies are spread over the first half of the MFMAs (after MFMA q for
    // q < NF, with q * NJ / NF stepping up): earlier than spread over all of
    // them, so each gets more cover, but not in one burst.  Measured on the
    // page-shape grouped FFN: 1.6% faster than all MFMAs, 0.4-1.6% faster than
    // the first quarter
    constexpr int NF = NM > 1 ? NM / 2 : 1;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        if (full || mi < mi_live) Op::mma(fb[buf % NBUF][ni], fa[buf % NBUF][mi], acc[mi][ni]);
        const int q = mi * NI + ni;
#pragma unroll
        for (int j = J0 + min(q, NF) * NJ / NF; j < J0 + min(q + 1, NF) * NJ / NF; ++j)
          if (copy) load_one(stage, kt, j);
      }
  };

  // ---- epilogue: store the accumulators of tile t (this wave's part).  Block
  //      (mi, ni): lane holds output row (lane % 32) and the columns
  //      8*q + 4*(lane/32) + i in acc[4*q + i], q, i = 0..3.  wbuf: this wave's
  //      LDS staging buffer (kEpiWaveBytes). -----------------------------------
  auto store_tile = [&](const TileInfo& t, char* wbuf) {
    const int64_t em0 = t.m0;
    const int en0 = t.n0, erows = t.rows_valid;

    const int h4 = 4 * (lane >> 5);
    // Staged through LDS, for an output element type OT (T, or float for
    // EPI_F32 / EPI_F32_BIAS): val(mi, ni, q, i) is the value of element 4 q + i of output
    // block (mi, ni), ni < NO; dstp the output matrix, row stride ld elements.
    auto staged = [&](auto ot_tag, auto val, void* dstp, int64_t ld) {
      typedef typename decltype(ot_tag)::type OT;
      // Staged through LDS (wbuf: this wave's 32 rows x 144 bytes, which nothing
      // else touches until the next barrier).  Per round
      // (one row block mi, 128 bytes of output columns) it parks its values there
      // (the 16-byte pad spreads rows over the banks and keeps every address a lane
      // base plus an immediate), then reads them back as 16-byte pieces, 8 lanes per
      // row, and stores whole 128-byte row segments.
      constexpr int NO = paired_epilogue(EPI) ? NI / 2 : NI;
      constexpr int CW = paired_epilogue(EPI) ? Cfg::WTN / 2 : Cfg::WTN;   // output columns per wave
      constexpr int ES = (int)sizeof(OT);
      constexpr int RC = 128 / ES;                                         // columns per round
      constexpr int ROUNDS = CW / RC;
      constexpr int RS = kEpiRowBytes;
      static_assert(CW % RC == 0, "whole rounds");
      char* wlane = wbuf + (lane & 31) * RS + h4 * ES;                     // this lane's row and column offset
      const char* rlane = wbuf + (lane >> 3) * RS + (lane & 7) * 16;
      // read-back rows r0 + 32 WM mi + 8 it of this wave (its row blocks are
      // wm + WM mi); one 64-bit address per lane, stepped by scalars (no per-row
      // 64-bit products to keep live)
      const int r0 = wm * 32 + (lane >> 3);
      const int rrem = erows - r0;
      const int c0l = en0 + wn * CW + (lane & 7) * (16 / ES);
      OT* cbase = static_cast<OT*>(dstp) + (em0 + r0) * ld + c0l;
      const int64_t rstep = 8 * ld;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        if (mi >= mi_live) break;
#pragma unroll
        for (int rd = 0; rd < ROUNDS; ++rd) {
#pragma unroll
          for (int ni = 0; ni < NO; ++ni)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int c0 = ni * 32 + 8 * q - rd * RC;                  // compile time
              if (c0 < 0 || c0 >= RC) continue;
              float v[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) v[i] = val(mi, ni, q, i);
              store4(reinterpret_cast<OT*>(wlane + c0 * ES), v);
            }
          wait_lgkmcnt0();
#pragma unroll
          for (int it = 0; it < 4; ++it) {
            const u32x4 piece = *reinterpret_cast<const u32x4*>(rlane + it * 8 * RS);
            const int cc = c0l + rd * RC;
            if constexpr (f32_epilogue(EPI)) {
              // N need not be a multiple of 4 here (a router's expert count)
              if (mi * 32 * WM + it * 8 < rrem) {
                OT* dst = cbase + (4 * WM * mi + it) * rstep + rd * RC;
                if (cc + 16 / ES <= p.N) {
                  *reinterpret_cast<u32x4*>(dst) = piece;
                } else if (cc < p.N) {
                  const OT* ev = reinterpret_cast<const OT*>(&piece);
                  for (int i = 0; i < 16 / ES && cc + i < p.N; ++i) dst[i] = ev[i];
                }
              }
            } else {
              if (mi * 32 * WM + it * 8 < rrem && cc < p.N)
                *reinterpret_cast<u32x4*>(cbase + (4 * WM * mi + it) * rstep + rd * RC) = piece;
            }
          }
          wait_lgkmcnt0();
        }
      }
    };
    // (EPI_SWIGLU_BWD's three outputs stay on the direct path: staging them costs
    // the K loop registers)
    constexpr bool kStaged = EPI != EPI_AXPBY && !swiglu_grad_epilogue(EPI) && NT == 512 && Cfg::WTM == 64 &&
                             8 * kEpiWaveBytes <= Cfg::kStageBytes;
    if constexpr (kStaged && EPI == EPI_SWIGLU_SAVE) {
      // h = silu(G) U, then G and U themselves into the two halves of C2's rows
      staged(
          TypeTag<T>{},
          [&](int mi, int ni, int q, int i) {
            const float gv = acc[mi][ni][4 * q + i];
            return gv / (1.0f + __expf(-gv)) * acc[mi][ni + NI / 2][4 * q + i];
          },
          p.C, (int64_t)p.N);
      staged(TypeTag<T>{}, [&](int mi, int ni, int q, int i) { return acc[mi][ni][4 * q + i]; }, p.C2,
             2 * (int64_t)p.N);
      staged(TypeTag<T>{}, [&](int mi, int ni, int q, int i) { return acc[mi][ni + NI / 2][4 * q + i]; },
             static_cast<T*>(p.C2) + p.N, 2 * (int64_t)p.N);
    } else if constexpr (kStaged) {
      typedef typename std::conditional<f32_epilogue(EPI), float, T>::type OT;
      staged(
          TypeTag<OT>{},
          [&](int mi, int ni, int q, int i) {
            if constexpr (EPI == EPI_SWIGLU) {
              const float gv = acc[mi][ni][4 * q + i];
              return gv / (1.0f + __expf(-gv)) * acc[mi][ni + NI / 2][4 * q + i];
            } else if constexpr (EPI == EPI_F32_BIAS) {
              const int col = en0 + wn * Cfg::WTN + ni * 32 + 8 * q + h4 + i;
              return acc[mi][ni][4 * q + i] + ((p.bias && col < p.N) ? p.bias[col] : 0.f);
            } else {
              return acc[mi][ni][4 * q + i];
            }
          },
          p.C, (int64_t)p.N);
    } else if constexpr (f32_epilogue(EPI) || EPI == EPI_SWIGLU_SAVE) {
      static_assert(!f32_epilogue(EPI) && EPI != EPI_SWIGLU_SAVE, "this epilogue takes the staged path");
    } else {
      constexpr int NO = paired_epilogue(EPI) ? NI / 2 : NI;
      constexpr int CW = paired_epilogue(EPI) ? Cfg::WTN / 2 : Cfg::WTN;
      const int64_t ldc = (swiglu_grad_epilogue(EPI) && p.ldc) ? p.ldc : p.N;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int r = (wm + WM * mi) * 32 + (lane & 31);
        if (r >= erows) continue;               // (lanes l and l + 32 share the row)
        T* crow = static_cast<T*>(p.C) + (em0 + r) * ldc;
#pragma unroll
        for (int ni = 0; ni < NO; ++ni)
#pragma unroll
          for (int q = 0; q < 4; q += 2) {
            // two 8-column groups q, q + 1; N is a multiple of 8 here, so both lanes of
            // a pair agree on every column test
            float v[2][3][4];                     // [group][output][element]
            // EPI_AXPBY with 16-bit D: this lane loads the 8 values of D at its
            // store columns (16 bytes) and the pair exchanges halves back into
            // the MFMA layout: dd[qq] = columns 8 (q + qq) + h4 .. + 3
            float dd[2][4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            if constexpr (EPI == EPI_AXPBY && sizeof(T) == 2) {
              const int colp = en0 + wn * CW + ni * 32 + 8 * (q + (lane >> 5));
              u32x4 ld = {0u, 0u, 0u, 0u};
              if (colp < p.N)
                ld = *reinterpret_cast<const u32x4*>(static_cast<const T*>(p.D) + (em0 + r) * (int64_t)p.N + colp);
              const bool lo = lane < 32;
              // lane l keeps columns 0-3 of group q and needs 0-3 of group q + 1 (the
              // partner's first half); lane l + 32 keeps 4-7 of group q + 1 and needs
              // 4-7 of group q (the partner's second half)
              const uint32_t s0 = lo ? ld[2] : ld[0], s1 = lo ? ld[3] : ld[1];
              const uint32_t r0 = (uint32_t)__shfl_xor((int)s0, 32, 64), r1 = (uint32_t)__shfl_xor((int)s1, 32, 64);
              const uint32_t own0 = lo ? ld[0] : ld[2], own1 = lo ? ld[1] : ld[3];
              auto lo16 = [](uint32_t w) { return __uint_as_float(w << 16); };
              auto hi16 = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
              // lo lane: group q = own, group q + 1 = received; hi lane: group q = received
              const uint32_t g0a = lo ? own0 : r0, g0b = lo ? own1 : r1;
              const uint32_t g1a = lo ? r0 : own0, g1b = lo ? r1 : own1;
              dd[0][0] = lo16(g0a); dd[0][1] = hi16(g0a); dd[0][2] = lo16(g0b); dd[0][3] = hi16(g0b);
              dd[1][0] = lo16(g1a); dd[1][1] = hi16(g1a); dd[1][2] = lo16(g1b); dd[1][3] = hi16(g1b);
            }
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
              const int col = en0 + wn * CW + ni * 32 + 8 * (q + qq) + h4;
              if constexpr (swiglu_grad_epilogue(EPI)) {
                // S = silu(G), H = S U, dU = dH S, dG = dH U silu'(G); dG and dU go to
                // the row's two halves.  EPI_SWIGLU_BWD: G, U recomputed (accumulators),
                // dH read; EPI_DH_SWIGLU: dH accumulated, G, U read (saved by the forward)
                float gg[4], uu[4], dh[4];
                if constexpr (EPI == EPI_SWIGLU_BWD) {
                  f32x4 dv4 = {0.f, 0.f, 0.f, 0.f};
                  if (col < p.N)
                    dv4 = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.D) +
                                                          (em0 + r) * (int64_t)p.N + col);
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    gg[i] = acc[mi][ni][4 * (q + qq) + i];
                    uu[i] = acc[mi][ni + NI / 2][4 * (q + qq) + i];
                    dh[i] = dv4[i];
                  }
                } else {
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    gg[i] = 0.f;
                    uu[i] = 0.f;
                    dh[i] = acc[mi][ni][4 * (q + qq) + i];
                  }
                  if (col < p.N) {
                    const T* gu = static_cast<const T*>(p.D) + (em0 + r) * 2 * (int64_t)p.N + col;
                    load4(gu, gg);
                    load4(gu + p.N, uu);
                  }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const float g = gg[i], u = uu[i];
                  const float sg = 1.0f / (1.0f + __expf(-g));
                  const float sv = g * sg;
                  v[qq][0][i] = dh[i] * u * (sg * (1.0f + g * (1.0f - sg)));
                  v[qq][1][i] = dh[i] * sv;
                  v[qq][2][i] = sv * u;
                }
              } else {
                float dv[4] = {dd[qq][0], dd[qq][1], dd[qq][2], dd[qq][3]};
                if constexpr (EPI == EPI_AXPBY && sizeof(T) != 2)
                  if (col < p.N) load4(static_cast<const T*>(p.D) + (em0 + r) * (int64_t)p.N + col, dv);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  if constexpr (EPI == EPI_SWIGLU) {
                    const float gv = acc[mi][ni][4 * (q + qq) + i];
                    const float uv = acc[mi][ni + NI / 2][4 * (q + qq) + i];
                    v[qq][0][i] = gv / (1.0f + __expf(-gv)) * uv;
                  } else if constexpr (EPI == EPI_AXPBY) {
                    v[qq][0][i] = p.alpha * acc[mi][ni][4 * (q + qq) + i] + p.beta * dv[i];
                  } else {
                    v[qq][0][i] = acc[mi][ni][4 * (q + qq) + i];
                  }
                }
              }
            }
            constexpr int NOUT_ = swiglu_grad_epilogue(EPI) ? 3 : 1;
            if constexpr (sizeof(T) == 2) {
              const int colp = en0 + wn * CW + ni * 32 + 8 * (q + (lane >> 5));   // this lane's 8 columns
#pragma unroll
              for (int o = 0; o < NOUT_; ++o) {
                const u32x4 w = pair_groups16(v[0][o], v[1][o], lane);
                if (colp < p.N) {
                  T* dst = o == 0 ? crow + colp
                                  : (o == 1 ? crow + p.N + colp : static_cast<T*>(p.C2) + (em0 + r) * (int64_t)p.N + colp);
                  *reinterpret_cast<u32x4*>(dst) = w;
                }
              }
            } else {
#pragma unroll
              for (int qq = 0; qq < 2; ++qq) {
                const int col = en0 + wn * CW + ni * 32 + 8 * (q + qq) + h4;
                if (col < p.N) {
#pragma unroll
                  for (int o = 0; o < NOUT_; ++o) {
                    T* dst = o == 0 ? crow + col
                                    : (o == 1 ? crow + p.N + col : static_cast<T*>(p.C2) + (em0 + r) * (int64_t)p.N + col);
                    store4(dst, v[qq][o]);
                  }
                }
              }
            }
          }
      }
    }
  };

  // Workgroups are dispatched to the 8 XCDs round-robin (workgroup b on XCD b % 8)
  // and each XCD has its own L2.  Give the workgroups of one XCD a contiguous run
  // of the tile list in every round, so that the tiles resident on an XCD share
  // their A rows (the column tiles of a row tile) and expert weights.
  const int grid = gridDim.x;
  int tile = blockIdx.x;
  const int step = grid, end = total;
  if (grid % kXcds == 0) tile = (blockIdx.x % kXcds) * (grid / kXcds) + blockIdx.x / kXcds;
  if (tile >= end) return;

  TileInfo cur = locate(tile), nxt = cur;
  int arow[CPA], arow_n[CPA];
  fetch_rows(cur, arow);
  setup(cur, arow);
  prologue(STR ? cur.nk : K / BK);

  while (true) {
    const int nk = STR ? cur.nk : K / BK;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[mi][ni][j] = 0.f;

    {
      // row blocks with a valid row; this wave's are blocks wm + WM mi
      const int nb = (cur.rows_valid + 31) / 32;
      mi_live = __builtin_amdgcn_readfirstlane(nb > wm ? min(MI, (nb - wm + WM - 1) / WM) : 0);
    }

    // k-tile 0 has landed (this wave's copies; the barrier covers the others)
    if (STAGES - 2 <= nk - 1) wait_vmcnt<(STAGES - 2) * CPT>();
    else wait_vmcnt<0>();
    block_barrier();
    // Look up the next tile.  With a gather map, before the next stage's copies
    // go out: the compiler waits for its own loads (the row numbers) with a full
    // memory-counter wait, which would also wait for copies issued ahead of them;
    // the row numbers then arrive during this K loop.  Without one the lookup only
    // reads LDS, so the copies go out first and the lookup runs under them.
    // (Only the SwiGLU epilogues' GEMMs read A through a gather map.)
    const int next_tile = tile + step;
    const bool more = next_tile < end;
    if constexpr (kMayGather) {
      if (more) {
        nxt = locate(next_tile);
        fetch_rows(nxt, arow_n);
      }
      if (STAGES - 1 < nk) load_stage((STAGES - 1) % STAGES, STAGES - 1);
    } else {
      if (STAGES - 1 < nk) load_stage((STAGES - 1) % STAGES, STAGES - 1);
      if (more) {
        nxt = locate(next_tile);
        fetch_rows(nxt, arow_n);
      }
    }
      // the K loop, compiled twice: without per-block checks for tiles whose row
    // blocks are all live, with them for ragged tiles (the checks cost the
    // compiler its exact tracking of outstanding LDS reads)
    auto kloop = [&](auto fullc) {
      constexpr bool FULL = decltype(fullc)::value;
#pragma unroll
      for (int s = 0; s < PD; ++s) read_frags(FULL, s, 0, s);

      for (int kt = 0; kt < nk; ++kt) {
        const int st = kt % STAGES;
        static_for<KSUB>([&](auto sc) {
          constexpr int s = decltype(sc)::value;
          if constexpr (s + PD < KSUB) {
            read_frags(FULL, s + PD, st, s + PD);
          } else {
            // every LDS read of stage st has been issued: wait for them (on every
            // path, so the compiler sees one state after the branch).  The
            // scheduling barrier keeps the previous sub-step's MFMAs above the wait:
            // they touch no memory, and the compiler otherwise sinks them below it,
            // exposing the latency of the reads just issued once per k-tile.
            if constexpr (s + PD == KSUB) {
              __builtin_amdgcn_sched_barrier(0);
              wait_lgkmcnt0();
            }
            if (kt + 1 < nk) {
              if constexpr (s + PD == KSUB) {
                // k-tile kt+1 has landed: recycle stage st for k-tile kt+STAGES
                if (kt + STAGES - 1 <= nk - 1) wait_vmcnt<(STAGES - 2) * CPT>();
                else wait_vmcnt<0>();
                block_barrier();
                if (kDmaSpread == 0 && kt + STAGES < nk) load_stage(st, kt + STAGES);
              }
              read_frags(FULL, s + PD - KSUB, (kt + 1) % STAGES, s + PD - KSUB);
            }
          }
          // copies threaded through sub-step KSUB-PD (this k-tile) and sub-steps
          // 0 .. kDmaSpread-2 of the next one: piece i of kDmaSpread, taken from the
          // end of the copy list, so the B (weight) copies go out first and get the
          // longest cover (0.9% faster on the page-shape grouped FFN than A first)
          constexpr int piece = (s + PD == KSUB) ? 0 : (s + 1 < kDmaSpread ? s + 1 : -1);
          if constexpr (kDmaSpread > 0 && piece >= 0) {
            constexpr int J0 = (kDmaSpread - 1 - piece) * CPT / (kDmaSpread > 0 ? kDmaSpread : 1);
            constexpr int J1 = (kDmaSpread - piece) * CPT / (kDmaSpread > 0 ? kDmaSpread : 1);
            if constexpr (piece == 0)
              mma_all_copy(std::integral_constant<int, J0>{}, std::integral_constant<int, J1>{}, FULL, s, st,
                           kt + STAGES, kt + 1 < nk && kt + STAGES < nk);
            else   // the copies of the stage recycled at the previous k-tile's barrier
              mma_all_copy(std::integral_constant<int, J0>{}, std::integral_constant<int, J1>{}, FULL, s,
                           (kt + STAGES - 1) % STAGES, kt - 1 + STAGES, kt >= 1 && kt - 1 + STAGES < nk);
          } else {
            mma_all(FULL, s);
          }
        });
      }
    };
    if (mi_live == MI) kloop(std::true_type{});
    else kloop(std::false_type{});

    // this tile's LDS reads are done everywhere: start the next tile's copies, then
    // store this tile while they are in flight
    wait_lgkmcnt0();
    block_barrier();
    if (more) {
      setup(nxt, arow_n);
      prologue(STR ? nxt.nk : K / BK);
    }
    store_tile(cur, smem + (STAGES - 1) * Cfg::kStageBytes + wave * kEpiWaveBytes);
    if (!more) break;
    tile = next_tile;
    cur = nxt;
  }
}

}  // namespace moe
