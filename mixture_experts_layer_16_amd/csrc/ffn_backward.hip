// Backward pass of the grouped SwiGLU expert FFN.
//
// The pages' workload is pre-training ("Training a 1T-Parameter MoE on EU public
// infrastructure with PyTorch and TorchTitan"), so every step also runs the
// layer backward.  For expert e with rows X (token rows, read in place through
// the gather map or from x_perm) and output gradient dY (rows of dy_perm):
//     dH = dY W_d,   S = silu(X W_g^T),  U = X W_u^T,  H = S U
//     dU = dH S,     dG = dH U silu'(X W_g^T)
//     dX = dG W_g + dU W_u
//     dW_d = dY^T H,   dW_g = dG^T X,   dW_u = dU^T X
//
// Everything runs on the grouped GEMM (C = A B^T, both operands read along the
// contraction, or C = A B with B stored along N):
//   * dH = dY W_d and dX = [dG | dU] [W_g ; W_u] contract along the weights'
//     first dimension: 16-bit weights are read in place (the GEMM's B-along-N
//     form, transposing LDS reads), float32 ones through transposed copies
//     ([E, F, d] and [E, d, 2F], made here); dH is float32, dX the I/O type;
//   * the I/O type is bf16 (MFMA bf16 products, float32 accumulation) or float32
//     (float32 MFMA products throughout);
//   * G and U are recomputed by the gate/up GEMM, whose epilogue turns them and
//     dH into dG, dU (one [n, 2F] buffer) and H; or, when the forward kept them
//     (G | U rounded to the I/O type), the dH GEMM's epilogue reads them and writes
//     dG, dU and H itself (no recompute, no float32 dH);
//   * the weight gradients contract over each expert's rows: the activations
//     are transposed into a layout where expert e owns columns
//     [poff[e], poff[e+1]) (its row count rounded up to 64, the gap zero-filled),
//     stored k-blocked (below), and one GEMM per gradient runs with one group per
//     expert whose k range is that column range, every group reading the same
//     operand rows.  An expert with no rows gets a zero gradient.
#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"
#include "transpose.h"

namespace moe {

namespace {

constexpr int kTile = 64;

// Tile order of the weight-gradient GEMMs inside an expert (see GemmArgs): row
// tiles in chunks of kWgradRowChunk, column tiles in groups of kWgradColumnGroup,
// so the 32 tiles an XCD runs side by side form a 4 x 8 block and share their A
// rows and B rows in that XCD's L2 (all row or all column tiles of an expert would
// stream one of the two operands once per XCD that holds part of the expert).
constexpr int kWgradRowChunk = 4;
constexpr int kWgradColumnGroup = 8;
// The same for the GEMMs over the expert rows (dH, recompute, dX); 0: not chunked.
constexpr int kRowsRowChunk = 0;
constexpr int kRowsColumnGroup = 0;

// The caller's offsets made consistent, then padded:
//   soff[e] = the running maximum of offsets[0..e] clamped to [0, n_max] (offsets
//             that are non-decreasing and end at most at n_max pass through
//             unchanged; any others still give disjoint segments inside the
//             buffers), and every later kernel reads soff, never offsets;
//   poff[e] = sum over e' < e of the row count of e' rounded up to 64 (one block).
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int E, int64_t n_max,
                                                           int32_t* __restrict__ soff, int32_t* __restrict__ poff) {
  __shared__ int wsum[16];
  __shared__ int wmax[16];
  __shared__ int bnd[kMaxExperts + 1];
  const int e = threadIdx.x;
  const int lane = e & 63, wv = e >> 6;
  int mx = e < E ? offsets[e] : INT32_MIN;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(mx, o, 64);
    if (lane >= o) mx = max(mx, t);
  }
  if (lane == 63) wmax[wv] = mx;
  __syncthreads();
  int before = INT32_MIN;
  for (int i = 0; i < wv; ++i) before = max(before, wmax[i]);
  const int run = max(before, mx);                 // maximum of offsets[0..e]
  if (e < E) bnd[e] = (int)clamp64(run, 0, n_max);
  if (e == E - 1) bnd[E] = (int)clamp64(max(run, offsets[E]), 0, n_max);
  __syncthreads();
  if (e < E) soff[e] = bnd[e];
  if (e == E - 1) soff[E] = bnd[E];
  const int v = e < E ? (bnd[e + 1] - bnd[e] + 63) / 64 * 64 : 0;
  int incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int sum_before = 0;
  for (int i = 0; i < wv; ++i) sum_before += wsum[i];
  if (e < E) poff[e] = sum_before + incl - v;
  if (e == E - 1) poff[E] = sum_before + incl;
}

// The transposed, padded activations are stored k-blocked: element (c, p) of an
// [R, n_pad] matrix (c < R a feature, p a padded row) sits at
// (p / KW) R KW + c KW + p % KW, i.e. every KW-wide column block is one contiguous
// [R, KW] piece.  A weight-gradient tile then reads each k-step (256 features x KW
// rows) as one contiguous 32 KB piece, where a plain [R, n_pad] layout would touch
// 256 rows a megabyte apart (one address-translation page each).
//
// Element (c, p) for padded row p of expert e = source row offsets[e] + (p - poff[e])
// (through rows[] when given, its entries clamped to [0, n_src)), column col0 + c of
// the source (row stride ld_src); zero past the expert's rows.  One 64 x 64 tile per block; blocks past poff[E] have
// nothing to do; pblk_expert[p / 64] is the expert owning padded rows p .. p + 63.
template <typename T, int KW>
__global__ __launch_bounds__(256) void pad_transpose_kernel(const T* __restrict__ src, int64_t ld_src, int col0,
                                                            const int32_t* __restrict__ rows, int64_t n_src,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ poff,
                                                            const int32_t* __restrict__ pblk_expert, int E,
                                                            T* __restrict__ dst, int64_t R) {
  __shared__ T tile[kTile][kTile + 2];
  const int p0 = blockIdx.x * kTile;
  if (p0 >= poff[E]) return;
  const int e = pblk_expert[blockIdx.x];
  const int r0 = p0 - poff[e];
  const int n_e = offsets[e + 1] - offsets[e];
  const int c0 = blockIdx.y * kTile;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int j = ty; j < kTile; j += 4) {
    T v = static_cast<T>(0.0f);
    if (r0 + j < n_e) {
      const int64_t sr = offsets[e] + r0 + j;
      const int64_t row = rows ? (int64_t)clamp_row(rows[sr], n_src) : sr;
      v = src[row * ld_src + col0 + c0 + tx];
    }
    tile[j][tx] = v;
  }
  __syncthreads();
  const int p = p0 + tx;
  T* out = dst + (int64_t)(p / KW) * R * KW + p % KW;
  for (int i = ty; i < kTile; i += 4) out[(int64_t)(c0 + i) * KW] = tile[tx][i];
}

// pblk_expert[b] = the expert owning padded rows 64 b .. 64 b + 63 (largest e with
// poff[e] <= 64 b), for every block b below poff[E] / 64.
__global__ __launch_bounds__(256) void pad_block_experts_kernel(const int32_t* __restrict__ poff, int E,
                                                                int32_t* __restrict__ pblk_expert) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  const int p0 = b * kTile;
  if (p0 >= poff[E]) return;
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (poff[mid] <= p0) lo = mid; else hi = mid;
  }
  pblk_expert[b] = lo;
}

// 16-bit elements: the same result as pad_transpose_kernel with KW = 64, in strips
// of up to 8 tiles (grid.y walks the strips of the R source columns).
__global__ __launch_bounds__(256) void pad_transpose16_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                                              int col0, const int32_t* __restrict__ rows, int64_t n_src,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ poff,
                                                              const int32_t* __restrict__ pblk_expert, int E,
                                                              uint16_t* __restrict__ dst, int64_t R) {
  const int p0 = blockIdx.x * kTile;
  if (p0 >= poff[E]) return;
  const int e = pblk_expert[blockIdx.x];
  const int r0 = p0 - poff[e];
  const int n_e = offsets[e + 1] - offsets[e];
  const int cs = blockIdx.y * 8 * kTile;                         // first source column of the strip
  const int ntile = min(8, (int)(R / kTile) - blockIdx.y * 8);
  uint16_t* blk = dst + (int64_t)(p0 / kTile) * R * kTile;
  transpose_strip16(
      ntile,
      [&](int r) -> const uint16_t* {
        if (r0 + r >= n_e) return nullptr;
        const int64_t sr = offsets[e] + r0 + r;
        const int64_t row = rows ? (int64_t)clamp_row(rows[sr], n_src) : sr;
        return src + row * ld_src + col0 + cs;
      },
      [&](int j, int c) { return blk + (int64_t)(cs + j * kTile + c) * kTile; });
}

// dst[b][c * ld_dst + coff + r] = src[b][r * cols + c] for b < batch: transposes
// of [rows, cols] matrices into column range [coff, coff + rows) of [cols, ld_dst].
template <typename T>
__global__ __launch_bounds__(256) void transpose_into_kernel(const T* __restrict__ src, int rows, int cols,
                                                             T* __restrict__ dst, int64_t ld_dst, int coff,
                                                             int64_t dst_batch) {
  __shared__ T tile[kTile][kTile + 2];
  const T* S = src + (int64_t)blockIdx.z * rows * cols;
  T* D = dst + (int64_t)blockIdx.z * dst_batch;
  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < kTile; i += 4) tile[i][tx] = S[(int64_t)(r0 + i) * cols + c0 + tx];
  __syncthreads();
  for (int i = ty; i < kTile; i += 4) D[(int64_t)(c0 + i) * ld_dst + coff + r0 + tx] = tile[tx][i];
}

GemmArgs args_grouped(const void* A, const int32_t* a_rows, const void* B0, const void* B1, int64_t b_stride,
                      const int32_t* seg, int G, int64_t M, int N, int K, void* C) {
  GemmArgs a{};
  a.A = A;
  a.a_rows = a_rows;
  a.B0 = B0;
  a.B1 = B1;
  a.b_stride = b_stride;
  a.seg = seg;
  a.G = G;
  a.M = M;
  a.N = N;
  a.K = K;
  a.C = C;
  return a;
}

template <typename T, int BK, int EPI, int FEAT = 0>
void gemm(GemmArgs a, int num_cu, hipStream_t s) {
  if (a.m_chunk == 0 && a.n_group == 0) {
    a.m_chunk = (FEAT & kFeatStrides) ? kWgradRowChunk : kRowsRowChunk;
    a.n_group = (FEAT & kFeatStrides) ? kWgradColumnGroup : kRowsColumnGroup;
  }
  hipLaunchKernelGGL((grouped_gemm_kernel<T, 256, 256, BK, 4, 2, 2, EPI, 1, FEAT>), dim3(num_cu), dim3(512), 0, s, a);
}

template <typename T, int BK>
hipError_t ffn_backward_t(int64_t n_max, int64_t d, int64_t E, int64_t F, const void* x_in, int64_t n_in,
                          const int32_t* a_rows, const int32_t* raw_offsets, const void* w_gate, const void* w_up, const void* w_down,
                          const void* dy_perm, const void* gu, void* dx_perm, float* dw_gate, float* dw_up,
                          float* dw_down, const FfnBackwardScratch& w, int num_cu, hipStream_t s) {
  const int64_t np = w.n_pad;   // columns of the padded transposed layouts
  const T* Wg = static_cast<const T*>(w_gate);
  const T* Wu = static_cast<const T*>(w_up);
  const T* Wd = static_cast<const T*>(w_down);

  // consistent and padded expert row ranges; transposed weights
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(1024), 0, s, raw_offsets, (int)E, n_max, w.soff, w.poff);
  const int32_t* offsets = w.soff;
  // (whole, regular matrices: one tile per block keeps the most tiles in flight)
  auto transpose_into = [&](const T* src, int rows, int cols, T* dst, int64_t ld_dst, int coff, int64_t batch) {
    hipLaunchKernelGGL((transpose_into_kernel<T>), dim3((unsigned)(cols / kTile), (unsigned)(rows / kTile), (unsigned)E),
                       dim3(256), 0, s, src, rows, cols, dst, ld_dst, coff, batch);
  };
  // 16-bit weights are read where they lie (B stored along N, transposing LDS
  // reads); float32 ones through transposed copies
  constexpr bool kBkn = sizeof(T) == 2;
  if constexpr (!kBkn) {
    transpose_into(Wd, (int)d, (int)F, static_cast<T*>(w.wd_t), d, 0, F * d);
    transpose_into(Wg, (int)F, (int)d, static_cast<T*>(w.wgu_t), 2 * F, 0, d * 2 * F);
    transpose_into(Wu, (int)F, (int)d, static_cast<T*>(w.wgu_t), 2 * F, (int)F, d * 2 * F);
  }

  if (gu) {
    // dH = dY W_d accumulated; the epilogue reads the saved G | U and writes dG | dU, H
    const void* wd = kBkn ? static_cast<const void*>(Wd) : static_cast<const void*>(w.wd_t);
    GemmArgs a1 = args_grouped(dy_perm, nullptr, wd, nullptr, d * F, offsets, (int)E, n_max, (int)F, (int)d, w.dgu);
    a1.D = gu;
    a1.C2 = w.h;
    a1.ldc = 2 * F;
    if constexpr (kBkn)
      gemm<T, BK, EPI_DH_SWIGLU, kFeatBKN>(a1, num_cu, s);
    else
      gemm<T, BK, EPI_DH_SWIGLU>(a1, num_cu, s);
  } else {
    // dH = dY W_d (float32)
    if constexpr (kBkn) {
      GemmArgs a1 = args_grouped(dy_perm, nullptr, Wd, nullptr, d * F, offsets, (int)E, n_max, (int)F, (int)d, w.dh);
      gemm<T, BK, EPI_F32, kFeatBKN>(a1, num_cu, s);
    } else {
      GemmArgs a1 = args_grouped(dy_perm, nullptr, w.wd_t, nullptr, F * d, offsets, (int)E, n_max, (int)F, (int)d,
                                 w.dh);
      gemm<T, BK, EPI_F32>(a1, num_cu, s);
    }
    // recompute G, U; dG | dU and H
    GemmArgs a2 = args_grouped(x_in, a_rows, w_gate, w_up, F * d, offsets, (int)E, n_max, (int)F, (int)d, w.dgu);
    a2.a_rows_n = n_in;
    a2.D = w.dh;
    a2.C2 = w.h;
    a2.ldc = 2 * F;
    gemm<T, BK, EPI_SWIGLU_BWD>(a2, num_cu, s);
  }
  // dX = [dG | dU] [W_g ; W_u]: k < F reads W_g's rows, k >= F W_u's
  if constexpr (kBkn) {
    GemmArgs a3 = args_grouped(w.dgu, nullptr, Wg, Wu, F * d, offsets, (int)E, n_max, (int)d, (int)(2 * F), dx_perm);
    a3.k_split = (int32_t)F;
    gemm<T, BK, EPI_STORE, kFeatBKN>(a3, num_cu, s);
  } else {
    GemmArgs a3 = args_grouped(w.dgu, nullptr, w.wgu_t, nullptr, d * 2 * F, offsets, (int)E, n_max, (int)d,
                               (int)(2 * F), dx_perm);
    gemm<T, BK, EPI_STORE>(a3, num_cu, s);
  }

  // transposed, padded, k-blocked activations for the weight gradients
  const unsigned nblk = (unsigned)(np / kTile);
  hipLaunchKernelGGL(pad_block_experts_kernel, dim3((nblk + 255) / 256), dim3(256), 0, s, w.poff, (int)E,
                     w.pblk_expert);
  auto pad_transpose = [&](const void* src, int64_t ld_src, int col0, const int32_t* rows, void* dst, int64_t R) {
    if constexpr (sizeof(T) == 2 && BK == kTile) {
      hipLaunchKernelGGL(pad_transpose16_kernel, dim3(nblk, (unsigned)((R / kTile + 7) / 8)), dim3(256), 0, s,
                         static_cast<const uint16_t*>(src), ld_src, col0, rows, n_in, offsets, w.poff,
                         w.pblk_expert, (int)E, static_cast<uint16_t*>(dst), R);
    } else {
      hipLaunchKernelGGL((pad_transpose_kernel<T, BK>), dim3(nblk, (unsigned)(R / kTile)), dim3(256), 0, s,
                         static_cast<const T*>(src), ld_src, col0, rows, n_in, offsets, w.poff, w.pblk_expert,
                         (int)E, static_cast<T*>(dst), R);
    }
  };
  pad_transpose(x_in, d, 0, a_rows, w.x_t, d);
  pad_transpose(dy_perm, d, 0, nullptr, w.dy_t, d);
  pad_transpose(w.h, F, 0, nullptr, w.h_t, F);
  pad_transpose(w.dgu, 2 * F, 0, nullptr, w.dg_t, F);
  pad_transpose(w.dgu, 2 * F, (int)F, nullptr, w.du_t, F);

  // weight gradients: one group per expert, k over its padded column range
  auto wgrad = [&](const void* A, int rows, const void* B, int N, float* C) {
    GemmArgs a = args_grouped(A, nullptr, B, nullptr, 0, nullptr, (int)E, E * rows, N, 0, C);
    a.group_rows = rows;
    a.a_shared = 1;
    a.lda = BK;
    a.ldb = BK;
    a.ksa = (int64_t)rows * BK;
    a.ksb = (int64_t)N * BK;
    a.kseg = w.poff;
    gemm<T, BK, EPI_F32, kFeatGroups | kFeatStrides>(a, num_cu, s);
  };
  wgrad(w.dy_t, (int)d, w.h_t, (int)F, dw_down);
  wgrad(w.dg_t, (int)F, w.x_t, (int)d, dw_gate);
  wgrad(w.du_t, (int)F, w.x_t, (int)d, dw_up);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_ffn_backward(int dtype, int64_t n_max, int64_t d, int64_t E, int64_t F, const void* x_in,
                                       int64_t n_in, const int32_t* a_rows, const int32_t* offsets,
                                       const void* w_gate, const void* w_up, const void* w_down, const void* dy_perm,
                                       const void* gu, void* dx_perm, float* dw_gate, float* dw_up, float* dw_down,
                                       const FfnBackwardScratch& w, int num_cu, hipStream_t s) {
  if (dtype == 1)
    return ffn_backward_t<bf16, 64>(n_max, d, E, F, x_in, n_in, a_rows, offsets, w_gate, w_up, w_down, dy_perm, gu,
                                    dx_perm, dw_gate, dw_up, dw_down, w, num_cu, s);
  return ffn_backward_t<float, 32>(n_max, d, E, F, x_in, n_in, a_rows, offsets, w_gate, w_up, w_down, dy_perm, gu,
                                   dx_perm, dw_gate, dw_up, dw_down, w, num_cu, s);
}

}  // namespace moe
