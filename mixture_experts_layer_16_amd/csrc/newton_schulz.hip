// Muon's Newton-Schulz orthogonalisation of a batch of whole matrices.
//
// Muon orthogonalises every update with a few Newton-Schulz iterations over the
// whole matrix, and whole experts are placed on one rank so each rank runs them
// on complete expert matrices without communication ("FlexShard: communication-
// free Muon" in "Training a 1T-Parameter MoE on EU public infrastructure with
// PyTorch and TorchTitan").  The iteration is Muon's quintic, on the wide
// orientation of each matrix (a tall one is transposed first and back at the
// end):
//     X = G / (||G||_F + eps);   repeat: A = X X^T,  B = b A + c A A,  X = a X + B X
//
// Layout and kernels (bf16 storage, fp32 accumulation):
//   * sum of squares per matrix: kNormBlocks partial sums, each over a fixed
//     contiguous chunk, then every consumer adds the partials in one fixed order
//     (deterministic, no atomics);
//   * init: X0 scaled and cast, written in the wide orientation Xw [R', C'] (a
//     tall G through a 64 x 64 LDS tile);
//   * per step, three launches of the grouped GEMM with one group per matrix:
//       A   = Xw Xw^T              (NT, K = C')
//       B   = c (A A^T) + b A      (NT, K = R'; A is symmetric, so A A^T = A A)
//       Xw' = B Xw + a Xw          (K = R'; Xw is read where it lies, as a B
//                                   operand stored along N), into the other Xw
//     A wide matrix's last step writes the caller's output directly; a tall
//     one's result is transposed once at the end.
#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int kTile = 64;

// partial[m * kNormBlocks + b] = sum of squares of chunk b of matrix m (chunks of
// per / kNormBlocks elements, a multiple of 8: R and C are multiples of 64), read as
// 16-byte vectors; each thread's running sum, then a fixed-order block reduction.
__global__ __launch_bounds__(256) void ns_sumsq_kernel(const bf16* __restrict__ g, int64_t per, float* __restrict__ partial) {
  __shared__ float wsum[4];
  const int m = blockIdx.y, b = blockIdx.x;
  const int64_t chunk = per / kNormBlocks;
  const bf16* p = g + (int64_t)m * per + (int64_t)b * chunk;
  float s = 0.f;
  for (int64_t i = (int64_t)threadIdx.x * 8; i < chunk; i += 256 * 8) {
    const bf16x8 q = *reinterpret_cast<const bf16x8*>(p + i);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = static_cast<float>(q[j]);
      s = fmaf(v, v, s);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) partial[(int64_t)m * kNormBlocks + b] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
}

// scale = 1 / (sqrt(sum of the partials in order) + eps); out_same = scale * G (G's
// orientation), out_t = its transpose, both rounded once to bf16 (either may be
// null: not written).  One 64 x 64 tile
// of one matrix per block: each thread reads 16 consecutive elements of one row
// (two 16-byte loads), writes them scaled in place order, and parks them in LDS
// column-wise; then reads 16 consecutive elements of one transposed row.
__global__ __launch_bounds__(256) void ns_init_kernel(const bf16* __restrict__ g, int R, int C,
                                                      const float* __restrict__ partial, float eps,
                                                      bf16* __restrict__ out_same, bf16* __restrict__ out_t) {
  __shared__ uint16_t tile[kTile][kTile + 2];
  const int m = blockIdx.z;
  float ss = 0.f;
  for (int i = 0; i < kNormBlocks; ++i) ss += partial[(int64_t)m * kNormBlocks + i];
  const float scale = 1.0f / (sqrtf(ss) + eps);
  const int64_t per = (int64_t)R * C;
  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  const int t = threadIdx.x, r = t >> 2, q = (t & 3) * 16;
  const int64_t off = m * per + (int64_t)(r0 + r) * C + c0 + q;
  bf16x8 v[2];
  v[0] = *reinterpret_cast<const bf16x8*>(g + off);
  v[1] = *reinterpret_cast<const bf16x8*>(g + off + 8);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 8; ++j) v[h][j] = static_cast<bf16>(static_cast<float>(v[h][j]) * scale);
  // park the 16 rounded values column-wise (halves taken from the packed words)
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const u32x4 w = __builtin_bit_cast(u32x4, v[h]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[q + 8 * h + 2 * e][r] = (uint16_t)(w[e] & 0xffffu);
      tile[q + 8 * h + 2 * e + 1][r] = (uint16_t)(w[e] >> 16);
    }
  }
  if (out_same) {
    *reinterpret_cast<bf16x8*>(out_same + off) = v[0];
    *reinterpret_cast<bf16x8*>(out_same + off + 8) = v[1];
  }
  if (out_t == nullptr) return;   // (the same for the whole block)
  __syncthreads();
  const int c = t >> 2, p = (t & 3) * 16;
  const uint32_t* row = reinterpret_cast<const uint32_t*>(&tile[c][0]) + p / 2;
  u32x4 o0, o1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o0[e] = row[e];
    o1[e] = row[4 + e];
  }
  uint16_t* d = reinterpret_cast<uint16_t*>(out_t) + m * per + (int64_t)(c0 + c) * R + r0 + p;
  *reinterpret_cast<u32x4*>(d) = o0;
  *reinterpret_cast<u32x4*>(d + 8) = o1;
}

// dst[m] = src[m]^T for [rows, cols] bf16 matrices; one 64 x 64 tile per block
// (for these whole, regular matrices one tile per block keeps more tiles in
// flight than the strip transposes, which pay off where rows are looked up).
__global__ __launch_bounds__(256) void ns_transpose_kernel(const bf16* __restrict__ src, int rows, int cols,
                                                           bf16* __restrict__ dst) {
  __shared__ bf16 tile[kTile][kTile + 2];
  const int64_t per = (int64_t)rows * cols;
  const bf16* S = src + blockIdx.z * per;
  bf16* D = dst + blockIdx.z * per;
  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < kTile; i += 4) tile[i][tx] = S[(int64_t)(r0 + i) * cols + c0 + tx];
  __syncthreads();
  for (int i = ty; i < kTile; i += 4) D[(int64_t)(c0 + i) * rows + r0 + tx] = tile[tx][i];
}

GemmArgs batch_gemm(const bf16* A, const bf16* B, int64_t b_stride, int n, int64_t rows, int N, int K, bf16* C) {
  GemmArgs a{};
  a.A = A;
  a.a_rows = nullptr;
  a.B0 = B;
  a.B1 = nullptr;
  a.b_stride = b_stride;
  a.seg = nullptr;
  a.G = n;
  a.M = (int64_t)n * rows;
  a.group_rows = rows;
  a.N = N;
  a.K = K;
  a.C = C;
  a.bias = nullptr;
  return a;
}

}  // namespace

hipError_t launch_newton_schulz(int64_t n, int64_t R, int64_t C, int64_t steps, float a, float b, float c,
                                float eps, const void* g, void* x, void* xw0, void* xw1, void* A, void* B,
                                float* partial, int num_cu, hipStream_t stream) {
  const bool tall = R > C;
  const int64_t Rw = tall ? C : R, Cw = tall ? R : C;   // wide orientation
  const int64_t per = R * C;
  const bf16* G = static_cast<const bf16*>(g);
  bf16* X = static_cast<bf16*>(x);
  bf16* Xw[2] = {static_cast<bf16*>(xw0), static_cast<bf16*>(xw1)};
  bf16* Ab = static_cast<bf16*>(A);
  bf16* Bb = static_cast<bf16*>(B);

  hipLaunchKernelGGL(ns_sumsq_kernel, dim3(kNormBlocks, (unsigned)n), dim3(256), 0, stream, G, per, partial);
  // X0: the output itself when there are no steps, else the wide orientation
  bf16* same = steps == 0 ? X : (tall ? nullptr : Xw[0]);
  bf16* trans = (steps == 0 || !tall) ? nullptr : Xw[0];
  hipLaunchKernelGGL(ns_init_kernel, dim3((unsigned)(C / kTile), (unsigned)(R / kTile), (unsigned)n), dim3(256), 0,
                     stream, G, (int)R, (int)C, partial, eps, same, trans);
  if (steps == 0) return hipGetLastError();

  constexpr int BK = 64, ST = 2, WM = 4, WN = 2;
  int cur = 0;
  for (int64_t s = 0; s < steps; ++s) {
    const bool last = s + 1 == steps;
    // A = Xw Xw^T
    GemmArgs p1 = batch_gemm(Xw[cur], Xw[cur], Rw * Cw, (int)n, Rw, (int)Rw, (int)Cw, Ab);
    hipLaunchKernelGGL((grouped_gemm_kernel<bf16, 256, 256, BK, WM, WN, ST, EPI_STORE, 1, kFeatGroups>), dim3(num_cu),
                       dim3(WM * WN * 64), 0, stream, p1);
    // B = c (A A^T) + b A
    GemmArgs p2 = batch_gemm(Ab, Ab, Rw * Rw, (int)n, Rw, (int)Rw, (int)Rw, Bb);
    p2.alpha = c;
    p2.beta = b;
    p2.D = Ab;
    hipLaunchKernelGGL((grouped_gemm_kernel<bf16, 256, 256, BK, WM, WN, ST, EPI_AXPBY, 1, kFeatGroups>), dim3(num_cu),
                       dim3(WM * WN * 64), 0, stream, p2);
    // Xw' = B Xw + a Xw (Xw [R', C'] read along C' as stored); a wide matrix's last
    // step writes the caller's output
    bf16* out = (last && !tall) ? X : Xw[cur ^ 1];
    GemmArgs p3 = batch_gemm(Bb, Xw[cur], Rw * Cw, (int)n, Rw, (int)Cw, (int)Rw, out);
    p3.alpha = 1.0f;
    p3.beta = a;
    p3.D = Xw[cur];
    hipLaunchKernelGGL((grouped_gemm_kernel<bf16, 256, 256, BK, WM, WN, ST, EPI_AXPBY, 1, kFeatGroups | kFeatBKN>),
                       dim3(num_cu), dim3(WM * WN * 64), 0, stream, p3);
    cur ^= 1;
  }
  // a tall matrix: its result is the transpose of the wide one
  if (tall)
    hipLaunchKernelGGL(ns_transpose_kernel, dim3((unsigned)(Cw / kTile), (unsigned)(Rw / kTile), (unsigned)n),
                       dim3(256), 0, stream, Xw[cur], (int)Rw, (int)Cw, X);
  return hipGetLastError();
}

}  // namespace moe
