// Permutation of token slots by expert: a deterministic counting sort.
//
// Tokens go to a few experts each (section 二 of "Domyn 团队在 Jupiter 超算完成
// 1 万亿参数 MoE 模型训练项目解析"), so the rows an expert works on must be
// gathered.  The order inside an expert's segment is ascending token index,
// which makes the result unique and bit-reproducible:
//   1. count:   each block of 256 tokens counts its slots per expert (LDS);
//   2. scan:    per expert, an exclusive prefix of the block counts (in place),
//               then an exclusive prefix over experts gives the offsets;
//   3. scatter: each block sets one bit per (expert, token) in an LDS bitmap;
//               a slot's rank among its block's rows of that expert is the
//               popcount of the bits of lower tokens, so
//               row = offsets[e] + block_prefix[b][e] + rank;
//               then (unless only indices are wanted) the block copies each
//               token's row to its k destinations with 16-byte vectors.
// No global atomics: two runs give identical bits.  A negative id (or one >= E)
// marks a slot that is skipped.  A token that names the same expert in two slots
// (top-k never does; pre-routed input might) gets two rows, in slot order, like
// any counting sort of the slots: the bitmap cannot count such a token twice, so
// an expert with a repeated (token, expert) pair in a block is ranked by a serial
// walk over the block's slots instead.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int TB = kPermuteBlockTokens;   // tokens per block
constexpr int WPB = TB / 32;              // bitmap words per expert

__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ ids, int T, int E, int k,
                                                            int32_t* __restrict__ counts) {
  __shared__ int hist[kMaxExperts];
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t s0 = (int64_t)blockIdx.x * TB * k;
  const int64_t s1 = min<int64_t>((int64_t)T * k, s0 + (int64_t)TB * k);
  for (int64_t s = s0 + threadIdx.x; s < s1; s += 256) {
    const int e = ids[s];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// One block of 1024 threads: thread e scans column e of the [nblk, E] counts.
__global__ __launch_bounds__(1024) void permute_scan_kernel(int32_t* __restrict__ counts, int nblk, int E,
                                                            int32_t* __restrict__ offsets) {
  __shared__ int wsum[16];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = counts[(int64_t)(b + i) * E + e];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        counts[(int64_t)(b + i) * E + e] = run;
        run += v[i];
      }
    }
    for (; b < nblk; ++b) {
      const int v = counts[(int64_t)b * E + e];
      counts[(int64_t)b * E + e] = run;
      run += v;
    }
  }
  // exclusive scan of the per-expert totals over e (1024 threads)
  const int lane = e & 63, wv = e >> 6;
  int incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int i = 0; i < wv; ++i) before += wsum[i];
  if (e < E) offsets[e] = before + incl - run;
  if (e == E - 1) offsets[E] = before + incl;
}

template <typename T>
__global__ __launch_bounds__(256) void permute_scatter_kernel(const T* __restrict__ x, const int32_t* __restrict__ ids,
                                                              int Tn, int d, int E, int k,
                                                              const int32_t* __restrict__ offsets,
                                                              const int32_t* __restrict__ block_prefix,
                                                              int32_t* __restrict__ row_token,
                                                              int32_t* __restrict__ slot_row, T* __restrict__ x_perm) {
  __shared__ uint32_t bits[kMaxExperts * WPB];
  __shared__ int base[kMaxExperts];
  __shared__ uint8_t repeated[kMaxExperts];   // expert e has a token naming it twice in this block
  __shared__ int any_repeated;
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < E * WPB; i += 256) bits[i] = 0u;
  for (int e = threadIdx.x; e < E; e += 256) {
    base[e] = offsets[e] + block_prefix[(int64_t)b * E + e];
    repeated[e] = 0;
  }
  if (threadIdx.x == 0) any_repeated = 0;
  __syncthreads();
  const int t0 = b * TB;
  const int64_t s0 = (int64_t)t0 * k;
  const int64_t s1 = min<int64_t>((int64_t)Tn * k, s0 + (int64_t)TB * k);
  for (int64_t s = s0 + threadIdx.x; s < s1; s += 256) {
    const int e = ids[s];
    if (e >= 0 && e < E) {
      const int tl = (int)(s / k) - t0;
      const uint32_t m = 1u << (tl & 31);
      if (atomicOr(&bits[e * WPB + (tl >> 5)], m) & m) {
        repeated[e] = 1;
        any_repeated = 1;
      }
    }
  }
  __syncthreads();

  // indices: one thread per slot (experts with a repeated pair: below)
  for (int64_t s = s0 + threadIdx.x; s < s1; s += 256) {
    const int e = ids[s];
    const int t = (int)(s / k);
    if (e >= 0 && e < E) {
      if (repeated[e]) continue;
      const int tl = t - t0;
      const uint32_t* w = bits + e * WPB;
      int rank = __popc(w[tl >> 5] & ((1u << (tl & 31)) - 1u));
      for (int q = 0; q < (tl >> 5); ++q) rank += __popc(w[q]);
      const int row = base[e] + rank;
      row_token[row] = t;
      slot_row[s] = row;
    } else {
      slot_row[s] = -1;
    }
  }
  if (any_repeated) {
    // one thread per such expert walks the block's slots in (token, slot) order
    for (int e = threadIdx.x; e < E; e += 256) {
      if (!repeated[e]) continue;
      int row = base[e];
      for (int64_t s = s0; s < s1; ++s)
        if (ids[s] == e) {
          row_token[row] = (int)(s / k);
          slot_row[s] = row++;
        }
    }
  }
  if (x_perm == nullptr) return;
  __syncthreads();   // this block's slot_row entries are written

  // rows: each wavefront copies its tokens' rows to their destinations with
  // 16-byte vectors
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nt = min(TB, Tn - t0);
  constexpr int EPC = 16 / sizeof(T);
  const int nchunk = d / EPC;
  for (int tl = wave; tl < nt; tl += 4) {
    const int t = t0 + tl;
    for (int j = 0; j < k; ++j) {
      const int row = slot_row[(int64_t)t * k + j];
      if (row < 0) continue;
      const u32x4* src = reinterpret_cast<const u32x4*>(x + (int64_t)t * d);
      u32x4* dst = reinterpret_cast<u32x4*>(x_perm + (int64_t)row * d);
      for (int c = lane; c < nchunk; c += 64) dst[c] = src[c];
    }
  }
}

}  // namespace

hipError_t launch_permute(int dtype, int64_t T, int64_t d, int64_t E, int64_t k, const void* x, const int32_t* ids,
                          int32_t* offsets, int32_t* row_token, int32_t* slot_row, void* x_perm,
                          int32_t* block_counts, hipStream_t stream) {
  const int nblk = (int)((T + TB - 1) / TB);
  hipLaunchKernelGGL(permute_count_kernel, dim3(nblk), dim3(256), 0, stream, ids, (int)T, (int)E, (int)k,
                     block_counts);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, stream, block_counts, nblk, (int)E, offsets);
  if (dtype == 1)
    hipLaunchKernelGGL(permute_scatter_kernel<bf16>, dim3(nblk), dim3(256), 0, stream, (const bf16*)x, ids, (int)T,
                       (int)d, (int)E, (int)k, offsets, block_counts, row_token, slot_row, (bf16*)x_perm);
  else
    hipLaunchKernelGGL(permute_scatter_kernel<float>, dim3(nblk), dim3(256), 0, stream, (const float*)x, ids,
                       (int)T, (int)d, (int)E, (int)k, offsets, block_counts, row_token, slot_row,
                       (float*)x_perm);
  return hipGetLastError();
}

}  // namespace moe
