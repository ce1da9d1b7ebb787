// Weighted un-permute: y[t] = sum_j w[t,j] * y_perm[slot_row[t,j]].
//
// Each token's output mixes the outputs of the few experts it was routed to
// (section 二 of "Domyn 团队在 Jupiter 超算完成 1 万亿参数 MoE 模型训练项目解析"),
// weighted by its renormalised gate weights.  A gather, not a scatter-add: one
// wavefront per token reads its k expert rows with 16-byte loads, sums in
// float32 in slot order, and stores the row once.  No atomics, so the result
// is bit-reproducible.  Negative rows (slots owned elsewhere) contribute 0.
#include "common.h"
#include "kernels.h"
#include "rows.h"

namespace moe {

namespace {

// KU > 0: k is the compile-time KU, so the token's KU row loads are all in
// flight before the first FMA; KU == 0: any k, in groups of 8.
template <typename T, int KU>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y_perm, const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ w, int Tn, int d, int k,
                                                      T* __restrict__ y) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= Tn) return;
  const int lane = threadIdx.x & 63;
  const int32_t* sr = slot_row + (int64_t)t * k;
  const float* wt = w + (int64_t)t * k;
  if constexpr (KU > 0) {
    int row[KU];
    float wj[KU];
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      row[j] = __builtin_amdgcn_readfirstlane(sr[j]);
      wj[j] = wt[j];
    }
    // two 512-column pieces per pass: 2 KU row loads in flight per lane
    for (int c0 = lane * 8; c0 < d; c0 += 2 * 64 * 8) {
      const int c1 = c0 + 64 * 8;
      const bool has1 = c1 < d;
      typename Raw16<T>::type v[2][KU];   // kept as loaded until the FMAs
#pragma unroll
      for (int j = 0; j < KU; ++j)
        if (row[j] >= 0) {
          v[0][j] = Raw16<T>::load(y_perm + (int64_t)row[j] * d + c0);
          if (has1) v[1][j] = Raw16<T>::load(y_perm + (int64_t)row[j] * d + c1);
        }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
        for (int j = 0; j < KU; ++j)
          if (row[j] >= 0) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj[j], Raw16<T>::get(v[h][j], i), acc[i]);
          }
        if (h == 0) store8(y + (int64_t)t * d + c0, acc);
        else if (has1) store8(y + (int64_t)t * d + c1, acc);
      }
    }
  } else {
    for (int c0 = lane * 8; c0 < d; c0 += 64 * 8) {
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
      for (int j = 0; j < k; ++j) {
        const int row = sr[j];
        if (row < 0) continue;
        const float wj = wt[j];
        float v[8];
        load8(y_perm + (int64_t)row * d + c0, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
      }
      store8(y + (int64_t)t * d + c0, acc);
    }
  }
}

template <typename T>
void launch_combine_t(int64_t T_, int64_t d, int64_t k, const T* y_perm, const int32_t* slot_row, const float* w,
                      T* y, hipStream_t stream) {
  const dim3 grid((unsigned)((T_ + 3) / 4)), block(256);
  const int Tn = (int)T_, dn = (int)d, kn = (int)k;
  switch (k) {
    case 1: hipLaunchKernelGGL((combine_kernel<T, 1>), grid, block, 0, stream, y_perm, slot_row, w, Tn, dn, kn, y); break;
    case 2: hipLaunchKernelGGL((combine_kernel<T, 2>), grid, block, 0, stream, y_perm, slot_row, w, Tn, dn, kn, y); break;
    case 4: hipLaunchKernelGGL((combine_kernel<T, 4>), grid, block, 0, stream, y_perm, slot_row, w, Tn, dn, kn, y); break;
    case 8: hipLaunchKernelGGL((combine_kernel<T, 8>), grid, block, 0, stream, y_perm, slot_row, w, Tn, dn, kn, y); break;
    default: hipLaunchKernelGGL((combine_kernel<T, 0>), grid, block, 0, stream, y_perm, slot_row, w, Tn, dn, kn, y);
  }
}

}  // namespace

hipError_t launch_combine(int dtype, int64_t T, int64_t d, int64_t k, const void* y_perm, const int32_t* slot_row,
                          const float* w, void* y, hipStream_t stream) {
  if (dtype == 1)
    launch_combine_t<bf16>(T, d, k, (const bf16*)y_perm, slot_row, w, (bf16*)y, stream);
  else
    launch_combine_t<float>(T, d, k, (const float*)y_perm, slot_row, w, (float*)y, stream);
  return hipGetLastError();
}

}  // namespace moe
