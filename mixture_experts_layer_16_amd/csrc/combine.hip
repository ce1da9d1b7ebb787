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

namespace moe {

namespace {

__device__ __forceinline__ void load8(const bf16* p, float* v) {
  const bf16x8 q = *reinterpret_cast<const bf16x8*>(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = static_cast<float>(q[i]);
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
  bf16x8 q;
#pragma unroll
  for (int i = 0; i < 8; ++i) q[i] = static_cast<bf16>(v[i]);
  *reinterpret_cast<bf16x8*>(p) = q;
}
__device__ __forceinline__ void load8(const float* p, float* v) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[i + 4] = b[i]; }
}
__device__ __forceinline__ void store8(float* p, const float* v) {
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) { a[i] = v[i]; b[i] = v[i + 4]; }
  *reinterpret_cast<f32x4*>(p) = a;
  *reinterpret_cast<f32x4*>(p + 4) = b;
}

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y_perm, const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ w, int Tn, int d, int k,
                                                      T* __restrict__ y) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= Tn) return;
  const int lane = threadIdx.x & 63;
  const int32_t* sr = slot_row + (int64_t)t * k;
  const float* wt = w + (int64_t)t * k;
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

}  // namespace

hipError_t launch_combine(int dtype, int64_t T, int64_t d, int64_t k, const void* y_perm, const int32_t* slot_row,
                          const float* w, void* y, hipStream_t stream) {
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (dtype == 1)
    hipLaunchKernelGGL(combine_kernel<bf16>, grid, block, 0, stream, (const bf16*)y_perm, slot_row, w, (int)T, (int)d,
                       (int)k, (bf16*)y);
  else
    hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, stream, (const float*)y_perm, slot_row, w, (int)T,
                       (int)d, (int)k, (float*)y);
  return hipGetLastError();
}

}  // namespace moe
