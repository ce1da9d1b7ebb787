// Routing: router GEMM (MFMA) and a wavefront-level softmax/top-k.
//
// The layer sends each token to the k experts with the largest router scores
// (model-configuration table of "Training a 1T-Parameter MoE on EU public
// infrastructure with PyTorch and TorchTitan": top-8 of 384 routed experts).
// Selection uses the float32 logits with -0.0 == +0.0 and ties going to the
// lower expert index; the weights are the selected softmax probabilities
// renormalised to sum to one, i.e. exp(l_j - l_max) / sum_S exp(l_i - l_max).
#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"

namespace moe {

namespace {

// Monotone map float32 -> uint32 (larger float, larger key); -0.0 is folded to +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float order_key_inv(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t other = __shfl_xor(v, o, 64);
    v = other > v ? other : v;
  }
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  // every lane ends with the same bits: at each level both partners add the
  // same two values, and float addition is commutative
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// One wavefront per token.  Each lane holds logits e = lane + 64*i as 64-bit
// keys (order_key(l) << 32 | ~e), so one unsigned max picks the larger logit
// and, among equal logits, the lower index.  k rounds of (lane max, wave max,
// remove winner) give the k selected experts in key order.
template <int VPL, int KPL>
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                           int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= T) return;
  const float* row = logits + (int64_t)t * E;

  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? ((uint64_t)order_key(row[e]) << 32) | (uint32_t)(0xffffffffu - (uint32_t)e) : 0ull;
  }

  uint64_t sel[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) sel[i] = 0ull;

  for (int r = 0; r < k; ++r) {
    uint64_t best = 0ull;
#pragma unroll
    for (int i = 0; i < VPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64(best);
    const uint32_t e = 0xffffffffu - (uint32_t)best;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if ((uint32_t)(lane + 64 * i) == e) key[i] = 0ull;
#pragma unroll
    for (int i = 0; i < KPL; ++i)
      if (lane + 64 * i == r) sel[i] = best;
  }

  // the first selection is the largest logit of the row
  const float lmax = order_key_inv((uint32_t)(__shfl(sel[0], 0, 64) >> 32));
  float part = 0.f;
  float ex[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int r = lane + 64 * i;
    ex[i] = 0.f;
    if (r < k) {
      ex[i] = expf(order_key_inv((uint32_t)(sel[i] >> 32)) - lmax);
      part += ex[i];
    }
  }
  const float denom = wave_sum(part);
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int r = lane + 64 * i;
    if (r < k) {
      ids[(int64_t)t * k + r] = (int32_t)(0xffffffffu - (uint32_t)sel[i]);
      w[(int64_t)t * k + r] = ex[i] / denom;
    }
  }
}

template <int VPL>
hipError_t launch_topk_vpl(int64_t T, int64_t E, int64_t k, const float* logits, int32_t* ids, float* w,
                           hipStream_t stream) {
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (k <= 64)
    hipLaunchKernelGGL((topk_softmax_kernel<VPL, 1>), grid, block, 0, stream, logits, (int)T, (int)E, (int)k, ids, w);
  else
    hipLaunchKernelGGL((topk_softmax_kernel<VPL, 16>), grid, block, 0, stream, logits, (int)T, (int)E, (int)k, ids, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(int64_t T, int64_t E, int64_t k, const float* logits, int32_t* ids, float* w,
                       hipStream_t stream) {
  if (E <= 64) return launch_topk_vpl<1>(T, E, k, logits, ids, w, stream);
  if (E <= 128) return launch_topk_vpl<2>(T, E, k, logits, ids, w, stream);
  if (E <= 256) return launch_topk_vpl<4>(T, E, k, logits, ids, w, stream);
  if (E <= 512) return launch_topk_vpl<8>(T, E, k, logits, ids, w, stream);
  return launch_topk_vpl<16>(T, E, k, logits, ids, w, stream);
}

hipError_t launch_router_gemm(int dtype, int64_t T, int64_t d, int64_t E, const void* x, const void* w_router,
                              const float* bias, float* logits, int num_cu, hipStream_t stream) {
  GemmArgs a{};
  a.A = x;
  a.a_rows = nullptr;
  a.B0 = w_router;
  a.B1 = nullptr;
  a.b_stride = 0;
  a.seg = nullptr;
  a.G = 1;
  a.M = T;
  a.N = (int32_t)E;
  a.K = (int32_t)d;
  a.C = logits;
  a.bias = bias;
  a.n_group = 0;
  a.m_chunk = 0;
  const dim3 grid((unsigned)num_cu), block(512);
  if (dtype == 1)
    hipLaunchKernelGGL((grouped_gemm_kernel<bf16, 256, 256, 64, 4, 2, 2, EPI_F32_BIAS>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<float, 256, 256, 32, 4, 2, 2, EPI_F32_BIAS>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
