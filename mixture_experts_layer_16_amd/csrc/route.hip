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

// One 16-lane DPP row per token (four tokens per wavefront) for E a multiple of 4,
// E <= 64 V4 and k <= 16: lane l of a row loads logits 64 i + 4 l .. + 3 as float4
// (i < V4), so each k round is a maximum over the lane's 4 V4 keys, then over the
// row through DPP moves (no LDS round trips); the same 64-bit keys and tie rule as
// topk_softmax_kernel, so the same selection.
template <int CTRL> __device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL> __device__ __forceinline__ uint64_t row_max_step(uint64_t v) {
  const uint64_t o = ((uint64_t)dpp32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp32<CTRL>((uint32_t)v);
  return o > v ? o : v;
}
template <int CTRL> __device__ __forceinline__ float row_sum_step(float v) {
  return v + __uint_as_float(dpp32<CTRL>(__float_as_uint(v)));
}
// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1] (partners 1 and 2 apart), half-row
// mirror (lane i <-> 7 - i within 8), row mirror (i <-> 15 - i within 16).  At every
// step both partners combine the same two values, so every lane of the row ends
// with the same bits.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
__device__ __forceinline__ uint64_t row16_max(uint64_t v) {
  v = row_max_step<kDppXor1>(v);
  v = row_max_step<kDppXor2>(v);
  v = row_max_step<kDppHalfMirror>(v);
  return row_max_step<kDppMirror>(v);
}
__device__ __forceinline__ float row16_sum(float v) {
  v = row_sum_step<kDppXor1>(v);
  v = row_sum_step<kDppXor2>(v);
  v = row_sum_step<kDppHalfMirror>(v);
  return row_sum_step<kDppMirror>(v);
}

template <int V4>
__global__ __launch_bounds__(256) void topk_softmax_row16_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                                 int32_t* __restrict__ ids, float* __restrict__ w) {
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15;
  const int t = blockIdx.x * 16 + (threadIdx.x >> 6) * 4 + (lane >> 4);
  const bool valid = t < T;
  // rows past T read the last row (in bounds) and store nothing; every lane of a
  // DPP row takes part in the row reductions
  const float* row = logits + (int64_t)(valid ? t : T - 1) * E;

  uint64_t key[4 * V4];
#pragma unroll
  for (int i = 0; i < V4; ++i) {
    const int e0 = 64 * i + 4 * l16;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (e0 < E) v = *reinterpret_cast<const f32x4*>(row + e0);
#pragma unroll
    for (int c = 0; c < 4; ++c)
      key[4 * i + c] =
          (e0 < E) ? ((uint64_t)order_key(v[c]) << 32) | (uint32_t)(0xffffffffu - (uint32_t)(e0 + c)) : 0ull;
  }

  uint64_t sel = 0ull, first = 0ull;
  for (int r = 0; r < k; ++r) {
    uint64_t best = 0ull;
#pragma unroll
    for (int j = 0; j < 4 * V4; ++j) best = key[j] > best ? key[j] : best;
    best = row16_max(best);
#pragma unroll
    for (int j = 0; j < 4 * V4; ++j) key[j] = key[j] == best ? 0ull : key[j];
    if (l16 == r) sel = best;
    if (r == 0) first = best;
  }

  // the first selection is the largest logit of the row
  const float lmax = order_key_inv((uint32_t)(first >> 32));
  const float ex = l16 < k ? expf(order_key_inv((uint32_t)(sel >> 32)) - lmax) : 0.f;
  const float denom = row16_sum(ex);
  if (valid && l16 < k) {
    ids[(int64_t)t * k + l16] = (int32_t)(0xffffffffu - (uint32_t)sel);
    w[(int64_t)t * k + l16] = ex / denom;
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
  if (E % 4 == 0 && k <= 16 && E > 64 && E <= 512) {
    const dim3 grid((unsigned)((T + 15) / 16)), block(256);
    const int Tn = (int)T, En = (int)E, kn = (int)k;
    if (E <= 128)
      hipLaunchKernelGGL((topk_softmax_row16_kernel<2>), grid, block, 0, stream, logits, Tn, En, kn, ids, w);
    else if (E <= 256)
      hipLaunchKernelGGL((topk_softmax_row16_kernel<4>), grid, block, 0, stream, logits, Tn, En, kn, ids, w);
    else if (E <= 384)
      hipLaunchKernelGGL((topk_softmax_row16_kernel<6>), grid, block, 0, stream, logits, Tn, En, kn, ids, w);
    else
      hipLaunchKernelGGL((topk_softmax_row16_kernel<8>), grid, block, 0, stream, logits, Tn, En, kn, ids, w);
    return hipGetLastError();
  }
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
  // bf16: the tile width of 192 or 256 columns that pads E less (E = 384 fits two
  // 192-wide tiles exactly, where 256-wide tiles would compute 512 columns)
  const bool narrow = (E + 191) / 192 * 192 < (E + 255) / 256 * 256;
  if (dtype == 1 && narrow)
    hipLaunchKernelGGL((grouped_gemm_kernel<bf16, 256, 192, 64, 4, 2, 2, EPI_F32_BIAS>), grid, block, 0, stream, a);
  else if (dtype == 1)
    hipLaunchKernelGGL((grouped_gemm_kernel<bf16, 256, 256, 64, 4, 2, 2, EPI_F32_BIAS>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((grouped_gemm_kernel<float, 256, 256, 32, 4, 2, 2, EPI_F32_BIAS>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace moe
