// Backward of the routing, permutation and combine steps of the layer.
//
// The pages' workload is pre-training ("Training a 1T-Parameter MoE on EU public
// infrastructure with PyTorch and TorchTitan": TL;DR and "The machine and its
// constraints"), so every step runs the layer backward.  With the forward
//     l = x W_r^T + b,  w[t,:] = renormalised softmax of the k selected logits,
//     x_perm[r] = x[row_token[r]],  y[t] = sum_j w[t,j] y_perm[slot_row[t,j]],
// the steps here are:
//   * combine backward (one wavefront per token, no atomics):
//       dy_perm[slot_row[t,j]] = w[t,j] dy[t],   g[t,j] = <dy[t], y_perm[slot_row[t,j]]>;
//   * gate-weight and router backward: the renormalised weights are a softmax of
//     the selected logits, so dl[t,S_j] = w_j (g_j - sum_i w_i g_i) and every
//     other logit gets zero; then
//       dx[t] = sum_j dl[t,S_j] W_r[S_j] + sum_j dx_perm[slot_row[t,j]]
//     (the router's input gradient and the permutation's backward, which meet in
//     dx; one wavefront per token reads the k rows of W_r, which stay in cache),
//       db[e] = sum_t dl[t,e]           (float32 column sums, two fixed-order passes),
//       dW_r = dl^T x                   (MFMA: dl and x transposed to [E, T'] and
//                                        [d, T'], T' = T rounded up to 64 with zero
//                                        columns, stored k-blocked; one NT GEMM split
//                                        over k ranges of tokens, the float32 partials
//                                        summed in order).
#include <algorithm>

#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"
#include "rows.h"

namespace moe {

namespace {

constexpr int kTile = 64;

// One wavefront per token.  KU > 0: k is the compile-time KU (the k row loads of
// a column chunk are in flight together); KU == 0: any k, slot by slot.
template <typename T, int KU>
__global__ __launch_bounds__(256) void combine_backward_kernel(const T* __restrict__ dy, const T* __restrict__ y_perm,
                                                               const int32_t* __restrict__ slot_row,
                                                               const float* __restrict__ w, int Tn, int d, int k,
                                                               T* __restrict__ dy_perm, float* __restrict__ g) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= Tn) return;
  const int lane = threadIdx.x & 63;
  const int32_t* sr = slot_row + (int64_t)t * k;
  const float* wt = w + (int64_t)t * k;
  const T* dyt = dy + (int64_t)t * d;
  if constexpr (KU > 0) {
    int row[KU];
    float wj[KU], dot[KU];
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      row[j] = __builtin_amdgcn_readfirstlane(sr[j]);
      wj[j] = wt[j];
      dot[j] = 0.f;
    }
    for (int c0 = lane * 8; c0 < d; c0 += 64 * 8) {
      float a[8], v[KU][8];
      load8(dyt + c0, a);
#pragma unroll
      for (int j = 0; j < KU; ++j)
        if (row[j] >= 0) load8(y_perm + (int64_t)row[j] * d + c0, v[j]);
#pragma unroll
      for (int j = 0; j < KU; ++j)
        if (row[j] >= 0) {
          float o[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            dot[j] = fmaf(a[i], v[j][i], dot[j]);
            o[i] = wj[j] * a[i];
          }
          store8(dy_perm + (int64_t)row[j] * d + c0, o);
        }
    }
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      const float s = wave_sum64(dot[j]);
      if (lane == j) g[(int64_t)t * k + j] = row[j] >= 0 ? s : 0.f;
    }
  } else {
    for (int j = 0; j < k; ++j) {
      const int row = __builtin_amdgcn_readfirstlane(sr[j]);
      if (row < 0) {
        if (lane == 0) g[(int64_t)t * k + j] = 0.f;
        continue;
      }
      const float wj = wt[j];
      float dot = 0.f;
      for (int c0 = lane * 8; c0 < d; c0 += 64 * 8) {
        float a[8], v[8], o[8];
        load8(dyt + c0, a);
        load8(y_perm + (int64_t)row * d + c0, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dot = fmaf(a[i], v[i], dot);
          o[i] = wj * a[i];
        }
        store8(dy_perm + (int64_t)row * d + c0, o);
      }
      const float s = wave_sum64(dot);
      if (lane == 0) g[(int64_t)t * k + j] = s;
    }
  }
}

// One wavefront per token: dl from (w, g) over the slots whose id is in [0, E)
// (ids of a token distinct, as the top-k gives them); dl scattered into the dense [T, E]
// logit gradient (zeroed beforehand) when given; dx[t] = sum_j dx_perm[row_j]
// (when given) + sum_j dl_j W_r[id_j] (when W_r is given), summed in float32 in
// that order.  Slots with a negative id or row contribute nothing.
template <typename T, int KU>
__global__ __launch_bounds__(256) void route_backward_token_kernel(
    const T* __restrict__ dx_perm, const int32_t* __restrict__ slot_row, const int32_t* __restrict__ ids,
    const float* __restrict__ w, const float* __restrict__ g, const T* __restrict__ w_router, int Tn, int d, int E,
    int k, float* __restrict__ dlogits, T* __restrict__ dx) {
  const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (t >= Tn) return;
  const int lane = threadIdx.x & 63;
  const int64_t s0 = (int64_t)t * k;
  const bool routed = w_router != nullptr;
  // s = sum_j w_j g_j over the valid slots, in slot order (same on every lane)
  float s = 0.f;
  if (routed)
    for (int j = 0; j < k; ++j) {
      const int e = ids[s0 + j];
      if (e >= 0 && e < E) s = fmaf(w[s0 + j], g[s0 + j], s);
    }
  if (dlogits)
    for (int j = lane; j < k; j += 64) {
      const int e = ids[s0 + j];
      if (e >= 0 && e < E) dlogits[(int64_t)t * E + e] = w[s0 + j] * (g[s0 + j] - s);
    }
  constexpr int KR = KU > 0 ? KU : 1;
  int row[KR], id[KR];
  float dl[KR];
  if constexpr (KU > 0) {
#pragma unroll
    for (int j = 0; j < KU; ++j) {
      row[j] = dx_perm ? __builtin_amdgcn_readfirstlane(slot_row[s0 + j]) : -1;
      id[j] = routed ? __builtin_amdgcn_readfirstlane(ids[s0 + j]) : -1;
      if (id[j] >= E) id[j] = -1;
      dl[j] = id[j] >= 0 ? w[s0 + j] * (g[s0 + j] - s) : 0.f;
    }
  }
  for (int c0 = lane * 8; c0 < d; c0 += 64 * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    if constexpr (KU > 0) {
      // rows kept as loaded until used (half the registers of float copies)
      typename Raw16<T>::type v[KU], r[KU];
#pragma unroll
      for (int j = 0; j < KU; ++j) {
        if (row[j] >= 0) v[j] = Raw16<T>::load(dx_perm + (int64_t)row[j] * d + c0);
        if (id[j] >= 0) r[j] = Raw16<T>::load(w_router + (int64_t)id[j] * d + c0);
      }
#pragma unroll
      for (int j = 0; j < KU; ++j)
        if (row[j] >= 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += Raw16<T>::get(v[j], i);
        }
#pragma unroll
      for (int j = 0; j < KU; ++j)
        if (id[j] >= 0) {
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(dl[j], Raw16<T>::get(r[j], i), acc[i]);
        }
    } else {
      float v[8];
      if (dx_perm)
        for (int j = 0; j < k; ++j) {
          const int rj = __builtin_amdgcn_readfirstlane(slot_row[s0 + j]);
          if (rj < 0) continue;
          load8(dx_perm + (int64_t)rj * d + c0, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] += v[i];
        }
      if (routed)
        for (int j = 0; j < k; ++j) {
          const int ej = __builtin_amdgcn_readfirstlane(ids[s0 + j]);
          if (ej < 0 || ej >= E) continue;
          const float dlj = w[s0 + j] * (g[s0 + j] - s);
          load8(w_router + (int64_t)ej * d + c0, v);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(dlj, v[i], acc[i]);
        }
    }
    store8(dx + (int64_t)t * d + c0, acc);
  }
}

// p[0 .. n) = 0 (a kernel rather than a memset, so the sequence can be captured in
// a graph).
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

// partial[c * E + e] = sum of dl[r, e] over rows r of chunk c (rows_per_chunk
// consecutive rows); 4 row phases x 64 columns per block, combined in a fixed order.
__global__ __launch_bounds__(256) void column_sum_partial_kernel(const float* __restrict__ dl, int Tn, int E,
                                                                 int rows_per_chunk, float* __restrict__ partial) {
  __shared__ float ps[4][64];
  const int e = blockIdx.x * 64 + (threadIdx.x & 63), ph = threadIdx.x >> 6;
  const int c = blockIdx.y;
  const int lo = c * rows_per_chunk, hi = min(Tn, lo + rows_per_chunk);
  float s = 0.f;
  if (e < E)
    for (int r = lo + ph; r < hi; r += 4) s += dl[(int64_t)r * E + e];
  ps[ph][threadIdx.x & 63] = s;
  __syncthreads();
  if (ph == 0 && e < E) partial[(int64_t)c * E + e] = ((ps[0][threadIdx.x] + ps[1][threadIdx.x]) + ps[2][threadIdx.x]) +
                                                      ps[3][threadIdx.x];
}

// out[e] = sum over c < chunks of partial[c * E + e], in order of c.
__global__ __launch_bounds__(256) void column_sum_final_kernel(const float* __restrict__ partial, int chunks, int E,
                                                               float* __restrict__ out) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  float s = 0.f;
  for (int c = 0; c < chunks; ++c) s += partial[(int64_t)c * E + e];
  out[e] = s;
}

// Transpose with zero padding, stored k-blocked: element (c, r) of the [cols, T']
// result (c < cols, r < T' = gridDim.y * 64) is src[r * cols + c] for r < rows and
// 0 beyond, at (r / KW) cols KW + c KW + r % KW (every KW-wide block of r is one
// contiguous [cols, KW] piece, which a GEMM k-step reads whole).  One 64 x 64 tile
// per block; values pass through float32 (exact for bf16 -> bf16 and float ->
// float; float -> bf16 rounds to nearest even).
template <typename Ts, typename Td, int KW>
__global__ __launch_bounds__(256) void transpose_pad_kernel(const Ts* __restrict__ src, int rows, int cols,
                                                            Td* __restrict__ dst) {
  __shared__ float tile[kTile][kTile + 1];
  const int r0 = blockIdx.y * kTile, c0 = blockIdx.x * kTile;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < kTile; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? to_f32(src[(int64_t)r * cols + c]) : 0.f;
  }
  __syncthreads();
  const int r = r0 + tx;
  Td* out = dst + (int64_t)(r / KW) * cols * KW + r % KW;
  for (int i = ty; i < kTile; i += 4) {
    const int c = c0 + i;
    if (c < cols) out[(int64_t)c * KW] = from_f32<Td>(tile[tx][i]);
  }
}

// kseg[i] = the first k of split i: nkt k-tiles of BK shared out as evenly as possible.
__global__ void split_offsets_kernel(int32_t* __restrict__ kseg, int splits, int nkt, int bk) {
  const int i = threadIdx.x;
  if (i <= splits) kseg[i] = (int32_t)((int64_t)nkt * i / splits) * bk;
}

// out[i] = sum over s < splits of part[s * n + i], in order of s (n a multiple of 4).
__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part, int splits, int64_t n,
                                                         float* __restrict__ out) {
  for (int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += (int64_t)gridDim.x * 256 * 4) {
    f32x4 s = *reinterpret_cast<const f32x4*>(part + i);
    for (int q = 1; q < splits; ++q) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(part + (int64_t)q * n + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] += v[j];
    }
    *reinterpret_cast<f32x4*>(out + i) = s;
  }
}

template <typename T>
void launch_combine_backward_t(int64_t T_, int64_t d, int64_t k, const T* dy, const T* y_perm,
                               const int32_t* slot_row, const float* w, T* dy_perm, float* g, hipStream_t s) {
  const dim3 grid((unsigned)((T_ + 3) / 4)), block(256);
  const int Tn = (int)T_, dn = (int)d, kn = (int)k;
#define MOE_CB(KU) hipLaunchKernelGGL((combine_backward_kernel<T, KU>), grid, block, 0, s, dy, y_perm, slot_row, w, \
                                      Tn, dn, kn, dy_perm, g)
  switch (k) {
    case 1: MOE_CB(1); break;
    case 2: MOE_CB(2); break;
    case 4: MOE_CB(4); break;
    case 8: MOE_CB(8); break;
    default: MOE_CB(0);
  }
#undef MOE_CB
}

template <typename T>
void launch_route_token_t(int64_t T_, int64_t d, int64_t E, int64_t k, const T* dx_perm, const int32_t* slot_row,
                          const int32_t* ids, const float* w, const float* g, const T* w_router, float* dlogits,
                          T* dx, hipStream_t s) {
  const dim3 grid((unsigned)((T_ + 3) / 4)), block(256);
  const int Tn = (int)T_, dn = (int)d, En = (int)E, kn = (int)k;
#define MOE_RB(KU) hipLaunchKernelGGL((route_backward_token_kernel<T, KU>), grid, block, 0, s, dx_perm, slot_row, ids, \
                                      w, g, w_router, Tn, dn, En, kn, dlogits, dx)
  switch (k) {
    case 1: MOE_RB(1); break;
    case 2: MOE_RB(2); break;
    case 4: MOE_RB(4); break;
    case 8: MOE_RB(8); break;
    default: MOE_RB(0);
  }
#undef MOE_RB
}

template <typename T, int BK>
hipError_t route_backward_t(int64_t T_, int64_t d, int64_t E, int64_t k, const T* x, const T* w_router,
                            const int32_t* ids, const float* w, const float* g, const T* dx_perm,
                            const int32_t* slot_row, T* dx, float* dw_router, float* dbias,
                            const RouteBackwardScratch& ws, int num_cu, hipStream_t s) {
  const int64_t tp = ws.t_pad;
  const int64_t nl = T_ * E;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)std::min<int64_t>((nl + 255) / 256, 8 * (int64_t)num_cu)),
                     dim3(256), 0, s, ws.dlogits, nl);
  launch_route_token_t<T>(T_, d, E, k, dx_perm, slot_row, ids, w, g, w_router, ws.dlogits, dx, s);

  // db: column sums of the dense logit gradient
  if (dbias) {
    const int rows_per_chunk = (int)((T_ + ws.bias_chunks - 1) / ws.bias_chunks);
    hipLaunchKernelGGL(column_sum_partial_kernel, dim3((unsigned)((E + 63) / 64), (unsigned)ws.bias_chunks),
                       dim3(256), 0, s, ws.dlogits, (int)T_, (int)E, rows_per_chunk, ws.bias_partial);
    hipLaunchKernelGGL(column_sum_final_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, s, ws.bias_partial,
                       ws.bias_chunks, (int)E, dbias);
  }

  // dW_r = dl^T x on the transposed, zero-padded operands
  T* dlt = static_cast<T*>(ws.dl_t);
  T* xt = static_cast<T*>(ws.x_t);
  hipLaunchKernelGGL((transpose_pad_kernel<float, T, BK>), dim3((unsigned)((E + 63) / 64), (unsigned)(tp / kTile)),
                     dim3(256), 0, s, ws.dlogits, (int)T_, (int)E, dlt);
  hipLaunchKernelGGL((transpose_pad_kernel<T, T, BK>), dim3((unsigned)(d / kTile), (unsigned)(tp / kTile)),
                     dim3(256), 0, s, x, (int)T_, (int)d, xt);
  hipLaunchKernelGGL(split_offsets_kernel, dim3(1), dim3(64), 0, s, ws.kseg, ws.splits, (int)(tp / BK), BK);
  GemmArgs a{};
  a.A = dlt;
  a.B0 = xt;
  a.b_stride = 0;
  a.G = ws.splits;
  a.M = (int64_t)ws.splits * E;
  a.group_rows = E;
  a.N = (int)d;
  a.K = 0;
  a.C = ws.splits > 1 ? static_cast<void*>(ws.split_partial) : static_cast<void*>(dw_router);
  a.a_shared = 1;
  a.lda = BK;
  a.ldb = BK;
  a.ksa = E * BK;
  a.ksb = d * BK;
  a.kseg = ws.kseg;
  hipLaunchKernelGGL((grouped_gemm_kernel<T, 256, 256, BK, 4, 2, 2, EPI_F32, 1, kFeatGroups | kFeatStrides>),
                     dim3(num_cu), dim3(512), 0, s, a);
  if (ws.splits > 1) {
    const int64_t n = E * d;
    const int64_t blocks = std::min<int64_t>((n / 4 + 255) / 256, 4 * (int64_t)num_cu);
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ws.split_partial, ws.splits, n,
                       dw_router);
  }
  return hipGetLastError();
}

}  // namespace

int route_backward_splits(int64_t E, int64_t d, int64_t t_pad) {
  // enough 256 x 256 output tiles for the 256 compute units of an MI355X; a fixed
  // count (not the device's) keeps the float32 summation order, and so the bits
  // of dW_r, the same on every device
  constexpr int64_t kTargetTiles = 256;
  const int64_t tiles = ((E + 255) / 256) * ((d + 255) / 256);
  const int64_t nkt = t_pad / 64;                      // k-tiles of the bf16 GEMM
  int64_t s = (kTargetTiles + tiles - 1) / tiles;
  s = std::min<int64_t>(s, std::max<int64_t>(1, nkt / 4));
  return (int)std::max<int64_t>(1, std::min<int64_t>(s, kMaxSplits));
}

hipError_t launch_combine_backward(int dtype, int64_t T, int64_t d, int64_t k, const void* dy, const void* y_perm,
                                   const int32_t* slot_row, const float* w, void* dy_perm, float* g,
                                   hipStream_t stream) {
  if (dtype == 1)
    launch_combine_backward_t<bf16>(T, d, k, (const bf16*)dy, (const bf16*)y_perm, slot_row, w, (bf16*)dy_perm, g,
                                    stream);
  else
    launch_combine_backward_t<float>(T, d, k, (const float*)dy, (const float*)y_perm, slot_row, w, (float*)dy_perm,
                                     g, stream);
  return hipGetLastError();
}

hipError_t launch_route_backward(int dtype, int64_t T, int64_t d, int64_t E, int64_t k, const void* x,
                                 const void* w_router, const int32_t* ids, const float* w, const float* g,
                                 const void* dx_perm, const int32_t* slot_row, void* dx, float* dw_router,
                                 float* dbias, const RouteBackwardScratch& ws, int num_cu, hipStream_t stream) {
  if (dtype == 1)
    return route_backward_t<bf16, 64>(T, d, E, k, (const bf16*)x, (const bf16*)w_router, ids, w, g,
                                      (const bf16*)dx_perm, slot_row, (bf16*)dx, dw_router, dbias, ws, num_cu, stream);
  return route_backward_t<float, 32>(T, d, E, k, (const float*)x, (const float*)w_router, ids, w, g,
                                     (const float*)dx_perm, slot_row, (float*)dx, dw_router, dbias, ws, num_cu,
                                     stream);
}

hipError_t launch_unpermute(int dtype, int64_t T, int64_t d, int64_t k, const void* dx_perm,
                            const int32_t* slot_row, void* dx, hipStream_t stream) {
  if (dtype == 1)
    launch_route_token_t<bf16>(T, d, 1, k, (const bf16*)dx_perm, slot_row, nullptr, nullptr, nullptr, nullptr,
                               nullptr, (bf16*)dx, stream);
  else
    launch_route_token_t<float>(T, d, 1, k, (const float*)dx_perm, slot_row, nullptr, nullptr, nullptr, nullptr,
                                nullptr, (float*)dx, stream);
  return hipGetLastError();
}

}  // namespace moe
