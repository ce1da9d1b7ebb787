// Host-side launchers of the layer's kernels (one translation unit per step).
// Every launcher only enqueues on `stream`; argument checks happen earlier,
// in the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Router GEMM: logits[T,E] (float32) = x[T,d] . W_r[E,d]^T + bias.
hipError_t launch_router_gemm(int dtype, int64_t T, int64_t d, int64_t E, const void* x,
                              const void* w_router, const float* bias, float* logits,
                              int num_cu, hipStream_t stream);

// Softmax + top-k + renormalisation, one wavefront per token.
hipError_t launch_topk(int64_t T, int64_t E, int64_t k, const float* logits, int32_t* ids,
                       float* w, hipStream_t stream);

// Permutation: counts per 256-token block, scan, stable scatter + row copy
// (x_perm == nullptr: indices only).
hipError_t launch_permute(int dtype, int64_t T, int64_t d, int64_t E, int64_t k, const void* x,
                          const int32_t* ids, int32_t* offsets, int32_t* row_token,
                          int32_t* slot_row, void* x_perm, int32_t* block_counts,
                          hipStream_t stream);
constexpr int kPermuteBlockTokens = 256;

// Grouped SwiGLU FFN: h = silu(X W_g^T) * (X W_u^T); y_perm = h W_d^T, where row r
// of X is x_perm[r], or x[a_rows[r]] when a gather map is given (x has n_in rows;
// map entries are clamped to them).  The offsets are clamped into consistent
// segments inside [0, n_max) on the device.
hipError_t launch_grouped_ffn(int dtype, int64_t n_max, int64_t d, int64_t E, int64_t F,
                              const void* x_perm, int64_t n_in, const int32_t* a_rows, const int32_t* offsets,
                              const void* w_gate,
                              const void* w_up, const void* w_down, void* y_perm, void* h,
                              void* gu_out, int num_cu, hipStream_t stream);

// Muon's Newton-Schulz orthogonalisation of n bf16 matrices [R, C] (R, C multiples
// of 64): g in, x out; xw0 and xw1 [n, R', C'], A and B [n, R', R']
// (R' = min(R, C), C' = max(R, C)) and partial [n * kNormBlocks] are scratch.
constexpr int kNormBlocks = 64;
hipError_t launch_newton_schulz(int64_t n, int64_t R, int64_t C, int64_t steps, float a, float b, float c,
                                float eps, const void* g, void* x, void* xw0, void* xw1, void* A, void* B,
                                float* partial, int num_cu, hipStream_t stream);

// Backward of the grouped SwiGLU FFN: dx_perm and the float32 weight gradients
// from dy_perm.  Scratch (caller-carved; "I/O" = the dtype's element type):
struct FfnBackwardScratch {
  int32_t* soff;   // [E+1] the caller's offsets clamped into consistent segments
  int32_t* poff;   // [E+1] padded expert column offsets
  int32_t* pblk_expert;  // [n_pad / 64] expert of each 64-wide padded column block
  void* wd_t;      // [E, F, d]   W_d transposed (float32 layers only)
  void* wgu_t;     // [E, d, 2F]  W_g and W_u transposed, side by side (float32 layers only)
  float* dh;       // [n_max, F]  dH (float32); nullptr when the forward kept G | U
  void* dgu;       // [n_max, 2F] dG | dU (I/O)
  void* h;         // [n_max, F]  H recomputed (I/O)
  void* x_t;       // [d, n_pad]  expert rows of the input, transposed and padded, stored
                   //             k-blocked ([n_pad / BK] blocks of [d, BK]) (I/O)
  void* dy_t;      // [d, n_pad]  k-blocked (I/O)
  void* h_t;       // [F, n_pad]  k-blocked (I/O)
  void* dg_t;      // [F, n_pad]  k-blocked (I/O)
  void* du_t;      // [F, n_pad]  k-blocked (I/O)
  int64_t n_pad;   // >= sum over experts of rows rounded up to 64; a multiple of 64
};
hipError_t launch_grouped_ffn_backward(int dtype, int64_t n_max, int64_t d, int64_t E, int64_t F, const void* x_in,
                                       int64_t n_in, const int32_t* a_rows, const int32_t* offsets, const void* w_gate,
                                       const void* w_up, const void* w_down, const void* dy_perm, const void* gu,
                                       void* dx_perm, float* dw_gate, float* dw_up, float* dw_down,
                                       const FfnBackwardScratch& w, int num_cu, hipStream_t stream);

// Weighted un-permute: y[t] = sum_j w[t,j] * y_perm[slot_row[t,j]].
hipError_t launch_combine(int dtype, int64_t T, int64_t d, int64_t k, const void* y_perm,
                          const int32_t* slot_row, const float* w, void* y, hipStream_t stream);

// Backward of the combine: dy_perm[slot_row[t,j]] = w[t,j] dy[t] and
// g[t,j] = <dy[t], y_perm[slot_row[t,j]]> (0 for slot_row < 0).
hipError_t launch_combine_backward(int dtype, int64_t T, int64_t d, int64_t k, const void* dy, const void* y_perm,
                                   const int32_t* slot_row, const float* w, void* dy_perm, float* g,
                                   hipStream_t stream);

// Backward of the routing (renormalised top-k softmax and router GEMM) plus the
// permutation: dx[t] = sum_j dl[t,j] W_r[ids[t,j]] + sum_j dx_perm[slot_row[t,j]]
// (dx_perm == nullptr: router part only), dW_r = dl^T x, db = column sums of dl
// (dbias == nullptr: skipped).  Scratch (caller-carved):
constexpr int kMaxSplits = 16;
struct RouteBackwardScratch {
  float* dlogits;        // [T, E] dense logit gradient
  void* dl_t;            // [E, t_pad] its transpose, k-blocked (I/O type)
  void* x_t;             // [d, t_pad] x transposed, k-blocked (I/O type)
  int32_t* kseg;         // [splits + 1] token ranges of the split GEMM
  float* split_partial;  // [splits, E, d] when splits > 1
  float* bias_partial;   // [bias_chunks, E]
  int64_t t_pad;         // T rounded up to 64
  int splits;            // 1 .. kMaxSplits (route_backward_splits)
  int bias_chunks;       // 1 .. 64
};
int route_backward_splits(int64_t E, int64_t d, int64_t t_pad);
hipError_t launch_route_backward(int dtype, int64_t T, int64_t d, int64_t E, int64_t k, const void* x,
                                 const void* w_router, const int32_t* ids, const float* w, const float* g,
                                 const void* dx_perm, const int32_t* slot_row, void* dx, float* dw_router,
                                 float* dbias, const RouteBackwardScratch& ws, int num_cu, hipStream_t stream);

// Backward of the permutation alone: dx[t] = sum_j dx_perm[slot_row[t,j]].
hipError_t launch_unpermute(int dtype, int64_t T, int64_t d, int64_t k, const void* dx_perm,
                            const int32_t* slot_row, void* dx, hipStream_t stream);

}  // namespace moe
