// Grouped per-expert SwiGLU FFN over the permuted rows.
//
// Expert e (of the 384 routed experts, hidden 6,144, expert hidden 1,792 in the
// model-configuration table of "Training a 1T-Parameter MoE on EU public
// infrastructure with PyTorch and TorchTitan") maps each of its rows v to
// W_d[e] (silu(W_g[e] v) * (W_u[e] v)).  The table's parameter counts fit
// exactly three d x F matrices per expert; SwiGLU is the reading of the gate.
//
// Two persistent launches of the grouped GEMM template:
//   gate/up: one A tile against the gate AND the up tile of the same columns,
//            SwiGLU in registers, h stored once (never the two halves); the A
//            rows are either x_perm's rows or, with a gather map, token rows of
//            x read in place (no permuted copy of x is ever written);
//   down:    y_perm = h W_d^T.
// Row counts per expert are read on the device from the offsets; experts with
// no rows own no tile.
#include "common.h"
#include "gemm_tile.h"
#include "kernels.h"

namespace moe {

namespace {

// Tile order inside an expert: chunks of row tiles, column groups inside a chunk
// (0 = no chunking / all columns together).  The 32 tiles an XCD runs side by side
// then cover 8 row tiles x 4 column tiles of a large expert, so each weight k-slice
// and each row k-slice is read by several of them from that XCD's L2.  Measured at
// 65,536 tokens (page shape, skewed routing), bytes read past L2 per call: 8 x 2
// chunks 59 GB (gate/up) and 23.4 GB (down); 16 x 2 65 and 26.5 GB; 16 x 4 60 and
// 23.6 GB; 8 x 4 62.6 and 24.7 GB; all at the same time (19.6 and 10.3 ms) and
// shader clock (1.64-1.65 GHz).  Without chunking: 30.9 ms for the two GEMMs.
constexpr int kGateUpRowChunk = 8;
constexpr int kGateUpColumnGroup = 2;
constexpr int kDownRowChunk = 8;
constexpr int kDownColumnGroup = 2;

// Tile configuration: 256 x 256 output tiles, BK-deep k-slices, STAGES-deep LDS
// ring, WM x WN wavefronts, MFMA operands read PD 16-k sub-steps ahead.
template <typename T, int BK, int STAGES, int WM, int WN, int PD>
void run(int64_t n_max, int64_t d, int64_t E, int64_t F, const void* x_perm, int64_t n_in, const int32_t* a_rows,
         const int32_t* offsets,
         const void* w_gate, const void* w_up, const void* w_down, void* y_perm, void* h, void* gu_out, int num_cu,
         hipStream_t stream) {
  GemmArgs gu{};
  gu.A = x_perm;
  gu.a_rows = a_rows;
  gu.a_rows_n = n_in;
  gu.B0 = w_gate;
  gu.B1 = w_up;
  gu.b_stride = F * d;
  gu.seg = offsets;
  gu.G = (int32_t)E;
  gu.M = n_max;
  gu.N = (int32_t)F;
  gu.K = (int32_t)d;
  gu.C = h;
  gu.bias = nullptr;
  gu.n_group = kGateUpColumnGroup;
  gu.m_chunk = kGateUpRowChunk;
  if (gu_out) {
    // G | U kept for the backward (rows of [n_max, 2F], G in the first F columns)
    gu.C2 = gu_out;
    hipLaunchKernelGGL((grouped_gemm_kernel<T, 256, 256, BK, WM, WN, STAGES, EPI_SWIGLU_SAVE, PD>), dim3(num_cu),
                       dim3(WM * WN * 64), 0, stream, gu);
  } else {
    hipLaunchKernelGGL((grouped_gemm_kernel<T, 256, 256, BK, WM, WN, STAGES, EPI_SWIGLU, PD>), dim3(num_cu),
                       dim3(WM * WN * 64), 0, stream, gu);
  }

  GemmArgs dn{};
  dn.A = h;
  dn.a_rows = nullptr;
  dn.B0 = w_down;
  dn.B1 = nullptr;
  dn.b_stride = d * F;
  dn.seg = offsets;
  dn.G = (int32_t)E;
  dn.M = n_max;
  dn.N = (int32_t)d;
  dn.K = (int32_t)F;
  dn.C = y_perm;
  dn.bias = nullptr;
  dn.n_group = kDownColumnGroup;
  dn.m_chunk = kDownRowChunk;
  hipLaunchKernelGGL((grouped_gemm_kernel<T, 256, 256, BK, WM, WN, STAGES, EPI_STORE, PD>), dim3(num_cu),
                     dim3(WM * WN * 64), 0,
                     stream, dn);
}

}  // namespace

hipError_t launch_grouped_ffn(int dtype, int64_t n_max, int64_t d, int64_t E, int64_t F, const void* x_perm,
                              int64_t n_in, const int32_t* a_rows, const int32_t* offsets, const void* w_gate,
                              const void* w_up, const void* w_down, void* y_perm, void* h, void* gu_out,
                              int num_cu, hipStream_t stream) {
  if (dtype == 1)
    run<bf16, 64, 2, 4, 2, 1>(n_max, d, E, F, x_perm, n_in, a_rows, offsets, w_gate, w_up, w_down, y_perm, h,
                              gu_out, num_cu, stream);
  else
    run<float, 32, 2, 4, 2, 1>(n_max, d, E, F, x_perm, n_in, a_rows, offsets, w_gate, w_up, w_down, y_perm, h,
                               gu_out, num_cu, stream);
  return hipGetLastError();
}

}  // namespace moe
