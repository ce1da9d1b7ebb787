// C ABI of the routed-MoE layer (forward, backward, Muon's Newton-Schulz): argument checks, workspace sizing and
// carving, launch geometry.  All checks run on the host before any HIP call, so
// a bad call returns a status without touching the device.  Kernels are only
// enqueued on the caller's stream; nothing here synchronises or allocates.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>

#include "kernels.h"
#include "moe.h"

namespace {

constexpr int64_t kMaxE = 1024;
constexpr int64_t kMaxDim = int64_t(1) << 20;
constexpr int64_t kIdxLimit = int64_t(1) << 31;
constexpr size_t kWsAlign = 256;

size_t round_up(size_t v) { return (v + kWsAlign - 1) / kWsAlign * kWsAlign; }
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool ok16(const void* p) { return p != nullptr && aligned(p, 16); }
bool ok4(const void* p) { return p != nullptr && aligned(p, 4); }
bool opt16(const void* p) { return p == nullptr || aligned(p, 16); }
bool opt4(const void* p) { return p == nullptr || aligned(p, 4); }
size_t elem_size(moe_dtype t) { return t == MOE_BF16 ? 2 : 4; }

// Compute units of the current device, cached per device.
std::atomic<int> g_cu_cache[64];

moe_status num_cu(int* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    const int c = g_cu_cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *out = c;
      return MOE_OK;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return MOE_ERR_HIP;
  if (dev >= 0 && dev < 64) g_cu_cache[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return MOE_OK;
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe_status check_dtype(moe_dtype t) { return (t == MOE_F32 || t == MOE_BF16) ? MOE_OK : MOE_ERR_UNSUPPORTED; }

// Shared size checks for T, d, E, k.
moe_status check_tdek(int64_t T, int64_t d, int64_t E, int64_t k) {
  if (T <= 0 || d <= 0 || E <= 0 || k <= 0 || k > E) return MOE_ERR_INVALID_ARG;
  if (d % 64 != 0 || d > kMaxDim || E > kMaxE || T * k >= kIdxLimit) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_ffn_dims(int64_t n_max, int64_t d, int64_t E, int64_t F) {
  if (n_max <= 0 || d <= 0 || E <= 0 || F <= 0) return MOE_ERR_INVALID_ARG;
  if (d % 64 != 0 || F % 64 != 0 || d > kMaxDim || F > kMaxDim || E > kMaxE || n_max >= kIdxLimit)
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t permute_ws(int64_t T, int64_t E) {
  const int64_t nblk = (T + moe::kPermuteBlockTokens - 1) / moe::kPermuteBlockTokens;
  return round_up((size_t)nblk * (size_t)E * 4);
}

// Resolve the workspace protocol: query (ws == NULL) or size check.
// Returns true when the caller should return `st` right away.
// ws == NULL with ws_bytes == NULL means "no workspace provided": fine only
// when none is needed.
bool workspace_step(void* ws, size_t* ws_bytes, size_t need, moe_status* st) {
  if (ws_bytes == nullptr) {
    if (ws == nullptr && need == 0) return false;
    *st = MOE_ERR_WORKSPACE;
    return true;
  }
  if (ws == nullptr) {
    *ws_bytes = need;
    *st = MOE_OK;
    return true;
  }
  if (*ws_bytes < need) {
    *st = MOE_ERR_WORKSPACE;
    return true;
  }
  if (!aligned(ws, kWsAlign)) {
    *st = MOE_ERR_INVALID_ARG;
    return true;
  }
  return false;
}

// Carves consecutive 256-byte aligned pieces out of the workspace.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* ws) : base(static_cast<char*>(ws)) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += round_up(bytes);
    return p;
  }
};

// Scratch of the grouped-FFN backward for n_max rows (element size es); saved: the
// forward's G | U are given (no float32 dH buffer).
void carve_ffn_backward(Carver& c, moe::FfnBackwardScratch& w, int64_t n_max, int64_t d, int64_t E, int64_t F,
                        size_t es, bool saved) {
  const int64_t n_pad = (n_max + 63 * E + 63) / 64 * 64;
  w.soff = static_cast<int32_t*>(c.take((size_t)(E + 1) * 4));
  w.poff = static_cast<int32_t*>(c.take((size_t)(E + 1) * 4));
  w.pblk_expert = static_cast<int32_t*>(c.take((size_t)(n_pad / 64) * 4));
  // transposed weight copies: float32 only (16-bit weights are read in place)
  w.wd_t = es == 4 ? c.take((size_t)E * F * d * es) : nullptr;
  w.wgu_t = es == 4 ? c.take((size_t)E * d * 2 * F * es) : nullptr;
  w.dh = saved ? nullptr : static_cast<float*>(c.take((size_t)n_max * F * 4));
  w.dgu = c.take((size_t)n_max * 2 * F * es);
  w.h = c.take((size_t)n_max * F * es);
  w.x_t = c.take((size_t)d * n_pad * es);
  w.dy_t = c.take((size_t)d * n_pad * es);
  w.h_t = c.take((size_t)F * n_pad * es);
  w.dg_t = c.take((size_t)F * n_pad * es);
  w.du_t = c.take((size_t)F * n_pad * es);
  w.n_pad = n_pad;
}

bool ffn_backward_fits(int64_t n_max, int64_t E) { return (n_max + 63 * E + 63) / 64 * 64 < kIdxLimit; }

// Scratch of the routing backward for T tokens (dlogits_out: the caller's buffer).
void carve_route_backward(Carver& c, moe::RouteBackwardScratch& w, int64_t T, int64_t d, int64_t E, size_t es,
                          float* dlogits_out) {
  const int64_t tp = (T + 63) / 64 * 64;
  w.t_pad = tp;
  w.splits = moe::route_backward_splits(E, d, tp);
  w.bias_chunks = (int)(T < 64 ? T : 64);
  w.dlogits = dlogits_out ? dlogits_out : static_cast<float*>(c.take((size_t)T * E * 4));
  w.dl_t = c.take((size_t)E * tp * es);
  w.x_t = c.take((size_t)d * tp * es);
  w.kseg = static_cast<int32_t*>(c.take((size_t)(moe::kMaxSplits + 1) * 4));
  w.split_partial = w.splits > 1 ? static_cast<float*>(c.take((size_t)w.splits * E * d * 4)) : nullptr;
  w.bias_partial = static_cast<float*>(c.take((size_t)w.bias_chunks * E * 4));
}

}  // namespace

extern "C" {

moe_status moe_route(int64_t T, int64_t d, int64_t E, int64_t k, moe_dtype dtype, const void* x,
                     const void* w_router, const float* bias, float* logits_out, int32_t* topk_ids, float* topk_w,
                     void* ws, size_t* ws_bytes, void* stream) {
  moe_status st = check_tdek(T, d, E, k);
  if (st != MOE_OK) return st;
  if ((st = check_dtype(dtype)) != MOE_OK) return st;
  const size_t need = logits_out ? 0 : round_up((size_t)T * (size_t)E * 4);
  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    return MOE_OK;
  }
  if (!ok16(x) || !ok16(w_router) || !opt4(bias) || !opt16(logits_out) || !ok4(topk_ids) || !ok4(topk_w))
    return MOE_ERR_INVALID_ARG;
  if (workspace_step(ws, ws_bytes, need, &st)) return st;
  int ncu = 0;
  if ((st = num_cu(&ncu)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* logits = logits_out ? logits_out : static_cast<float*>(ws);
  if ((st = hip_status(moe::launch_router_gemm(dtype, T, d, E, x, w_router, bias, logits, ncu, s))) != MOE_OK)
    return st;
  return hip_status(moe::launch_topk(T, E, k, logits, topk_ids, topk_w, s));
}

moe_status moe_permute(int64_t T, int64_t d, int64_t E, int64_t k, moe_dtype dtype, const void* x,
                       const int32_t* topk_ids, int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                       void* x_perm, void* ws, size_t* ws_bytes, void* stream) {
  moe_status st = check_tdek(T, d, E, k);
  if (st != MOE_OK) return st;
  if ((st = check_dtype(dtype)) != MOE_OK) return st;
  const size_t need = permute_ws(T, E);
  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    return MOE_OK;
  }
  if (!ok16(x) || !ok4(topk_ids) || !ok4(offsets) || !ok4(row_token) || !ok4(slot_row) || !opt16(x_perm))
    return MOE_ERR_INVALID_ARG;
  if (workspace_step(ws, ws_bytes, need, &st)) return st;
  return hip_status(moe::launch_permute(dtype, T, d, E, k, x, topk_ids, offsets, row_token, slot_row, x_perm,
                                        static_cast<int32_t*>(ws), static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_ffn(int64_t n_max, int64_t d, int64_t E, int64_t F, moe_dtype dtype, const void* x_in,
                           int64_t n_in, const int32_t* a_rows, const int32_t* offsets, const void* w_gate,
                           const void* w_up, const void* w_down, void* y_perm, void* gu_out, void* ws,
                           size_t* ws_bytes, void* stream) {
  moe_status st = check_ffn_dims(n_max, d, E, F);
  if (st != MOE_OK) return st;
  if ((st = check_dtype(dtype)) != MOE_OK) return st;
  if (a_rows != nullptr) {
    if (n_in <= 0) return MOE_ERR_INVALID_ARG;
    if ((uint64_t)n_in * (uint64_t)d * elem_size(dtype) >= (uint64_t(1) << 32)) return MOE_ERR_UNSUPPORTED;
  }
  const size_t need = round_up((size_t)n_max * (size_t)F * elem_size(dtype));
  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    return MOE_OK;
  }
  if (!ok16(x_in) || !opt4(a_rows) || !ok4(offsets) || !ok16(w_gate) || !ok16(w_up) || !ok16(w_down) ||
      !ok16(y_perm) || !opt16(gu_out))
    return MOE_ERR_INVALID_ARG;
  if (workspace_step(ws, ws_bytes, need, &st)) return st;
  int ncu = 0;
  if ((st = num_cu(&ncu)) != MOE_OK) return st;
  return hip_status(moe::launch_grouped_ffn(dtype, n_max, d, E, F, x_in, a_rows ? n_in : n_max, a_rows, offsets,
                                            w_gate, w_up, w_down, y_perm, ws, gu_out, ncu,
                                            static_cast<hipStream_t>(stream)));
}

moe_status moe_grouped_ffn_backward(int64_t n_max, int64_t d, int64_t E, int64_t F, moe_dtype dtype,
                                    const void* x_in, int64_t n_in, const int32_t* a_rows, const int32_t* offsets,
                                    const void* w_gate, const void* w_up, const void* w_down, const void* dy_perm,
                                    const void* gu, void* dx_perm, float* dw_gate, float* dw_up, float* dw_down,
                                    void* ws, size_t* ws_bytes, void* stream) {
  moe_status st = check_ffn_dims(n_max, d, E, F);
  if (st != MOE_OK) return st;
  if ((st = check_dtype(dtype)) != MOE_OK) return st;
  const size_t es = elem_size(dtype);
  if (a_rows != nullptr) {
    if (n_in <= 0) return MOE_ERR_INVALID_ARG;
    if ((uint64_t)n_in * (uint64_t)d * es >= (uint64_t(1) << 32)) return MOE_ERR_UNSUPPORTED;
  }
  if (!ffn_backward_fits(n_max, E)) return MOE_ERR_UNSUPPORTED;
  moe::FfnBackwardScratch w{};
  Carver c0(nullptr);
  carve_ffn_backward(c0, w, n_max, d, E, F, es, gu != nullptr);
  const size_t need = c0.used;
  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    return MOE_OK;
  }
  if (!ok16(x_in) || !opt4(a_rows) || !ok4(offsets) || !ok16(w_gate) || !ok16(w_up) || !ok16(w_down) ||
      !ok16(dy_perm) || !opt16(gu) || !ok16(dx_perm) || !ok16(dw_gate) || !ok16(dw_up) || !ok16(dw_down))
    return MOE_ERR_INVALID_ARG;
  if (workspace_step(ws, ws_bytes, need, &st)) return st;
  int ncu = 0;
  if ((st = num_cu(&ncu)) != MOE_OK) return st;
  Carver cv(ws);
  carve_ffn_backward(cv, w, n_max, d, E, F, es, gu != nullptr);
  return hip_status(moe::launch_grouped_ffn_backward(dtype, n_max, d, E, F, x_in, a_rows ? n_in : n_max, a_rows,
                                                     offsets, w_gate, w_up, w_down, dy_perm, gu, dx_perm, dw_gate,
                                                     dw_up, dw_down, w, ncu, static_cast<hipStream_t>(stream)));
}

moe_status moe_combine_backward(int64_t T, int64_t d, int64_t k, moe_dtype dtype, const void* dy,
                                const void* y_perm, const int32_t* slot_row, const float* topk_w, void* dy_perm,
                                float* d_topk_w, void* stream) {
  if (T <= 0 || d <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
  if (d % 64 != 0 || d > kMaxDim || T * k >= kIdxLimit) return MOE_ERR_UNSUPPORTED;
  moe_status st = check_dtype(dtype);
  if (st != MOE_OK) return st;
  if (!ok16(dy) || !ok16(y_perm) || !ok4(slot_row) || !ok4(topk_w) || !ok16(dy_perm) || !ok4(d_topk_w))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine_backward(dtype, T, d, k, dy, y_perm, slot_row, topk_w, dy_perm, d_topk_w,
                                                 static_cast<hipStream_t>(stream)));
}

moe_status moe_route_backward(int64_t T, int64_t d, int64_t E, int64_t k, moe_dtype dtype, const void* x,
                              const void* w_router, const int32_t* topk_ids, const float* topk_w,
                              const float* d_topk_w, const void* dx_perm, const int32_t* slot_row, void* dx,
                              float* dw_router, float* dbias, float* dlogits_out, void* ws, size_t* ws_bytes,
                              void* stream) {
  moe_status st = check_tdek(T, d, E, k);
  if (st != MOE_OK) return st;
  if ((st = check_dtype(dtype)) != MOE_OK) return st;
  const size_t es = elem_size(dtype);
  moe::RouteBackwardScratch w{};
  Carver c0(nullptr);
  carve_route_backward(c0, w, T, d, E, es, dlogits_out);
  const size_t need = c0.used;
  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    return MOE_OK;
  }
  if (!ok16(x) || !ok16(w_router) || !ok4(topk_ids) || !ok4(topk_w) || !ok4(d_topk_w) || !ok16(dx) ||
      !ok16(dw_router) || !opt4(dbias) || !opt16(dlogits_out) || !opt16(dx_perm) || !opt4(slot_row))
    return MOE_ERR_INVALID_ARG;
  if ((dx_perm == nullptr) != (slot_row == nullptr)) return MOE_ERR_INVALID_ARG;
  if (workspace_step(ws, ws_bytes, need, &st)) return st;
  int ncu = 0;
  if ((st = num_cu(&ncu)) != MOE_OK) return st;
  Carver cv(ws);
  carve_route_backward(cv, w, T, d, E, es, dlogits_out);
  return hip_status(moe::launch_route_backward(dtype, T, d, E, k, x, w_router, topk_ids, topk_w, d_topk_w, dx_perm,
                                               slot_row, dx, dw_router, dbias, w, ncu,
                                               static_cast<hipStream_t>(stream)));
}

moe_status moe_layer_backward(int64_t T, int64_t d, int64_t E, int64_t k, int64_t F, moe_dtype dtype,
                              const void* x, const void* w_router, const void* w_gate, const void* w_up,
                              const void* w_down, const int32_t* topk_ids, const float* topk_w, const void* y_perm,
                              const void* gu, const void* dy, void* dx, float* dw_router, float* dbias, float* dw_gate,
                              float* dw_up, float* dw_down, float* d_topk_w_out, void* ws, size_t* ws_bytes,
                              void* stream) {
  moe_status st = check_tdek(T, d, E, k);
  if (st != MOE_OK) return st;
  if (F <= 0) return MOE_ERR_INVALID_ARG;
  if (F % 64 != 0 || F > kMaxDim) return MOE_ERR_UNSUPPORTED;
  if ((st = check_dtype(dtype)) != MOE_OK) return st;
  const bool routed = w_router != nullptr;
  const size_t es = elem_size(dtype);
  const int64_t slots = T * k;
  if (!ffn_backward_fits(slots, E)) return MOE_ERR_UNSUPPORTED;
  // token rows read in place through row_token when x's byte size fits the GEMM's
  // 32-bit row offsets; otherwise they are first copied to x_perm
  const bool in_place = (uint64_t)T * (uint64_t)d * es < (uint64_t(1) << 32);

  moe::FfnBackwardScratch fw{};
  moe::RouteBackwardScratch rw{};
  auto carve = [&](Carver& c, int32_t*& offsets, int32_t*& row_token, int32_t*& slot_row, int32_t*& counts,
                   float*& g, void*& dy_perm, void*& dx_perm, void*& x_perm) {
    offsets = static_cast<int32_t*>(c.take((size_t)(E + 1) * 4));
    row_token = static_cast<int32_t*>(c.take((size_t)slots * 4));
    slot_row = static_cast<int32_t*>(c.take((size_t)slots * 4));
    counts = static_cast<int32_t*>(c.take(permute_ws(T, E)));
    g = d_topk_w_out ? d_topk_w_out : static_cast<float*>(c.take((size_t)slots * 4));
    dy_perm = c.take((size_t)slots * d * es);
    dx_perm = c.take((size_t)slots * d * es);
    x_perm = in_place ? nullptr : c.take((size_t)slots * d * es);
    carve_ffn_backward(c, fw, slots, d, E, F, es, gu != nullptr);
    if (routed) carve_route_backward(c, rw, T, d, E, es, nullptr);
  };
  int32_t *offsets, *row_token, *slot_row, *counts;
  float* g;
  void *dy_perm, *dx_perm, *x_perm;
  Carver c0(nullptr);
  carve(c0, offsets, row_token, slot_row, counts, g, dy_perm, dx_perm, x_perm);
  const size_t need = c0.used;
  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    return MOE_OK;
  }
  if (!ok16(x) || !ok16(w_gate) || !ok16(w_up) || !ok16(w_down) || !ok4(topk_ids) || !ok4(topk_w) ||
      !ok16(y_perm) || !opt16(gu) || !ok16(dy) || !ok16(dx) || !ok16(dw_gate) || !ok16(dw_up) ||
      !ok16(dw_down) || !opt4(d_topk_w_out))
    return MOE_ERR_INVALID_ARG;
  if (routed) {
    if (!ok16(w_router) || !ok16(dw_router) || !opt4(dbias)) return MOE_ERR_INVALID_ARG;
  } else {
    if (dw_router || dbias) return MOE_ERR_INVALID_ARG;
  }
  if (workspace_step(ws, ws_bytes, need, &st)) return st;
  int ncu = 0;
  if ((st = num_cu(&ncu)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  Carver cv(ws);
  carve(cv, offsets, row_token, slot_row, counts, g, dy_perm, dx_perm, x_perm);

  if ((st = hip_status(moe::launch_permute(dtype, T, d, E, k, x, topk_ids, offsets, row_token, slot_row, x_perm,
                                           counts, s))) != MOE_OK)
    return st;
  if ((st = hip_status(moe::launch_combine_backward(dtype, T, d, k, dy, y_perm, slot_row, topk_w, dy_perm, g, s))) !=
      MOE_OK)
    return st;
  if ((st = hip_status(moe::launch_grouped_ffn_backward(dtype, slots, d, E, F, in_place ? x : x_perm,
                                                        in_place ? T : slots, in_place ? row_token : nullptr,
                                                        offsets, w_gate, w_up, w_down, dy_perm, gu, dx_perm, dw_gate,
                                                        dw_up, dw_down, fw, ncu, s))) != MOE_OK)
    return st;
  if (routed)
    return hip_status(moe::launch_route_backward(dtype, T, d, E, k, x, w_router, topk_ids, topk_w, g, dx_perm,
                                                 slot_row, dx, dw_router, dbias, rw, ncu, s));
  return hip_status(moe::launch_unpermute(dtype, T, d, k, dx_perm, slot_row, dx, s));
}

moe_status moe_newton_schulz(int64_t n, int64_t R, int64_t C, moe_dtype dtype, int64_t steps, float a, float b,
                             float c, float eps, const void* g, void* x, void* ws, size_t* ws_bytes, void* stream) {
  if (n <= 0 || R <= 0 || C <= 0 || steps < 0 || !(eps >= 0.0f)) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_BF16 || R % 64 != 0 || C % 64 != 0 || R > kMaxDim || C > kMaxDim || n > (int64_t(1) << 16) ||
      R * C >= kIdxLimit || n * (R / 256 + 1) * (C / 256 + 1) >= kIdxLimit)
    return MOE_ERR_UNSUPPORTED;
  const size_t per = (size_t)R * (size_t)C * 2, sq = (size_t)(R < C ? R : C) * (size_t)(R < C ? R : C) * 2;
  Carver c0(nullptr);
  c0.take(n * per);                               // X, wide orientation, two of them
  c0.take(n * per);
  c0.take(n * sq);                                // A = X X^T
  c0.take(n * sq);                                // B = b A + c A A
  c0.take((size_t)n * moe::kNormBlocks * 4);      // partial sums of squares
  const size_t need = c0.used;
  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    return MOE_OK;
  }
  if (!ok16(g) || !ok16(x)) return MOE_ERR_INVALID_ARG;
  moe_status st = MOE_OK;
  if (workspace_step(ws, ws_bytes, need, &st)) return st;
  int ncu = 0;
  if ((st = num_cu(&ncu)) != MOE_OK) return st;
  Carver cv(ws);
  void* xw0 = cv.take(n * per);
  void* xw1 = cv.take(n * per);
  void* A = cv.take(n * sq);
  void* B = cv.take(n * sq);
  float* partial = static_cast<float*>(cv.take((size_t)n * moe::kNormBlocks * 4));
  return hip_status(moe::launch_newton_schulz(n, R, C, steps, a, b, c, eps, g, x, xw0, xw1, A, B, partial, ncu,
                                              static_cast<hipStream_t>(stream)));
}

moe_status moe_combine(int64_t T, int64_t d, int64_t k, moe_dtype dtype, const void* y_perm,
                       const int32_t* slot_row, const float* topk_w, void* y, void* stream) {
  if (T <= 0 || d <= 0 || k <= 0) return MOE_ERR_INVALID_ARG;
  if (d % 64 != 0 || d > kMaxDim || T * k >= kIdxLimit) return MOE_ERR_UNSUPPORTED;
  moe_status st = check_dtype(dtype);
  if (st != MOE_OK) return st;
  if (!ok16(y_perm) || !ok4(slot_row) || !ok4(topk_w) || !ok16(y)) return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_combine(dtype, T, d, k, y_perm, slot_row, topk_w, y,
                                        static_cast<hipStream_t>(stream)));
}

moe_status moe_layer_forward(int64_t T, int64_t d, int64_t E, int64_t k, int64_t F, moe_dtype dtype, const void* x,
                             const void* w_router, const float* bias, const void* w_gate, const void* w_up,
                             const void* w_down, void* y, float* logits_out, int32_t* topk_ids, float* topk_w,
                             int32_t* offsets_out, void* y_perm_out, void* gu_out, void* ws, size_t* ws_bytes,
                             void* stream) {
  moe_status st = check_tdek(T, d, E, k);
  if (st != MOE_OK) return st;
  if (F <= 0) return MOE_ERR_INVALID_ARG;
  if (F % 64 != 0 || F > kMaxDim) return MOE_ERR_UNSUPPORTED;
  if ((st = check_dtype(dtype)) != MOE_OK) return st;
  const bool routed = w_router != nullptr;
  const size_t es = elem_size(dtype);
  const size_t slots = (size_t)T * (size_t)k;

  // workspace layout (each piece 256-byte aligned)
  Carver c(ws);
  float* logits = routed ? (logits_out ? logits_out : static_cast<float*>(c.take((size_t)T * E * 4))) : nullptr;
  int32_t* ids = (routed && !topk_ids) ? static_cast<int32_t*>(c.take(slots * 4)) : topk_ids;
  float* w = (routed && !topk_w) ? static_cast<float*>(c.take(slots * 4)) : topk_w;
  int32_t* offsets = offsets_out ? offsets_out : static_cast<int32_t*>(c.take((size_t)(E + 1) * 4));
  int32_t* row_token = static_cast<int32_t*>(c.take(slots * 4));
  int32_t* slot_row = static_cast<int32_t*>(c.take(slots * 4));
  int32_t* counts = static_cast<int32_t*>(c.take(permute_ws(T, E)));
  // also holds x_perm when x is not read in place
  void* y_perm = y_perm_out ? y_perm_out : c.take(slots * (size_t)d * es);
  void* h = c.take(slots * (size_t)F * es);
  const size_t need = c.used;

  if (ws == nullptr && ws_bytes != nullptr) {
    *ws_bytes = need;
    return MOE_OK;
  }
  if (!ok16(x) || !ok16(w_gate) || !ok16(w_up) || !ok16(w_down) || !ok16(y) || !opt16(logits_out) ||
      !opt4(offsets_out) || !opt16(y_perm_out) || !opt16(gu_out))
    return MOE_ERR_INVALID_ARG;
  if (routed) {
    if (!ok16(w_router) || !opt4(bias) || !opt4(topk_ids) || !opt4(topk_w)) return MOE_ERR_INVALID_ARG;
  } else {
    if (bias || logits_out || !ok4(topk_ids) || !ok4(topk_w)) return MOE_ERR_INVALID_ARG;
  }
  if (workspace_step(ws, ws_bytes, need, &st)) return st;
  int ncu = 0;
  if ((st = num_cu(&ncu)) != MOE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);

  if (routed) {
    if ((st = hip_status(moe::launch_router_gemm(dtype, T, d, E, x, w_router, bias, logits, ncu, s))) != MOE_OK)
      return st;
    if ((st = hip_status(moe::launch_topk(T, E, k, logits, ids, w, s))) != MOE_OK) return st;
  }
  // The gate/up GEMM reads token rows of x in place through row_token (no permuted
  // copy of x) whenever x's byte size fits the kernel's 32-bit row offsets.
  // Otherwise x is first copied to x_perm in y_perm's buffer; the down GEMM then
  // overwrites it, after the gate/up GEMM (same stream) has finished reading it.
  const bool in_place = (uint64_t)T * (uint64_t)d * es < (uint64_t(1) << 32);
  if ((st = hip_status(moe::launch_permute(dtype, T, d, E, k, x, ids, offsets, row_token, slot_row,
                                           in_place ? nullptr : y_perm, counts, s))) != MOE_OK)
    return st;
  if ((st = hip_status(moe::launch_grouped_ffn(dtype, (int64_t)slots, d, E, F, in_place ? x : y_perm,
                                               in_place ? T : (int64_t)slots, in_place ? row_token : nullptr, offsets, w_gate, w_up, w_down,
                                               y_perm, h, gu_out, ncu, s))) != MOE_OK)
    return st;
  return hip_status(moe::launch_combine(dtype, T, d, k, y_perm, slot_row, w, y, s));
}

}  // extern "C"
