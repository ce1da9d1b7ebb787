/*
 * moe.h - C ABI of the MI355X (gfx950) routed Mixture-of-Experts layer: forward,
 * backward, and Muon's Newton-Schulz step for whole expert matrices.
 *
 * The layer (one Mixture-of-Experts block of the ~1T-parameter model in
 * "Training a 1T-Parameter MoE on EU public infrastructure with PyTorch and
 * TorchTitan", TL;DR, model-configuration table: hidden 6,144, 384 routed
 * experts, top-8, expert hidden 1,792) sends every token to the k experts with
 * the largest router logits and mixes their SwiGLU outputs:
 *
 *   l[t,e]  = x[t,:] . W_r[e,:] + b[e]                        (router GEMM)
 *   S_t     = k largest l[t,:], ties to the lower expert index  (top-k)
 *   w[t,j]  = softmax(l[t,:])[S_tj] / sum_j' softmax(l[t,:])[S_tj']
 *   y[t]    = sum_j w[t,j] * FFN_{S_tj}(x[t])
 *   FFN_e(v) = W_d[e] (silu(W_g[e] v) * (W_u[e] v)),  silu(z) = z/(1+exp(-z))
 *
 * "Domyn 团队在 Jupiter 超算完成 1 万亿参数 MoE 模型训练项目解析", section 二,
 * states the routing idea (each token uses a few experts).  Routing is dropless
 * (no capacity limit), as in the Pangu Ultra MoE page.  Softmax scoring, SwiGLU
 * and the tie rule are readings the pages leave open.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  T tokens, d hidden size, E experts (on this GPU), k experts per token,
 *  F expert hidden size.  All matrices are row-major and dense.  Weights are
 *  stored output-major (like a linear layer): W_r [E,d], W_g and W_u [E,F,d],
 *  W_d [E,d,F], so both operands of every GEMM are contiguous along the
 *  contraction.
 *  dtype (MOE_F32 or MOE_BF16) is the type of x, the expert/router weights,
 *  x_perm, y_perm and y.  Logits, gate weights and bias are always float32;
 *  indices are always int32.  bf16 work accumulates in float32 and rounds to
 *  nearest-even when it stores bf16.
 *  Every pointer is a device pointer (HBM) that the caller allocates and owns;
 *  the library never allocates or frees device memory.  Data pointers must be
 *  16-byte aligned; the workspace must be 256-byte aligned.
 *  stream is a hipStream_t (NULL = the default stream).  Every call only
 *  enqueues work on that stream and returns at once: it never synchronises and
 *  never copies device memory to the host.  Faults inside kernels surface at
 *  the caller's next synchronisation.
 *  Workspace: call with ws == NULL and ws_bytes != NULL to have the required
 *  byte count written to *ws_bytes (MOE_OK, nothing launched, no HIP call
 *  made); call again with a buffer of at least that many bytes in ws and its
 *  size in *ws_bytes.  ws == NULL with ws_bytes == NULL runs without a
 *  workspace, which is allowed only when the required size is 0.
 *  Argument checks run on the host before anything is launched.
 *
 * Limits: d and F multiples of 64; 1 <= k <= E <= 1024; T*k < 2^31.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null required pointer, size <= 0, k > E, misaligned pointer */
  MOE_ERR_UNSUPPORTED = 2, /* d or F not a multiple of 64, E > 1024, T*k >= 2^31, unknown dtype */
  MOE_ERR_WORKSPACE = 3,   /* *ws_bytes smaller than the required size, or no workspace given when one is needed */
  MOE_ERR_HIP = 4          /* a launch or device query failed */
} moe_status;

/*
 * moe_route: router GEMM, softmax and top-k (first two steps of the layer).
 * Passage: the model-configuration table in the TL;DR of "Training a
 * 1T-Parameter MoE on EU public infrastructure with PyTorch and TorchTitan"
 * (384 routed experts, each token uses the top 8); the score function (softmax
 * over all routed experts), the tie rule and the renormalisation are readings.
 *   x          [T,d]  dtype      input tokens
 *   w_router   [E,d]  dtype      router weights
 *   bias       [E]    float32    per-expert routing bias added to the logits, or NULL
 *   logits_out [T,E]  float32    router logits l (bias included), or NULL
 *   topk_ids   [T,k]  int32      out: chosen experts, larger logit first, ties to the lower index
 *   topk_w     [T,k]  float32    out: renormalised gate weights (sum 1 per token, non-increasing)
 *   ws                           workspace: T*E*4 bytes (logits) when logits_out is NULL, else 0
 */
moe_status moe_route(int64_t T, int64_t d, int64_t E, int64_t k, moe_dtype dtype,
                     const void* x, const void* w_router, const float* bias,
                     float* logits_out, int32_t* topk_ids, float* topk_w,
                     void* ws, size_t* ws_bytes, void* stream);

/*
 * moe_permute: group the (token, slot) pairs by expert and copy token rows.
 * Passage: section 二 of "Domyn 团队在 Jupiter 超算完成 1 万亿参数 MoE 模型训练项目解析"
 * (each token is routed to a few expert sub-networks, so each expert's rows must
 * be gathered); dropless routing as on the Pangu Ultra MoE page (every slot gets
 * a row, no capacity limit).  The result is the stable counting sort of the slots
 * taken token by token, slot by slot.
 *   x          [T,d]   dtype     input tokens
 *   topk_ids   [T,k]   int32     expert of each slot; a negative id (or one >= E)
 *                                 marks a slot whose expert is not on this GPU: it
 *                                 is skipped.  A token naming the same expert in
 *                                 several slots (top-k never does) gets one row per
 *                                 slot, in slot order, like any other slot.
 *   offsets    [E+1]   int32     out: rows offsets[e]..offsets[e+1]-1 belong to expert e;
 *                                 offsets[E] = number of valid slots N
 *   row_token  [T*k]   int32     out: row r copies token row_token[r]; rows of one
 *                                 expert are in ascending token order (first N written)
 *   slot_row   [T*k]   int32     out: row of slot (t,j), or -1 for a skipped slot
 *   x_perm     [T*k,d] dtype     out: x_perm[r] = x[row_token[r]] (first N rows written);
 *                                 NULL: only the indices are produced (the grouped FFN
 *                                 can read x in place through row_token)
 *   ws                           workspace: ceil(T/256)*E*4 bytes
 */
moe_status moe_permute(int64_t T, int64_t d, int64_t E, int64_t k, moe_dtype dtype,
                       const void* x, const int32_t* topk_ids, int32_t* offsets,
                       int32_t* row_token, int32_t* slot_row, void* x_perm,
                       void* ws, size_t* ws_bytes, void* stream);

/*
 * moe_grouped_ffn: the SwiGLU FFN of every expert over its own rows.
 * Passage: the model-configuration table of "Training a 1T-Parameter MoE on EU
 * public infrastructure with PyTorch and TorchTitan" (hidden 6,144, expert hidden
 * 1,792; its parameter counts fit three d x F matrices per expert, a gated FFN);
 * SwiGLU is the reading of the gate.
 *   n_max              capacity (rows) of y_perm (and of x_in without a_rows)
 *   offsets are read on the device (nothing is copied back) and are not trusted:
 *                       the kernels use the running maximum of offsets[0..e],
 *                       clamped to [0, n_max], as expert e's first row.  Offsets
 *                       as moe_permute writes them (non-decreasing, offsets[E] <=
 *                       n_max) pass through unchanged; any others give unspecified
 *                       output (and may take long) but no access outside x_in,
 *                       a_rows, y_perm or the workspace.
 *   x_in               the FFN's input rows, one of:
 *                        a_rows == NULL: x_perm [n_max,d], rows grouped by expert;
 *                        a_rows != NULL: the token matrix x [n_in,d]; row r of the
 *                          FFN input is x[a_rows[r]] (a_rows = row_token from
 *                          moe_permute), read in place without a permuted copy.
 *                          Requires n_in*d*sizeof(dtype) < 2^32; entries outside
 *                          [0, n_in) are clamped into it on the device.
 *   n_in               rows of x_in when a_rows != NULL (ignored otherwise)
 *   a_rows   [n_max]   int32   NULL or the gather map described above
 *   offsets  [E+1]     int32   device array as written by moe_permute; empty experts allowed
 *   w_gate   [E,F,d]   dtype
 *   w_up     [E,F,d]   dtype
 *   w_down   [E,d,F]   dtype
 *   y_perm   [n_max,d] dtype   out: y_perm[r] = W_d[e](silu(W_g[e] v_r) * (W_u[e] v_r)) for
 *                               input row v_r of expert e (first offsets[E] rows); may be
 *                               the same buffer as x_perm
 *   gu_out [n_max,2F] dtype    NULL, or out: the gate and up pre-activations kept for
 *                               the backward (moe_grouped_ffn_backward's gu): row r
 *                               holds G = W_g[e] v_r in columns [0,F) and U = W_u[e] v_r
 *                               in [F,2F), float32 sums rounded to dtype (first
 *                               offsets[E] rows).  y_perm is the same with or without it.
 *                               16-byte aligned.
 *   ws                          workspace: n_max*F*sizeof(dtype) bytes (the hidden activations h)
 */
moe_status moe_grouped_ffn(int64_t n_max, int64_t d, int64_t E, int64_t F, moe_dtype dtype,
                           const void* x_in, int64_t n_in, const int32_t* a_rows,
                           const int32_t* offsets, const void* w_gate, const void* w_up,
                           const void* w_down, void* y_perm, void* gu_out, void* ws, size_t* ws_bytes,
                           void* stream);

/*
 * moe_combine: weighted un-permute.
 * Passage: section 二 of "Domyn 团队在 Jupiter 超算完成 1 万亿参数 MoE 模型训练项目解析"
 * (a token's output comes from the few experts it was routed to), mixed with the
 * renormalised gate weights of moe_route.
 *   y_perm    [*,d]  dtype     expert outputs by row
 *   slot_row  [T,k]  int32     row of slot (t,j), negative = skipped; every
 *                               non-negative row must exist in y_perm (the library
 *                               does not know y_perm's row count: this is the
 *                               caller's promise, kept by moe_permute's output)
 *   topk_w    [T,k]  float32   gate weights
 *   y         [T,d]  dtype     out: y[t] = sum_j topk_w[t,j] * y_perm[slot_row[t,j]]
 *                               (float32 sum); a token with no valid slot gets 0
 */
moe_status moe_combine(int64_t T, int64_t d, int64_t k, moe_dtype dtype,
                       const void* y_perm, const int32_t* slot_row, const float* topk_w,
                       void* y, void* stream);

/*
 * moe_layer_forward: the whole layer, route -> permute -> grouped FFN -> combine.
 * Passages: those of the four calls above (the layer of the configuration table of
 * "Training a 1T-Parameter MoE on EU public infrastructure with PyTorch and
 * TorchTitan", routed as in section 二 of the Domyn page, dropless as in Pangu).
 *   x [T,d], w_router [E,d] | NULL, bias [E] | NULL, w_gate, w_up [E,F,d], w_down [E,d,F]
 *   y [T,d] out.
 *   When w_router is not NULL the router runs and topk_ids / topk_w, if not
 *   NULL, receive its choice; logits_out [T,E], if not NULL, receives the logits.
 *   When w_router is NULL the slots are pre-routed (one expert-parallel rank's
 *   share): topk_ids [T,k] and topk_w [T,k] are then required INPUTS, with
 *   negative ids for slots owned elsewhere; bias and logits_out must be NULL.
 *   offsets_out [E+1] int32, if not NULL, receives the expert row offsets.
 *   y_perm_out [T*k,d] dtype, if not NULL, receives the expert outputs in the
 *   permutation's order (moe_layer_backward's y_perm) instead of the workspace.
 *   gu_out [T*k,2F] dtype, if not NULL, receives the gate and up pre-activations
 *   in the same row order (moe_grouped_ffn's gu_out; moe_layer_backward's gu).
 *   Both 16-byte aligned; y is the same with or without them.
 *   ws: query with ws == NULL (size grows with T*k*(2d+F); T*k*F without
 *   y_perm_out).
 */
moe_status moe_layer_forward(int64_t T, int64_t d, int64_t E, int64_t k, int64_t F, moe_dtype dtype,
                             const void* x, const void* w_router, const float* bias,
                             const void* w_gate, const void* w_up, const void* w_down,
                             void* y, float* logits_out, int32_t* topk_ids, float* topk_w,
                             int32_t* offsets_out, void* y_perm_out, void* gu_out, void* ws,
                             size_t* ws_bytes, void* stream);

/*
 * moe_layer_forward_noalloc: moe_layer_forward without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Its workspace is a device
 * array inside this library of MOE_NOALLOC_SCRATCH_BYTES bytes, which every GPU
 * the library runs on holds until the process ends; a call whose workspace query
 * (moe_layer_forward with ws == NULL) exceeds it returns MOE_ERR_WORKSPACE before
 * anything is launched.  At the page's layer shape (d 6,144, E 384, top-8, F
 * 1,792, bf16) that is up to 521 routed tokens per call (2,211 with y_perm_out
 * given, which takes y_perm out of the workspace).  Same kernels and results as
 * moe_layer_forward; it calls no allocator.  Calls that overlap on one GPU share
 * the array and race: order them on one stream (or synchronise between them).
 * Arguments and errors as moe_layer_forward.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status moe_layer_forward_noalloc(int64_t T, int64_t d, int64_t E, int64_t k, int64_t F, moe_dtype dtype,
                                     const void* x, const void* w_router, const float* bias,
                                     const void* w_gate, const void* w_up, const void* w_down,
                                     void* y, float* logits_out, int32_t* topk_ids, float* topk_w,
                                     int32_t* offsets_out, void* y_perm_out, void* gu_out, void* stream);

/*
 * moe_grouped_ffn_backward: gradients of the grouped SwiGLU FFN (the layer
 * backward's matrix products; the pages' workload is pre-training, "Training a
 * 1T-Parameter MoE on EU public infrastructure with PyTorch and TorchTitan").
 * For expert e and its rows X (as in moe_grouped_ffn) with output gradient dY:
 *   dH = dY W_d, S = silu(X W_g^T), U = X W_u^T, H = S U,
 *   dU = dH S, dG = dH U silu'(X W_g^T),
 *   dX = dG W_g + dU W_u,  dW_d = dY^T H,  dW_g = dG^T X,  dW_u = dU^T X.
 * G and U are recomputed from the inputs, or read from gu when the forward kept
 * them (moe_grouped_ffn's gu_out): the backward then skips the gate/up product
 * (a third of its matrix work) and holds no float32 dH.
 *   n_max, d, E, F, x_in, n_in, a_rows, offsets, w_gate, w_up, w_down: as in
 *                        moe_grouped_ffn
 *   dy_perm  [n_max,d] dtype   dY, rows grouped by expert (rows offsets[E].. unused)
 *   gu     [n_max,2F] dtype   NULL (recompute G and U), or the forward's gu_out for
 *                              the same rows, 16-byte aligned
 *   dx_perm  [n_max,d] dtype   out: dX (first offsets[E] rows written)
 *   dw_gate, dw_up [E,F,d] f32, dw_down [E,d,F] f32   out; zero for an expert with
 *                        no rows
 *   ws: query with ws == NULL (holds dH in float32, dG|dU, H and transposed
 *       activations: 3 n_max F dtype elements, n_max F float32 and
 *       (2 d + 3 F) (n_max + 63 E) dtype elements; float32 layers add transposed
 *       weight copies, 3 E d F elements; bf16 weights are read in place).
 * bf16: bf16 products, float32 accumulation; dG, dU and H are rounded to bf16
 * before the products that use them (with gu, G and U come in rounded to bf16
 * as well).  float32: float32 throughout.  The workspace query depends on
 * whether gu is NULL.
 * Errors as moe_grouped_ffn.
 */
moe_status moe_grouped_ffn_backward(int64_t n_max, int64_t d, int64_t E, int64_t F, moe_dtype dtype,
                                    const void* x_in, int64_t n_in, const int32_t* a_rows,
                                    const int32_t* offsets, const void* w_gate, const void* w_up,
                                    const void* w_down, const void* dy_perm, const void* gu,
                                    void* dx_perm, float* dw_gate, float* dw_up, float* dw_down,
                                    void* ws, size_t* ws_bytes, void* stream);

/*
 * Backward of the whole layer.  The pages' workload is pre-training ("Training
 * a 1T-Parameter MoE on EU public infrastructure with PyTorch and TorchTitan",
 * TL;DR and "The machine and its constraints"), so every step runs the layer
 * backward after the forward.  Given the output gradient dy, the chain rule of
 * the forward above gives, step by step in reverse:
 *   combine:       dy_perm[slot_row[t,j]] = w[t,j] dy[t]
 *                  g[t,j] = <dy[t], y_perm[slot_row[t,j]]>          (gradient of w)
 *   experts:       moe_grouped_ffn_backward on the permuted rows
 *   gate weights:  w[t,:] is a softmax of the selected logits (the full softmax's
 *                  denominator cancels when renormalising), so
 *                  dl[t,S_tj] = w[t,j] (g[t,j] - sum_i w[t,i] g[t,i]); every
 *                  other logit gets 0 (the selection is piecewise constant)
 *   router:        dx += dl W_r,  dW_r = dl^T x,  db = sum over tokens of dl
 *   permutation:   dx[t] += sum_j dx_perm[slot_row[t,j]]
 * Every reduction runs in a fixed order (no atomics): results are
 * bit-reproducible for the same inputs and sizes.
 */

/*
 * moe_combine_backward: backward of moe_combine.
 *   dy        [T,d]   dtype    output gradient
 *   y_perm    [*,d]   dtype    the forward's expert outputs (rows slot_row refers to)
 *   slot_row  [T,k]   int32    the forward's map (from moe_permute); < 0: skipped slot
 *   topk_w    [T,k]   float32  the forward's gate weights
 *   dy_perm   [*,d]   dtype    out: row slot_row[t,j] = topk_w[t,j] dy[t] (float32
 *                              product, rounded to dtype); rows no slot refers to
 *                              are left untouched
 *   d_topk_w  [T,k]   float32  out: g[t,j] = <dy[t], y_perm[slot_row[t,j]]> (float32
 *                              sum), 0 for a skipped slot
 * slot_row must hold distinct in-range rows (as moe_permute writes them).  No
 * workspace.  Errors: sizes <= 0 or null/misaligned pointers:
 * MOE_ERR_INVALID_ARG; d not a multiple of 64 or T*k >= 2^31: MOE_ERR_UNSUPPORTED.
 */
moe_status moe_combine_backward(int64_t T, int64_t d, int64_t k, moe_dtype dtype, const void* dy,
                                const void* y_perm, const int32_t* slot_row, const float* topk_w,
                                void* dy_perm, float* d_topk_w, void* stream);

/*
 * moe_route_backward: backward of moe_route (renormalised top-k softmax and
 * router GEMM), plus the permutation's backward when dx_perm is given, since both
 * end in dx.
 *   x, w_router            as in moe_route
 *   topk_ids, topk_w [T,k] the forward's routing (ids distinct per token; ids
 *                          outside [0, E) are skipped)
 *   d_topk_w  [T,k] f32    gradient of the gate weights (moe_combine_backward's g)
 *   dx_perm   [*,d] dtype  gradient of the permuted rows, or NULL
 *   slot_row  [T,k] int32  the forward's map; required exactly when dx_perm is given
 *   dx        [T,d] dtype  out: sum_j dl[t,j] W_r[ids[t,j]] (+ sum_j dx_perm[slot_row[t,j]])
 *                          summed in float32, rounded once
 *   dw_router [E,d] f32    out: dl^T x (bf16: dl rounded to bf16 for the
 *                          product, float32 accumulation)
 *   dbias     [E]   f32    out: float32 column sums of dl, or NULL to skip
 *   dlogits_out [T,E] f32  out: the dense logit gradient dl, or NULL (then it lives
 *                          in the workspace)
 *   ws: query with ws == NULL (about T E 4 + (E + d) T' dtype bytes, T' = T rounded
 *       up to 64, plus up to 16 E d float32 partial sums).
 * Errors as moe_route; dx_perm given without slot_row or the reverse:
 * MOE_ERR_INVALID_ARG.
 */
moe_status moe_route_backward(int64_t T, int64_t d, int64_t E, int64_t k, moe_dtype dtype,
                              const void* x, const void* w_router, const int32_t* topk_ids,
                              const float* topk_w, const float* d_topk_w, const void* dx_perm,
                              const int32_t* slot_row, void* dx, float* dw_router, float* dbias,
                              float* dlogits_out, void* ws, size_t* ws_bytes, void* stream);

/*
 * moe_layer_backward: the whole layer backward from the forward's saved routing
 * and expert outputs.
 *   T, d, E, k, F, dtype, x, w_router, w_gate, w_up, w_down: as in moe_layer_forward
 *                          (w_router NULL: pre-routed slots, no router gradient)
 *   topk_ids, topk_w [T,k] the forward's routing (negative id: slot owned elsewhere)
 *   y_perm  [T*k,d] dtype  the forward's expert outputs, rows in the permutation's
 *                          order (experts ascending, tokens ascending within an
 *                          expert; moe_permute's order, recomputed here from topk_ids)
 *   gu    [T*k,2F]  dtype  NULL, or the forward's gate/up pre-activations in the same
 *                          row order (moe_layer_forward's gu_out): no recompute
 *   dy      [T,d]   dtype  output gradient
 *   dx      [T,d]   dtype  out: input gradient (experts, permutation and router)
 *   dw_router [E,d] f32    out (NULL when pre-routed); dbias [E] f32 out or NULL
 *                          (must be NULL when pre-routed)
 *   dw_gate, dw_up [E,F,d], dw_down [E,d,F] f32   out (zero for an expert with no rows)
 *   d_topk_w_out [T,k] f32 out: gradient of the gate weights, or NULL
 *   ws: query with ws == NULL (the grouped-FFN backward's workspace for T*k rows,
 *       plus dy_perm and dx_perm, plus moe_route_backward's when routed).
 * Errors as moe_layer_forward; dw_router or dbias given when pre-routed:
 * MOE_ERR_INVALID_ARG.
 */
moe_status moe_layer_backward(int64_t T, int64_t d, int64_t E, int64_t k, int64_t F, moe_dtype dtype,
                              const void* x, const void* w_router, const void* w_gate, const void* w_up,
                              const void* w_down, const int32_t* topk_ids, const float* topk_w,
                              const void* y_perm, const void* gu, const void* dy, void* dx, float* dw_router,
                              float* dbias, float* dw_gate, float* dw_up, float* dw_down, float* d_topk_w_out,
                              void* ws, size_t* ws_bytes, void* stream);

/*
 * moe_newton_schulz: Muon's orthogonalisation of a batch of whole matrices
 * ("Training a 1T-Parameter MoE on EU public infrastructure with PyTorch and
 * TorchTitan", section "FlexShard: communication-free Muon": a few
 * Newton-Schulz iterations over each whole matrix, experts kept whole on one
 * rank).  For each of the n matrices G [R,C], working on its wide orientation
 * (a tall G is transposed first and the result transposed back):
 *     X = G / (||G||_F + eps);  `steps` times: A = X X^T, B = b A + c A A, X = a X + B X
 * Muon's published quintic uses (a, b, c) = (3.4445, -4.7750, 2.0315), 5 steps,
 * eps = 1e-7.  bf16 storage of X, A and B between the products, fp32
 * accumulation and fp32 Frobenius norm (summed in a fixed order: results are
 * bit-reproducible).
 *   n                  matrices (<= 65536)
 *   R, C               rows and columns of each, multiples of 64
 *   dtype              MOE_BF16 only (MOE_F32: MOE_ERR_UNSUPPORTED)
 *   steps              >= 0 (0: the normalised input)
 *   g   [n,R,C] bf16   input, row-major, matrices back to back
 *   x   [n,R,C] bf16   out, same layout; must not overlap g or ws
 *   ws: query with ws == NULL; about 2 n R C + 2 n min(R,C)^2 bf16 elements.
 * Errors: n, R, C <= 0, steps < 0 or eps < 0 or NaN: MOE_ERR_INVALID_ARG;
 * R or C not a multiple of 64, dtype not bf16, sizes past the limits:
 * MOE_ERR_UNSUPPORTED; g, x, ws not 16-byte aligned: MOE_ERR_INVALID_ARG.
 */
moe_status moe_newton_schulz(int64_t n, int64_t R, int64_t C, moe_dtype dtype, int64_t steps,
                             float a, float b, float c, float eps, const void* g, void* x,
                             void* ws, size_t* ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
