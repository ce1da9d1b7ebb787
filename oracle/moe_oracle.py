"""Plain CPU oracle for the forward pass of one routed Mixture-of-Experts layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the CPU-baseline
leg of the benchmark use it.  It shares no code with the HIP path.

Every floating-point step runs in float64 with numpy.  Inputs given in bf16
(or fp32) are converted exactly to float64 first; the oracle never rounds
anything back to a narrower type.

What the layer computes, and where it comes from
------------------------------------------------
* "Training a 1T-Parameter MoE on EU public infrastructure with PyTorch and
  TorchTitan" (PyTorch blog, Chinese rendering), TL;DR, model-configuration
  table: hidden size 6,144, 384 routed experts of which each token uses the
  top 8, expert hidden size 1,792.  The same table's parameter counts (951.9B
  total, 32.8B active, 74 layers) fit exactly three d x F matrices per expert,
  i.e. a gated FFN.
* "Domyn 团队在 Jupiter 超算完成 1 万亿参数 MoE 模型训练项目解析", section 二
  (MoE architecture): each input token is routed to a few expert sub-networks;
  the other parameters stay inactive for that token.
* "华为揭秘：国产昇腾训出世界一流大模型" (Pangu Ultra MoE): dropless training,
  i.e. no capacity limit and no dropped tokens.
* The pages do not name the score function, the activation, the weight
  normalisation or the tie rule.  The readings used here are: softmax over all
  routed experts, selection of the k largest logits with ties going to the
  lower expert index, selected probabilities renormalised to sum to one, and a
  SwiGLU expert h = silu(x W_g^T) * (x W_u^T), y = h W_d^T with
  silu(z) = z / (1 + exp(-z)).  Rows of one expert's segment are ordered by
  ascending token index.

Every function here has a pin in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import numpy as np


def to_f64(a) -> np.ndarray:
    """Exact conversion to float64.  uint16 arrays are read as bf16 bit patterns
    (the upper half of an IEEE binary32); anything else goes through numpy."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


# ----------------------------------------------------------------------------
# Routing
# ----------------------------------------------------------------------------

def router_logits(x, w_router, bias=None) -> np.ndarray:
    """l[t, e] = sum_i x[t, i] * W_r[e, i] + b[e]   (router GEMM; weights stored
    [E, d] like a linear layer).  The bias is the per-expert routing bias of the
    skewed-routing workload; None means zero."""
    l = to_f64(x) @ to_f64(w_router).T
    if bias is not None:
        l = l + to_f64(bias)[None, :]
    return l


def softmax(logits) -> np.ndarray:
    """Softmax over the routed experts of each token (max-shifted)."""
    l = to_f64(logits)
    m = l.max(axis=1, keepdims=True)
    p = np.exp(l - m)
    return p / p.sum(axis=1, keepdims=True)


def select_topk(logits, k: int):
    """Top-k of each row by the key (larger logit first, then lower expert
    index), and the renormalised gate weights of the chosen experts.

    Selection works on the logits themselves (softmax is monotone, so this is the
    same set as selecting on probabilities, without rounding ties).  -0.0 and
    +0.0 are the same value.  Returns (ids [T, k] int32, w [T, k] float64), each
    row in key order, so w is non-increasing along a row.
    """
    l = to_f64(logits) + 0.0                      # -0.0 + 0.0 == +0.0
    T, E = l.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    expert = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((expert, -l), axis=-1)     # primary key -l, then e
    ids = order[:, :k].astype(np.int32)
    p = softmax(l)
    p_sel = np.take_along_axis(p, order[:, :k], axis=1)
    w = p_sel / p_sel.sum(axis=1, keepdims=True)
    return ids, w


def route(x, w_router, bias, k: int):
    """Router GEMM, softmax and top-k.  Returns (logits, ids, w)."""
    l = router_logits(x, w_router, bias)
    ids, w = select_topk(l, k)
    return l, ids, w


# ----------------------------------------------------------------------------
# Permutation (counting sort of the (token, slot) pairs by expert)
# ----------------------------------------------------------------------------

def permute(ids, num_experts: int):
    """Group the (token, slot) pairs by expert.

    ids[t, j] is token t's j-th expert; a negative id marks a slot whose expert
    lives elsewhere (pre-routed input of one expert-parallel rank) and is
    skipped.  Within an expert's segment the rows follow ascending token index:
    a stable sort of the slots, taken in token-major order, by expert id.

    Returns (offsets [E+1] int32, row_token [N] int32, slot_row [T, k] int32)
    where N is the number of valid slots, rows offsets[e]..offsets[e+1]-1 belong
    to expert e, row_token[r] is the token that row r copies, and slot_row[t, j]
    is the row of slot (t, j) or -1.
    """
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    valid = np.nonzero(flat >= 0)[0]              # slot numbers s = t*k + j
    if np.any(flat[valid] >= num_experts):
        raise ValueError("expert id out of range")
    counts = np.bincount(flat[valid], minlength=num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = valid[np.argsort(flat[valid], kind="stable")]
    row_token = (order // k).astype(np.int32)
    slot_row = np.full(T * k, -1, dtype=np.int64)
    slot_row[order] = np.arange(order.size)
    return offsets.astype(np.int32), row_token, slot_row.reshape(T, k).astype(np.int32)


def gather_rows(x, row_token) -> np.ndarray:
    """x_perm[r] = x[row_token[r]] (an exact copy, kept in the input's dtype)."""
    return np.asarray(x)[np.asarray(row_token, dtype=np.int64)]


# ----------------------------------------------------------------------------
# Expert FFN
# ----------------------------------------------------------------------------

def silu(z) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = to_f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_ffn(X, w_gate_e, w_up_e, w_down_e) -> np.ndarray:
    """One SwiGLU expert on the rows X [n, d]:
    G = X W_g^T, U = X W_u^T, H = silu(G) * U, Y = H W_d^T.
    W_g, W_u are [F, d]; W_d is [d, F] (output-major, like a linear layer)."""
    X = to_f64(X)
    G = X @ to_f64(w_gate_e).T
    U = X @ to_f64(w_up_e).T
    H = silu(G) * U
    return H @ to_f64(w_down_e).T


def grouped_ffn(x_perm, offsets, w_gate, w_up, w_down) -> np.ndarray:
    """Apply expert e to rows offsets[e]..offsets[e+1]-1 of x_perm, for every e;
    experts with no rows are skipped.  w_gate[e], w_up[e], w_down[e] are read one
    expert at a time, so they may be lazy per-expert loaders."""
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.size - 1
    n = int(offsets[-1])
    d = np.asarray(x_perm).shape[1]
    y_perm = np.zeros((n, d), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y_perm[lo:hi] = expert_ffn(np.asarray(x_perm)[lo:hi], w_gate[e], w_up[e], w_down[e])
    return y_perm


# ----------------------------------------------------------------------------
# Combine (weighted un-permute)
# ----------------------------------------------------------------------------

def combine(y_perm, slot_row, weights) -> np.ndarray:
    """y[t] = sum_j w[t, j] * y_perm[slot_row[t, j]], skipping slot_row < 0.
    A token with no valid slot gets a zero row."""
    y_perm = to_f64(y_perm)
    slot_row = np.asarray(slot_row, dtype=np.int64)
    w = to_f64(weights)
    T, k = slot_row.shape
    y = np.zeros((T, y_perm.shape[1]), dtype=np.float64)
    for j in range(k):
        ok = slot_row[:, j] >= 0
        y[ok] += w[ok, j][:, None] * y_perm[slot_row[ok, j]]
    return y


# ----------------------------------------------------------------------------
# Whole layer
# ----------------------------------------------------------------------------

def layer_forward(x, w_router, bias, w_gate, w_up, w_down, k: int,
                  selection_logits=None, ids=None, weights=None) -> dict:
    """The whole layer: route, permute, grouped SwiGLU FFN, combine.

    selection_logits: if given, top-k selection and gate weights are taken from
      these logits instead of the oracle's own (the oracle's logits are still
      returned for a separate comparison).
    ids, weights: pre-routed slots (negative id = skipped); then no router runs.
    Returns a dict with logits (None when pre-routed), ids, w, offsets,
    row_token, slot_row, x_perm, y_perm and y.
    """
    x = np.asarray(x)
    if ids is None:
        logits = router_logits(x, w_router, bias)
        ids, w = select_topk(logits if selection_logits is None else selection_logits, k)
        E = np.asarray(w_router).shape[0]
    else:
        logits = None
        w = to_f64(weights)
        E = len(w_gate)
    offsets, row_token, slot_row = permute(ids, E)
    x_perm = gather_rows(x, row_token)
    y_perm = grouped_ffn(x_perm, offsets, w_gate, w_up, w_down)
    y = combine(y_perm, slot_row, w)
    return dict(logits=logits, ids=np.asarray(ids, dtype=np.int32), w=w, offsets=offsets,
                row_token=row_token, slot_row=slot_row, x_perm=x_perm, y_perm=y_perm, y=y)
