"""Plain CPU oracle for the backward pass of the whole routed MoE layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite and the CPU-baseline leg of the
benchmark use it.  It shares no code with the HIP path.

What it computes, and where it comes from
-----------------------------------------
The pages' workload is pre-training ("Training a 1T-Parameter MoE on EU public
infrastructure with PyTorch and TorchTitan": TL;DR and "The machine and its
constraints"), so each step runs the layer backward after the forward.  The
forward is the one in moe_oracle (router GEMM, softmax over all routed
experts, top-k, renormalised gate weights, permutation, SwiGLU experts,
weighted combine).  Its backward, given the output gradient dy [T, d] and the
forward's saved routing and expert outputs y_perm, is the chain rule taken
step by step in reverse:

  combine      y[t] = sum_j w[t,j] y_perm[slot_row[t,j]]
               -> dy_perm[slot_row[t,j]] = w[t,j] dy[t]
               -> g[t,j] = <dy[t], y_perm[slot_row[t,j]]>        (gradient of w)
  experts      moe_backward_oracle.grouped_ffn_backward on the permuted rows
               -> dx_perm, dW_g, dW_u, dW_d
  gate weights w[t,:] = softmax of the selected logits l[t, S_t]  (the full
               softmax's denominator cancels in the renormalisation), so with
               J = diag(w) - w w^T:  dl[t, S_t] = J g[t,:]; every other logit
               gets zero (the selection is piecewise constant in the logits)
  router       l = x W_r^T + b -> dx += dl W_r,  dW_r = dl^T x,  db = sum_t dl[t]
  permutation  x_perm[r] = x[row_token[r]] -> dx[t] += sum of dx_perm over the
               rows that copy token t

Every floating-point step runs in float64 with numpy.  Every function here has
a pin in tests/pins_layer_backward.py.
"""
from __future__ import annotations

import numpy as np

from . import moe_backward_oracle as ffn_bwd
from . import moe_oracle as fwd


def to_f64(a) -> np.ndarray:
    return fwd.to_f64(a)


def combine_backward(dy, y_perm, slot_row, weights):
    """Backward of the weighted un-permute.  Returns (dy_perm [N, d], g [T, k]):
    dy_perm[slot_row[t,j]] = w[t,j] dy[t] and g[t,j] = <dy[t], y_perm[slot_row[t,j]]>;
    a slot with slot_row < 0 has g = 0 and no row."""
    dy, y_perm, w = to_f64(dy), to_f64(y_perm), to_f64(weights)
    slot_row = np.asarray(slot_row, dtype=np.int64)
    T, k = slot_row.shape
    dy_perm = np.zeros_like(y_perm)
    g = np.zeros((T, k))
    for j in range(k):
        ok = slot_row[:, j] >= 0
        rows = slot_row[ok, j]
        dy_perm[rows] = w[ok, j][:, None] * dy[ok]
        g[ok, j] = np.einsum("td,td->t", dy[ok], y_perm[rows])
    return dy_perm, g


def gate_weights_backward(weights, g):
    """Gradient of the selected logits from the gradient g of the renormalised
    gate weights w = softmax(selected logits): dl = (diag(w) - w w^T) g per token
    (the Jacobian of a softmax is symmetric).  Returns dl_sel [T, k]."""
    w, g = to_f64(weights), to_f64(g)
    T, k = w.shape
    dl = np.zeros((T, k))
    for t in range(T):
        J = np.diag(w[t]) - np.outer(w[t], w[t])
        dl[t] = J @ g[t]
    return dl


def scatter_logit_grad(ids, dl_sel, num_experts: int):
    """Dense dlogits [T, E] from the selected positions (zero elsewhere)."""
    ids = np.asarray(ids, dtype=np.int64)
    T, k = ids.shape
    dl = np.zeros((T, num_experts))
    for j in range(k):
        ok = ids[:, j] >= 0
        dl[np.nonzero(ok)[0], ids[ok, j]] = to_f64(dl_sel)[ok, j]
    return dl


def router_backward(x, w_router, dlogits):
    """Backward of l = x W_r^T + b: returns (dx [T, d], dW_r [E, d], db [E])."""
    x, Wr, dl = to_f64(x), to_f64(w_router), to_f64(dlogits)
    return dl @ Wr, dl.T @ x, dl.sum(axis=0)


def permute_backward(dx_perm, row_token, num_tokens: int):
    """Backward of x_perm[r] = x[row_token[r]]: dx[t] = sum of dx_perm[r] over
    the rows r with row_token[r] = t (zero for a token with no row)."""
    dx_perm = to_f64(dx_perm)
    row_token = np.asarray(row_token, dtype=np.int64)
    dx = np.zeros((num_tokens, dx_perm.shape[1]))
    np.add.at(dx, row_token, dx_perm)
    return dx


def layer_backward(x, w_router, w_gate, w_up, w_down, ids, weights, y_perm, dy) -> dict:
    """The whole layer backward from the forward's routing (ids [T, k], weights
    [T, k]) and expert outputs y_perm (rows in the permutation's order), for the
    output gradient dy [T, d].  With w_router None (pre-routed slots) no router
    gradient is taken.  The bias gradient equals the sum of the logit gradient
    over tokens whether or not the forward had a bias.

    Returns a dict: offsets, row_token, slot_row, dy_perm, g, dl_sel, dlogits,
    dx_perm, dx, dw_router, dbias, dw_gate, dw_up, dw_down."""
    x = np.asarray(x)
    T = x.shape[0]
    E = len(w_gate)
    offsets, row_token, slot_row = fwd.permute(ids, E)
    dy_perm, g = combine_backward(dy, y_perm, slot_row, weights)
    x_perm = fwd.gather_rows(x, row_token)
    dx_perm, dwg, dwu, dwd = ffn_bwd.grouped_ffn_backward(x_perm, offsets, w_gate, w_up, w_down, dy_perm)
    dx = permute_backward(dx_perm, row_token, T)
    out = dict(offsets=offsets, row_token=row_token, slot_row=slot_row, dy_perm=dy_perm, g=g, dx_perm=dx_perm,
               dw_gate=dwg, dw_up=dwu, dw_down=dwd, dl_sel=None, dlogits=None, dw_router=None, dbias=None)
    if w_router is not None:
        dl_sel = gate_weights_backward(weights, g)
        dlogits = scatter_logit_grad(ids, dl_sel, E)
        dx_r, dwr, db = router_backward(x, w_router, dlogits)
        dx = dx + dx_r
        out.update(dl_sel=dl_sel, dlogits=dlogits, dw_router=dwr, dbias=db)
    out["dx"] = dx
    return out
