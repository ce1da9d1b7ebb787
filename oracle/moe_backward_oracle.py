"""Plain CPU oracle for the backward pass of the grouped SwiGLU expert FFN.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite and the CPU-baseline leg of the
benchmark use it.  It shares no code with the HIP path.

What it computes, and where it comes from
-----------------------------------------
The pages' workload is pre-training ("Training a 1T-Parameter MoE on EU public
infrastructure with PyTorch and TorchTitan": TL;DR and "The machine and its
constraints"), so every step runs the layer backward as well.  This module
covers the expert part of it, which carries the backward's matrix products:
for expert e with input rows X [n, d] (the forward's permuted rows) and the
gradient dY [n, d] of its output rows,

    G = X W_g^T,  U = X W_u^T,  S = silu(G),  H = S * U,  Y = H W_d^T     (forward)
    dH   = dY W_d                          dW_d = dY^T H
    dU   = dH * S                          dS   = dH * U
    dG   = dS * silu'(G),   silu'(z) = sigma(z) (1 + z (1 - sigma(z)))
    dX   = dG W_g + dU W_u                 dW_g = dG^T X,   dW_u = dU^T X

with sigma(z) = 1 / (1 + exp(-z)).  These are the chain rule written out for
the forward in moe_oracle.expert_ffn (the same SwiGLU reading).

Every floating-point step runs in float64 with numpy.  Every function here has
a pin in tests/pins_backward.py.
"""
from __future__ import annotations

import numpy as np


def to_f64(a) -> np.ndarray:
    """Exact conversion to float64; uint16 arrays are bf16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def sigmoid(z) -> np.ndarray:
    z = to_f64(z)
    return 1.0 / (1.0 + np.exp(-z))


def silu_grad(z) -> np.ndarray:
    """d/dz [z sigma(z)] = sigma(z) + z sigma(z) (1 - sigma(z))."""
    z = to_f64(z)
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def expert_ffn_backward(X, w_gate_e, w_up_e, w_down_e, dY):
    """Gradients of one expert: returns (dX [n,d], dW_g [F,d], dW_u [F,d], dW_d [d,F])."""
    X, dY = to_f64(X), to_f64(dY)
    Wg, Wu, Wd = to_f64(w_gate_e), to_f64(w_up_e), to_f64(w_down_e)
    G = X @ Wg.T
    U = X @ Wu.T
    S = G * sigmoid(G)
    H = S * U
    dH = dY @ Wd
    dWd = dY.T @ H
    dU = dH * S
    dG = dH * U * silu_grad(G)
    dX = dG @ Wg + dU @ Wu
    return dX, dG.T @ X, dU.T @ X, dWd


def grouped_ffn_backward(x_perm, offsets, w_gate, w_up, w_down, dy_perm):
    """Every expert's backward on its rows offsets[e] .. offsets[e+1]-1.
    Returns (dx_perm [n,d], dW_g [E,F,d], dW_u [E,F,d], dW_d [E,d,F]); an expert
    with no rows gets zero weight gradients."""
    offsets = np.asarray(offsets, dtype=np.int64)
    E = offsets.size - 1
    n = int(offsets[-1])
    x_perm = np.asarray(x_perm)
    d = x_perm.shape[1]
    F = np.asarray(w_gate[0]).shape[0]
    dx = np.zeros((n, d))
    dwg = np.zeros((E, F, d))
    dwu = np.zeros((E, F, d))
    dwd = np.zeros((E, d, F))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            dx[lo:hi], dwg[e], dwu[e], dwd[e] = expert_ffn_backward(
                x_perm[lo:hi], w_gate[e], w_up[e], w_down[e], np.asarray(dy_perm)[lo:hi])
    return dx, dwg, dwu, dwd
