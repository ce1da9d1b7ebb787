"""Plain CPU oracle for Muon's Newton-Schulz orthogonalisation of whole matrices.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the test suite and the CPU-baseline leg of the
benchmark use it.  It shares no code with the HIP path.

What it computes, and where it comes from
-----------------------------------------
* "Training a 1T-Parameter MoE on EU public infrastructure with PyTorch and
  TorchTitan" (PyTorch blog, Chinese rendering), section "FlexShard:
  communication-free Muon": every weight matrix except the router and the
  embeddings is trained with Muon; Muon orthogonalises each update with a few
  Newton-Schulz iterations that act on the whole matrix; experts are placed
  whole on one rank, so each rank runs the iterations on complete expert
  matrices with no communication.  The same section and its Figure 3 measure
  the iterations moved from the host CPU to the GPU.
* The pages give neither the iteration's polynomial nor the number of steps.
  Reading used here: Muon's published quintic iteration
      A = X X^T,   B = b A + c A A,   X <- a X + B X
  with (a, b, c) = (3.4445, -4.7750, 2.0315) and five steps, started from
  X = G / (||G||_F + eps), eps = 1e-7, on the wide orientation of the matrix
  (a tall matrix is transposed first and the result transposed back).
  On the singular values this is the scalar map s -> a s + b s^3 + c s^5,
  applied five times to s / ||s||_2; the singular vectors are unchanged.

Precision
---------
float64 with numpy by default.  With round_bf16=True the oracle rounds X, A
and B to bfloat16 (round to nearest even, from float32) at the points where a
bfloat16 implementation stores them: X after the normalisation and after every
step, A, and B (formed from the bf16 A and the exact A A).  Each rounding here
is written out below; the comparison with a GPU path then only sees the
difference of summation order.

Every function here has a pin in tests/pins_muon.py.
"""
from __future__ import annotations

import numpy as np

MUON_COEFFS = (3.4445, -4.7750, 2.0315)
MUON_STEPS = 5
MUON_EPS = 1e-7


def to_f64(a) -> np.ndarray:
    """Exact conversion to float64; uint16 arrays are bf16 bit patterns."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_bf16(a) -> np.ndarray:
    """Round to bfloat16 (nearest, ties to even) by way of float32, returned as
    float64.  bfloat16 is the upper 16 bits of an IEEE binary32: add half an ulp
    of the kept part (plus the kept part's lowest bit, for ties to even) to the
    32-bit pattern and clear the low 16 bits.  Inputs are finite."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def normalise(G, eps=MUON_EPS) -> np.ndarray:
    """X0 = G / (||G||_F + eps), one matrix."""
    G = to_f64(G)
    return G / (np.sqrt(np.sum(G * G)) + eps)


def ns_step(X, coeffs=MUON_COEFFS, bf16=False) -> np.ndarray:
    """One quintic step on a wide matrix X [R, C] (R <= C)."""
    a, b, c = coeffs
    r = round_bf16 if bf16 else (lambda v: v)
    A = r(X @ X.T)
    B = r(b * A + c * (A @ A))
    return r(a * X + B @ X)


def newton_schulz(G, steps=MUON_STEPS, coeffs=MUON_COEFFS, eps=MUON_EPS, bf16=False) -> np.ndarray:
    """Orthogonalise one matrix G [R, C] or a batch G [n, R, C]."""
    G = to_f64(G)
    if G.ndim == 3:
        return np.stack([newton_schulz(g, steps, coeffs, eps, bf16) for g in G])
    tall = G.shape[0] > G.shape[1]
    X = normalise(G.T if tall else G, eps)
    if bf16:
        X = round_bf16(X)
    for _ in range(steps):
        X = ns_step(X, coeffs, bf16)
    return X.T if tall else X


def ns_scalar(s, steps=MUON_STEPS, coeffs=MUON_COEFFS) -> np.ndarray:
    """The iteration on one singular value: s -> a s + b s^3 + c s^5, `steps` times."""
    a, b, c = coeffs
    s = np.asarray(s, dtype=np.float64)
    for _ in range(steps):
        s = a * s + b * s ** 3 + c * s ** 5
    return s
