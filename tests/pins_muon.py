"""Pins of the Newton-Schulz oracle to things other than itself.

Each pin takes an oracle module (the real one, or a copy with a planted
mistake) and raises AssertionError when it disagrees with:
  * the closed form on singular values: for G = U diag(s) V^T the iteration
    returns U diag(q(s / ||s||_2)) V^T, q = five applications of the scalar
    polynomial s -> a s + b s^3 + c s^5 (evaluated here with Horner's rule,
    independently of the oracle's helper);
  * invariances: orthogonal factors on either side pass through; a tall matrix
    gives the transpose of its wide transpose; a positive scale drops out;
  * brute force with Python loops on a tiny matrix;
  * torch's own bfloat16 rounding at the storage points of the bf16 reading.
"""
from __future__ import annotations

import numpy as np
import torch

A_, B_, C_ = 3.4445, -4.7750, 2.0315


def _rng(seed):
    return np.random.default_rng(seed)


def _orthonormal(r, n, k):
    q, _ = np.linalg.qr(r.standard_normal((n, k)))
    return q


def _q(s, steps=5):
    s = np.asarray(s, dtype=np.float64)
    for _ in range(steps):
        s2 = s * s
        s = s * (A_ + s2 * (B_ + s2 * C_))
    return s


def pin_ns_closed_form_on_singular_values(orc):
    r = _rng(11)
    R, C = 24, 40
    U = _orthonormal(r, R, R)
    V = _orthonormal(r, C, R)
    s = np.sort(r.uniform(0.02, 3.0, R))[::-1]
    G = U @ np.diag(s) @ V.T
    want = U @ np.diag(_q(s / np.linalg.norm(s))) @ V.T
    got = orc.newton_schulz(G, eps=0.0)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-10)


def pin_ns_singular_value_band(orc):
    # five quintic steps put every singular value of a well-spread spectrum in
    # the band the polynomial oscillates in (about 0.68 .. 1.13)
    r = _rng(12)
    G = r.standard_normal((64, 160))
    s = np.linalg.svd(orc.newton_schulz(G), compute_uv=False)
    assert 0.6 < s.min() and s.max() < 1.2, (s.min(), s.max())


def pin_ns_orthogonal_invariance(orc):
    r = _rng(13)
    R, C = 16, 28
    G = r.standard_normal((R, C))
    Q1 = _orthonormal(r, R, R)
    Q2 = _orthonormal(r, C, C)
    np.testing.assert_allclose(orc.newton_schulz(Q1 @ G @ Q2), Q1 @ orc.newton_schulz(G) @ Q2, rtol=0,
                               atol=1e-10)


def pin_ns_tall_is_transposed_wide(orc):
    r = _rng(14)
    G = r.standard_normal((20, 36))
    np.testing.assert_allclose(orc.newton_schulz(G.T), orc.newton_schulz(G).T, rtol=0, atol=1e-12)
    # and a tall input is really worked on as its wide transpose: the result's
    # singular vectors are G's (column space of G^T for the tall case)
    X = orc.newton_schulz(G.T)
    assert X.shape == (36, 20)


def pin_ns_scale_drops_out(orc):
    r = _rng(15)
    G = r.standard_normal((12, 30))
    np.testing.assert_allclose(orc.newton_schulz(7.5 * G, eps=0.0), orc.newton_schulz(G, eps=0.0), rtol=0,
                               atol=1e-10)


def pin_ns_brute_force_tiny(orc):
    r = _rng(16)
    R, C, steps, eps = 3, 5, 2, 1e-7
    G = r.standard_normal((R, C))
    nrm = sum(float(G[i, j]) ** 2 for i in range(R) for j in range(C)) ** 0.5
    X = [[float(G[i, j]) / (nrm + eps) for j in range(C)] for i in range(R)]
    for _ in range(steps):
        A = [[sum(X[i][k] * X[j][k] for k in range(C)) for j in range(R)] for i in range(R)]
        AA = [[sum(A[i][k] * A[k][j] for k in range(R)) for j in range(R)] for i in range(R)]
        B = [[B_ * A[i][j] + C_ * AA[i][j] for j in range(R)] for i in range(R)]
        BX = [[sum(B[i][k] * X[k][j] for k in range(R)) for j in range(C)] for i in range(R)]
        X = [[A_ * X[i][j] + BX[i][j] for j in range(C)] for i in range(R)]
    np.testing.assert_allclose(orc.newton_schulz(G, steps=steps, eps=eps), np.array(X), rtol=0, atol=1e-12)


def pin_ns_bf16_rounding_points(orc):
    # the bf16 reading against the same steps written with torch's bfloat16
    # rounding (float64 products, rounded through float32 like the oracle says)
    r = _rng(17)
    G = r.standard_normal((8, 24))

    def rb(v):
        return torch.from_numpy(np.asarray(v, dtype=np.float64).astype(np.float32)).bfloat16().double().numpy()

    X = rb(G / (np.linalg.norm(G) + 1e-7))
    for _ in range(3):
        A = rb(X @ X.T)
        B = rb(B_ * A + C_ * (A @ A))
        X = rb(A_ * X + B @ X)
    np.testing.assert_array_equal(orc.newton_schulz(G, steps=3, bf16=True), X)


def pin_ns_batch_is_per_matrix(orc):
    r = _rng(18)
    G = r.standard_normal((3, 6, 10))
    got = orc.newton_schulz(G)
    for i in range(3):
        np.testing.assert_array_equal(got[i], orc.newton_schulz(G[i]))


def pin_to_f64_reads_bf16_bits(orc):
    """uint16 inputs are bf16 bit patterns: all 65,536 against torch's conversion."""
    from pin_bits import check_bf16_bits
    check_bf16_bits(orc.to_f64)


PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
