"""Pins of the expert-FFN backward oracle to things other than itself.

Each pin takes an oracle module (the real one, or a copy with a planted
mistake) and raises AssertionError when it disagrees with:
  * torch.autograd differentiating the SwiGLU expert (torch's linear and silu)
    in float64;
  * central finite differences of the forward on a tiny expert;
  * the closed-form derivative of silu, and its value at 0;
  * the grouped form being the per-expert form on each segment, with empty
    experts getting zero weight gradients.
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as Fn


def _rng(seed):
    return np.random.default_rng(seed)


def _expert(r, n, d, F):
    X = r.standard_normal((n, d))
    Wg = r.standard_normal((F, d)) / np.sqrt(d)
    Wu = r.standard_normal((F, d)) / np.sqrt(d)
    Wd = r.standard_normal((d, F)) / np.sqrt(F)
    dY = r.standard_normal((n, d))
    return X, Wg, Wu, Wd, dY


def _fwd(X, Wg, Wu, Wd):
    return ((X @ Wg.T) / (1 + np.exp(-(X @ Wg.T))) * (X @ Wu.T)) @ Wd.T


def pin_backward_matches_torch_autograd(orc):
    r = _rng(21)
    X, Wg, Wu, Wd, dY = _expert(r, 13, 10, 7)
    t = [torch.tensor(a, requires_grad=True) for a in (X, Wg, Wu, Wd)]
    Y = Fn.linear(Fn.silu(Fn.linear(t[0], t[1])) * Fn.linear(t[0], t[2]), t[3])
    Y.backward(torch.from_numpy(dY))
    got = orc.expert_ffn_backward(X, Wg, Wu, Wd, dY)
    for g, ref in zip(got, (t[0].grad, t[1].grad, t[2].grad, t[3].grad)):
        np.testing.assert_allclose(g, ref.numpy(), rtol=0, atol=1e-12)


def pin_backward_finite_differences(orc):
    r = _rng(22)
    X, Wg, Wu, Wd, dY = _expert(r, 3, 4, 2)
    got = orc.expert_ffn_backward(X, Wg, Wu, Wd, dY)
    h = 1e-6
    for idx, (name, A) in enumerate((("X", X), ("Wg", Wg), ("Wu", Wu), ("Wd", Wd))):
        num = np.zeros_like(A)
        for i in np.ndindex(A.shape):
            args_p = [X.copy(), Wg.copy(), Wu.copy(), Wd.copy()]
            args_m = [X.copy(), Wg.copy(), Wu.copy(), Wd.copy()]
            args_p[idx][i] += h
            args_m[idx][i] -= h
            num[i] = np.sum(dY * (_fwd(*args_p) - _fwd(*args_m))) / (2 * h)
        np.testing.assert_allclose(got[idx], num, rtol=0, atol=1e-7, err_msg=name)


def pin_silu_grad_closed_form(orc):
    z = np.linspace(-12, 12, 97)
    s = 1 / (1 + np.exp(-z))
    np.testing.assert_allclose(orc.silu_grad(z), s + z * s * (1 - s), rtol=0, atol=1e-14)
    assert abs(orc.silu_grad(np.array([0.0]))[0] - 0.5) < 1e-15
    # the derivative of torch's silu, elementwise
    zt = torch.tensor(z, requires_grad=True)
    Fn.silu(zt).sum().backward()
    np.testing.assert_allclose(orc.silu_grad(z), zt.grad.numpy(), rtol=0, atol=1e-14)


def pin_grouped_backward_is_per_expert(orc):
    r = _rng(23)
    d, F = 6, 5
    counts = [3, 0, 4, 1]
    off = np.concatenate([[0], np.cumsum(counts)])
    E = len(counts)
    X = r.standard_normal((off[-1], d))
    dY = r.standard_normal((off[-1], d))
    Wg = r.standard_normal((E, F, d))
    Wu = r.standard_normal((E, F, d))
    Wd = r.standard_normal((E, d, F))
    dx, dwg, dwu, dwd = orc.grouped_ffn_backward(X, off, Wg, Wu, Wd, dY)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            assert not dwg[e].any() and not dwu[e].any() and not dwd[e].any()
            continue
        t = [torch.tensor(a, requires_grad=True) for a in (X[lo:hi], Wg[e], Wu[e], Wd[e])]
        Y = Fn.linear(Fn.silu(Fn.linear(t[0], t[1])) * Fn.linear(t[0], t[2]), t[3])
        Y.backward(torch.from_numpy(dY[lo:hi]))
        np.testing.assert_allclose(dx[lo:hi], t[0].grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dwg[e], t[1].grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dwu[e], t[2].grad.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(dwd[e], t[3].grad.numpy(), rtol=0, atol=1e-12)


def pin_to_f64_reads_bf16_bits(orc):
    """uint16 inputs are bf16 bit patterns: all 65,536 against torch's conversion."""
    from pin_bits import check_bf16_bits
    check_bf16_bits(orc.to_f64)


PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
