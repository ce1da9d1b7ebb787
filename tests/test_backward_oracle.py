"""The expert-FFN backward oracle against torch.autograd, finite differences and
closed forms (no GPU needed); plus planted mistakes that the pins must catch."""
import importlib.util

import numpy as np
import pytest

import oracle.moe_backward_oracle as real
from pins_backward import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_backward_oracle_pin(pin):
    pin(real)


def fresh_copy():
    spec = importlib.util.spec_from_file_location("moe_backward_oracle_copy", real.__file__)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _m_silu_grad_missing_term(m):
    m.silu_grad = lambda z: m.sigmoid(z)


def _m_dwd_uses_silu_not_h(m):
    # dW_d from silu(G) instead of H = silu(G) * U
    def expert_ffn_backward(X, Wg, Wu, Wd, dY):
        X, dY = m.to_f64(X), m.to_f64(dY)
        Wg, Wu, Wd = m.to_f64(Wg), m.to_f64(Wu), m.to_f64(Wd)
        G = X @ Wg.T
        U = X @ Wu.T
        S = G * m.sigmoid(G)
        dH = dY @ Wd
        dU = dH * S
        dG = dH * U * m.silu_grad(G)
        return dG @ Wg + dU @ Wu, dG.T @ X, dU.T @ X, dY.T @ S
    m.expert_ffn_backward = expert_ffn_backward


def _m_swap_gate_up_grads(m):
    orig = m.expert_ffn_backward

    def expert_ffn_backward(X, Wg, Wu, Wd, dY):
        dX, dWg, dWu, dWd = orig(X, Wg, Wu, Wd, dY)
        return dX, dWu, dWg, dWd
    m.expert_ffn_backward = expert_ffn_backward


def _m_dx_drops_up_path(m):
    def expert_ffn_backward(X, Wg, Wu, Wd, dY):
        X, dY = m.to_f64(X), m.to_f64(dY)
        Wg, Wu, Wd = m.to_f64(Wg), m.to_f64(Wu), m.to_f64(Wd)
        G = X @ Wg.T
        U = X @ Wu.T
        S = G * m.sigmoid(G)
        H = S * U
        dH = dY @ Wd
        dU = dH * S
        dG = dH * U * m.silu_grad(G)
        return dG @ Wg, dG.T @ X, dU.T @ X, dY.T @ H
    m.expert_ffn_backward = expert_ffn_backward


def _m_grouped_off_by_one(m):
    orig = m.expert_ffn_backward

    def grouped_ffn_backward(x_perm, offsets, w_gate, w_up, w_down, dy_perm):
        offsets = np.asarray(offsets, dtype=np.int64)
        E = offsets.size - 1
        n = int(offsets[-1])
        x_perm = np.asarray(x_perm)
        d = x_perm.shape[1]
        F = np.asarray(w_gate[0]).shape[0]
        dx = np.zeros((n, d)); dwg = np.zeros((E, F, d)); dwu = np.zeros((E, F, d)); dwd = np.zeros((E, d, F))
        for e in range(E):
            lo, hi = int(offsets[e]), int(offsets[e + 1])
            if hi > lo:
                w = (e + 1) % E
                dx[lo:hi], dwg[e], dwu[e], dwd[e] = orig(x_perm[lo:hi], w_gate[w], w_up[w], w_down[w],
                                                         np.asarray(dy_perm)[lo:hi])
        return dx, dwg, dwu, dwd
    m.grouped_ffn_backward = grouped_ffn_backward


MUTATIONS = [_m_silu_grad_missing_term, _m_dwd_uses_silu_not_h, _m_swap_gate_up_grads, _m_dx_drops_up_path,
             _m_grouped_off_by_one]


@pytest.mark.parametrize("mut", MUTATIONS, ids=[f.__name__ for f in MUTATIONS])
def test_pins_catch_planted_mistake(mut):
    m = fresh_copy()
    mut(m)
    caught = []
    for pin in PINS:
        try:
            pin(m)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mut.__name__}"
