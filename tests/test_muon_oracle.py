"""The Newton-Schulz oracle against closed forms, invariances, brute force and
torch's bfloat16 rounding (no GPU needed); plus planted mistakes that the pins
must catch."""
import importlib.util

import numpy as np
import pytest

import oracle.muon_oracle as real
from pins_muon import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_muon_oracle_pin(pin):
    pin(real)


def fresh_copy():
    spec = importlib.util.spec_from_file_location("muon_oracle_copy", real.__file__)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _m_b_sign(m):
    a, b, c = m.MUON_COEFFS
    m.MUON_COEFFS = (a, -b, c)
    m.newton_schulz.__defaults__ = (m.MUON_STEPS, m.MUON_COEFFS, m.MUON_EPS, False)
    m.ns_step.__defaults__ = (m.MUON_COEFFS, False)


def _m_gram_wrong_side(m):
    def ns_step(X, coeffs=m.MUON_COEFFS, bf16=False):
        a, b, c = coeffs
        A = X.T @ X
        B = b * A + c * (A @ A)
        return a * X + X @ B
    m.ns_step = ns_step


def _m_no_normalise(m):
    m.normalise = lambda G, eps=m.MUON_EPS: m.to_f64(G)


def _m_tall_not_transposed(m):
    orig = m.newton_schulz

    def newton_schulz(G, steps=m.MUON_STEPS, coeffs=m.MUON_COEFFS, eps=m.MUON_EPS, bf16=False):
        G = m.to_f64(G)
        if G.ndim == 3:
            return np.stack([newton_schulz(g, steps, coeffs, eps, bf16) for g in G])
        X = m.normalise(G, eps)
        for _ in range(steps):
            X = m.ns_step(X, coeffs, bf16)
        return X
    m.newton_schulz = newton_schulz


def _m_cubic_term_dropped(m):
    def ns_step(X, coeffs=m.MUON_COEFFS, bf16=False):
        a, b, c = coeffs
        A = X @ X.T
        return a * X + c * (A @ A) @ X
    m.ns_step = ns_step


def _m_round_toward_zero(m):
    def round_bf16(a):
        f = np.asarray(a, dtype=np.float64).astype(np.float32)
        u = f.view(np.uint32) & np.uint32(0xFFFF0000)
        return u.view(np.float32).astype(np.float64)
    m.round_bf16 = round_bf16


def _m_one_step_short(m):
    orig = m.newton_schulz

    def newton_schulz(G, steps=m.MUON_STEPS, coeffs=m.MUON_COEFFS, eps=m.MUON_EPS, bf16=False):
        return orig(G, max(steps - 1, 0), coeffs, eps, bf16)
    m.newton_schulz = newton_schulz


MUTATIONS = [_m_b_sign, _m_gram_wrong_side, _m_no_normalise, _m_tall_not_transposed, _m_cubic_term_dropped,
             _m_round_toward_zero, _m_one_step_short]


@pytest.mark.parametrize("mut", MUTATIONS, ids=[f.__name__ for f in MUTATIONS])
def test_pins_catch_planted_mistake(mut):
    m = fresh_copy()
    mut(m)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(m)
        except (AssertionError, np.linalg.LinAlgError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mut.__name__}"
