"""The whole-layer backward oracle against torch.autograd, finite differences,
adjoint identities and closed forms (no GPU needed); plus planted mistakes
that the pins must catch."""
import importlib.util

import numpy as np
import pytest

import oracle.moe_layer_backward_oracle as real
from pins_layer_backward import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_layer_backward_oracle_pin(pin):
    pin(real)


def fresh_copy():
    spec = importlib.util.spec_from_file_location("oracle.moe_layer_backward_oracle_copy", real.__file__)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _m_jacobian_drops_outer_term(m):
    m.gate_weights_backward = lambda w, g: m.to_f64(w) * m.to_f64(g)


def _m_jacobian_sign(m):
    orig = m.gate_weights_backward
    m.gate_weights_backward = lambda w, g: -orig(w, g)


def _m_dy_perm_unweighted(m):
    orig = m.combine_backward

    def combine_backward(dy, y_perm, slot_row, weights):
        _, g = orig(dy, y_perm, slot_row, weights)
        dy_perm, _ = orig(dy, y_perm, slot_row, np.ones_like(m.to_f64(weights)))
        return dy_perm, g
    m.combine_backward = combine_backward


def _m_g_from_weighted_rows(m):
    orig = m.combine_backward

    def combine_backward(dy, y_perm, slot_row, weights):
        dy_perm, g = orig(dy, y_perm, slot_row, weights)
        return dy_perm, g * m.to_f64(weights)
    m.combine_backward = combine_backward


def _m_router_dx_dropped(m):
    orig = m.router_backward

    def router_backward(x, w_router, dlogits):
        dx, dwr, db = orig(x, w_router, dlogits)
        return np.zeros_like(dx), dwr, db
    m.router_backward = router_backward


def _m_permute_backward_drops_repeats(m):
    def permute_backward(dx_perm, row_token, num_tokens):
        dx = np.zeros((num_tokens, np.asarray(dx_perm).shape[1]))
        dx[np.asarray(row_token, dtype=np.int64)] = m.to_f64(dx_perm)
        return dx
    m.permute_backward = permute_backward


def _m_bias_grad_mean(m):
    orig = m.router_backward

    def router_backward(x, w_router, dlogits):
        dx, dwr, db = orig(x, w_router, dlogits)
        return dx, dwr, db / np.asarray(dlogits).shape[0]
    m.router_backward = router_backward


def _m_scatter_wrong_slot(m):
    orig = m.scatter_logit_grad

    def scatter_logit_grad(ids, dl_sel, num_experts):
        return orig(ids, np.roll(m.to_f64(dl_sel), 1, axis=1), num_experts)
    m.scatter_logit_grad = scatter_logit_grad


MUTATIONS = [_m_jacobian_drops_outer_term, _m_jacobian_sign, _m_dy_perm_unweighted, _m_g_from_weighted_rows,
             _m_router_dx_dropped, _m_permute_backward_drops_repeats, _m_bias_grad_mean, _m_scatter_wrong_slot]


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
