"""Plant plausible mistakes in a fresh copy of the oracle (on the CPU) and check
that at least one pin catches each of them.  This shows the pins are strong
enough to catch a dropped term, a wrong sign or index, or a transposed operand."""
import importlib.util
import os

import numpy as np
import pytest

import oracle.moe_oracle as real
from pins import PINS


def fresh_copy():
    spec = importlib.util.spec_from_file_location("moe_oracle_copy", real.__file__)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _m_swap_gate_up(m):
    def expert_ffn(X, wg, wu, wd):
        X = m.to_f64(X)
        return (m.silu(X @ m.to_f64(wu).T) * (X @ m.to_f64(wg).T)) @ m.to_f64(wd).T
    m.expert_ffn = expert_ffn


def _m_drop_up(m):
    def expert_ffn(X, wg, wu, wd):
        X = m.to_f64(X)
        G = X @ m.to_f64(wg).T
        return (m.silu(G) * G) @ m.to_f64(wd).T
    m.expert_ffn = expert_ffn


def _m_down_not_transposed(m):
    def expert_ffn(X, wg, wu, wd):
        X = m.to_f64(X)
        H = m.silu(X @ m.to_f64(wg).T) * (X @ m.to_f64(wu).T)
        return H @ m.to_f64(wd)
    m.expert_ffn = expert_ffn


def _m_silu_sign(m):
    m.silu = lambda z: m.to_f64(z) / (1.0 + np.exp(m.to_f64(z)))


def _m_no_renorm(m):
    orig = m.select_topk
    def select_topk(logits, k):
        ids, _ = orig(logits, k)
        p = m.softmax(logits)
        return ids, np.take_along_axis(p, ids.astype(np.int64), axis=1)
    m.select_topk = select_topk


def _m_ties_higher_index(m):
    def select_topk(logits, k):
        l = m.to_f64(logits) + 0.0
        T, E = l.shape
        order = np.lexsort((-np.broadcast_to(np.arange(E), (T, E)), -l), axis=-1)
        p = np.take_along_axis(m.softmax(l), order[:, :k], axis=1)
        return order[:, :k].astype(np.int32), p / p.sum(1, keepdims=True)
    m.select_topk = select_topk


def _m_smallest_logits(m):
    orig = m.select_topk
    m.select_topk = lambda logits, k: orig(-m.to_f64(logits), k)


def _m_softmax_sign(m):
    def softmax(logits):
        l = m.to_f64(logits)
        p = np.exp(l.max(1, keepdims=True) - l)
        return p / p.sum(1, keepdims=True)
    m.softmax = softmax


def _m_drop_bias(m):
    orig = m.router_logits
    m.router_logits = lambda x, w, b=None: orig(x, w, None)


def _m_descending_rows(m):
    orig = m.permute
    def permute(ids, E):
        off, rt, sr = orig(ids, E)
        rt2, sr2 = rt.copy(), sr.copy()
        for e in range(E):
            lo, hi = off[e], off[e + 1]
            rt2[lo:hi] = rt[lo:hi][::-1]
            mask = (sr >= lo) & (sr < hi)
            sr2[mask] = lo + hi - 1 - sr[mask]
        return off, rt2, sr2
    m.permute = permute


def _m_offsets_shifted(m):
    orig = m.permute
    def permute(ids, E):
        off, rt, sr = orig(ids, E)
        off2 = off.copy()
        off2[1:-1] = off[2:]
        return off2, rt, sr
    m.permute = permute


def _m_row_token_is_slot(m):
    orig = m.permute
    def permute(ids, E):
        off, rt, sr = orig(ids, E)
        k = np.asarray(ids).shape[1]
        s = np.full(rt.shape, 0, dtype=np.int64)
        s[sr[sr >= 0]] = np.nonzero(sr.reshape(-1) >= 0)[0]
        return off, np.minimum(s, len(np.asarray(ids)) - 1).astype(np.int32), sr
    m.permute = permute


def _m_combine_unweighted(m):
    orig = m.combine
    m.combine = lambda y_perm, slot_row, w: orig(y_perm, slot_row, np.ones_like(m.to_f64(w)))


def _m_combine_first_slot_only(m):
    orig = m.combine
    def combine(y_perm, slot_row, w):
        sr = np.array(slot_row, copy=True)
        sr[:, 1:] = -1
        return orig(y_perm, sr, w)
    m.combine = combine


def _m_grouped_skip_last_expert(m):
    orig = m.grouped_ffn
    def grouped_ffn(x_perm, offsets, wg, wu, wd):
        off = np.array(offsets, copy=True)
        y = orig(x_perm, off, wg, wu, wd)
        y[off[-2]:off[-1]] = 0.0
        return y
    m.grouped_ffn = grouped_ffn


def _m_bf16_bits_misread(m):
    def to_f64(a):
        a = np.asarray(a)
        if a.dtype == np.uint16:                  # read as IEEE half instead of bf16
            return a.view(np.float16).astype(np.float64)
        return a.astype(np.float64)
    m.to_f64 = to_f64


MUTATIONS = [v for k, v in sorted(globals().items()) if k.startswith("_m_")]


@pytest.mark.parametrize("mutate", MUTATIONS, ids=[f.__name__[3:] for f in MUTATIONS])
def test_some_pin_catches_planted_mistake(mutate):
    m = fresh_copy()
    mutate(m)
    caught = []
    for pin in PINS:
        try:
            pin(m)
        except Exception:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutation {mutate.__name__}"


def test_unmutated_copy_passes_every_pin():
    m = fresh_copy()
    for pin in PINS:
        pin(m)
