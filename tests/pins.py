"""Pins of the CPU oracle to things other than itself.

Each pin takes an oracle module (the real one, or a copy with a planted
mistake) and raises AssertionError when the oracle disagrees with:
  * brute force on tiny inputs (Python loops, math.exp, sorted());
  * closed forms (two-expert softmax is a logistic function; k = 1 is argmax;
    equal logits give 1/k);
  * library routines the layer reduces to (torch's linear/silu/softmax/sort,
    scipy's expit) in float64;
  * the page's configuration table (three d x F matrices per expert).
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import scipy.special
import torch
import torch.nn.functional as Fn

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _dense_swiglu_torch(x, wg, wu, wd):
    """The dense SwiGLU FFN through torch's library ops, float64."""
    xt = torch.from_numpy(np.asarray(x, dtype=np.float64))
    h = Fn.silu(Fn.linear(xt, torch.from_numpy(wg))) * Fn.linear(xt, torch.from_numpy(wu))
    return Fn.linear(h, torch.from_numpy(wd)).numpy()


# ----------------------------------------------------------------------------
# brute force
# ----------------------------------------------------------------------------

def _brute_route(x, wr, b, k):
    T, d = x.shape
    E = wr.shape[0]
    ids, ws, ls = [], [], []
    for t in range(T):
        l = [sum(float(x[t, i]) * float(wr[e, i]) for i in range(d)) + float(b[e]) for e in range(E)]
        m = max(l)
        ex = [math.exp(v - m) for v in l]
        z = sum(ex)
        p = [v / z for v in ex]
        order = sorted(range(E), key=lambda e: (-l[e], e))[:k]
        s = sum(p[e] for e in order)
        ids.append(order)
        ws.append([p[e] / s for e in order])
        ls.append(l)
    return np.array(ls), np.array(ids), np.array(ws)


def pin_brute_force_routing(orc):
    r = _rng(1)
    T, d, E, k = 40, 7, 11, 3
    x = r.standard_normal((T, d))
    wr = r.standard_normal((E, d))
    b = r.standard_normal(E)
    l, ids, w = orc.route(x, wr, b, k)
    bl, bids, bw = _brute_route(x, wr, b, k)
    np.testing.assert_allclose(l, bl, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(ids, bids)
    np.testing.assert_allclose(w, bw, rtol=0, atol=1e-12)


def pin_brute_force_routing_ties(orc):
    # integer-valued inputs give integer logits with many exact ties
    r = _rng(2)
    T, d, E, k = 64, 3, 9, 4
    x = r.integers(-1, 2, (T, d)).astype(np.float64)
    wr = r.integers(-1, 2, (E, d)).astype(np.float64)
    b = np.zeros(E)
    l, ids, w = orc.route(x, wr, b, k)
    bl, bids, bw = _brute_route(x, wr, b, k)
    np.testing.assert_array_equal(ids, bids)
    np.testing.assert_allclose(w, bw, rtol=0, atol=1e-12)


def pin_signed_zero_is_a_tie(orc):
    l = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0], [-1.0, -0.0, 0.0]])
    ids, w = orc.select_topk(l, 2)
    np.testing.assert_array_equal(ids, [[0, 1], [0, 1], [1, 2]])
    np.testing.assert_allclose(w, 0.5, rtol=0, atol=1e-15)


def _brute_permute(ids, E):
    T, k = ids.shape
    offsets, row_token = [0], []
    slot_row = [[-1] * k for _ in range(T)]
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t][j] == e:
                    slot_row[t][j] = len(row_token)
                    row_token.append(t)
        offsets.append(len(row_token))
    return np.array(offsets), np.array(row_token, dtype=np.int64), np.array(slot_row)


def pin_brute_force_permute(orc):
    r = _rng(3)
    T, E, k = 50, 9, 4
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)])
    ids[r.random((T, k)) < 0.3] = -1               # pre-routed: some slots elsewhere
    off, rt, sr = orc.permute(ids, E)
    boff, brt, bsr = _brute_permute(ids, E)
    np.testing.assert_array_equal(off, boff)
    np.testing.assert_array_equal(rt, brt)
    np.testing.assert_array_equal(sr, bsr)


def pin_brute_force_layer(orc):
    r = _rng(4)
    T, d, E, k, F = 24, 6, 5, 2, 4
    x = r.standard_normal((T, d))
    wr = r.standard_normal((E, d))
    b = 0.5 * r.standard_normal(E)
    wg = r.standard_normal((E, F, d))
    wu = r.standard_normal((E, F, d))
    wd = r.standard_normal((E, d, F))
    out = orc.layer_forward(x, wr, b, wg, wu, wd, k)
    _, bids, bw = _brute_route(x, wr, b, k)
    y = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            e = bids[t][j]
            h = []
            for f in range(F):
                g = sum(x[t, i] * wg[e, f, i] for i in range(d))
                u = sum(x[t, i] * wu[e, f, i] for i in range(d))
                h.append(g / (1.0 + math.exp(-g)) * u)
            for i in range(d):
                y[t, i] += bw[t][j] * sum(h[f] * wd[e, i, f] for f in range(F))
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-12)


def pin_brute_force_pre_routed_layer(orc):
    r = _rng(5)
    T, d, E, k, F = 20, 5, 6, 3, 5
    ids = np.stack([r.permutation(E)[:k] for _ in range(T)])
    ids[r.random((T, k)) < 0.4] = -1
    ids[0, :] = -1                                   # a token with no local slot
    w = r.random((T, k))
    wg = r.standard_normal((E, F, d))
    wu = r.standard_normal((E, F, d))
    wd = r.standard_normal((E, d, F))
    x = r.standard_normal((T, d))
    out = orc.layer_forward(x, None, None, wg, wu, wd, k, ids=ids, weights=w)
    y = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            e = ids[t][j]
            if e < 0:
                continue
            for i in range(d):
                acc = 0.0
                for f in range(F):
                    g = sum(x[t, q] * wg[e, f, q] for q in range(d))
                    u = sum(x[t, q] * wu[e, f, q] for q in range(d))
                    acc += g / (1.0 + math.exp(-g)) * u * wd[e, i, f]
                y[t, i] += w[t][j] * acc
    np.testing.assert_allclose(out["y"], y, rtol=1e-12, atol=1e-12)
    assert np.all(out["y"][0] == 0.0)


# ----------------------------------------------------------------------------
# reductions to library routines and closed forms
# ----------------------------------------------------------------------------

def pin_logits_match_torch_linear(orc):
    r = _rng(6)
    x, wr, b = r.standard_normal((33, 20)), r.standard_normal((13, 20)), r.standard_normal(13)
    ref = Fn.linear(torch.from_numpy(x), torch.from_numpy(wr), torch.from_numpy(b)).numpy()
    np.testing.assert_allclose(orc.router_logits(x, wr, b), ref, rtol=1e-13, atol=1e-13)


def pin_silu_matches_library(orc):
    z = np.linspace(-30, 30, 2001)
    ref = z * scipy.special.expit(z)
    np.testing.assert_allclose(orc.silu(z), ref, rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(orc.silu(z), Fn.silu(torch.from_numpy(z)).numpy(), rtol=1e-13, atol=1e-300)
    assert orc.silu(np.array([0.0]))[0] == 0.0


def pin_identical_experts_give_dense_ffn(orc):
    # all experts equal and weights summing to 1 => the layer is the dense FFN
    r = _rng(7)
    T, d, E, k, F = 64, 12, 10, 3, 12                # d == F: a transposed W_d would not raise
    x = r.standard_normal((T, d))
    wr = r.standard_normal((E, d))
    wg0, wu0, wd0 = r.standard_normal((F, d)), r.standard_normal((F, d)), r.standard_normal((d, F))
    rep = lambda a: np.repeat(a[None], E, axis=0)
    out = orc.layer_forward(x, wr, None, rep(wg0), rep(wu0), rep(wd0), k)
    np.testing.assert_allclose(out["y"], _dense_swiglu_torch(x, wg0, wu0, wd0), rtol=1e-11, atol=1e-11)


def pin_single_expert_is_dense_ffn(orc):
    r = _rng(8)
    T, d, F = 30, 8, 16
    x = r.standard_normal((T, d))
    wg, wu, wd = r.standard_normal((1, F, d)), r.standard_normal((1, F, d)), r.standard_normal((1, d, F))
    out = orc.layer_forward(x, r.standard_normal((1, d)), None, wg, wu, wd, 1)
    assert np.all(out["w"] == 1.0)
    np.testing.assert_allclose(out["y"], _dense_swiglu_torch(x, wg[0], wu[0], wd[0]), rtol=1e-11, atol=1e-11)


def pin_k_equals_E_is_sorted_softmax(orc):
    r = _rng(9)
    l = r.standard_normal((50, 7))
    l[:, 3] = l[:, 1]                                 # ties, broken by index
    ids, w = orc.select_topk(l, 7)
    lt = torch.from_numpy(l)
    p = torch.softmax(lt, dim=1)
    _, order = torch.sort(lt, dim=1, descending=True, stable=True)
    np.testing.assert_array_equal(ids, order.numpy())
    np.testing.assert_allclose(w, torch.gather(p, 1, order).numpy(), rtol=1e-13, atol=1e-15)


def pin_k1_is_argmax(orc):
    r = _rng(10)
    l = np.round(r.standard_normal((200, 9)), 1)      # rounding makes ties common
    ids, w = orc.select_topk(l, 1)
    np.testing.assert_array_equal(ids[:, 0], np.argmax(l, axis=1))
    assert np.all(w == 1.0)


def pin_equal_logits_give_uniform_weights(orc):
    x = _rng(11).standard_normal((17, 5))
    l, ids, w = orc.route(x, np.zeros((12, 5)), None, 5)
    np.testing.assert_array_equal(ids, np.broadcast_to(np.arange(5), (17, 5)))
    np.testing.assert_allclose(w, 0.2, rtol=0, atol=1e-15)


def pin_two_experts_logistic(orc):
    r = _rng(12)
    l = r.standard_normal((100, 2)) * 3
    ids, w = orc.select_topk(l, 2)
    gap = np.abs(l[:, 0] - l[:, 1])
    np.testing.assert_allclose(w[:, 0], scipy.special.expit(gap), rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(ids[:, 0], np.where(l[:, 0] >= l[:, 1], 0, 1))


def pin_routing_invariants(orc):
    r = _rng(13)
    T, d, E, k = 500, 16, 37, 5
    _, ids, w = orc.route(r.standard_normal((T, d)), r.standard_normal((E, d)), r.standard_normal(E), k)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)
    assert np.all(np.diff(w, axis=1) <= 0)
    assert np.all((ids >= 0) & (ids < E))
    assert all(len(set(row)) == k for row in ids.tolist())
    off, rt, sr = orc.permute(ids, E)
    N = T * k
    assert off[0] == 0 and off[-1] == N and np.all(np.diff(off) >= 0)
    assert np.all(np.bincount(rt, minlength=T) == k)
    for e in range(E):
        seg = rt[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)
    assert np.array_equal(np.sort(sr.reshape(-1)), np.arange(N))
    t_idx = np.repeat(np.arange(T), k).reshape(T, k)
    assert np.array_equal(rt[sr], t_idx)
    seg_of_row = np.searchsorted(off, sr, side="right") - 1
    assert np.array_equal(seg_of_row, ids)


def pin_page_parameter_identity(orc):
    """The configuration table's parameter counts fix three d x F matrices per
    expert: (E - k) experts per layer are inactive for a token, and their
    parameters over all layers make up total minus active."""
    with open(os.path.join(GOLDEN, "page_config_table.json")) as f:
        g = json.load(f)
    d, F, E, k, L = g["hidden"], g["expert_hidden"], g["routed_experts"], g["top_k"], g["layers"]
    # structure of the oracle's expert: which of its three matrices matter
    r = _rng(14)
    dd, ff = 6, 5
    X = r.standard_normal((4, dd))
    mats = [r.standard_normal((ff, dd)), r.standard_normal((ff, dd)), r.standard_normal((dd, ff))]
    base = orc.expert_ffn(X, *mats)
    used = 0
    for i, m in enumerate(mats):
        pert = list(mats)
        pert[i] = m * 1.5
        if not np.allclose(orc.expert_ffn(X, *pert), base):
            used += m.size
    per_expert = used // (dd * ff) * d * F        # matrices that matter, at the page's shape
    inactive = (E - k) * per_expert * L / 1e9
    active_routed = k * per_expert * L / 1e9
    page_inactive = g["total_params_billion"] - g["active_params_billion_per_token"]
    assert abs(inactive - page_inactive) <= 2 * g["printed_precision_billion"], (inactive, page_inactive)
    assert active_routed <= g["active_params_billion_per_token"]


def pin_to_f64_reads_bf16_bits(orc):
    """uint16 inputs are bf16 bit patterns: all 65,536 against torch's conversion."""
    from pin_bits import check_bf16_bits
    check_bf16_bits(orc.to_f64)


PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
