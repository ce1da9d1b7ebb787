"""Pins of the whole-layer backward oracle to things other than itself.

Each pin takes an oracle module (the real one, or a copy with a planted
mistake) and raises AssertionError when it disagrees with:
  * torch.autograd through an independent float64 forward written per token
    (torch's linear, softmax, topk and silu; no permutation), with and without
    a router bias, and with pre-routed slots (negative ids, leaf gate weights);
  * central finite differences of a numpy forward on a tiny layer whose top-k
    selection is far from any tie;
  * adjoint (dot-product) identities of the linear steps: combine, permutation,
    router GEMM;
  * closed forms of the renormalised gate weights' gradient: it sums to zero
    over a token's slots, vanishes for k = 1 and for a constant upstream
    gradient, and for k = E equals the full softmax's (torch.autograd).
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as Fn

from oracle import moe_oracle as fwd


def _rng(seed):
    return np.random.default_rng(seed)


def _layer_inputs(r, T, d, E, F, bias=True):
    x = r.standard_normal((T, d))
    Wr = r.standard_normal((E, d)) / np.sqrt(d)
    b = r.standard_normal(E) * 0.3 if bias else np.zeros(E)
    Wg = r.standard_normal((E, F, d)) / np.sqrt(d)
    Wu = r.standard_normal((E, F, d)) / np.sqrt(d)
    Wd = r.standard_normal((E, d, F)) / np.sqrt(F)
    dy = r.standard_normal((T, d))
    return x, Wr, b, Wg, Wu, Wd, dy


def _torch_layer(x, Wr, b, Wg, Wu, Wd, k):
    """Per-token float64 forward: y[t] = sum_j w[t,j] FFN_{S_tj}(x[t])."""
    l = Fn.linear(x, Wr, b)
    p = torch.softmax(l, dim=1)
    idx = torch.topk(l, k, dim=1).indices
    ps = torch.gather(p, 1, idx)
    w = ps / ps.sum(dim=1, keepdim=True)
    rows = []
    for t in range(x.shape[0]):
        acc = torch.zeros(x.shape[1], dtype=x.dtype)
        for j in range(k):
            e = int(idx[t, j])
            h = Fn.silu(Fn.linear(x[t], Wg[e])) * Fn.linear(x[t], Wu[e])
            acc = acc + w[t, j] * Fn.linear(h, Wd[e])
        rows.append(acc)
    return torch.stack(rows), idx, w


def _y_perm(x, ids, Wg, Wu, Wd):
    E = Wg.shape[0]
    offsets, row_token, _ = fwd.permute(ids, E)
    return fwd.grouped_ffn(fwd.gather_rows(x, row_token), offsets, Wg, Wu, Wd)


def _check_against_autograd(orc, T, d, E, k, F, seed, bias):
    r = _rng(seed)
    x, Wr, b, Wg, Wu, Wd, dy = _layer_inputs(r, T, d, E, F, bias)
    t = [torch.tensor(a, requires_grad=True) for a in (x, Wr, b, Wg, Wu, Wd)]
    y, idx, w = _torch_layer(*t, k)
    y.backward(torch.from_numpy(dy))
    ids = idx.numpy().astype(np.int32)
    wn = w.detach().numpy()
    got = orc.layer_backward(x, Wr, Wg, Wu, Wd, ids, wn, _y_perm(x, ids, Wg, Wu, Wd), dy)
    for name, ref in (("dx", t[0]), ("dw_router", t[1]), ("dbias", t[2]), ("dw_gate", t[3]),
                      ("dw_up", t[4]), ("dw_down", t[5])):
        np.testing.assert_allclose(got[name], ref.grad.numpy(), rtol=0, atol=1e-11, err_msg=name)


def pin_layer_backward_matches_torch_autograd(orc):
    _check_against_autograd(orc, T=11, d=7, E=6, k=3, F=5, seed=31, bias=True)
    _check_against_autograd(orc, T=9, d=5, E=4, k=2, F=3, seed=32, bias=False)


def pin_pre_routed_backward_matches_torch_autograd(orc):
    # slots with a negative id are skipped; gate weights are leaves, so their
    # gradient is g, and no router gradient is taken
    r = _rng(33)
    T, d, E, k, F = 7, 5, 4, 3, 3
    x, _, _, Wg, Wu, Wd, dy = _layer_inputs(r, T, d, E, F)
    ids = np.full((T, k), -1, dtype=np.int32)
    for t in range(T):
        m = int(r.integers(0, k + 1))
        ids[t, :m] = np.sort(r.choice(E, size=m, replace=False))
    wv = r.uniform(0.1, 1.0, (T, k))
    tx, tg, tu, td, tw = [torch.tensor(a, requires_grad=True) for a in (x, Wg, Wu, Wd, wv)]
    rows = []
    for t in range(T):
        acc = torch.zeros(d, dtype=torch.float64)
        for j in range(k):
            e = int(ids[t, j])
            if e >= 0:
                h = Fn.silu(Fn.linear(tx[t], tg[e])) * Fn.linear(tx[t], tu[e])
                acc = acc + tw[t, j] * Fn.linear(h, td[e])
        rows.append(acc)
    torch.stack(rows).backward(torch.from_numpy(dy))
    got = orc.layer_backward(x, None, Wg, Wu, Wd, ids, wv, _y_perm(x, ids, Wg, Wu, Wd), dy)
    np.testing.assert_allclose(got["dx"], tx.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(got["dw_gate"], tg.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(got["dw_up"], tu.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(got["dw_down"], td.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(got["g"], tw.grad.numpy(), rtol=0, atol=1e-11)
    assert got["dw_router"] is None


def _np_layer(x, Wr, b, Wg, Wu, Wd, k):
    l = x @ Wr.T + b
    out = np.zeros_like(x)
    for t in range(x.shape[0]):
        order = sorted(range(Wr.shape[0]), key=lambda e: (-l[t, e], e))[:k]
        z = np.exp(l[t, order] - l[t, order].max())
        w = z / z.sum()
        for j, e in enumerate(order):
            G = Wg[e] @ x[t]
            h = G / (1 + np.exp(-G)) * (Wu[e] @ x[t])
            out[t] += w[j] * (Wd[e] @ h)
    return out


def pin_layer_backward_finite_differences(orc):
    r = _rng(34)
    T, d, E, k, F = 3, 3, 4, 2, 2
    x, Wr, b, Wg, Wu, Wd, dy = _layer_inputs(r, T, d, E, F)
    l = np.sort(x @ Wr.T + b, axis=1)[:, ::-1]
    assert (l[:, k - 1] - l[:, k]).min() > 1e-3          # no selection change within h
    ids, w = fwd.select_topk(x @ Wr.T + b, k)
    got = orc.layer_backward(x, Wr, Wg, Wu, Wd, ids, w, _y_perm(x, ids, Wg, Wu, Wd), dy)
    h = 1e-6
    params = [x, Wr, b, Wg, Wu, Wd]
    for idx, name in enumerate(("dx", "dw_router", "dbias", "dw_gate", "dw_up", "dw_down")):
        A = params[idx]
        num = np.zeros_like(A)
        for i in np.ndindex(A.shape):
            pp = [a.copy() for a in params]
            pm = [a.copy() for a in params]
            pp[idx][i] += h
            pm[idx][i] -= h
            num[i] = np.sum(dy * (_np_layer(*pp, k) - _np_layer(*pm, k))) / (2 * h)
        np.testing.assert_allclose(got[name], num, rtol=0, atol=1e-7, err_msg=name)


def pin_adjoint_identities(orc):
    r = _rng(35)
    T, d, E, k = 10, 6, 5, 3
    ids = np.stack([r.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    ids[2, 1] = -1
    offsets, row_token, slot_row = fwd.permute(ids, E)
    N = int(offsets[-1])
    w = r.uniform(0.1, 1.0, (T, k))
    y_perm = r.standard_normal((N, d))
    dy = r.standard_normal((T, d))
    # combine is bilinear in (w, y_perm): <y, dy> = <y_perm, dy_perm> = sum w g
    y = fwd.combine(y_perm, slot_row, w)
    dy_perm, g = orc.combine_backward(dy, y_perm, slot_row, w)
    assert abs(np.sum(y * dy) - np.sum(y_perm * dy_perm)) < 1e-11
    assert abs(np.sum(y * dy) - np.sum(w * g)) < 1e-11
    assert g[2, 1] == 0.0
    # permutation: <gather(x), dx_perm> = <x, permute_backward(dx_perm)>
    x = r.standard_normal((T, d))
    dx_perm = r.standard_normal((N, d))
    lhs = np.sum(fwd.gather_rows(x, row_token) * dx_perm)
    assert abs(lhs - np.sum(x * orc.permute_backward(dx_perm, row_token, T))) < 1e-11
    # router GEMM: <x W_r^T + b, dl> = <x, dx> + <W_r, dW_r> - <x W_r^T, dl> + <b, db>
    Wr = r.standard_normal((E, d))
    b = r.standard_normal(E)
    dl = r.standard_normal((T, E))
    dx, dwr, db = orc.router_backward(x, Wr, dl)
    assert abs(np.sum((x @ Wr.T) * dl) - np.sum(x * dx)) < 1e-11
    assert abs(np.sum((x @ Wr.T) * dl) - np.sum(Wr * dwr)) < 1e-11
    assert abs(np.sum(b[None, :] * dl) - np.sum(b * db)) < 1e-11


def pin_gate_weight_grad_closed_forms(orc):
    r = _rng(36)
    T, k = 12, 4
    z = r.standard_normal((T, k))
    w = np.exp(z) / np.exp(z).sum(axis=1, keepdims=True)
    g = r.standard_normal((T, k))
    dl = orc.gate_weights_backward(w, g)
    np.testing.assert_allclose(dl.sum(axis=1), 0.0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(orc.gate_weights_backward(w, np.repeat(g[:, :1], k, axis=1)), 0.0, rtol=0,
                               atol=1e-15)
    assert not orc.gate_weights_backward(np.ones((T, 1)), g[:, :1]).any()
    # k = E: the renormalised weights are the full softmax
    zt = torch.tensor(z, requires_grad=True)
    torch.softmax(zt, dim=1).backward(torch.from_numpy(g))
    np.testing.assert_allclose(dl, zt.grad.numpy(), rtol=0, atol=1e-14)
    # dense scatter puts each token's k values at its experts and nothing else
    ids = np.stack([r.choice(9, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    D = orc.scatter_logit_grad(ids, dl, 9)
    for t in range(T):
        for e in range(9):
            want = dl[t, list(ids[t]).index(e)] if e in ids[t] else 0.0
            assert D[t, e] == want


PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
