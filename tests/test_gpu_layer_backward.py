"""The layer backward on the GPU (moe_layer_backward, moe_combine_backward,
moe_route_backward) against the float64 oracle in
oracle/moe_layer_backward_oracle.py.

Inputs are given to both sides and none comes from the GPU: x and the weights
from the seeded workload generator; the routing (ids, gate weights) from the
oracle's router on those inputs (small layers) or from the generator's seeded
routing table (page shape); y_perm from the oracle's forward rounded to the
layer's dtype (small layers) or seeded noise; dy seeded.

Tolerances (from the arithmetic):
  * float32 layers: max |g - o| <= 1e-5 max |o| for every output (float32
    arithmetic throughout, float32 MFMA products);
  * bf16 layers, outputs that pass through bf16 products or bf16 roundings (dx,
    the weight gradients; dW_r uses dl rounded to bf16): the forward's bf16
    rule relative to each output's scale, |g - o| <= 1e-2 max|o| + 2e-2 |o|
    and max |g - o| <= 1e-2 max |o|;
  * d_topk_w, the logit gradient and db are float32 sums of exact products of
    bf16 inputs: max |g - o| <= 1e-4 max |o|;
  * dy_perm = topk_w * dy rounded once to bf16: |g - o| <= 2^-8 |o| (half an ulp,
    plus the float32 product's own rounding).
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_16_amd import binding as B
from mixture_experts_layer_16_amd import workloads as W
from oracle import moe_layer_backward_oracle as lbo
from oracle import moe_oracle as fwd

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def close_bf16(g, o, what):
    m = np.abs(o).max()
    d = np.abs(g - o)
    assert (d <= 1e-2 * m + 2e-2 * np.abs(o)).all(), (what, d.max(), m)
    assert d.max() <= 1e-2 * m, (what, d.max(), m)


def close_rel(g, o, tol, what):
    m = np.abs(o).max()
    assert np.abs(g - o).max() <= tol * m, (what, np.abs(g - o).max(), m)


def small_layer(T, d, E, k, F, dtype, seed, bias=False):
    wl = W.Workload(f"t{T}_d{d}_E{E}_k{k}_F{F}", T, d, E, k, F, dtype, routing="router_bias" if bias else "router",
                    seed=seed)
    inp = W.make_inputs(wl, device=DEV)
    X, Wr = f64(inp["x"]), f64(inp["w_router"])
    b = f64(inp["bias"]) if bias else None
    Wg, Wu, Wd = f64(inp["w_gate"]), f64(inp["w_up"]), f64(inp["w_down"])
    _, ids, w = fwd.route(X, Wr, b, k)
    w32 = w.astype(np.float32)
    off, rt, _ = fwd.permute(ids, E)
    y_perm = fwd.grouped_ffn(fwd.gather_rows(X, rt), off, Wg, Wu, Wd)
    y_perm_t = torch.from_numpy(y_perm).to(DEV).to(dtype)
    dy = W.output_grad(T, d, dtype, DEV, seed)
    gpu = dict(inp=inp, ids=torch.from_numpy(ids).to(DEV), w=torch.from_numpy(w32).to(DEV), y_perm=y_perm_t, dy=dy)
    ref = lbo.layer_backward(X, Wr, Wg, Wu, Wd, ids, w32, f64(y_perm_t), f64(dy))
    return gpu, ref


def run_layer(gpu, routed=True):
    inp = gpu["inp"]
    return B.moe_layer_backward(inp["x"], inp["w_router"] if routed else None, inp["w_gate"], inp["w_up"],
                                inp["w_down"], gpu["ids"], gpu["w"], gpu["y_perm"], gpu["dy"], want_bias=routed,
                                want_d_topk_w=True)


def check_layer(L, ref, dtype, routed=True):
    if dtype == torch.float32:
        close = lambda g, o, what: close_rel(g, o, 1e-5, what)   # noqa: E731
        exact = close
    else:
        close = close_bf16
        exact = lambda g, o, what: close_rel(g, o, 1e-4, what)   # noqa: E731
    exact(f64(L.d_topk_w), ref["g"], "d_topk_w")
    close(f64(L.dx), ref["dx"], "dx")
    E = ref["dw_gate"].shape[0]
    counts = np.diff(ref["offsets"].astype(np.int64))
    for e in range(E):
        for got, want, nm in ((L.dw_gate, ref["dw_gate"], "dW_gate"), (L.dw_up, ref["dw_up"], "dW_up"),
                              (L.dw_down, ref["dw_down"], "dW_down")):
            if counts[e] == 0:
                assert not got[e].any(), (nm, e)
            else:
                close(f64(got[e]), want[e], f"{nm}[{e}]")
    if routed:
        close(f64(L.dw_router), ref["dw_router"], "dW_router")
        exact(f64(L.dbias), ref["dbias"], "dbias")
    else:
        assert L.dw_router is None and L.dbias is None


LAYERS = [
    # (T, d, E, k, F, dtype, seed, bias)
    (256, 128, 16, 2, 64, torch.float32, 0, False),      # the tiny fp32 layer
    (4096, 1024, 64, 8, 512, torch.bfloat16, 0, False),  # the small bf16 layer
    (100, 64, 5, 2, 64, torch.bfloat16, 1, True),        # ragged T, router bias
    (70, 128, 7, 3, 128, torch.bfloat16, 2, False),      # k without a specialised kernel
    (130, 192, 9, 3, 64, torch.float32, 3, True),
]


@pytest.mark.parametrize("T,d,E,k,F,dtype,seed,bias", LAYERS)
def test_layer_backward_matches_oracle(T, d, E, k, F, dtype, seed, bias):
    print(f"[lbwd] T={T} d={d} E={E} k={k} F={F} {dtype}", flush=True)
    gpu, ref = small_layer(T, d, E, k, F, dtype, seed, bias)
    L = run_layer(gpu)
    torch.cuda.synchronize()
    check_layer(L, ref, dtype)


def test_layer_backward_pre_routed():
    # one expert-parallel rank's share: negative ids are slots owned elsewhere; no router
    T, d, E, k, F = 300, 128, 6, 4, 64
    print(f"[lbwd] pre-routed T={T} E={E}", flush=True)
    wl = W.Workload("pre", T, d, E, k, F, torch.bfloat16, routing="pre_routed", n_slots=600, n_empty=1,
                    hot_frac=0.3, seed=4)
    inp = W.make_inputs(wl, device=DEV)
    ids, w = f64(inp["topk_ids"]).astype(np.int32), f64(inp["topk_w"]).astype(np.float32)
    X, Wg, Wu, Wd = f64(inp["x"]), f64(inp["w_gate"]), f64(inp["w_up"]), f64(inp["w_down"])
    off, rt, _ = fwd.permute(ids, E)
    n = int(off[-1])
    g = torch.Generator(device=DEV).manual_seed(9)
    y_perm = torch.randn(T * k, d, generator=g, device=DEV).to(torch.bfloat16)
    dy = W.output_grad(T, d, torch.bfloat16, DEV, 4)
    gpu = dict(inp=inp, ids=inp["topk_ids"], w=inp["topk_w"], y_perm=y_perm, dy=dy)
    ref = lbo.layer_backward(X, None, Wg, Wu, Wd, ids, w, f64(y_perm[:n]), f64(dy))
    L = run_layer(gpu, routed=False)
    torch.cuda.synchronize()
    check_layer(L, ref, torch.bfloat16, routed=False)
    assert not L.d_topk_w[torch.from_numpy(ids < 0).to(DEV)].any()
    # the same share from the gate/up pre-activations its forward kept
    Lf = B.moe_layer_forward(inp["x"], None, None, inp["w_gate"], inp["w_up"], inp["w_down"], k,
                             topk_ids=inp["topk_ids"], topk_w=inp["topk_w"], want_gu=True)
    K = B.moe_layer_backward(inp["x"], None, inp["w_gate"], inp["w_up"], inp["w_down"], inp["topk_ids"],
                             inp["topk_w"], y_perm, dy, want_bias=False, want_d_topk_w=True, gu=Lf.gu)
    torch.cuda.synchronize()
    check_layer(K, ref, torch.bfloat16, routed=False)
    assert torch.equal(K.d_topk_w, L.d_topk_w)          # the combine backward does not see G | U


def test_layer_backward_is_deterministic_and_equals_its_steps():
    T, d, E, k, F = 300, 256, 12, 4, 128
    print("[lbwd] determinism and step composition", flush=True)
    gpu, _ = small_layer(T, d, E, k, F, torch.bfloat16, 5, True)
    a = run_layer(gpu)
    torch.cuda.synchronize()
    snap = [t.clone() for t in (a.dx, a.dw_router, a.dbias, a.dw_gate, a.dw_up, a.dw_down, a.d_topk_w)]
    b = run_layer(gpu)
    torch.cuda.synchronize()
    for s, t in zip(snap, (b.dx, b.dw_router, b.dbias, b.dw_gate, b.dw_up, b.dw_down, b.d_topk_w)):
        assert torch.equal(s.view(torch.int16) if s.dtype == torch.bfloat16 else s,
                           t.view(torch.int16) if t.dtype == torch.bfloat16 else t)
    # the same result from the step entry points called one after another
    inp = gpu["inp"]
    off, rt, sr, _ = B.moe_permute(inp["x"], gpu["ids"], E, copy_rows=False)
    dy_perm, gw = B.moe_combine_backward(gpu["dy"], gpu["y_perm"], sr, gpu["w"])
    dxp, dwg, dwu, dwd = B.moe_grouped_ffn_backward(inp["x"], off, inp["w_gate"], inp["w_up"], inp["w_down"],
                                                    dy_perm, a_rows=rt)
    dx, dwr, db, _ = B.moe_route_backward(inp["x"], inp["w_router"], gpu["ids"], gpu["w"], gw, dx_perm=dxp,
                                          slot_row=sr)
    torch.cuda.synchronize()
    assert torch.equal(gw, b.d_topk_w)
    assert torch.equal(dx.view(torch.int16), b.dx.view(torch.int16))
    for s, t in ((dwr, b.dw_router), (db, b.dbias), (dwg, b.dw_gate), (dwu, b.dw_up), (dwd, b.dw_down)):
        assert torch.equal(s, t)


def page_routing(seed):
    wl = W.WORKLOADS["page_seq64k_skewed"]
    ids, w = W.synthetic_routing(wl.T, wl.E, wl.k, seed)
    off, rt, sr = fwd.permute(ids, wl.E)
    return wl, ids, w, off, rt, sr


def test_combine_backward_page_shape_sampled():
    wl, ids, w, off, rt, sr = page_routing(21)
    N = int(off[-1])
    print(f"[lbwd] combine backward T={wl.T} d={wl.d} N={N}", flush=True)
    g = torch.Generator(device=DEV).manual_seed(22)
    y_perm = torch.randn(N, wl.d, generator=g, device=DEV).to(torch.bfloat16)
    dy = W.output_grad(wl.T, wl.d, torch.bfloat16, DEV, 23)
    srt = torch.from_numpy(sr).to(DEV)
    wt = torch.from_numpy(w).to(DEV)
    dy_perm, gw = B.moe_combine_backward(dy, y_perm, srt, wt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(24)
    S = np.unique(np.concatenate([[0, wl.T - 1], rng.integers(0, wl.T, 62)]))
    rows = sr[S].reshape(-1)
    sub_sr = np.arange(rows.size, dtype=np.int32).reshape(S.size, wl.k)
    rows_t = torch.from_numpy(rows.astype(np.int64)).to(DEV)
    ref_dyp, ref_g = lbo.combine_backward(f64(dy[torch.from_numpy(S).to(DEV)]), f64(y_perm[rows_t]), sub_sr, w[S])
    close_rel(f64(gw)[S], ref_g, 1e-4, "d_topk_w")
    got = f64(dy_perm[rows_t])
    assert (np.abs(got - ref_dyp) <= 2.0 ** -8 * (1 + 1e-6) * np.abs(ref_dyp)).all()


def test_route_backward_page_shape_sampled():
    wl, ids, w, off, rt, sr = page_routing(31)
    N = int(off[-1])
    print(f"[lbwd] route backward T={wl.T} d={wl.d} E={wl.E}", flush=True)
    inp = W.make_inputs(wl, device=DEV)
    x, wr = inp["x"], inp["w_router"]
    del inp
    g = torch.Generator(device=DEV).manual_seed(32)
    gw = torch.randn(wl.T, wl.k, generator=g, device=DEV)
    dxp = torch.randn(N, wl.d, generator=g, device=DEV).to(torch.bfloat16)
    dx, dwr, db, dl = B.moe_route_backward(x, wr, torch.from_numpy(ids).to(DEV), torch.from_numpy(w).to(DEV), gw,
                                           dx_perm=dxp, slot_row=torch.from_numpy(sr).to(DEV), want_dlogits=True)
    torch.cuda.synchronize()
    ref_sel = lbo.gate_weights_backward(w, f64(gw))
    ref_dl = lbo.scatter_logit_grad(ids, ref_sel, wl.E)
    rng = np.random.default_rng(33)
    S = np.unique(np.concatenate([[0, wl.T - 1], rng.integers(0, wl.T, 62)]))
    St = torch.from_numpy(S).to(DEV)
    close_rel(f64(dl[St]), ref_dl[S], 1e-4, "dlogits (sampled tokens)")
    close_rel(f64(db), ref_dl.sum(axis=0), 1e-4, "dbias")
    cols = np.unique(np.concatenate([[0, wl.d - 1], rng.integers(0, wl.d, 30)]))
    Xc = f64(x[:, torch.from_numpy(cols).to(DEV)])
    close_bf16(f64(dwr)[:, cols], ref_dl.T @ Xc, "dW_router (sampled columns)")
    rows = sr[S].reshape(-1)
    sub_rt = np.repeat(np.arange(S.size), wl.k)
    dx_perm_part = lbo.permute_backward(f64(dxp[torch.from_numpy(rows.astype(np.int64)).to(DEV)]), sub_rt, S.size)
    dx_router_part = ref_dl[S] @ f64(wr)
    close_bf16(f64(dx[St]), dx_perm_part + dx_router_part, "dx (sampled tokens)")


@pytest.mark.parametrize("T,d,E,k,F,dtype,seed,bias", LAYERS)
def test_layer_backward_from_kept_gate_up(T, d, E, k, F, dtype, seed, bias):
    # The forward (fed the oracle's routing, so no oracle input comes from the GPU)
    # keeps G | U; the backward reads them.  bf16: G and U are rounded once more than
    # on the recompute path, within the same rule.  float32: the kept values are the
    # recompute path's accumulators, so every output equals that path's bit for bit.
    print(f"[lbwd-gu] T={T} d={d} E={E} k={k} F={F} {dtype}", flush=True)
    gpu, ref = small_layer(T, d, E, k, F, dtype, seed, bias)
    inp = gpu["inp"]
    Lf = B.moe_layer_forward(inp["x"], None, None, inp["w_gate"], inp["w_up"], inp["w_down"], k,
                             topk_ids=gpu["ids"], topk_w=gpu["w"], want_y_perm=True, want_gu=True)
    L = B.moe_layer_backward(inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"], gpu["ids"],
                             gpu["w"], gpu["y_perm"], gpu["dy"], want_bias=True, want_d_topk_w=True, gu=Lf.gu)
    torch.cuda.synchronize()
    check_layer(L, ref, dtype)
    if dtype == torch.float32:
        R = run_layer(gpu)
        torch.cuda.synchronize()
        for a, b in ((L.dx, R.dx), (L.dw_gate, R.dw_gate), (L.dw_up, R.dw_up), (L.dw_down, R.dw_down),
                     (L.dw_router, R.dw_router), (L.dbias, R.dbias), (L.d_topk_w, R.d_topk_w)):
            assert torch.equal(a, b)


def test_layer_forward_training_outputs():
    # y_perm_out and gu_out change nothing in y; y_perm_out is the stage path's y_perm
    T, d, E, k, F = 300, 256, 12, 4, 128
    print("[lbwd-gu] forward outputs for training", flush=True)
    wl = W.Workload("train_fwd", T, d, E, k, F, torch.bfloat16, routing="router_bias", seed=6)
    inp = W.make_inputs(wl, device=DEV)
    a = B.moe_layer_forward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"], inp["w_down"], k,
                            want_routing=True, want_offsets=True)
    b = B.moe_layer_forward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"], inp["w_down"], k,
                            want_routing=True, want_offsets=True, want_y_perm=True, want_gu=True)
    torch.cuda.synchronize()
    assert torch.equal(a.y.view(torch.int16), b.y.view(torch.int16))
    off, rt, sr, _ = B.moe_permute(inp["x"], b.topk_ids, E, copy_rows=False)
    gu = torch.empty(T * k, 2 * F, dtype=torch.bfloat16, device=DEV)
    yp = B.moe_grouped_ffn(inp["x"], off, inp["w_gate"], inp["w_up"], inp["w_down"], a_rows=rt, gu_out=gu)
    torch.cuda.synchronize()
    n = int(off[-1])
    assert torch.equal(yp[:n].view(torch.int16), b.y_perm[:n].view(torch.int16))
    assert torch.equal(gu[:n].view(torch.int16), b.gu[:n].view(torch.int16))
