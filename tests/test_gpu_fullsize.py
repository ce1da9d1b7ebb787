"""The three full-size workloads, through the same entry point and launch
configuration that bench.py times (moe_layer_forward).  The oracle checks:
  * routing of EVERY token: ids bit-exact and gate weights within 1e-6 when the
    oracle selects on the GPU's logits; the logits themselves on a token sample;
  * the expert offsets, bit-exact;
  * the grouped FFN (stage entry points) on EVERY row of the largest expert's
    first four chunks of 8 row tiles and of its last chunk (the tile order walks
    a large expert chunk by chunk), and on sampled rows of the smallest non-empty
    expert and two random ones;
  * the layer output on 256 sampled tokens (plus a token with no local slot);
  * the layer entry point equals the stage-by-stage path bit for bit.
"""
import numpy as np
import pytest
import torch

from mixture_experts_layer_16_amd import binding as B
from mixture_experts_layer_16_amd import workloads as W
from oracle import moe_oracle as orc
from parity_util import assert_close, assert_logits_close, bits_equal, f64, i64, routing_disagreement

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FULL = ["page_balanced", "page_seq64k_skewed", "ep_rank_share"]


def expert_f64(inp, e):
    """Exact float64 host copies of expert e's three matrices (widened on the device)."""
    return tuple(inp[n][e].to(torch.float64).cpu().numpy() for n in ("w_gate", "w_up", "w_down"))


ROW_CHUNK = 8 * 256    # rows of one chunk of the forward GEMMs' tile order


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_parity(name):
    wl = W.WORKLOADS[name]
    print(f"[full-size] {name}: T={wl.T} d={wl.d} E={wl.E} k={wl.k} F={wl.F}", flush=True)
    inp = W.make_inputs(wl, device=DEV)
    routed = inp["w_router"] is not None
    L = B.LayerForward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"], inp["w_down"], wl.k,
                       topk_ids=inp.get("topk_ids"), topk_w=inp.get("topk_w"), want_logits=routed,
                       want_routing=routed, want_offsets=True)
    L()
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    T = wl.T

    if routed:
        gl = L.logits.cpu().numpy().astype(np.float64)
        ref_ids, ref_w = orc.select_topk(gl, wl.k)
        assert np.array_equal(i64(L.topk_ids), ref_ids)
        assert np.abs(f64(L.topk_w) - ref_w).max() <= 1e-6
        S = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 62, replace=False)]))
        own = orc.router_logits(f64(inp["x"][S]), f64(inp["w_router"]), f64(inp["bias"]))
        assert_logits_close(gl[S], own, wl.dtype)
        routing_disagreement(own, gl[S], wl.k)
    else:
        ref_ids, ref_w = i64(inp["topk_ids"]), f64(inp["topk_w"])
    r_off, r_rt, r_sr = orc.permute(ref_ids, wl.E)
    assert np.array_equal(i64(L.offsets), r_off)
    counts = np.diff(r_off)
    print(f"[full-size] {name}: expert rows min {counts.min()} max {counts.max()} empty {(counts == 0).sum()}",
          flush=True)

    # layer output on 256 sampled tokens (a token with no local slot included when
    # present), the reference one expert at a time
    has = (ref_ids >= 0).any(1)
    St = list(rng.choice(np.nonzero(has)[0], 256, replace=False))
    if (~has).any():
        St.append(int(np.nonzero(~has)[0][0]))
    St = np.array(St)
    xs = f64(inp["x"][torch.from_numpy(St).to(DEV)])
    y_ref = np.zeros((St.size, wl.d))
    for e in np.unique(ref_ids[St][ref_ids[St] >= 0]):
        pos, slot = np.nonzero(ref_ids[St] == e)
        ye = orc.expert_ffn(xs[pos], *expert_f64(inp, int(e)))
        y_ref[pos] += ref_w[St[pos], slot][:, None] * ye
    assert_close(f64(L.y[torch.from_numpy(St).to(DEV)]), y_ref, wl.dtype, "y (256 sampled tokens)")

    # the stage entry points: bit-equal to the layer entry point
    if routed:
        ids, w, _ = B.moe_route(inp["x"], inp["w_router"], wl.k, bias=inp["bias"], want_logits=False)
    else:
        ids, w = inp["topk_ids"], inp["topk_w"]
    off, rt, sr, _ = B.moe_permute(inp["x"], ids, wl.E, copy_rows=False)
    yp = B.moe_grouped_ffn(inp["x"], off, inp["w_gate"], inp["w_up"], inp["w_down"], a_rows=rt)
    y = B.moe_combine(yp, sr, w)
    torch.cuda.synchronize()
    assert bits_equal(y, L.y)

    def check_rows(e, rows, what):
        idx = torch.from_numpy(rows.astype(np.int64)).to(DEV)
        X = inp["x"][torch.from_numpy(r_rt[rows].astype(np.int64)).to(DEV)].to(torch.float64).cpu().numpy()
        ref = orc.expert_ffn(X, *expert_f64(inp, e))
        assert_close(f64(yp[idx]), ref, wl.dtype, what)

    # every row of the largest expert's first four chunks and of its last chunk
    big = int(np.argmax(counts))
    lo, hi = int(r_off[big]), int(r_off[big + 1])
    last = lo + (hi - lo - 1) // ROW_CHUNK * ROW_CHUNK
    rows = np.unique(np.concatenate([np.arange(lo, min(hi, lo + 4 * ROW_CHUNK)), np.arange(last, hi)]))
    print(f"[full-size] {name}: expert {big} ({hi - lo} rows): {rows.size} rows compared", flush=True)
    check_rows(big, rows, f"y_perm rows of expert {big}")
    # sampled rows of the smallest non-empty expert and two random ones
    nz = np.nonzero(counts)[0]
    pick = {int(nz[np.argmin(counts[nz])])} | set(rng.choice(nz, 2, replace=False).tolist())
    for e in sorted(pick - {big}):
        lo, hi = int(r_off[e]), int(r_off[e + 1])
        rows = np.unique(np.concatenate([[lo, hi - 1], rng.integers(lo, hi, 14)]))
        check_rows(e, rows, f"y_perm rows of expert {e}")
