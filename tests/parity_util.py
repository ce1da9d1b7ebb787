"""Helpers shared by the GPU parity tests: exact host copies and the tolerance.

Tolerance for floating-point outputs of the layer:
  bf16:    every element |g - o| <= 1e-2 + 2e-2 |o|, and max |g - o| <= 1e-2 max |o|
  float32: max |g - o| <= 1e-5 max |o|
Router logits (inputs and weights in bf16, products exact in float32, only the
summation order differs): |g - o| <= 1e-4 for bf16, <= 1e-5 max |l| for float32.
Gate weights: |g - o| <= 1e-6.  Integer and index outputs: bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch


def f64(t) -> np.ndarray:
    """Exact float64 host copy of a bf16/fp32 tensor (None stays None)."""
    if t is None:
        return None
    return t.detach().to("cpu").to(torch.float64).numpy()


def i64(t) -> np.ndarray:
    return t.detach().to("cpu").to(torch.int64).numpy()


class LazyExperts:
    """Per-expert float64 host copies of a [E, r, c] device tensor, made on demand."""

    def __init__(self, t):
        self.t = t

    def __len__(self):
        return self.t.shape[0]

    def __getitem__(self, e):
        return f64(self.t[e])


def assert_close(g, o, dtype, what=""):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    err = np.abs(g - o)
    scale = np.abs(o).max() if o.size else 0.0
    if dtype == torch.float32:
        assert err.max(initial=0.0) <= 1e-5 * scale, f"{what}: max err {err.max():.3e} > 1e-5 * {scale:.3e}"
    else:
        assert err.max(initial=0.0) <= 1e-2 * scale, f"{what}: max err {err.max():.3e} > 1e-2 * {scale:.3e}"
        bad = err > 1e-2 + 2e-2 * np.abs(o)
        assert not bad.any(), f"{what}: {bad.sum()} elements outside atol 1e-2 / rtol 2e-2 (worst {err.max():.3e})"
    return float(err.max(initial=0.0)), float(scale)


def assert_logits_close(g, o, dtype, what="logits"):
    err = np.abs(np.asarray(g, np.float64) - np.asarray(o, np.float64))
    bound = 1e-5 * np.abs(o).max() if dtype == torch.float32 else 1e-4
    assert err.max(initial=0.0) <= bound, f"{what}: max err {err.max():.3e} > {bound:.3e}"
    return float(err.max(initial=0.0))


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    """Bitwise equality of two tensors of the same dtype."""
    if a.dtype != b.dtype or a.shape != b.shape:
        return False
    view = {torch.bfloat16: torch.int16, torch.float32: torch.int32}.get(a.dtype)
    if view is not None:
        a, b = a.view(view), b.view(view)
    return bool(torch.equal(a, b))


def routing_disagreement(own_logits, gpu_logits, k):
    """Tokens where selection on the oracle's own logits differs from selection
    on the GPU's logits; each must sit on a near-tie (gap between the k-th and
    (k+1)-th logit within twice the largest logit difference)."""
    from oracle import moe_oracle as orc
    ids_own, _ = orc.select_topk(own_logits, k)
    ids_gpu, _ = orc.select_topk(gpu_logits, k)
    diff = np.nonzero((np.sort(ids_own, 1) != np.sort(ids_gpu, 1)).any(1))[0]
    dl = np.abs(own_logits - gpu_logits).max()
    for t in diff:
        srt = np.sort(own_logits[t])[::-1]
        gap = srt[k - 1] - srt[k] if k < srt.size else np.inf
        assert gap <= 2 * dl, f"token {t} selects differently with a gap {gap:.3e} > 2 * {dl:.3e}"
    return diff.size
