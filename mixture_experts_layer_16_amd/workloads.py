"""Seeded synthetic inputs for the layer, shared by the HIP path's tests and
benchmark and by the oracle's checks.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Shapes come from the model-configuration table of
"Training a 1T-Parameter MoE on EU public infrastructure with PyTorch and
TorchTitan" (hidden 6,144, 384 routed experts, top-8, expert hidden 1,792,
65,536-token pre-training sequences).  No data set or trained weight exists
here, so every tensor is drawn from a fixed distribution:

  x                      ~ N(0, 1)
  W_r (router)           ~ N(0, 1)/sqrt(d), or N(0, 0.02^2) at the page's shape
  W_g, W_u [E, F, d]     ~ N(0, 1)/sqrt(d)
  W_d      [E, d, F]     ~ N(0, 1)/sqrt(F)
  routing bias (skewed)  b_e = -1.5 * log10(rank_e), ranks a seeded permutation of 1..E
  pre-routed slots       12 empty experts, one holding 20% of the slots, the rest
                         multinomial; a token's slots hold distinct experts in
                         ascending order, -1 elsewhere; gate weights ~ U(0, 1)
                         normalised over the token's local slots
  backward inputs        output gradient dy ~ N(0, 1); where a routing table is
                         drawn rather than computed: k distinct experts per token
                         sampled without replacement with probability
                         proportional to 1/rank_e (Zipf), gate weights ~ U(0.05, 1)
                         normalised and sorted in descending order

bf16 tensors are the fp32 draws rounded to nearest even.  Tensors are drawn on
the requested device with torch's generator for that device; the discrete
routing structure is drawn with numpy's PCG64 on the host.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    dtype: torch.dtype
    routing: str = "router"          # "router", "router_bias" or "pre_routed"
    router_std: Optional[float] = None  # None: 1/sqrt(d)
    n_slots: int = 0                  # pre_routed: valid slots on this GPU
    n_empty: int = 0                  # pre_routed: experts with no slot
    hot_frac: float = 0.0             # pre_routed: share of slots on one expert
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def N(self) -> int:
        return self.n_slots if self.routing == "pre_routed" else self.T * self.k

    def expert_flops(self) -> float:
        """Algorithmic FLOPs of the grouped SwiGLU FFN (gate, up and down GEMMs)."""
        return 6.0 * self.N * self.d * self.F

    def router_flops(self) -> float:
        return 0.0 if self.routing == "pre_routed" else 2.0 * self.T * self.d * self.E


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32", 256, 128, 16, 2, 64, torch.float32,
                 note="tiny fp32 layer, seed 0"),
        Workload("small_bf16", 4096, 1024, 64, 8, 512, torch.bfloat16,
                 note="small bf16 layer, near-uniform router logits"),
        Workload("page_balanced", 8192, 6144, 384, 8, 1792, torch.bfloat16, router_std=0.02,
                 note="page's layer shape, 8,192 tokens, balanced routing"),
        Workload("page_seq64k_skewed", 65536, 6144, 384, 8, 1792, torch.bfloat16, routing="router_bias",
                 router_std=0.02, note="page's layer shape, one 65,536-token sequence, Zipf-like routing bias"),
        Workload("ep_rank_share", 65536, 6144, 96, 8, 1792, torch.bfloat16, routing="pre_routed",
                 n_slots=131072, n_empty=12, hot_frac=0.2,
                 note="one expert-parallel rank's share: 96 local experts, 131,072 pre-routed slots"),
    ]
}


def _normal(shape, std, gen, device, dtype):
    t = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def _experts(E, rows, cols, std, gen, device, dtype):
    out = torch.empty(E, rows, cols, dtype=dtype, device=device)
    for e in range(E):             # one expert at a time bounds the fp32 scratch
        out[e] = _normal((rows, cols), std, gen, device, dtype)
    return out


def routing_bias(E: int, seed: int) -> np.ndarray:
    """Zipf-like per-expert bias b_e = -1.5 * log10(rank_e) (float32)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))
    ranks = rng.permutation(E) + 1
    return (-1.5 * np.log10(ranks)).astype(np.float32)


def pre_routed_slots(T: int, E: int, k: int, n_slots: int, n_empty: int, hot_frac: float, seed: int):
    """Seeded ragged slot table of one expert-parallel rank: ids [T, k] int32
    (-1 = slot owned elsewhere) and gate weights [T, k] float32."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2])))
    perm = rng.permutation(E)
    empty, hot, rest = perm[:n_empty], perm[n_empty], perm[n_empty + 1:]
    counts = np.zeros(E, dtype=np.int64)
    counts[hot] = int(round(hot_frac * n_slots))
    counts[rest] = rng.multinomial(n_slots - counts[hot], np.full(rest.size, 1.0 / rest.size))
    assert counts[empty].sum() == 0 and counts.sum() == n_slots
    used = np.zeros(T, dtype=np.int64)
    toks, exps = [], []
    for e in range(E):
        if counts[e] == 0:
            continue
        avail = np.nonzero(used < k)[0]
        pick = rng.choice(avail, size=int(counts[e]), replace=False)
        used[pick] += 1
        toks.append(pick)
        exps.append(np.full(pick.size, e))
    toks = np.concatenate(toks)
    exps = np.concatenate(exps)
    order = np.lexsort((exps, toks))            # by token, then expert
    toks, exps = toks[order], exps[order]
    first = np.searchsorted(toks, toks, side="left")
    pos = np.arange(toks.size) - first
    ids = np.full((T, k), -1, dtype=np.int32)
    ids[toks, pos] = exps
    w = rng.random((T, k)).astype(np.float32)
    w[ids < 0] = 0.0
    s = w.sum(axis=1, keepdims=True)
    w = np.divide(w, s, out=np.zeros_like(w), where=s > 0).astype(np.float32)
    return ids, w


def synthetic_routing(T: int, E: int, k: int, seed: int):
    """Seeded routing table (ids [T, k] int32, distinct per token; gate weights
    [T, k] float32, each row summing to one and non-increasing).  Experts are
    drawn without replacement with probability proportional to 1/rank_e (ranks a
    seeded permutation of 1..E), by adding Gumbel noise to the log-probabilities
    and keeping the k largest."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 3])))
    ranks = rng.permutation(E) + 1
    logp = -np.log(ranks.astype(np.float64))
    keys = logp[None, :] + rng.gumbel(size=(T, E))
    ids = np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)
    w = rng.uniform(0.05, 1.0, (T, k))
    w = -np.sort(-(w / w.sum(axis=1, keepdims=True)), axis=1)
    return ids, w.astype(np.float32)


def output_grad(T: int, d: int, dtype, device="cuda", seed: int = 0) -> torch.Tensor:
    """Seeded output gradient dy [T, d] ~ N(0, 1) in dtype."""
    gen = torch.Generator(device=torch.device(device))
    gen.manual_seed(seed + 7919)
    return _normal((T, d), 1.0, gen, torch.device(device), dtype)


def make_inputs(wl: Workload, device="cuda", seed: Optional[int] = None) -> dict:
    """All input tensors of one workload, on `device`."""
    seed = wl.seed if seed is None else seed
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    dt = wl.dtype
    out = {"x": _normal((wl.T, wl.d), 1.0, gen, dev, dt)}
    if wl.routing == "pre_routed":
        out["w_router"] = None
        out["bias"] = None
    else:
        std = wl.router_std if wl.router_std is not None else 1.0 / math.sqrt(wl.d)
        out["w_router"] = _normal((wl.E, wl.d), std, gen, dev, dt)
        out["bias"] = (torch.from_numpy(routing_bias(wl.E, seed)).to(dev)
                       if wl.routing == "router_bias" else None)
    out["w_gate"] = _experts(wl.E, wl.F, wl.d, 1.0 / math.sqrt(wl.d), gen, dev, dt)
    out["w_up"] = _experts(wl.E, wl.F, wl.d, 1.0 / math.sqrt(wl.d), gen, dev, dt)
    out["w_down"] = _experts(wl.E, wl.d, wl.F, 1.0 / math.sqrt(wl.F), gen, dev, dt)
    if wl.routing == "pre_routed":
        ids, w = pre_routed_slots(wl.T, wl.E, wl.k, wl.n_slots, wl.n_empty, wl.hot_frac, seed)
        out["topk_ids"] = torch.from_numpy(ids).to(dev)
        out["topk_w"] = torch.from_numpy(w).to(dev)
    return out
