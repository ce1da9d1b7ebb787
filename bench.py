"""Benchmark: routed-MoE layer forward on one MI355X.

A step is one moe_layer_forward call (router GEMM, softmax top-k, permute,
grouped SwiGLU FFN, combine) over the whole workload, with every input already
resident in HBM.  The default workload is the page's layer shape (hidden 6,144,
384 routed experts, top-8, expert hidden 1,792, bf16) on one 65,536-token
sequence with Zipf-like routing skew.

Prints one JSON line.  `roofline` covers the grouped FFN (its gate/up and down
GEMM launches, timed together with HIP events on the launch stream) against
the bf16 dense MFMA peak; `stages_ms` gives each step's average duration from
a second, stage-by-stage pass; `kernels` gives every kernel's average device
time from a third pass traced with torch's profiler (HIP activity records), and
each kernel's fraction of its roofline (MFMA peak for the GEMMs, HBM peak for
route's top-k, permute and combine); `other_workloads` times the 8,192-token
balanced workload and the expert-parallel rank's share the same way;
`cpu_baseline` times the float64 CPU oracle, step by step, on a bounded slice of
the same workload, and `cpu_oracle` on the whole small workload.

`--cpu-only NAME[,NAME...]` times only the oracle, step by step, on whole
workloads (inputs drawn on the GPU, copied to the host) and prints one JSON line
per workload.

`--path backward` measures the layer backward (moe_layer_backward: combine,
grouped expert FFN, gate-weight/router and permutation backward) from the
forward's routing and expert outputs of the same workload; its roofline covers
the grouped expert-FFN backward, timed alone in a stage-by-stage pass.

`--path newton_schulz` measures the next row instead: Muon's Newton-Schulz
orthogonalisation of whole expert matrices (one step = the gate, up and down
matrices of the 96 experts one expert-parallel rank owns, five quintic steps
each), on the same contract.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/s + grouped-GEMM % bf16 MFMA peak (d6144,E384,top8)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3        # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="page_seq64k_skewed")
    ap.add_argument("--path", default="layer", choices=["layer", "newton_schulz", "backward"],
                    help="layer: the MoE layer forward (default); newton_schulz: Muon's orthogonalisation "
                         "of whole expert matrices; backward: the grouped expert-FFN backward")
    ap.add_argument("--ns-experts", type=int, default=96,
                    help="newton_schulz: experts whose gate, up and down matrices one step orthogonalises")
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="tokens of the workload the CPU oracle runs on (0 = skip; default 8192 for the forward, "
                         "1024 for the backward); the oracle's fixed cost of widening each expert it touches from "
                         "bf16 dominates much smaller samples")
    ap.add_argument("--other-workloads", default="page_balanced,ep_rank_share",
                    help="workloads timed after the main one (comma-separated; empty: none)")
    ap.add_argument("--no-kernel-split", action="store_true",
                    help="skip the per-kernel pass traced with torch's profiler (for runs under rocprofv3)")
    ap.add_argument("--cpu-only", default="",
                    help="comma-separated workloads: time only the CPU oracle on each whole workload")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run one 1 GiB device copy, then one grouped FFN call, and exit "
                         "(for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs)")
    args = ap.parse_args()
    if args.cpu_tokens is None:
        args.cpu_tokens = 1024 if args.path == "backward" else 8192
    return args


# HBM traffic of one grouped-FFN call (gate/up + down launches) at 65,536 tokens
# of the page shape, from rocprofv3 FETCH_SIZE and WRITE_SIZE runs of
# `bench.py --traffic-probe`, each scaled by the same counter's reading for a
# 1 GiB device copy.  Valid only for the kernel sources it was measured on.
TRAFFIC = {"workload": "page_seq64k_skewed", "kernel_source_hash": "f7fafd382b194657", "bytes": 99547995081,
           "fetch_scale": 1.9999, "write_scale": 1.0000}
KERNEL_SOURCES = ["mixture_experts_layer_16_amd/csrc/gemm_tile.h", "mixture_experts_layer_16_amd/csrc/grouped_ffn.hip",
                  "mixture_experts_layer_16_amd/csrc/common.h", "mixture_experts_layer_16_amd/csrc/tile_walk.h"]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_probe(torch, B, W, wl):
    """One plain 1 GiB copy (the counters' calibration) and one grouped FFN call."""
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    inp = W.make_inputs(wl, device="cuda:0")
    if inp["w_router"] is not None:
        ids, w, _ = B.moe_route(inp["x"], inp["w_router"], wl.k, bias=inp["bias"], want_logits=False)
    else:
        ids, w = inp["topk_ids"], inp["topk_w"]
    off, rt, sr, _ = B.moe_permute(inp["x"], ids, wl.E, copy_rows=False)
    yp = torch.empty(rt.numel(), wl.d, dtype=inp["x"].dtype, device="cuda:0")
    torch.cuda.synchronize()
    B.moe_grouped_ffn(inp["x"], off, inp["w_gate"], inp["w_up"], inp["w_down"], y_perm=yp, a_rows=rt)
    torch.cuda.synchronize()
    print(json.dumps({"traffic_probe": wl.name, "kernel_source_hash": kernel_source_hash()}), flush=True)


def stage_pass(torch, B, inp, wl, steps):
    """Average per-stage durations (ms) with events on the current stream."""
    routed = inp["w_router"] is not None
    names = (["route"] if routed else []) + ["permute", "grouped_ffn", "combine"]
    acc = {n: 0.0 for n in names}
    for _ in range(steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        ev[0].record()
        i = 0
        if routed:
            ids, w, _ = B.moe_route(inp["x"], inp["w_router"], wl.k, bias=inp["bias"], want_logits=False)
            i += 1
            ev[i].record()
        else:
            ids, w = inp["topk_ids"], inp["topk_w"]
        off, rt, sr, _ = B.moe_permute(inp["x"], ids, wl.E, copy_rows=False)
        i += 1
        ev[i].record()
        yp = B.moe_grouped_ffn(inp["x"], off, inp["w_gate"], inp["w_up"], inp["w_down"], a_rows=rt)
        i += 1
        ev[i].record()
        B.moe_combine(yp, sr, w)
        i += 1
        ev[i].record()
        torch.cuda.synchronize()
        for j, n in enumerate(names):
            acc[n] += ev[j].elapsed_time(ev[j + 1])
        del off, rt, sr, yp
    return {n: v / steps for n, v in acc.items()}


def host_info():
    """CPU model, core count and the BLAS library numpy's products run on."""
    from threadpoolctl import threadpool_info
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p.get("num_threads", 1) for p in blas] + [1])
    lib = ", ".join(f"{p.get('internal_api')} {p.get('version')}" for p in blas) or "unknown"
    return {"cpu_model": model, "host_cpus": os.cpu_count(), "blas": lib, "blas_threads": threads}


def oracle_stages(orc, x, wr, b, wg, wu, wd, k, ids=None, weights=None):
    """The oracle's own steps in layer_forward's order, each timed (seconds)."""
    t = {}
    t0 = time.perf_counter()
    if ids is None:
        logits = orc.router_logits(x, wr, b)
        ids, w = orc.select_topk(logits, k)
    else:
        w = orc.to_f64(weights)
    t1 = time.perf_counter()
    offsets, row_token, slot_row = orc.permute(ids, len(wg))
    x_perm = orc.gather_rows(x, row_token)
    t2 = time.perf_counter()
    y_perm = orc.grouped_ffn(x_perm, offsets, wg, wu, wd)
    t3 = time.perf_counter()
    orc.combine(y_perm, slot_row, w)
    t4 = time.perf_counter()
    if wr is not None:
        t["route"] = t1 - t0
    t.update(permute=t2 - t1, expert_ffn=t3 - t2, combine=t4 - t3, layer=t4 - t0)
    return t, int(offsets[-1])


class _HostExperts:
    """Per-expert weights on the host as stored: bf16 as uint16 bit patterns
    (the oracle widens one expert at a time), float32 as it is."""

    def __init__(self, torch, t, progress=""):
        import numpy as np
        self.h = t.cpu()
        self.bits = t.dtype == torch.bfloat16
        self.np, self.torch = np, torch
        self.progress = progress

    def __len__(self):
        return self.h.shape[0]

    def __getitem__(self, e):
        if self.progress and e % 48 == 0:
            print(f"[{self.progress}] expert {e} of {len(self)}", file=sys.stderr, flush=True)
        if self.bits:
            return self.h[e].view(self.torch.int16).numpy().view(self.np.uint16)
        return self.h[e].numpy()


def _host_tokens(torch, t):
    """Token rows on the host as stored (bf16 as uint16 bit patterns)."""
    import numpy as np
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def cpu_oracle_run(torch, inp, wl, n_tokens, repeats=1, progress=""):
    """The float64 oracle step by step on the first n_tokens tokens (0 = all) of
    the workload's inputs; the median run of `repeats`."""
    import numpy as np
    from oracle import moe_oracle as orc
    n = wl.T if n_tokens <= 0 else min(n_tokens, wl.T)
    x = _host_tokens(torch, inp["x"][:n])
    routed = inp["w_router"] is not None
    wr = _host_tokens(torch, inp["w_router"]) if routed else None
    b = inp["bias"].cpu().numpy() if inp.get("bias") is not None else None
    ew = [_HostExperts(torch, inp[k], progress if k == "w_gate" else "") for k in ("w_gate", "w_up", "w_down")]
    kw = {} if routed else dict(ids=inp["topk_ids"][:n].cpu().numpy(), weights=inp["topk_w"][:n].cpu().numpy())
    runs = []
    for _ in range(repeats):
        t, slots = oracle_stages(orc, x, wr, b, *ew, wl.k, **kw)
        runs.append(t)
    runs.sort(key=lambda r: r["layer"])
    t = runs[len(runs) // 2]
    flops = 6.0 * slots * wl.d * wl.F + (2.0 * n * wl.d * wl.E if routed else 0.0)
    return n, slots, t, flops


def cpu_baseline(torch, inp, wl, n_tokens):
    """The float64 oracle on the first n_tokens tokens of the workload (their
    routing, permutation, every expert FFN they use, and the combine), step by
    step."""
    info = host_info()
    n, slots, t, flops = cpu_oracle_run(torch, inp, wl, n_tokens)
    return {"value": round(n / t["layer"], 3), "unit": "tokens/s", "cores": info["blas_threads"], "kind": "oracle",
            "sample": f"first {n} of {wl.T} tokens of {wl.name} ({slots} slots): the float64 oracle's steps "
                      f"(routing, permutation, SwiGLU FFN of every expert they use, combine) in "
                      f"{t['layer']:.1f} s on {info['blas_threads']} BLAS threads of {info['host_cpus']} host CPUs",
            "stages_s": {k_: round(v, 4) for k_, v in t.items()},
            "gflops": round(flops / t["layer"] / 1e9, 2), **info}


def cpu_only(args, torch, W):
    """Time the oracle, step by step, on whole workloads (one JSON line each)."""
    info = host_info()
    for name in [w for w in args.cpu_only.split(",") if w]:
        wl = W.WORKLOADS[name]
        inp = W.make_inputs(wl, device="cuda:0")
        reps = 3 if wl.T * wl.k * wl.d * wl.F <= 4096 * 8 * 1024 * 512 else 1
        n, slots, t, flops = cpu_oracle_run(torch, inp, wl, 0, repeats=reps, progress=name)
        del inp
        torch.cuda.empty_cache()
        print(json.dumps({"cpu_oracle": name, "tokens": n, "slots": slots, "runs": reps,
                          "note": "float64 oracle (numpy), the median of the runs" if reps > 1 else
                                  "float64 oracle (numpy), one run",
                          "stages_s": {k_: round(v, 4) for k_, v in t.items()},
                          "tokens_per_s": round(n / t["layer"], 3), "gflops": round(flops / t["layer"] / 1e9, 2),
                          **info}), flush=True)


def kernel_split(torch, L, routed, reps=3):
    """Average device time (ms) of every kernel of one layer call, from torch's
    profiler (HIP activity records of the library's launches)."""
    from torch.profiler import ProfilerActivity, profile
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for _ in range(reps):
            L()
        torch.cuda.synchronize()
    evs = [e for e in prof.events() if e.device_type == torch.autograd.DeviceType.CUDA]
    evs.sort(key=lambda e: e.time_range.start)
    gemms = (["router_gemm"] if routed else []) + ["gate_up_gemm", "down_gemm"]
    acc, gi = {}, 0
    for e in evs:
        n = e.name
        if "grouped_gemm_kernel" in n:
            role = gemms[gi % len(gemms)]
            gi += 1
        elif "topk" in n:
            role = "topk"
        elif "permute" in n:
            role = "permute"
        elif "combine_kernel" in n:
            role = "combine"
        else:
            continue
        us = e.device_time if hasattr(e, "device_time") else e.cuda_time
        acc[role] = acc.get(role, 0.0) + us
    if gi != reps * len(gemms):
        raise RuntimeError(f"profiler saw {gi} GEMM launches, expected {reps * len(gemms)}")
    return {k_: v / reps / 1e3 for k_, v in acc.items()}


def kernel_fractions(wl, es, km):
    """Each kernel's algorithmic work per launch over its measured time, as a
    fraction of its roofline.  Bytes count every tensor read or written once."""
    import math
    nblk = math.ceil(wl.T / 256)
    out = {}
    def mfma(name, flops):
        if name in km:
            out[name] = {"ms": round(km[name], 4), "tflops": round(flops / km[name] / 1e9, 1),
                         "mfma_frac": round(flops / km[name] / 1e9 / PEAK_BF16_TFLOPS, 4), "flops": flops}
    def hbm(name, nbytes):
        if name in km:
            out[name] = {"ms": round(km[name], 4), "gbs": round(nbytes / km[name] / 1e6, 1),
                         "hbm_frac": round(nbytes / km[name] / 1e6 / PEAK_HBM_GBS, 4), "bytes": nbytes}
    if wl.routing != "pre_routed":
        mfma("router_gemm", 2.0 * wl.T * wl.d * wl.E)
        out["router_gemm"]["bytes"] = wl.T * wl.d * es + wl.E * wl.d * es + wl.T * wl.E * 4
        hbm("topk", wl.T * wl.E * 4 + wl.T * wl.k * 8)
    # ids read twice; block counts written, scanned and read; row_token and slot_row written
    hbm("permute", wl.T * wl.k * 4 * 2 + nblk * wl.E * 4 * 4 + (wl.E + 1) * 4 + wl.N * 4 + wl.T * wl.k * 4)
    mfma("gate_up_gemm", 4.0 * wl.N * wl.d * wl.F)
    mfma("down_gemm", 2.0 * wl.N * wl.d * wl.F)
    hbm("combine", wl.N * wl.d * es + wl.T * wl.d * es + wl.T * wl.k * 8)
    return out


def time_layer(torch, L, steps):
    """Mean ms per call of L over `steps` calls, one event before and after."""
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(steps):
        L()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def other_workload(torch, B, W, name, steps, warmup):
    """The layer forward on another workload: tokens/s, the grouped FFN's MFMA
    fraction and (weight-streaming case) its fraction of the HBM floor."""
    wl = W.WORKLOADS[name]
    inp = W.make_inputs(wl, device="cuda:0")
    L = B.LayerForward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"], inp["w_down"], wl.k,
                       topk_ids=inp.get("topk_ids"), topk_w=inp.get("topk_w"))
    for _ in range(warmup):
        L()
    ms = time_layer(torch, L, steps)
    stages = stage_pass(torch, B, inp, wl, 3)
    es = 2 if wl.dtype == torch.bfloat16 else 4
    ffn = stages["grouped_ffn"]
    tflops = wl.expert_flops() / (ffn / 1e3) / 1e12
    # the grouped FFN's minimum HBM traffic: every expert's weights once, its input
    # rows read, h written and read, y_perm written
    wbytes = 3.0 * wl.E * wl.d * wl.F * es
    act = wl.N * (wl.d * es * 2 + wl.F * es * 2)
    floor_ms = max(wl.expert_flops() / PEAK_BF16_TFLOPS / 1e9, (wbytes + act) / PEAK_HBM_GBS / 1e6)
    out = {"tokens_per_s": round(wl.T / (ms / 1e3), 1), "ms_per_step": round(ms, 4), "steps": steps,
           "tokens": wl.T, "experts": wl.E, "slots": wl.N, "routing": wl.routing,
           "grouped_ffn_ms": round(ffn, 4), "grouped_ffn_tflops": round(tflops, 1),
           "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
           "roofline_floor_ms": round(floor_ms, 4), "frac_of_roofline_floor": round(floor_ms / ffn, 4),
           "stages_ms": {k_: round(v, 4) for k_, v in stages.items()}}
    del L, inp
    torch.cuda.empty_cache()
    return out


NS_METRIC = "Muon Newton-Schulz expert matrices/s (5 quintic steps, d6144 x F1792, bf16)"


def ns_flops(R, C, steps):
    """Algorithmic FLOPs of the iteration on one R x C matrix (wide side C):
    X X^T, A A and B X per step."""
    r, c = min(R, C), max(R, C)
    return steps * (2 * r * r * c + 2 * r * r * r + 2 * r * r * c)


def bench_newton_schulz(args, torch, B):
    """One step: the gate and up matrices [F, d] and the down matrices [d, F] of
    args.ns_experts experts (two calls: one per orientation)."""
    import numpy as np
    d, F, steps = 6144, 1792, 5
    n = args.ns_experts
    g = torch.Generator(device="cuda:0").manual_seed(0)
    wide = torch.randn(2 * n, F, d, generator=g, device="cuda:0").to(torch.bfloat16)
    tall = torch.randn(n, d, F, generator=g, device="cuda:0").to(torch.bfloat16)
    calls = [B.NewtonSchulz(wide, steps), B.NewtonSchulz(tall, steps)]
    for _ in range(args.warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        for c in calls:
            c()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    mats = 3 * n
    flops = mats * ns_flops(F, d, steps)
    tflops = flops / (ms / 1e3) / 1e12
    out = {
        "metric": NS_METRIC, "value": round(mats / (ms / 1e3), 2), "unit": "matrices/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded random bf16 matrices of the page's expert shapes)",
        "config": {"workload": f"muon_ns_{n}_experts", "matrices": mats, "wide": [2 * n, F, d],
                   "tall": [n, d, F], "ns_steps": steps},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "moe_newton_schulz (3 batched GEMM launches per step)",
                     "flops_per_launch": flops, "ms_per_launch": round(ms, 3)},
    }
    if args.cpu_tokens > 0:
        from threadpoolctl import threadpool_info
        from oracle import muon_oracle as orc
        G = wide[0].float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        orc.newton_schulz(G, steps=steps)
        dt = time.perf_counter() - t0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        out["cpu_baseline"] = {"value": round(1.0 / dt, 4), "unit": "matrices/s", "cores": threads,
                               "kind": "oracle",
                               "sample": f"one {F}x{d} matrix, float64 oracle, {steps} steps: {dt:.1f} s on "
                                         f"{threads} BLAS threads of {os.cpu_count()} host CPUs"}
    print(json.dumps(out), flush=True)


BWD_METRIC = "MoE-layer backward tokens/s + expert-backward % bf16 MFMA peak (d6144,E384,top8)"


class _ExpertBits:
    """Per-expert bf16 weights as uint16 bit patterns on the host (the oracle
    widens them to float64 one expert at a time)."""

    def __init__(self, torch, t):
        import numpy as np
        self.h = t.cpu()
        self.np, self.torch = np, torch

    def __len__(self):
        return self.h.shape[0]

    def __getitem__(self, e):
        return self.h[e].view(self.torch.int16).numpy().view(self.np.uint16)


def bench_backward(args, torch, B, W):
    """One step: moe_layer_backward over the whole workload from the forward's
    routing, expert outputs and kept gate/up pre-activations (computed once,
    beforehand, by the forward's own entry points) and a seeded output gradient.
    Algorithmic work of the expert part 12 N d F (dH, dX, three weight
    gradients).  The same step with G and U recomputed instead (4 N d F more
    work, no kept activations) is timed too and reported under "recompute"."""
    import numpy as np
    wl = W.WORKLOADS[args.workload]
    dev = "cuda:0"
    inp = W.make_inputs(wl, device=dev)
    x, wr, wg, wu, wd = inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"]
    if wr is not None:
        ids, w, _ = B.moe_route(x, wr, wl.k, bias=inp["bias"], want_logits=False)
    else:
        ids, w = inp["topk_ids"], inp["topk_w"]
    off, rt, sr, _ = B.moe_permute(x, ids, wl.E, copy_rows=False)
    gu = torch.empty(rt.numel(), 2 * wl.F, dtype=wl.dtype, device=dev)
    y_perm = B.moe_grouped_ffn(x, off, wg, wu, wd, a_rows=rt, n_max=rt.numel(), gu_out=gu)
    dy = W.output_grad(wl.T, wl.d, wl.dtype, dev, seed=1)
    n = int(off[-1])

    def timed(fn, reps):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / reps

    def layer_ms(kept):
        L = B.LayerBackward(x, wr, wg, wu, wd, ids, w, y_perm, dy, gu=kept)
        for _ in range(args.warmup):
            L()
        torch.cuda.synchronize()
        t = timed(L, args.steps)
        del L
        torch.cuda.empty_cache()
        return t

    ms = layer_ms(gu)
    ms_recompute = layer_ms(None)

    # stage by stage, each on its own (same kernels as inside moe_layer_backward)
    dy_perm = torch.empty(rt.numel(), wl.d, dtype=wl.dtype, device=dev)
    stages = {}
    stages["permute"] = timed(lambda: B.moe_permute(x, ids, wl.E, copy_rows=False), 2)
    stages["combine_backward"] = timed(lambda: B.moe_combine_backward(dy, y_perm, sr, w, dy_perm=dy_perm), 2)
    _, gw = B.moe_combine_backward(dy, y_perm, sr, w, dy_perm=dy_perm)
    ffn = B.GroupedFfnBackward(x, off, wg, wu, wd, dy_perm, a_rows=rt, gu=gu)
    ffn()
    ffn_ms = timed(ffn, 2)
    stages["grouped_ffn_backward"] = ffn_ms
    dxp = ffn.dx
    del ffn
    torch.cuda.empty_cache()
    ffn = B.GroupedFfnBackward(x, off, wg, wu, wd, dy_perm, a_rows=rt)
    ffn()
    ffn_ms_recompute = timed(ffn, 2)
    del ffn
    torch.cuda.empty_cache()
    if wr is not None:
        stages["route_backward"] = timed(lambda: B.moe_route_backward(x, wr, ids, w, gw, dx_perm=dxp, slot_row=sr), 2)
    flops = 12 * n * wl.d * wl.F
    tflops = flops / (ffn_ms / 1e3) / 1e12
    tflops_recompute = flops / (ffn_ms_recompute / 1e3) / 1e12
    out = {
        "metric": BWD_METRIC, "value": round(wl.T / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded random inputs, weights and output gradient of the page's layer shape; routing, "
                "expert outputs and gate/up pre-activations from the forward's entry points)",
        "config": {"workload": wl.name + "_backward", "tokens": wl.T, "hidden": wl.d, "experts": wl.E,
                   "top_k": wl.k, "expert_hidden": wl.F, "slots": n},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "kernel": "grouped expert-FFN backward from the kept G | U (5 GEMM launches, activation "
                               "transposes; weights read in place)",
                     "flops_per_launch": flops, "ms_per_launch": round(ffn_ms, 4),
                     "note": "achieved counts 12 N d F (dH, dX, three weight gradients)"},
        "stages_ms": {k_: round(v, 4) for k_, v in stages.items()},
        "recompute": {"ms_per_step": round(ms_recompute, 4), "tokens_per_s": round(wl.T / (ms_recompute / 1e3), 1),
                      "grouped_ffn_backward_ms": round(ffn_ms_recompute, 4),
                      "grouped_ffn_backward_tflops": round(tflops_recompute, 1),
                      "mfma_frac": round(tflops_recompute / PEAK_BF16_TFLOPS, 4),
                      "note": "G and U recomputed by a gate/up GEMM (4 N d F more work) instead of kept by the "
                              "forward; achieved counts 12 N d F"},
    }
    if args.cpu_tokens > 0:
        from threadpoolctl import threadpool_info
        from oracle import moe_layer_backward_oracle as lbo
        nt = min(args.cpu_tokens, wl.T)
        ids_h = ids[:nt].cpu().numpy()
        w_h = w[:nt].cpu().numpy()
        f64 = lambda t: t.float().cpu().numpy().astype(np.float64)
        slots = int((ids_h >= 0).sum())
        rng = np.random.default_rng(2)
        yp = rng.standard_normal((slots, wl.d))
        dyh = rng.standard_normal((nt, wl.d))
        Xh = f64(x[:nt])
        Wr = f64(wr) if wr is not None else None
        ew = [_ExpertBits(torch, t) for t in (wg, wu, wd)]
        t0 = time.perf_counter()
        lbo.layer_backward(Xh, Wr, ew[0], ew[1], ew[2], ids_h, w_h, yp, dyh)
        dt = time.perf_counter() - t0
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        used = len(np.unique(ids_h[ids_h >= 0]))
        out["cpu_baseline"] = {"value": round(nt / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"first {nt} of {wl.T} tokens ({slots} slots, {used} experts): float64 "
                                         f"layer backward (combine, expert, gate-weight/router and permutation "
                                         f"backward) {dt:.1f} s on {threads} BLAS threads"}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(expert-parallel sharding of the layer is a design, not code).", file=sys.stderr)
        sys.exit(2)

    import torch
    from mixture_experts_layer_16_amd import binding as B
    from mixture_experts_layer_16_amd import workloads as W

    torch.cuda.set_device(0)
    if args.path == "newton_schulz":
        bench_newton_schulz(args, torch, B)
        return
    if args.path == "backward":
        bench_backward(args, torch, B, W)
        return
    if args.cpu_only:
        cpu_only(args, torch, W)
        return
    wl = W.WORKLOADS[args.workload]
    if args.traffic_probe:
        traffic_probe(torch, B, W, wl)
        return
    inp = W.make_inputs(wl, device="cuda:0")
    L = B.LayerForward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"], inp["w_down"], wl.k,
                       topk_ids=inp.get("topk_ids"), topk_w=inp.get("topk_w"))
    for _ in range(args.warmup):
        L()
    torch.cuda.synchronize()

    # one event between consecutive steps (no synchronisation inside the timed region)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(args.steps):
        L()
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    tokens_per_s = wl.T / (ms / 1e3)

    stages = stage_pass(torch, B, inp, wl, max(2, min(args.steps, 5)))
    ffn_ms = stages["grouped_ffn"]
    peak = PEAK_BF16_TFLOPS if wl.dtype == torch.bfloat16 else PEAK_F32_TFLOPS
    ffn_tflops = wl.expert_flops() / (ffn_ms / 1e3) / 1e12
    total_tflops = (wl.expert_flops() + wl.router_flops()) / (ms / 1e3) / 1e12
    es = 2 if wl.dtype == torch.bfloat16 else 4
    traffic = None
    if TRAFFIC and TRAFFIC["kernel_source_hash"] == kernel_source_hash() and TRAFFIC["workload"] == wl.name:
        traffic = TRAFFIC["bytes"]
    if args.no_kernel_split:
        kernels = {"skipped": "--no-kernel-split"}
    else:
        try:
            km = kernel_split(torch, L, inp["w_router"] is not None)
            kernels = kernel_fractions(wl, es, km)
        except Exception as exc:          # the profiler is a measurement aid, not the product
            kernels = {"error": f"{type(exc).__name__}: {exc}"}
    route = None
    if "router_gemm" in kernels and "topk" in kernels:
        route = {"router_gemm_ms": kernels["router_gemm"]["ms"], "router_mfma_frac": kernels["router_gemm"]["mfma_frac"],
                 "topk_ms": kernels["topk"]["ms"], "topk_hbm_frac": kernels["topk"]["hbm_frac"],
                 "route_ms": round(stages["route"], 4)}

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded random inputs and weights of the page's layer shape)",
        "config": {"workload": wl.name, "tokens": wl.T, "hidden": wl.d, "experts": wl.E, "top_k": wl.k,
                   "expert_hidden": wl.F, "routing": wl.routing, "slots": wl.N},
        "roofline": {"bound": "mfma", "achieved": round(ffn_tflops, 1), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(ffn_tflops / peak, 4), "traffic": traffic,
                     "kernel": "grouped SwiGLU FFN (gate/up + down GEMM launches)",
                     "flops_per_launch": wl.expert_flops(), "ms_per_launch": round(ffn_ms, 4)},
        "tflops_layer": round(total_tflops, 1),
        "step_ms": {"median": round(per_step[len(per_step) // 2], 4), "min": round(per_step[0], 4)},
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "route": route,
        "kernels": kernels,
    }
    # the same forward for training: y_perm and the gate/up pre-activations G | U
    # written to the caller's buffers for the backward
    LT = B.LayerForward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"], inp["w_down"], wl.k,
                        topk_ids=inp.get("topk_ids"), topk_w=inp.get("topk_w"), want_y_perm=True, want_gu=True)
    LT()
    ms_train = time_layer(torch, LT, max(2, min(args.steps, 5)))
    out["training_forward"] = {"ms_per_step": round(ms_train, 4), "tokens_per_s": round(wl.T / (ms_train / 1e3), 1),
                               "note": "moe_layer_forward also writing y_perm and G | U for the backward"}
    del LT
    torch.cuda.empty_cache()
    if args.cpu_tokens > 0:
        out["cpu_baseline"] = cpu_baseline(torch, inp, wl, args.cpu_tokens)
    del L, inp
    torch.cuda.empty_cache()
    others = {}
    for name in [w for w in args.other_workloads.split(",") if w and w != wl.name]:
        others[name] = other_workload(torch, B, W, name, min(args.steps, 10), max(1, min(args.warmup, 3)))
    if others:
        out["other_workloads"] = others
    if args.cpu_tokens > 0:
        small = W.WORKLOADS["small_bf16"]
        sinp = W.make_inputs(small, device="cuda:0")
        n, slots, t, flops = cpu_oracle_run(torch, sinp, small, 0, repeats=3)
        out["cpu_oracle"] = {"small_bf16": {"tokens": n, "slots": slots, "runs": 3,
                                            "stages_s": {k_: round(v, 4) for k_, v in t.items()},
                                            "tokens_per_s": round(n / t["layer"], 2),
                                            "gflops": round(flops / t["layer"] / 1e9, 2)}}
        del sinp
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
