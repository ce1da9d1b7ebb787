"""The layer's entry points under HIP graph capture.

Every entry point only enqueues kernels on the caller's stream (no allocation,
no memset node, no host synchronisation), so a whole layer forward, a whole
layer backward or a Newton-Schulz call can be captured once and replayed.  Each
test captures one call with its outputs and workspace allocated beforehand,
replays the graph several times with eager work and synchronisations between the
replays, and checks every replay bit for bit against the eager call.
"""
import pytest
import torch

from mixture_experts_layer_16_amd import binding as B
from mixture_experts_layer_16_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def replay_and_check(graph, outputs, expected, scribble):
    for i in range(4):
        for o in outputs:                      # make stale results visible
            o.fill_(float("nan")) if o.is_floating_point() else o.fill_(-7)
        scribble()                             # unrelated eager work on the same stream
        graph.replay()
        torch.cuda.synchronize()
        for o, e in zip(outputs, expected):
            assert torch.equal(bits(o), bits(e)), f"replay {i} differs"


def test_layer_forward_graph_replays_match_eager():
    print("[graph] layer forward", flush=True)
    wl = W.WORKLOADS["small_bf16"]
    inp = W.make_inputs(wl, device=DEV)
    L = B.LayerForward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"], inp["w_down"], wl.k,
                       want_logits=True, want_routing=True)
    L()
    torch.cuda.synchronize()
    expected = [L.y.clone(), L.logits.clone(), L.topk_ids.clone(), L.topk_w.clone()]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            L()
    torch.cuda.current_stream().wait_stream(s)
    junk = torch.randn(1 << 20, device=DEV)
    replay_and_check(g, [L.y, L.logits, L.topk_ids, L.topk_w], expected, lambda: junk.mul_(1.0001))


def test_layer_backward_graph_replays_match_eager():
    print("[graph] layer backward", flush=True)
    T, d, E, k, F = 1000, 256, 16, 4, 128
    wl = W.Workload("graph_bwd", T, d, E, k, F, torch.bfloat16, routing="router_bias")
    inp = W.make_inputs(wl, device=DEV)
    ids, w, _ = B.moe_route(inp["x"], inp["w_router"], k, bias=inp["bias"], want_logits=False)
    off, rt, sr, _ = B.moe_permute(inp["x"], ids, E, copy_rows=False)
    y_perm = B.moe_grouped_ffn(inp["x"], off, inp["w_gate"], inp["w_up"], inp["w_down"], a_rows=rt, n_max=T * k)
    dy = W.output_grad(T, d, torch.bfloat16, DEV, seed=3)
    L = B.LayerBackward(inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"], ids, w, y_perm, dy,
                        want_d_topk_w=True)
    L()
    torch.cuda.synchronize()
    outs = [L.dx, L.dw_router, L.dbias, L.dw_gate, L.dw_up, L.dw_down, L.d_topk_w]
    expected = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            L()
    torch.cuda.current_stream().wait_stream(s)
    junk = torch.randn(1 << 20, device=DEV)
    replay_and_check(g, outs, expected, lambda: junk.mul_(1.0001))


def test_training_step_graph_replays_match_eager():
    # one training step's layer work in one graph: the forward keeping y_perm and
    # G | U, then the backward reading them
    print("[graph] forward keeping G|U + backward from it", flush=True)
    T, d, E, k, F = 900, 256, 16, 4, 192
    wl = W.Workload("graph_train", T, d, E, k, F, torch.bfloat16, routing="router_bias", seed=2)
    inp = W.make_inputs(wl, device=DEV)
    LF = B.LayerForward(inp["x"], inp["w_router"], inp["bias"], inp["w_gate"], inp["w_up"], inp["w_down"], k,
                        want_routing=True, want_y_perm=True, want_gu=True)
    LF()
    torch.cuda.synchronize()
    dy = W.output_grad(T, d, torch.bfloat16, DEV, seed=5)
    LB = B.LayerBackward(inp["x"], inp["w_router"], inp["w_gate"], inp["w_up"], inp["w_down"], LF.topk_ids,
                         LF.topk_w, LF.y_perm, dy, want_d_topk_w=True, gu=LF.gu)
    LB()
    torch.cuda.synchronize()
    outs = [LF.y, LF.topk_ids, LF.topk_w, LB.dx, LB.dw_router, LB.dbias, LB.dw_gate, LB.dw_up, LB.dw_down,
            LB.d_topk_w]
    expected = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            LF()
            LB()
    torch.cuda.current_stream().wait_stream(s)
    junk = torch.randn(1 << 20, device=DEV)
    replay_and_check(g, outs, expected, lambda: junk.mul_(1.0001))


def test_newton_schulz_graph_replays_match_eager():
    print("[graph] newton-schulz", flush=True)
    gen = torch.Generator(device=DEV).manual_seed(4)
    gm = torch.randn(3, 192, 448, generator=gen, device=DEV).to(torch.bfloat16)
    ns = B.NewtonSchulz(gm)
    ns()
    torch.cuda.synchronize()
    expected = [ns.x.clone()]
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            ns()
    torch.cuda.current_stream().wait_stream(s)
    junk = torch.randn(1 << 20, device=DEV)
    replay_and_check(g, [ns.x], expected, lambda: junk.mul_(1.0001))
