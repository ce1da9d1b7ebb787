"""Thin ctypes binding of libmoe.so.

Argument marshalling only: each function takes torch device tensors, allocates
outputs and the workspace with torch on the same device, passes raw pointers
and the current HIP stream to the C ABI, and turns a non-zero status into an
exception.  Every step of the layer runs in the library's HIP kernels; there is
no fallback of any kind, and a missing library is an error.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}
EXPORTS = ("moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer_forward", "moe_newton_schulz",
           "moe_grouped_ffn_backward", "moe_combine_backward", "moe_route_backward", "moe_layer_backward",
           "moe_layer_forward_noalloc")


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}")
        self.status = status


_lib: Optional[ctypes.CDLL] = None

_i64, _int, _vp, _szp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)
_f32 = ctypes.c_float
_SIGS = {
    "moe_route": [_i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _szp, _vp],
    "moe_permute": [_i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _szp, _vp],
    "moe_grouped_ffn": [_i64, _i64, _i64, _i64, _int, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _szp, _vp],
    "moe_combine": [_i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp],
    "moe_layer_forward": [_i64, _i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                          _vp, _vp, _vp, _vp, _szp, _vp],
    "moe_layer_forward_noalloc": [_i64, _i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                  _vp, _vp, _vp, _vp, _vp],
    "moe_newton_schulz": [_i64, _i64, _i64, _int, _i64, _f32, _f32, _f32, _f32, _vp, _vp, _vp, _szp, _vp],
    "moe_grouped_ffn_backward": [_i64, _i64, _i64, _i64, _int, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp, _szp, _vp],
    "moe_combine_backward": [_i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp],
    "moe_route_backward": [_i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           _szp, _vp],
    "moe_layer_backward": [_i64, _i64, _i64, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _szp, _vp],
}

MUON_COEFFS = (3.4445, -4.7750, 2.0315)


def lib() -> ctypes.CDLL:
    """Load libmoe.so (built in-tree by __graft_entry__.build())."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def dtype_code(dt: torch.dtype) -> int:
    if dt == torch.float32:
        return MOE_F32
    if dt == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(fn: str, st: int):
    if st != 0:
        raise MoEError(fn, st)


def _query(fn: str, *args) -> int:
    """Workspace size for a call (the same arguments with ws = NULL)."""
    n = ctypes.c_size_t(0)
    _check(fn, getattr(lib(), fn)(*args, None, ctypes.byref(n), None))
    return n.value


def _ws(nbytes: int, dev) -> torch.Tensor:
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)


def moe_route(x, w_router, k: int, bias=None, want_logits: bool = True):
    """Router GEMM + softmax + top-k.  Returns (topk_ids, topk_w, logits|None)."""
    T, d = x.shape
    E = w_router.shape[0]
    dev = x.device
    ids = torch.empty(T, k, dtype=torch.int32, device=dev)
    w = torch.empty(T, k, dtype=torch.float32, device=dev)
    logits = torch.empty(T, E, dtype=torch.float32, device=dev) if want_logits else None
    head = (T, d, E, k, dtype_code(x.dtype), _p(x), _p(w_router), _p(bias), _p(logits), _p(ids), _p(w))
    need = _query("moe_route", *head)
    ws = _ws(need, dev)
    n = ctypes.c_size_t(ws.numel())
    _check("moe_route", lib().moe_route(*head, _p(ws), ctypes.byref(n), _stream(dev)))
    return ids, w, logits


def moe_permute(x, topk_ids, num_experts: int, copy_rows: bool = True):
    """Returns (offsets [E+1], row_token [T*k], slot_row [T,k], x_perm [T*k, d] | None).
    copy_rows=False produces only the indices (x_perm is None)."""
    T, d = x.shape
    k = topk_ids.shape[1]
    dev = x.device
    offsets = torch.empty(num_experts + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(T * k, dtype=torch.int32, device=dev)
    slot_row = torch.empty(T, k, dtype=torch.int32, device=dev)
    x_perm = torch.empty(T * k, d, dtype=x.dtype, device=dev) if copy_rows else None
    head = (T, d, num_experts, k, dtype_code(x.dtype), _p(x), _p(topk_ids), _p(offsets), _p(row_token),
            _p(slot_row), _p(x_perm))
    ws = _ws(_query("moe_permute", *head), dev)
    n = ctypes.c_size_t(ws.numel())
    _check("moe_permute", lib().moe_permute(*head, _p(ws), ctypes.byref(n), _stream(dev)))
    return offsets, row_token, slot_row, x_perm


def moe_grouped_ffn(x_in, offsets, w_gate, w_up, w_down, y_perm=None, a_rows=None, n_max=None, gu_out=None):
    """y_perm [n_max, d]: the SwiGLU FFN of each expert over its rows.  Without
    a_rows, x_in is x_perm (rows grouped by expert); with a_rows (row_token from
    moe_permute), x_in is the token matrix x read in place.  gu_out [n_max, 2F]
    (optional) receives the gate and up pre-activations for the backward."""
    d = x_in.shape[1]
    if a_rows is None:
        n_max, n_in = x_in.shape[0], 0
    else:
        n_max, n_in = (a_rows.numel() if n_max is None else n_max), x_in.shape[0]
    E, F, _ = w_gate.shape
    dev = x_in.device
    if y_perm is None:
        y_perm = torch.empty(n_max, d, dtype=x_in.dtype, device=dev)
    head = (n_max, d, E, F, dtype_code(x_in.dtype), _p(x_in), n_in, _p(a_rows), _p(offsets), _p(w_gate), _p(w_up),
            _p(w_down), _p(y_perm), _p(gu_out))
    ws = _ws(_query("moe_grouped_ffn", *head), dev)
    n = ctypes.c_size_t(ws.numel())
    _check("moe_grouped_ffn", lib().moe_grouped_ffn(*head, _p(ws), ctypes.byref(n), _stream(dev)))
    return y_perm


def moe_combine(y_perm, slot_row, topk_w, out=None):
    """y [T, d] = sum_j topk_w[t, j] * y_perm[slot_row[t, j]]."""
    T, k = slot_row.shape
    d = y_perm.shape[1]
    y = torch.empty(T, d, dtype=y_perm.dtype, device=y_perm.device) if out is None else out
    _check("moe_combine", lib().moe_combine(T, d, k, dtype_code(y_perm.dtype), _p(y_perm), _p(slot_row),
                                            _p(topk_w), _p(y), _stream(y_perm.device)))
    return y


class GroupedFfnBackward:
    """moe_grouped_ffn_backward with its outputs and workspace allocated once.
    x_in is x_perm, or (a_rows given) the token matrix read through a_rows; gu
    the forward's gate/up pre-activations (moe_grouped_ffn's gu_out), or None to
    recompute them."""

    def __init__(self, x_in, offsets, w_gate, w_up, w_down, dy_perm, a_rows=None, gu=None):
        E, F, d = w_gate.shape
        n_max = dy_perm.shape[0]
        dev = dy_perm.device
        n_in = x_in.shape[0] if a_rows is not None else 0
        self.t = (x_in, offsets, w_gate, w_up, w_down, dy_perm, a_rows, gu)
        self.dx = torch.empty(n_max, d, dtype=dy_perm.dtype, device=dev)
        self.dwg = torch.empty(E, F, d, dtype=torch.float32, device=dev)
        self.dwu = torch.empty(E, F, d, dtype=torch.float32, device=dev)
        self.dwd = torch.empty(E, d, F, dtype=torch.float32, device=dev)
        self.head = (n_max, d, E, F, dtype_code(dy_perm.dtype))
        self.mid = (_p(x_in), n_in, _p(a_rows), _p(offsets), _p(w_gate), _p(w_up), _p(w_down), _p(dy_perm),
                    _p(gu), _p(self.dx), _p(self.dwg), _p(self.dwu), _p(self.dwd))
        self.ws = _ws(_query("moe_grouped_ffn_backward", *self.head, *self.mid), dev)

    def __call__(self):
        n = ctypes.c_size_t(self.ws.numel())
        _check("moe_grouped_ffn_backward",
               lib().moe_grouped_ffn_backward(*self.head, *self.mid, _p(self.ws), ctypes.byref(n),
                                              _stream(self.dx.device)))
        return self.dx, self.dwg, self.dwu, self.dwd


def moe_grouped_ffn_backward(x_in, offsets, w_gate, w_up, w_down, dy_perm, a_rows=None, gu=None):
    """(dx_perm, dW_gate, dW_up, dW_down) of the grouped SwiGLU FFN."""
    return GroupedFfnBackward(x_in, offsets, w_gate, w_up, w_down, dy_perm, a_rows, gu)()


def moe_combine_backward(dy, y_perm, slot_row, topk_w, dy_perm=None):
    """Backward of moe_combine: returns (dy_perm, d_topk_w).  dy_perm rows that no
    slot refers to are left as allocated (zero when allocated here)."""
    T, k = slot_row.shape
    d = dy.shape[1]
    dev = dy.device
    if dy_perm is None:
        dy_perm = torch.zeros(y_perm.shape[0], d, dtype=dy.dtype, device=dev)
    g = torch.empty(T, k, dtype=torch.float32, device=dev)
    _check("moe_combine_backward",
           lib().moe_combine_backward(T, d, k, dtype_code(dy.dtype), _p(dy), _p(y_perm), _p(slot_row), _p(topk_w),
                                      _p(dy_perm), _p(g), _stream(dev)))
    return dy_perm, g


def moe_route_backward(x, w_router, topk_ids, topk_w, d_topk_w, dx_perm=None, slot_row=None, want_bias=True,
                       want_dlogits=False):
    """Backward of moe_route (plus the permutation's when dx_perm and slot_row are
    given).  Returns (dx, dW_router, dbias | None, dlogits | None)."""
    T, d = x.shape
    E = w_router.shape[0]
    k = topk_ids.shape[1]
    dev = x.device
    dx = torch.empty(T, d, dtype=x.dtype, device=dev)
    dwr = torch.empty(E, d, dtype=torch.float32, device=dev)
    db = torch.empty(E, dtype=torch.float32, device=dev) if want_bias else None
    dl = torch.empty(T, E, dtype=torch.float32, device=dev) if want_dlogits else None
    head = (T, d, E, k, dtype_code(x.dtype), _p(x), _p(w_router), _p(topk_ids), _p(topk_w), _p(d_topk_w),
            _p(dx_perm), _p(slot_row), _p(dx), _p(dwr), _p(db), _p(dl))
    ws = _ws(_query("moe_route_backward", *head), dev)
    n = ctypes.c_size_t(ws.numel())
    _check("moe_route_backward", lib().moe_route_backward(*head, _p(ws), ctypes.byref(n), _stream(dev)))
    return dx, dwr, db, dl


class LayerBackward:
    """moe_layer_backward with its outputs and workspace allocated once.  The
    forward's routing (topk_ids, topk_w) and expert outputs y_perm (rows in the
    permutation's order) are inputs; w_router None means pre-routed slots; gu the
    forward's gate/up pre-activations (moe_layer_forward's want_gu), or None to
    recompute them."""

    def __init__(self, x, w_router, w_gate, w_up, w_down, topk_ids, topk_w, y_perm, dy, want_bias: bool = True,
                 want_d_topk_w: bool = False, gu=None):
        T, d = x.shape
        E, F, _ = w_gate.shape
        k = topk_ids.shape[1]
        dev = x.device
        routed = w_router is not None
        self.t = (x, w_router, w_gate, w_up, w_down, topk_ids, topk_w, y_perm, gu, dy)
        self.dx = torch.empty(T, d, dtype=x.dtype, device=dev)
        self.dw_router = torch.empty(E, d, dtype=torch.float32, device=dev) if routed else None
        self.dbias = torch.empty(E, dtype=torch.float32, device=dev) if (routed and want_bias) else None
        self.dw_gate = torch.empty(E, F, d, dtype=torch.float32, device=dev)
        self.dw_up = torch.empty(E, F, d, dtype=torch.float32, device=dev)
        self.dw_down = torch.empty(E, d, F, dtype=torch.float32, device=dev)
        self.d_topk_w = torch.empty(T, k, dtype=torch.float32, device=dev) if want_d_topk_w else None
        self._head = (T, d, E, k, F, dtype_code(x.dtype), _p(x), _p(w_router), _p(w_gate), _p(w_up), _p(w_down),
                      _p(topk_ids), _p(topk_w), _p(y_perm), _p(gu), _p(dy), _p(self.dx), _p(self.dw_router),
                      _p(self.dbias), _p(self.dw_gate), _p(self.dw_up), _p(self.dw_down), _p(self.d_topk_w))
        self.ws = _ws(_query("moe_layer_backward", *self._head), dev)
        self._n = ctypes.c_size_t(self.ws.numel())
        self._ws_p = _p(self.ws)

    def __call__(self):
        _check("moe_layer_backward", lib().moe_layer_backward(*self._head, self._ws_p, ctypes.byref(self._n),
                                                              _stream(self.dx.device)))
        return self


def moe_layer_backward(x, w_router, w_gate, w_up, w_down, topk_ids, topk_w, y_perm, dy, want_bias=True,
                       want_d_topk_w=False, gu=None):
    """One call of the whole layer backward; returns the LayerBackward object
    holding dx, dw_router, dbias, dw_gate, dw_up, dw_down and d_topk_w."""
    return LayerBackward(x, w_router, w_gate, w_up, w_down, topk_ids, topk_w, y_perm, dy, want_bias,
                         want_d_topk_w, gu)()


class NewtonSchulz:
    """moe_newton_schulz on a fixed batch [n, R, C] (bf16) with its output and
    workspace allocated once."""

    def __init__(self, g, steps: int = 5, coeffs=MUON_COEFFS, eps: float = 1e-7):
        if g.dim() == 2:
            g = g.unsqueeze(0)
        self.g, self.steps, self.coeffs, self.eps = g, steps, coeffs, eps
        n, R, C = g.shape
        self.args = (n, R, C, dtype_code(g.dtype), steps, *coeffs, eps)
        self.x = torch.empty_like(g)
        self.ws = _ws(_query("moe_newton_schulz", *self.args, _p(g), _p(self.x)), g.device)

    def __call__(self):
        n = ctypes.c_size_t(self.ws.numel())
        _check("moe_newton_schulz", lib().moe_newton_schulz(*self.args, _p(self.g), _p(self.x), _p(self.ws),
                                                            ctypes.byref(n), _stream(self.g.device)))
        return self.x


def moe_newton_schulz(g, steps: int = 5, coeffs=MUON_COEFFS, eps: float = 1e-7):
    """Muon's Newton-Schulz orthogonalisation of g [R, C] or [n, R, C] (bf16)."""
    out = NewtonSchulz(g, steps, coeffs, eps)()
    return out if g.dim() == 3 else out[0]


class LayerForward:
    """moe_layer_forward with its outputs and workspace allocated once, so that
    repeated calls (benchmarks, graph capture) allocate nothing."""

    def __init__(self, x, w_router, bias, w_gate, w_up, w_down, k: int, topk_ids=None, topk_w=None,
                 want_logits: bool = False, want_routing: bool = False, want_offsets: bool = False,
                 want_y_perm: bool = False, want_gu: bool = False):
        self.x, self.w_router, self.bias = x, w_router, bias
        self.w_gate, self.w_up, self.w_down = w_gate, w_up, w_down
        T, d = x.shape
        E, F, _ = w_gate.shape
        self.T, self.d, self.E, self.k, self.F = T, d, E, k, F
        dev = x.device
        self.y = torch.empty(T, d, dtype=x.dtype, device=dev)
        routed = w_router is not None
        self.logits = torch.empty(T, E, dtype=torch.float32, device=dev) if (routed and want_logits) else None
        if routed:
            self.topk_ids = torch.empty(T, k, dtype=torch.int32, device=dev) if want_routing else None
            self.topk_w = torch.empty(T, k, dtype=torch.float32, device=dev) if want_routing else None
        else:
            self.topk_ids, self.topk_w = topk_ids, topk_w
        self.offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if want_offsets else None
        # training: the expert outputs and gate/up pre-activations the backward takes
        self.y_perm = torch.empty(T * k, d, dtype=x.dtype, device=dev) if want_y_perm else None
        self.gu = torch.empty(T * k, 2 * F, dtype=x.dtype, device=dev) if want_gu else None
        self._head = (T, d, E, k, F, dtype_code(x.dtype), _p(x), _p(w_router), _p(bias), _p(w_gate), _p(w_up),
                      _p(w_down), _p(self.y), _p(self.logits), _p(self.topk_ids), _p(self.topk_w),
                      _p(self.offsets), _p(self.y_perm), _p(self.gu))
        self.ws = _ws(_query("moe_layer_forward", *self._head), dev)
        self._n = ctypes.c_size_t(self.ws.numel())
        self._ws_p = _p(self.ws)

    def __call__(self):
        _check("moe_layer_forward", lib().moe_layer_forward(*self._head, self._ws_p, ctypes.byref(self._n),
                                                            _stream(self.x.device)))
        return self.y


def moe_layer_forward(x, w_router, bias, w_gate, w_up, w_down, k: int, topk_ids=None, topk_w=None,
                      want_logits=False, want_routing=False, want_offsets=False, want_y_perm=False, want_gu=False):
    """One call of the whole layer; returns the LayerForward object holding y
    and the optional outputs."""
    L = LayerForward(x, w_router, bias, w_gate, w_up, w_down, k, topk_ids, topk_w, want_logits, want_routing,
                     want_offsets, want_y_perm, want_gu)
    L()
    return L
