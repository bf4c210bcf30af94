"""ctypes marshalling for libgdr.so.  No arithmetic of the operator lives here."""
from __future__ import annotations

import ctypes
import os
import threading

import torch

GATE_NONE, GATE_SCALAR, GATE_CHANNEL = 0, 1, 2
ROUTE_VALUE, ROUTE_ERROR = 0, 1
PROLOGUE_NONE, PROLOGUE_ALPHA_SIGMOID, PROLOGUE_ALPHA_FORGET = 0, 1, 2
_BF16, _FP32 = 0, 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdr.so")
_lock = threading.Lock()
_lib = None


class GdrError(RuntimeError):
    """A non-OK status from libgdr (``code`` is the gdr_status value)."""

    def __init__(self, code: int, msg: str):
        super().__init__("%s: %s" % (_STATUS.get(code, "GDR_ERR_%d" % code), msg))
        self.code = code


_STATUS = {0: "GDR_OK", 1: "GDR_ERR_INVALID_ARG", 2: "GDR_ERR_UNSUPPORTED", 3: "GDR_ERR_WORKSPACE",
           4: "GDR_ERR_DEVICE"}


class Desc(ctypes.Structure):
    """Mirror of ``gdr_desc`` in include/gdr.h."""

    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("H", ctypes.c_int64),
                ("dk", ctypes.c_int64), ("dv", ctypes.c_int64), ("gate", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("scale", ctypes.c_float), ("chunk", ctypes.c_int32), ("route", ctypes.c_int32),
                ("prologue", ctypes.c_int32)]


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Loads libgdr.so once; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libgdr.so is not built; run `python -m gated_delta_rule_37_amd.build` "
                              "(or __graft_entry__.build())")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I64, I32, F32, SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float,
                                ctypes.c_size_t)
        D = ctypes.POINTER(Desc)
        lib.gdr_workspace_size.argtypes = [D, ctypes.c_int]
        lib.gdr_workspace_size.restype = SZ
        lib.gdr_forward_chunked.argtypes = [D] + [P] * 10 + [P, SZ, P]
        lib.gdr_forward_chunked.restype = ctypes.c_int
        lib.gdr_forward_chunked_gated.argtypes = [D] + [P] * 12 + [P, SZ, P]
        lib.gdr_forward_chunked_gated.restype = ctypes.c_int
        lib.gdr_backward.argtypes = [D] + [P] * 17 + [P, SZ, P]
        lib.gdr_backward.restype = ctypes.c_int
        lib.gdr_forward_train.argtypes = [D] + [P] * 10 + [P, SZ, P]
        lib.gdr_forward_train.restype = ctypes.c_int
        lib.gdr_backward_saved.argtypes = [D] + [P] * 17 + [P, SZ, P]
        lib.gdr_backward_saved.restype = ctypes.c_int
        lib.gdr_decode_step.argtypes = [I64] * 4 + [I32] * 3 + [F32] + [P] * 7 + [P]
        lib.gdr_decode_step.restype = ctypes.c_int
        lib.gdr_output_gate_forward.argtypes = [D] + [P] * 4 + [P]
        lib.gdr_output_gate_forward.restype = ctypes.c_int
        lib.gdr_output_gate_workspace_size.argtypes = [D]
        lib.gdr_output_gate_workspace_size.restype = SZ
        lib.gdr_output_gate_backward.argtypes = [D] + [P] * 8 + [SZ, P]
        lib.gdr_output_gate_backward.restype = ctypes.c_int
        lib.gdr_status_string.argtypes = [ctypes.c_int]
        lib.gdr_status_string.restype = ctypes.c_char_p
        lib.gdr_last_error.argtypes = []
        lib.gdr_last_error.restype = ctypes.c_char_p
        lib.gdr_version.argtypes = []
        lib.gdr_version.restype = I32
        lib.gdr_gdn2_workspace_size.argtypes = [D]
        lib.gdr_gdn2_workspace_size.restype = SZ
        lib.gdr_gdn2_forward_chunked.argtypes = [D] + [P] * 9 + [P, SZ, P]
        lib.gdr_gdn2_forward_chunked.restype = ctypes.c_int
        lib.gdr_gdn2_decode_step.argtypes = [I64] * 4 + [I32] * 3 + [F32] + [P] * 8 + [P]
        lib.gdr_gdn2_decode_step.restype = ctypes.c_int
        _lib = lib
        return lib


def _check(code: int):
    if code != 0:
        raise GdrError(code, load_library().gdr_last_error().decode())


def _dt(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return _BF16
    if t == torch.float32:
        return _FP32
    raise TypeError("unsupported dtype %s (bf16 or fp32)" % t)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name, dtype=None, shape=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a GPU (got %s)" % (name, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


def _gate_of(alpha, q):
    if alpha is None:
        return GATE_NONE
    return GATE_SCALAR if alpha.dim() == 3 else GATE_CHANNEL


def _route(route):
    if route in (ROUTE_VALUE, "value"):
        return ROUTE_VALUE
    if route in (ROUTE_ERROR, "error"):
        return ROUTE_ERROR
    raise ValueError("route must be 'value' (CLVR) or 'error' (CLER-H), got %r" % (route,))


_PROLOGUES = {None: PROLOGUE_NONE, "none": PROLOGUE_NONE, "sigmoid": PROLOGUE_ALPHA_SIGMOID,
              "forget": PROLOGUE_ALPHA_FORGET}


def _prologue(p):
    if p in (PROLOGUE_NONE, PROLOGUE_ALPHA_SIGMOID, PROLOGUE_ALPHA_FORGET):
        return int(p)
    if p in _PROLOGUES:
        return _PROLOGUES[p]
    raise ValueError("prologue must be None, 'sigmoid' or 'forget' (or 0, 1, 2), got %r" % (p,))


def _desc(q, v, alpha, out_dtype, scale, route=ROUTE_VALUE, prologue=None):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    return Desc(B, T, H, dk, dv, _gate_of(alpha, q), _dt(q.dtype),
                _dt(out_dtype if out_dtype is not None else q.dtype), float(scale), 0, _route(route),
                _prologue(prologue))


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace_size(B, T, H, d, gate=GATE_CHANNEL, in_dtype=torch.bfloat16, out_dtype=None,
                   backward=False, route=ROUTE_VALUE, prologue=None) -> int:
    desc = Desc(B, T, H, d, d, gate, _dt(in_dtype), _dt(out_dtype or in_dtype), 1.0, 0, _route(route),
                _prologue(prologue))
    n = load_library().gdr_workspace_size(ctypes.byref(desc), 1 if backward else 0)
    if n == 0 and B * H * T > 0:
        _check(1)
    return int(n)


def _check_inputs(q, k, v, beta, alpha, S0):
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q")
    _need(k, "k", q.dtype, (B, T, H, dk))
    _need(v, "v", q.dtype, (B, T, H, dv))
    _need(beta, "beta", torch.float32, (B, T, H))
    if alpha is not None:
        if alpha.dim() == 3:
            _need(alpha, "alpha", torch.float32, (B, T, H))
        else:
            _need(alpha, "alpha", torch.float32, (B, T, H, dk))
    _need(S0, "S0", torch.float32, (B, H, dk, dv))
    return B, T, H, dk, dv


def forward(q, k, v, beta, alpha=None, S0=None, *, scale=1.0, out_dtype=None, h=None,
            clvr_scale=None, output_final_state=True, workspace=None, save_for_backward=False,
            route="value", prologue=None):
    """Chunked forward.  Returns ``(o, S_T)`` (``S_T`` None unless requested).

    ``h`` ([B, T, H*dv], q's dtype) is updated in place by the hidden-stream
    epilogue when given: ``h += clvr_scale * v`` (``route="value"``, CLVR) or
    ``h += clvr_scale * e`` with the write errors ``e_t = u_t / beta_t``
    (``route="error"``, CLER-H; every beta must be nonzero).

    ``prologue="sigmoid"`` or ``"forget"``: q and k are passed unnormalised and
    beta, alpha as logits; the library L2-normalises q and k and applies
    beta = sigmoid(b) and alpha = sigmoid(a) resp. exp(-softplus(a)).

    ``save_for_backward=True`` runs the training forward: ``workspace`` (a uint8
    tensor of ``workspace_size(..., backward=True)`` bytes, required) then holds
    the intermediates that ``backward(..., saved_workspace=workspace)`` reuses."""
    B, T, H, dk, dv = _check_inputs(q, k, v, beta, alpha, S0)
    _need(h, "h", q.dtype, (B, T, H * dv))
    _need(clvr_scale, "clvr_scale", torch.float32, (H * dv,))
    lib = load_library()
    desc = _desc(q, v, alpha, out_dtype, scale, route, prologue)
    o = torch.empty((B, T, H, dv), dtype=out_dtype or q.dtype, device=q.device)
    ST = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if output_final_state else None
    need = lib.gdr_workspace_size(ctypes.byref(desc), 1 if save_for_backward else 0)
    if save_for_backward:
        if workspace is None:
            raise ValueError("save_for_backward needs a workspace tensor that the backward will reuse")
        _need(workspace, "workspace", torch.uint8)
        if workspace.numel() < need:
            raise ValueError("workspace has %d bytes, the training forward needs %d" % (workspace.numel(), need))
    elif workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    fn = lib.gdr_forward_train if save_for_backward else lib.gdr_forward_chunked
    _check(fn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S0), _ptr(o),
              _ptr(ST), _ptr(h), _ptr(clvr_scale), _ptr(workspace), need, _stream(q.device)))
    return o, ST


def forward_gated(q, k, v, beta, alpha, g, w=None, S0=None, *, scale=1.0, out_dtype=None, h=None,
                  clvr_scale=None, output_final_state=True, workspace=None, route="value", prologue=None):
    """Inference forward with the output-gate epilogue (``gdr_forward_chunked_gated``).
    Returns ``(y, S_T)`` with ``y = sigmoid(g) * w * RMSNorm(o)`` per head, equal
    to :func:`output_gate` applied to :func:`forward`'s ``o``; ``o`` itself is
    not kept.  ``g`` is [B, T, H, dv] in q's dtype, ``w`` [H*dv] fp32 or None
    (ones).  The other arguments are those of :func:`forward`."""
    B, T, H, dk, dv = _check_inputs(q, k, v, beta, alpha, S0)
    _need(g, "g", q.dtype, (B, T, H, dv))
    _need(w, "w", torch.float32, (H * dv,))
    _need(h, "h", q.dtype, (B, T, H * dv))
    _need(clvr_scale, "clvr_scale", torch.float32, (H * dv,))
    lib = load_library()
    desc = _desc(q, v, alpha, out_dtype, scale, route, prologue)
    y = torch.empty((B, T, H, dv), dtype=out_dtype or q.dtype, device=q.device)
    ST = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if output_final_state else None
    need = lib.gdr_workspace_size(ctypes.byref(desc), 0)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(lib.gdr_forward_chunked_gated(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha),
                                         _ptr(S0), _ptr(g), _ptr(w), _ptr(y), _ptr(ST), _ptr(h), _ptr(clvr_scale),
                                         _ptr(workspace), need, _stream(q.device)))
    return y, ST


def backward(q, k, v, beta, alpha, S0, dO, dST=None, *, scale=1.0, out_dtype=None, dh=None,
             clvr_scale=None, want_dclvr_scale=False, workspace=None, saved_workspace=None,
             route="value", prologue=None):
    """Gradients of :func:`forward`.  Returns a dict with ``dq, dk, dv, dbeta,
    dalpha`` (None for DeltaNet), ``dS0`` and ``dclvr_scale`` (when asked).
    ``dh`` is the gradient at the hidden stream after the epilogue of the given
    ``route``.

    ``saved_workspace``: the workspace of a preceding ``forward(...,
    save_for_backward=True)`` with the same inputs; the forward's intermediates
    are then read from it instead of being recomputed."""
    B, T, H, dk, dv = _check_inputs(q, k, v, beta, alpha, S0)
    _need(dO, "dO", q.dtype, (B, T, H, dv))
    _need(dST, "dST", torch.float32, (B, H, dk, dv))
    _need(dh, "dh", q.dtype, (B, T, H * dv))
    _need(clvr_scale, "clvr_scale", torch.float32, (H * dv,))
    lib = load_library()
    desc = _desc(q, v, alpha, out_dtype, scale, route, prologue)
    od = out_dtype or q.dtype
    dq = torch.empty_like(q, dtype=od)
    dk_ = torch.empty_like(k, dtype=od)
    dv_ = torch.empty_like(v, dtype=od)
    dbeta = torch.empty_like(beta)
    dalpha = None if alpha is None else torch.empty_like(alpha)
    dS0 = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    dlam = torch.empty((H * dv,), dtype=torch.float32, device=q.device) if want_dclvr_scale else None
    need = lib.gdr_workspace_size(ctypes.byref(desc), 1)
    fn = lib.gdr_backward
    if saved_workspace is not None:
        _need(saved_workspace, "saved_workspace", torch.uint8)
        if saved_workspace.numel() < need:
            raise ValueError("saved_workspace has %d bytes, needs %d" % (saved_workspace.numel(), need))
        workspace, fn = saved_workspace, lib.gdr_backward_saved
    elif workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _check(fn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha),
              _ptr(S0), _ptr(dO), _ptr(dST), _ptr(dh), _ptr(clvr_scale), _ptr(dq),
              _ptr(dk_), _ptr(dv_), _ptr(dbeta), _ptr(dalpha), _ptr(dS0), _ptr(dlam),
              _ptr(workspace), need, _stream(q.device)))
    return {"dq": dq, "dk": dk_, "dv": dv_, "dbeta": dbeta, "dalpha": dalpha, "dS0": dS0,
            "dclvr_scale": dlam}


def decode_step(q, k, v, beta, alpha, S, *, scale=1.0, out_dtype=None, out=None):
    """One recurrence step for N sequences; ``S`` [N,H,dk,dv] fp32 is updated in
    place.  Returns ``o`` [N,H,dv]."""
    if q.dim() != 3:
        raise ValueError("q must be [N, H, dk]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q")
    _need(k, "k", q.dtype, (N, H, dk))
    _need(v, "v", q.dtype, (N, H, dv))
    _need(beta, "beta", torch.float32, (N, H))
    gate = GATE_NONE
    if alpha is not None:
        gate = GATE_SCALAR if alpha.dim() == 2 else GATE_CHANNEL
        _need(alpha, "alpha", torch.float32, (N, H) if gate == GATE_SCALAR else (N, H, dk))
    _need(S, "S", torch.float32, (N, H, dk, dv))
    od = out_dtype or q.dtype
    o = out if out is not None else torch.empty((N, H, dv), dtype=od, device=q.device)
    _need(o, "out", od, (N, H, dv))
    lib = load_library()
    _check(lib.gdr_decode_step(N, H, dk, dv, gate, _dt(q.dtype), _dt(od), float(scale), _ptr(q),
                               _ptr(k), _ptr(v), _ptr(beta), _ptr(alpha), _ptr(S), _ptr(o),
                               _stream(q.device)))
    return o


def gdn2_workspace_size(B, T, H, d, gate=GATE_CHANNEL, in_dtype=torch.bfloat16, out_dtype=None) -> int:
    desc = Desc(B, T, H, d, d, gate, _dt(in_dtype), _dt(out_dtype or in_dtype), 1.0, 0, ROUTE_VALUE, PROLOGUE_NONE)
    n = load_library().gdr_gdn2_workspace_size(ctypes.byref(desc))
    if n == 0 and B * H * T > 0:
        _check(1)
    return int(n)


def gdn2_forward(q, k, v, erase, write, alpha=None, S0=None, *, scale=1.0, out_dtype=None,
                 output_final_state=True, workspace=None):
    """Gated DeltaNet-2 chunked forward: separate erase and write gates
    ``erase``, ``write`` [B, T, H, dk] fp32,
    ``S_t = (I - (e_t*k_t) k_t^T) Diag(alpha_t) S_{t-1} + (w_t*k_t) v_t^T``,
    ``o_t = scale S_t^T q_t``.  Returns ``(o, S_T)``."""
    if q.dim() != 4:
        raise ValueError("q must be [B, T, H, dk]")
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q")
    _need(k, "k", q.dtype, (B, T, H, dk))
    _need(v, "v", q.dtype, (B, T, H, dv))
    if alpha is not None:
        _need(alpha, "alpha", torch.float32, (B, T, H) if alpha.dim() == 3 else (B, T, H, dk))
    _need(S0, "S0", torch.float32, (B, H, dk, dv))
    _need(erase, "erase", torch.float32, (B, T, H, dk))
    _need(write, "write", torch.float32, (B, T, H, dk))
    lib = load_library()
    desc = _desc(q, v, alpha, out_dtype, scale)
    o = torch.empty((B, T, H, dv), dtype=out_dtype or q.dtype, device=q.device)
    ST = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device) if output_final_state else None
    need = lib.gdr_gdn2_workspace_size(ctypes.byref(desc))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    _check(lib.gdr_gdn2_forward_chunked(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(erase), _ptr(write),
                                        _ptr(alpha), _ptr(S0), _ptr(o), _ptr(ST), _ptr(workspace), need,
                                        _stream(q.device)))
    return o, ST


def gdn2_decode_step(q, k, v, erase, write, alpha, S, *, scale=1.0, out_dtype=None, out=None):
    """One Gated DeltaNet-2 step for N sequences (``erase``, ``write`` [N, H, dk]
    fp32); ``S`` [N, H, dk, dv] fp32 is updated in place.  Returns ``o``."""
    if q.dim() != 3:
        raise ValueError("q must be [N, H, dk]")
    N, H, dk = q.shape
    dv = v.shape[-1]
    _need(q, "q")
    _need(k, "k", q.dtype, (N, H, dk))
    _need(v, "v", q.dtype, (N, H, dv))
    _need(erase, "erase", torch.float32, (N, H, dk))
    _need(write, "write", torch.float32, (N, H, dk))
    gate = GATE_NONE
    if alpha is not None:
        gate = GATE_SCALAR if alpha.dim() == 2 else GATE_CHANNEL
        _need(alpha, "alpha", torch.float32, (N, H) if gate == GATE_SCALAR else (N, H, dk))
    _need(S, "S", torch.float32, (N, H, dk, dv))
    od = out_dtype or q.dtype
    o = out if out is not None else torch.empty((N, H, dv), dtype=od, device=q.device)
    _need(o, "out", od, (N, H, dv))
    lib = load_library()
    _check(lib.gdr_gdn2_decode_step(N, H, dk, dv, gate, _dt(q.dtype), _dt(od), float(scale), _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(erase), _ptr(write), _ptr(alpha), _ptr(S), _ptr(o),
                                    _stream(q.device)))
    return o


def _gate_desc(o, g):
    if o.dim() != 4:
        raise ValueError("o must be [B, T, H, dv]")
    B, T, H, dv = o.shape
    return Desc(B, T, H, dv, dv, GATE_NONE, _dt(g.dtype), _dt(o.dtype), 1.0, 0, ROUTE_VALUE, PROLOGUE_NONE)


def output_gate(o, g, w=None, *, out=None):
    """Output-gate epilogue ``y = sigmoid(g) * w * RMSNorm(o)`` per head (KDA
    blog 4.1).  o [B,T,H,dv] (bf16 or fp32), g of o's shape (bf16 or fp32),
    w [H*dv] fp32 or None.  ``out`` may be ``o`` itself."""
    _need(o, "o")
    _need(g, "g", None, tuple(o.shape))
    B, T, H, dv = o.shape
    _need(w, "w", torch.float32, (H * dv,))
    y = out if out is not None else torch.empty_like(o)
    _need(y, "out", o.dtype, tuple(o.shape))
    lib = load_library()
    desc = _gate_desc(o, g)
    _check(lib.gdr_output_gate_forward(ctypes.byref(desc), _ptr(o), _ptr(g), _ptr(w), _ptr(y), _stream(o.device)))
    return y


def output_gate_backward(o, g, w, dy, *, want_dw=True):
    """Returns ``(dO, dg, dw)`` for :func:`output_gate`; dO and dg have g's
    dtype (dO is what :func:`backward` takes), dw is None unless asked."""
    _need(o, "o")
    _need(g, "g", None, tuple(o.shape))
    _need(dy, "dy", o.dtype, tuple(o.shape))
    B, T, H, dv = o.shape
    _need(w, "w", torch.float32, (H * dv,))
    lib = load_library()
    desc = _gate_desc(o, g)
    dO = torch.empty_like(g)
    dg = torch.empty_like(g)
    dw = torch.empty((H * dv,), dtype=torch.float32, device=o.device) if want_dw else None
    need = lib.gdr_output_gate_workspace_size(ctypes.byref(desc)) if want_dw else 0
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=o.device) if want_dw else None
    _check(lib.gdr_output_gate_backward(ctypes.byref(desc), _ptr(o), _ptr(g), _ptr(w), _ptr(dy), _ptr(dO),
                                        _ptr(dg), _ptr(dw), _ptr(ws), need, _stream(o.device)))
    return dO, dg, dw
