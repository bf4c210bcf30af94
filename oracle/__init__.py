"""fp64 reference ("oracle") for the gated delta-rule operator -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU product path
(``gated_delta_rule_37_amd``) never imports it and shares no code with it.

The arithmetic lives in ``gdr_oracle.c`` (plain C, fp64, token by token); this
module only marshals NumPy arrays through ctypes.  The recurrence it follows is
the state update of the Kimi Delta Attention blog, section 2.1,
``S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T`` with
``o_t = S_t^T q_t``; see the C file's header for the step-by-step statement.

Parity of every function here is pinned by ``tests/test_oracle_pins.py``
(closed forms, reductions between gate kinds, brute-force unrolled products,
finite differences) rather than by comparison with any implementation.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

GATE_NONE, GATE_SCALAR, GATE_CHANNEL = 0, 1, 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compiles ``liboracle.so`` with the host C compiler (no HIP, no BLAS)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build(force=False)
            lib = ctypes.CDLL(_LIB)
            i64, dbl, ptr, cint = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
            lib.oracle_forward.argtypes = [i64] * 5 + [cint, dbl] + [ptr] * 8 + [cint]
            lib.oracle_backward.argtypes = [i64] * 5 + [cint, dbl] + [ptr] * 14 + [cint]
            lib.oracle_decode.argtypes = [i64] * 4 + [cint, dbl] + [ptr] * 7 + [cint]
            lib.oracle_gdn2_forward.argtypes = [i64] * 5 + [cint, dbl] + [ptr] * 9 + [cint]
            lib.oracle_gdn2_decode.argtypes = [i64] * 4 + [cint, dbl] + [ptr] * 8 + [cint]
            lib.oracle_clvr_forward.argtypes = [i64] * 4 + [ptr] * 4
            lib.oracle_clvr_backward.argtypes = [i64] * 4 + [ptr] * 5
            lib.oracle_forward_errors.argtypes = [i64] * 5 + [cint, dbl] + [ptr] * 9 + [cint]
            lib.oracle_backward_errors.argtypes = [i64] * 5 + [cint, dbl] + [ptr] * 15 + [cint]
            for f in (lib.oracle_forward, lib.oracle_backward, lib.oracle_decode,
                      lib.oracle_clvr_forward, lib.oracle_clvr_backward,
                      lib.oracle_forward_errors, lib.oracle_backward_errors,
                      lib.oracle_gdn2_forward, lib.oracle_gdn2_decode):
                f.restype = cint
            _lib = lib
    return _lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(x):
    return None if x is None else x.ctypes.data_as(ctypes.c_void_p)


def _threads(nthreads):
    if nthreads is None or nthreads <= 0:
        try:
            return len(os.sched_getaffinity(0))
        except AttributeError:  # pragma: no cover
            return os.cpu_count() or 1
    return int(nthreads)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError("%s failed with status %d" % (name, rc))


def gate_kind(alpha, q):
    """NONE when alpha is None, SCALAR for [B,T,H], CHANNEL for [B,T,H,dk]."""
    if alpha is None:
        return GATE_NONE
    return GATE_SCALAR if np.ndim(alpha) == 3 else GATE_CHANNEL


def forward(q, k, v, beta, alpha=None, S0=None, scale=1.0, nthreads=None, want_errors=False):
    """Token-by-token forward.  Returns ``(o [B,T,H,dv], S_T [B,H,dk,dv])``, and
    with ``want_errors`` also the write errors
    ``E [B,T,H,dv]``, ``e_t = v_t - (Diag(alpha_t) S_{t-1})^T k_t``."""
    q, k, v, beta, alpha, S0 = map(_f64, (q, k, v, beta, alpha, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    gate = gate_kind(alpha, q)
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    if want_errors:
        E = np.zeros((B, T, H, dv))
        rc = _load().oracle_forward_errors(B, T, H, dk, dv, gate, float(scale), _p(q), _p(k), _p(v),
                                           _p(beta), _p(alpha), _p(S0), _p(o), _p(ST), _p(E),
                                           _threads(nthreads))
        _check(rc, "oracle_forward_errors")
        return o, ST, E
    rc = _load().oracle_forward(B, T, H, dk, dv, gate, float(scale), _p(q), _p(k), _p(v),
                                _p(beta), _p(alpha), _p(S0), _p(o), _p(ST), _threads(nthreads))
    _check(rc, "oracle_forward")
    return o, ST


def backward(q, k, v, beta, alpha, S0, dO, dST=None, scale=1.0, nthreads=None, dE=None):
    """Adjoint of :func:`forward`.

    Returns a dict with ``dq, dk, dv, dbeta, dalpha`` (None for DeltaNet) and
    ``dS0``.  ``dalpha`` is the derivative with respect to alpha itself.
    ``dE`` [B,T,H,dv], when given, is a gradient arriving at the write errors
    that ``forward(..., want_errors=True)`` returns.
    """
    q, k, v, beta, alpha, S0, dO, dST, dE = map(_f64, (q, k, v, beta, alpha, S0, dO, dST, dE))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    gate = gate_kind(alpha, q)
    dq = np.zeros_like(q)
    dk_ = np.zeros_like(k)
    dv_ = np.zeros_like(v)
    dbeta = np.zeros_like(beta)
    dalpha = None if alpha is None else np.zeros_like(alpha)
    dS0 = np.zeros((B, H, dk, dv))
    if dE is not None:
        rc = _load().oracle_backward_errors(B, T, H, dk, dv, gate, float(scale), _p(q), _p(k), _p(v),
                                            _p(beta), _p(alpha), _p(S0), _p(dO), _p(dST), _p(dE),
                                            _p(dq), _p(dk_), _p(dv_), _p(dbeta), _p(dalpha), _p(dS0),
                                            _threads(nthreads))
        _check(rc, "oracle_backward_errors")
    else:
        rc = _load().oracle_backward(B, T, H, dk, dv, gate, float(scale), _p(q), _p(k), _p(v),
                                     _p(beta), _p(alpha), _p(S0), _p(dO), _p(dST), _p(dq), _p(dk_),
                                     _p(dv_), _p(dbeta), _p(dalpha), _p(dS0), _threads(nthreads))
        _check(rc, "oracle_backward")
    return {"dq": dq, "dk": dk_, "dv": dv_, "dbeta": dbeta, "dalpha": dalpha, "dS0": dS0}


def decode(q, k, v, beta, alpha, S, scale=1.0, nthreads=None):
    """One step for N sequences.  Returns ``(o [N,H,dv], S_new [N,H,dk,dv])``;
    the input state is not modified."""
    q, k, v, beta, alpha = map(_f64, (q, k, v, beta, alpha))
    S = np.array(S, dtype=np.float64, order="C", copy=True)
    N, H, dk = q.shape
    dv = v.shape[-1]
    gate = GATE_NONE if alpha is None else (GATE_SCALAR if alpha.ndim == 2 else GATE_CHANNEL)
    o = np.zeros((N, H, dv))
    rc = _load().oracle_decode(N, H, dk, dv, gate, float(scale), _p(q), _p(k), _p(v), _p(beta),
                               _p(alpha), _p(S), _p(o), _threads(nthreads))
    _check(rc, "oracle_decode")
    return o, S


def gdn2_forward(q, k, v, erase, write, alpha=None, S0=None, scale=1.0, nthreads=None):
    """Gated DeltaNet-2, token by token (erase and write gates [B,T,H,dk]):
    ``S_t = (I - (e_t*k_t) k_t^T) Diag(alpha_t) S_{t-1} + (w_t*k_t) v_t^T``,
    ``o_t = scale S_t^T q_t``.  Returns ``(o, S_T)``."""
    q, k, v, erase, write, alpha, S0 = map(_f64, (q, k, v, erase, write, alpha, S0))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    rc = _load().oracle_gdn2_forward(B, T, H, dk, dv, gate_kind(alpha, q), float(scale), _p(q), _p(k), _p(v),
                                     _p(erase), _p(write), _p(alpha), _p(S0), _p(o), _p(ST), _threads(nthreads))
    _check(rc, "oracle_gdn2_forward")
    return o, ST


def gdn2_decode(q, k, v, erase, write, alpha, S, scale=1.0, nthreads=None):
    """One Gated DeltaNet-2 step for N sequences (erase, write [N,H,dk]).
    Returns ``(o [N,H,dv], S_new)``; the input state is not modified."""
    q, k, v, erase, write, alpha = map(_f64, (q, k, v, erase, write, alpha))
    S = np.array(S, dtype=np.float64, order="C", copy=True)
    N, H, dk = q.shape
    dv = v.shape[-1]
    gate = GATE_NONE if alpha is None else (GATE_SCALAR if alpha.ndim == 2 else GATE_CHANNEL)
    o = np.zeros((N, H, dv))
    rc = _load().oracle_gdn2_decode(N, H, dk, dv, gate, float(scale), _p(q), _p(k), _p(v), _p(erase), _p(write),
                                    _p(alpha), _p(S), _p(o), _threads(nthreads))
    _check(rc, "oracle_gdn2_decode")
    return o, S


def clvr_forward(h, v, lam=None):
    """``h + lam * v`` routed per hidden channel ``h*dv + j``; h is [B,T,H*dv]."""
    h, v, lam = map(_f64, (h, v, lam))
    B, T, H, dv = v.shape
    out = np.zeros_like(h)
    rc = _load().oracle_clvr_forward(B, T, H, dv, _p(h), _p(v), _p(lam), _p(out))
    _check(rc, "oracle_clvr_forward")
    return out


def clvr_backward(dh, v, lam=None):
    """Returns ``(dv_from_clvr [B,T,H,dv], dlam [H*dv])``."""
    dh, v, lam = map(_f64, (dh, v, lam))
    B, T, H, dv = v.shape
    dv_acc = np.zeros_like(v)
    dlam = np.zeros(H * dv)
    rc = _load().oracle_clvr_backward(B, T, H, dv, _p(dh), _p(v), _p(lam), _p(dv_acc), _p(dlam))
    _check(rc, "oracle_clvr_backward")
    return dv_acc, dlam


def cler_forward(h, E, lam=None):
    """Error routing into the hidden stream (CLER-H): ``h + lam * e`` per hidden
    channel ``h*dv + j``, with E the write errors from
    ``forward(..., want_errors=True)``.  The routing is CLVR's with the write
    error in place of the value."""
    return clvr_forward(h, E, lam)


def cler_backward(dh, E, lam=None):
    """Returns ``(dE [B,T,H,dv], dlam [H*dv])`` for :func:`cler_forward`; dE is
    then passed to :func:`backward`."""
    return clvr_backward(dh, E, lam)


# --------------------------------------------------------------------------
# Prologue: L2-normalised q and k, activated gates
# --------------------------------------------------------------------------
# The KDA blog applies an L2 norm to q and k after their projections (section
# 7.1, also section 2.1's remark on numerical stability) and drives the gates
# through a sigmoid; its section 7.1 sets the forget-gate bias to -3, which
# makes the forgotten fraction sigmoid(-3) ~ 0.05 at initialisation.  Two gate
# readings are offered:
#   PRO_ALPHA_SIGMOID : alpha = sigmoid(a)
#   PRO_ALPHA_FORGET  : alpha = exp(-softplus(a)) = 1 - sigmoid(a)  (a is the
#                       forget-gate logit; bias -3 keeps ~95 % per token)
# and beta = sigmoid(b) in both.  The norm is x / max(|x|_2, NORM_EPS).
PRO_NONE, PRO_ALPHA_SIGMOID, PRO_ALPHA_FORGET = 0, 1, 2
NORM_EPS = 1e-6


def _sigmoid(x):
    x = np.asarray(x, np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def l2_normalise(x):
    """Rows of the last axis divided by max(|row|, NORM_EPS)."""
    x = np.asarray(x, np.float64)
    n = np.sqrt((x * x).sum(-1, keepdims=True))
    return x / np.maximum(n, NORM_EPS)


def prologue_forward(q, k, beta_logit, alpha_logit, mode):
    """Raw inputs -> (q_hat, k_hat, beta, alpha) as the operator consumes them."""
    if mode not in (PRO_ALPHA_SIGMOID, PRO_ALPHA_FORGET):
        raise ValueError("prologue mode %r" % (mode,))
    alpha = None
    if alpha_logit is not None:
        a = np.asarray(alpha_logit, np.float64)
        alpha = _sigmoid(a) if mode == PRO_ALPHA_SIGMOID else _sigmoid(-a)
    return l2_normalise(q), l2_normalise(k), _sigmoid(beta_logit), alpha


def _l2_normalise_backward(x, dxh):
    x = np.asarray(x, np.float64)
    n = np.sqrt((x * x).sum(-1, keepdims=True))
    big = n > NORM_EPS
    xh = x / np.maximum(n, NORM_EPS)
    proj = dxh - xh * (xh * dxh).sum(-1, keepdims=True)
    return np.where(big, proj / np.where(big, n, 1.0), dxh / NORM_EPS)


def prologue_backward(q, k, beta_logit, alpha_logit, mode, g):
    """Takes the gradients ``g`` of :func:`backward` (with respect to q_hat,
    k_hat, beta, alpha) back to the raw inputs; returns a new dict."""
    out = dict(g)
    out["dq"] = _l2_normalise_backward(q, g["dq"])
    out["dk"] = _l2_normalise_backward(k, g["dk"])
    bt = _sigmoid(beta_logit)
    out["dbeta"] = g["dbeta"] * bt * (1.0 - bt)
    if alpha_logit is not None:
        a = np.asarray(alpha_logit, np.float64)
        s = 1.0 if mode == PRO_ALPHA_SIGMOID else -1.0
        al = _sigmoid(s * a)
        out["dalpha"] = g["dalpha"] * s * al * (1.0 - al)
    return out


# --------------------------------------------------------------------------
# Output gate: y = sigmoid(g) * RMSNorm(o) per head (KDA blog section 4.1)
# --------------------------------------------------------------------------
# The page's best output gate is o_t = W_o(Sigmoid(W_up W_down x_t) * RMSNorm(KDA(...))).
# The projections are GEMMs outside the operator; the elementwise part takes the
# gate pre-activation g (the low-rank projection's output) from the caller.
# RMSNorm is taken per head over dv with a weight w [H*dv]:
#   y = sigmoid(g) * w * o / sqrt(mean_j o_j^2 + GATE_EPS)
GATE_EPS = 1e-6


def output_gate_forward(o, g, w=None):
    """o, g [B,T,H,dv]; w [H*dv] or None (ones).  Returns (y, rstd [B,T,H])."""
    o = np.asarray(o, np.float64)
    g = np.asarray(g, np.float64)
    B, T, H, dv = o.shape
    w = np.ones((H, dv)) if w is None else np.asarray(w, np.float64).reshape(H, dv)
    rstd = 1.0 / np.sqrt((o * o).mean(-1) + GATE_EPS)
    return _sigmoid(g) * w * o * rstd[..., None], rstd


def output_gate_backward(o, g, w, dy):
    """Returns (do, dg, dw [H*dv]) for :func:`output_gate_forward`."""
    o = np.asarray(o, np.float64)
    g = np.asarray(g, np.float64)
    dy = np.asarray(dy, np.float64)
    B, T, H, dv = o.shape
    w = np.ones((H, dv)) if w is None else np.asarray(w, np.float64).reshape(H, dv)
    rstd = 1.0 / np.sqrt((o * o).mean(-1) + GATE_EPS)
    n = o * rstd[..., None]
    s = _sigmoid(g)
    dn = dy * s * w
    do = rstd[..., None] * (dn - n * (dn * n).mean(-1, keepdims=True))
    dg = dy * w * n * s * (1.0 - s)
    dw = (dy * s * n).sum((0, 1)).reshape(H * dv)
    return do, dg, dw
