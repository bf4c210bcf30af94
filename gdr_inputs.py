"""Seeded synthetic inputs for the gated delta-rule operator.

This module only draws random numbers and rounds them to the declared storage
precision.  It holds none of the operator's arithmetic, so both the GPU path's
tests/bench and the fp64 oracle can consume the same inputs.

Recipe (fixed draw order per seed, NumPy ``default_rng``):
  q, k  ~ N(0, 1), L2-normalised per (token, head) in fp64 -- the caller-side
        normalisation the KDA blog asks for after the q/k projections
        (section 7.1); then rounded to the input dtype
  v     ~ N(0, 1), rounded to the input dtype
  beta  = sigmoid(N(0, 1)) per token and head, rounded to fp32
  alpha = sigmoid(N(3, 1)), one per token and head (Gated DeltaNet) or one per
        token, head and key channel (Kimi Delta Attention), rounded to fp32;
        absent for DeltaNet
  S0    ~ N(0, 0.02^2) fp32 (standard deviation 0.02) where a config asks for it
  dO    ~ N(0, 1) in the input dtype (backward configs)
  h     ~ N(0, 1) in the input dtype, [B, T, H*dv] (CLVR configs)
With ``prologue`` ("sigmoid" or "forget") the operator's own prologue is
exercised instead: q and k ~ N(0, 1) times a per-row scale drawn from
U(0.2, 5), not normalised; beta is a logit ~ N(0, 1); alpha a logit
~ N(3, 1) ("sigmoid": alpha = sigmoid(a)) or ~ N(-3, 1) ("forget": alpha =
1 - sigmoid(a), the forget-gate bias -3 of KDA blog section 7.1), so that
alpha lands near 0.95 either way.
All arrays come back as float32 NumPy arrays whose values are exactly
representable in the declared dtype (bf16 values are exact in fp32).
"""
from __future__ import annotations

import numpy as np

GATES = ("none", "scalar", "channel")

# Workload shapes of the study's 350M-parameter, 4K-32K token runs restated as
# operator inputs.  "c5b" is the 32K-token prefill that throughput is quoted on.
CONFIGS = {
    "c1": dict(desc="DeltaNet fp32 parity case", B=1, H=2, T=256, d=64, gate="none",
               dtype="fp32", s0=False, seed=1),
    "c2": dict(desc="Gated DeltaNet forward", B=4, H=16, T=4096, d=128, gate="scalar",
               dtype="bf16", s0=False, seed=2),
    "c3": dict(desc="Kimi Delta Attention forward, random initial state", B=1, H=16,
               T=16384, d=128, gate="channel", dtype="bf16", s0=True, seed=3),
    "c4": dict(desc="KDA forward+backward with CLVR, 350M layer (d_model 1024)", B=8, H=8,
               T=4096, d=128, gate="channel", dtype="bf16", s0=False, seed=4, bwd=True,
               clvr=True),
    "c5b": dict(desc="KDA prefill at 32K tokens", B=1, H=16, T=32768, d=128, gate="channel",
                dtype="bf16", s0=False, seed=6),
}
DECODE_CONFIG = dict(desc="KDA decode step, 256 sequences", N=256, H=16, d=128,
                     gate="channel", dtype="bf16", seed=5)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even to bfloat16, returned as float32."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(x)
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(dtype)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def make(B, T, H, d, gate="channel", dtype="bf16", seed=0, s0=False, bwd=False, clvr=False,
         alpha_recipe="sigmoid(N(3,1))", beta_recipe="sigmoid(N(0,1))", prologue=None, **_unused):
    """Draws one batch of chunked-path inputs.  Returns a dict of float32 arrays
    (``alpha`` None for DeltaNet, ``S0`` None for a zero start)."""
    if gate not in GATES:
        raise ValueError(gate)
    if prologue not in (None, "sigmoid", "forget"):
        raise ValueError(prologue)
    rng = np.random.default_rng(seed)
    out = {}
    if prologue is None:
        out["q"] = round_to(_unit_rows(rng.standard_normal((B, T, H, d))), dtype)
        out["k"] = round_to(_unit_rows(rng.standard_normal((B, T, H, d))), dtype)
    else:
        out["q"] = round_to(rng.standard_normal((B, T, H, d)) * rng.uniform(0.2, 5, (B, T, H, 1)), dtype)
        out["k"] = round_to(rng.standard_normal((B, T, H, d)) * rng.uniform(0.2, 5, (B, T, H, 1)), dtype)
    out["v"] = round_to(rng.standard_normal((B, T, H, d)), dtype)
    if prologue is None:
        out["beta"] = _beta(rng, (B, T, H), beta_recipe)
    else:
        out["beta"] = rng.standard_normal((B, T, H)).astype(np.float32)
    if gate == "none":
        out["alpha"] = None
    else:
        shape = (B, T, H) if gate == "scalar" else (B, T, H, d)
        if prologue is None:
            out["alpha"] = _alpha(rng, shape, alpha_recipe)
        else:
            mu = 3.0 if prologue == "sigmoid" else -3.0
            out["alpha"] = (mu + rng.standard_normal(shape)).astype(np.float32)
    out["S0"] = (0.02 * rng.standard_normal((B, H, d, d))).astype(np.float32) if s0 else None
    if bwd:
        out["dO"] = round_to(rng.standard_normal((B, T, H, d)), dtype)
    if clvr:
        out["h"] = round_to(rng.standard_normal((B, T, H * d)), dtype)
        out["lam"] = np.ones(H * d, dtype=np.float32)
    return out


def _beta(rng, shape, recipe):
    if recipe == "sigmoid(N(0,1))":
        return _sigmoid(rng.standard_normal(shape)).astype(np.float32)
    if recipe.startswith("const:"):
        return np.full(shape, float(recipe[6:]), dtype=np.float32)
    if recipe == "choice{0,1,2}":
        return rng.integers(0, 3, size=shape).astype(np.float32)
    raise ValueError(recipe)


def _alpha(rng, shape, recipe):
    if recipe == "sigmoid(N(3,1))":
        a = _sigmoid(3.0 + rng.standard_normal(shape))
    elif recipe == "sigmoid(N(-1,1))":
        a = _sigmoid(-1.0 + rng.standard_normal(shape))
    elif recipe == "uniform[1e-6,1e-3]":
        a = rng.uniform(1e-6, 1e-3, size=shape)
    elif recipe == "ones":
        a = np.ones(shape)
    else:
        raise ValueError(recipe)
    a = a.astype(np.float32)
    # keep alpha inside (0, 1]: fp32 rounding of sigmoid can reach exactly 1.0,
    # which is allowed; it can never reach 0 for these recipes
    return a


def make_config(name, **overrides):
    cfg = dict(CONFIGS[name])
    cfg.update(overrides)
    return make(**cfg), cfg


def make_decode(N, H, d, gate="channel", dtype="bf16", seed=5, nstates=1, **_unused):
    """Draws decode inputs: q,k,v [N,H,d], beta [N,H], alpha [N,H] or [N,H,d],
    and ``nstates`` independent fp32 states [N,H,d,d] ~ N(0, 0.02^2)."""
    rng = np.random.default_rng(seed)
    out = {}
    out["q"] = round_to(_unit_rows(rng.standard_normal((N, H, d))), dtype)
    out["k"] = round_to(_unit_rows(rng.standard_normal((N, H, d))), dtype)
    out["v"] = round_to(rng.standard_normal((N, H, d)), dtype)
    out["beta"] = _sigmoid(rng.standard_normal((N, H))).astype(np.float32)
    if gate == "none":
        out["alpha"] = None
    else:
        shape = (N, H) if gate == "scalar" else (N, H, d)
        out["alpha"] = _sigmoid(3.0 + rng.standard_normal(shape)).astype(np.float32)
    out["S"] = [(0.02 * rng.standard_normal((N, H, d, d))).astype(np.float32)
                for _ in range(nstates)]
    return out
