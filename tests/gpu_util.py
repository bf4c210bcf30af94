"""Helpers shared by the GPU parity tests (marshalling and error metrics only)."""
import numpy as np
import pytest
import torch

# Tolerances, as max|x - y| / max|y| per output tensor against the fp64 oracle:
#   bf16 inputs (fp32 state, fp32-stored outputs): 2e-3
#   fp32 inputs: 1e-5
#   bf16-stored outputs add bf16's unit roundoff 2^-8 (rounding an exact value
#   to bf16 alone moves it by up to that much relative to max|y|)
TOL = {"bf16": 2e-3, "fp32": 1e-5}
BF16_ULP = 2.0 ** -8


def tol(in_dtype, out_dtype=None):
    t = TOL[in_dtype]
    if (out_dtype or in_dtype) == "bf16":
        t += BF16_ULP
    return t


TORCH = {"bf16": torch.bfloat16, "fp32": torch.float32}


def device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return torch.device("cuda:0")


def to_dev(a, dtype=torch.float32):
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to(device()).to(dtype)


def inputs_to_dev(inp, in_dtype):
    dt = TORCH[in_dtype]
    out = {}
    for n, a in inp.items():
        if a is None:
            out[n] = None
        elif n in ("q", "k", "v", "dO", "h"):
            out[n] = to_dev(a, dt)
        else:
            out[n] = to_dev(a, torch.float32)
    return out


def rel(x, y):
    x = np.asarray(x.detach().float().cpu().numpy() if isinstance(x, torch.Tensor) else x, np.float64)
    y = np.asarray(y, np.float64)
    den = np.abs(y).max()
    return float(np.abs(x - y).max() / (den if den > 0 else 1.0))


def report(**errs):
    """Prints the measured errors of a case (shown with pytest -s)."""
    print("[gpu-err] " + " ".join("%s=%.3e" % (k, float(v)) for k, v in errs.items()), flush=True)


def announce(msg):
    print("[gpu-case] " + msg, flush=True)


gpu = pytest.mark.gpu
