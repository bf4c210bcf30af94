"""gated_delta_rule_37_amd -- the gated delta-rule operator on AMD MI355X (gfx950).

A thin Python binding over ``libgdr.so`` (C ABI in ``include/gdr.h``).  Every
step of the operator runs in the library's HIP kernels; this module only checks
tensors, allocates outputs and workspace with PyTorch, and passes raw device
pointers plus the current HIP stream.  There is no CPU fallback: if the library
is missing or the tensors are not on a GPU, the calls raise.

The operator (KDA blog, section 2.1):
    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    o_t = scale * S_t^T q_t
with alpha absent (DeltaNet), one value per token and head (Gated DeltaNet) or
one value per token, head and key channel (Kimi Delta Attention).  Gated
DeltaNet-2 (``gdn2_forward``, ``gdn2_decode_step``) replaces beta by separate
erase and write gates per key channel.
"""
from __future__ import annotations

from ._lib import (GATE_CHANNEL, GATE_NONE, GATE_SCALAR, PROLOGUE_ALPHA_FORGET, PROLOGUE_ALPHA_SIGMOID,
                   PROLOGUE_NONE, ROUTE_ERROR, ROUTE_VALUE, GdrError, backward, decode_step, forward,
                   forward_gated,
                   gdn2_decode_step, gdn2_forward, gdn2_workspace_size, library_path, load_library, output_gate,
                   output_gate_backward, workspace_size)

__all__ = [
    "GATE_NONE", "GATE_SCALAR", "GATE_CHANNEL", "ROUTE_VALUE", "ROUTE_ERROR", "PROLOGUE_NONE",
    "PROLOGUE_ALPHA_SIGMOID", "PROLOGUE_ALPHA_FORGET", "GdrError", "forward", "forward_gated", "backward",
    "decode_step", "output_gate", "output_gate_backward", "workspace_size", "load_library", "library_path",
    "gdn2_forward", "gdn2_decode_step", "gdn2_workspace_size",
]
