"""Tensors past 2^31 elements: the chunked forward and backward at B=1 H=16
d=128 with T = 1,048,704 tokens (q holds 2,147,745,792 elements), and a decode
step with N = 8200 sequences (the state holds 2,149,580,800 elements).

Offsets into such tensors do not fit 32-bit integers, so a kernel that formed
one in 32 bits would read or write the wrong tokens at the end of the sequence.
The inputs are drawn on the GPU (seeded); only windows go to the host.

What pins the long run without an oracle pass over a million tokens: with
alpha in U[0.6, 0.75] the state forgets (each token keeps at most 0.75 of it),
so over the last 384 tokens the operator equals the oracle run on those tokens
alone from a zero state, up to 0.75^192 ~ 1e-24 of what entered before.  The
last 192 tokens of o, of every gradient (dO given only inside the window), and
S_T are compared there for two heads; the decode step is compared slab by slab
for the first and the last sequence."""
import numpy as np
import pytest
import torch

import gated_delta_rule_37_amd as gdr
import oracle
from gpu_util import announce, rel, report

pytestmark = pytest.mark.gpu

B, H, D = 1, 16, 128
T = 1_048_704  # T * H * D = 2,147,745,792 > 2^31
WIN, CHK = 384, 192
HEADS = (0, 15)


def _bf16_unit_rows(shape, gen):
    x = torch.randn(shape, device="cuda", generator=gen)
    x = torch.nn.functional.normalize(x, dim=-1)
    return x.to(torch.bfloat16)


def _host(x, t0=None, t1=None, h=None):
    """fp64 host copy of x[:, t0:t1, h:h+1] (or x[:, :, h:h+1] for [B,T,H])."""
    y = x[:, t0:t1] if t0 is not None else x
    if h is not None:
        y = y[:, :, h:h + 1]
    return y.float().cpu().double().numpy()


@pytest.fixture(scope="module")
def big_inputs():
    if torch.cuda.get_device_properties(0).total_memory < 200 * 2**30:
        pytest.skip("needs a GPU with at least 200 GiB")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7001)
    t = {"q": _bf16_unit_rows((B, T, H, D), gen), "k": _bf16_unit_rows((B, T, H, D), gen),
         "v": torch.randn((B, T, H, D), device="cuda", generator=gen).to(torch.bfloat16),
         "beta": torch.sigmoid(torch.randn((B, T, H), device="cuda", generator=gen)),
         "alpha": 0.6 + 0.15 * torch.rand((B, T, H, D), device="cuda", generator=gen)}
    t["dO"] = torch.zeros((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    t["dO"][:, T - WIN:] = torch.randn((B, WIN, H, D), device="cuda", generator=gen).to(torch.bfloat16)
    assert t["q"].numel() > 2**31
    yield t
    del t
    torch.cuda.empty_cache()


def window_oracle(t, h):
    w = {n: _host(t[n], T - WIN, T, h) for n in ("q", "k", "v", "beta", "alpha", "dO")}
    o, ST = oracle.forward(w["q"], w["k"], w["v"], w["beta"], w["alpha"], None)
    g = oracle.backward(w["q"], w["k"], w["v"], w["beta"], w["alpha"], None, w["dO"])
    return o, ST, g


def test_forward_and_backward_past_2g_elements(big_inputs):
    t = big_inputs
    announce("forward + backward, B=1 H=16 T=%d d=128 (q: %d elements)" % (T, t["q"].numel()))
    o, ST = gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], None, out_dtype=torch.bfloat16)
    g = gdr.backward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], None, t["dO"], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    errs = {}
    for h in HEADS:
        o_ref, ST_ref, ref = window_oracle(t, h)
        errs["o%d" % h] = rel(_host(o, T - CHK, T, h), o_ref[:, WIN - CHK:])
        errs["S_T%d" % h] = rel(ST[:, h:h + 1], ST_ref)
        for n in ("dq", "dk", "dv"):
            errs["%s%d" % (n, h)] = rel(_host(g[n], T - CHK, T, h), ref[n][:, WIN - CHK:])
        for n in ("dbeta", "dalpha"):
            errs["%s%d" % (n, h)] = rel(_host(g[n], T - CHK, T, h), ref[n][:, WIN - CHK:])
    report(**errs)
    # bf16-stored o, dq, dk, dv: 2e-3 plus bf16's unit roundoff; fp32 S_T, dbeta, dalpha: 2e-3
    bf = [v for n, v in errs.items() if n[:2] in ("o0", "o1") or n.startswith(("dq", "dk", "dv"))]
    f32 = [v for n, v in errs.items() if n.startswith(("S_T", "dbeta", "dalpha"))]
    assert max(bf) < 2e-3 + 2**-8 and max(f32) < 2e-3, errs
    del o, ST, g
    torch.cuda.empty_cache()


def test_decode_step_past_2g_state_elements():
    if torch.cuda.get_device_properties(0).total_memory < 64 * 2**30:
        pytest.skip("needs a GPU with at least 64 GiB")
    N = 8200  # N * H * D * D = 2,149,580,800 > 2^31
    announce("decode step, N=%d H=16 d=128 (state: %d elements)" % (N, N * H * D * D))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7002)
    q = _bf16_unit_rows((N, H, D), gen)
    k = _bf16_unit_rows((N, H, D), gen)
    v = torch.randn((N, H, D), device="cuda", generator=gen).to(torch.bfloat16)
    beta = torch.sigmoid(torch.randn((N, H), device="cuda", generator=gen))
    alpha = torch.sigmoid(3 + torch.randn((N, H, D), device="cuda", generator=gen))
    S = 0.02 * torch.randn((N, H, D, D), device="cuda", generator=gen)
    assert S.numel() > 2**31
    S_in = {n: S[n].double().cpu().numpy() for n in (0, N - 1)}
    o = gdr.decode_step(q, k, v, beta, alpha, S, out_dtype=torch.float32)
    torch.cuda.synchronize()
    errs = {}
    for n in (0, N - 1):
        sl = lambda x: x[n:n + 1].float().double().cpu().numpy()  # noqa: E731
        o_ref, S_ref = oracle.decode(sl(q), sl(k), sl(v), sl(beta), sl(alpha), S_in[n][None])
        errs["o%d" % n] = rel(o[n:n + 1], o_ref)
        errs["S%d" % n] = rel(S[n:n + 1], S_ref)
    report(**errs)
    assert max(errs.values()) < 1e-5, errs
    del q, k, v, beta, alpha, S, o
    torch.cuda.empty_cache()
