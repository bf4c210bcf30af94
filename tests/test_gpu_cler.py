"""GPU parity of the error-routing epilogue (CLER-H, route="error").

The hidden stream gains lam * e_t per channel, with e_t the write error of the
delta rule (the popular article on the study, cross-layer section).  The
oracle gives e_t directly (``forward(..., want_errors=True)``) and takes the
gradient arriving at it (``backward(..., dE=...)``); dE = lam * dh and
dlam = sum_t dh * e_t come from the same routing adjoint as CLVR's.

Tolerances as in gpu_util: 2e-3 for bf16 inputs, 1e-5 for fp32 inputs, plus
bf16's unit roundoff where the compared tensor is stored in bf16 (the hidden
stream has the input dtype)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_37_amd as gdr
import gdr_inputs
import oracle
from gpu_util import TOL, announce, inputs_to_dev, rel, report, to_dev, tol

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "fp32": torch.float32}


def gpu_fwd(t, h, lam, out_dtype=torch.float32, route="error", **kw):
    o, ST = gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], out_dtype=out_dtype, h=h,
                        clvr_scale=lam, route=route, **kw)
    torch.cuda.synchronize()
    return o, ST


def gpu_bwd(t, dh, lam, dST=None, out_dtype=torch.float32, route="error", want=True, **kw):
    g = gdr.backward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], t["dO"], dST, out_dtype=out_dtype,
                     dh=dh, clvr_scale=lam, want_dclvr_scale=want and dh is not None, route=route, **kw)
    torch.cuda.synchronize()
    return g


def case(gate, d, in_dt, seed, B=2, T=200, H=2):
    inp = gdr_inputs.make(B=B, T=T, H=H, d=d, gate=gate, dtype=in_dt, seed=seed, s0=True, bwd=True, clvr=True)
    r = np.random.default_rng(seed + 1)
    lam = r.standard_normal(H * d).astype(np.float32)
    dh = gdr_inputs.round_to(r.standard_normal((B, T, H * d)), in_dt)
    dST = (0.1 * r.standard_normal((B, H, d, d))).astype(np.float32)
    return inp, lam, dh, dST


def oracle_cler(inp, lam, dh, dST):
    o, ST, E = oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], inp["S0"], want_errors=True)
    h = oracle.cler_forward(inp["h"], E, lam)
    dE, dlam = oracle.cler_backward(dh, E, lam)
    g = oracle.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], inp["S0"], inp["dO"], dST, dE=dE)
    g["dclvr_scale"] = dlam
    return o, ST, h, g


def dev_inputs(inp, in_dt):
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("h", "lam")}, in_dt)
    return t, to_dev(inp["h"], TD[in_dt])


@pytest.mark.parametrize("gate,d,in_dt", [("none", 128, "bf16"), ("scalar", 128, "bf16"),
                                          ("channel", 128, "bf16"), ("channel", 64, "bf16"),
                                          ("scalar", 64, "fp32"), ("channel", 64, "fp32"),
                                          ("scalar", 128, "fp32"), ("channel", 128, "fp32")])
def test_cler_forward_and_backward_match_oracle(gate, d, in_dt):
    announce("cler gate=%s d=%d in=%s" % (gate, d, in_dt))
    inp, lam, dh, dST = case(gate, d, in_dt, seed=500 + d + (7 if in_dt == "fp32" else 0))
    t, h = dev_inputs(inp, in_dt)
    o, ST = gpu_fwd(t, h, to_dev(lam))
    g = gpu_bwd(t, to_dev(dh, TD[in_dt]), to_dev(lam), to_dev(dST))
    o_ref, ST_ref, h_ref, ref = oracle_cler(inp, lam, dh, dST)
    errs = {"o": rel(o, o_ref), "S": rel(ST, ST_ref), "h": rel(h, h_ref)}
    for n in ("dq", "dk", "dv", "dbeta", "dalpha", "dS0", "dclvr_scale"):
        if ref[n] is not None:
            errs[n] = rel(g[n], ref[n])
    report(**errs)
    t_h = tol(in_dt, in_dt)
    assert errs["h"] < t_h, errs
    assert max(v for n, v in errs.items() if n != "h") < TOL[in_dt], errs


def test_cler_output_and_state_equal_the_plain_forward():
    """The epilogue only adds to the hidden stream: o and S_T are the plain
    forward's, bit for bit, for both operand precisions."""
    for in_dt, d in (("bf16", 128), ("fp32", 64)):
        inp, lam, _, _ = case("channel", d, in_dt, seed=520)
        t, h = dev_inputs(inp, in_dt)
        o1, S1 = gpu_fwd(t, h, to_dev(lam))
        o2, S2 = gpu_fwd(t, None, None)
        assert torch.equal(o1, o2) and torch.equal(S1, S2), in_dt


def test_cler_zero_scale_is_a_bitwise_no_op():
    """lam = 0 leaves the hidden stream unchanged and gives the gradients of the
    layer without the epilogue, bit for bit (dlam is then sum dh * e)."""
    announce("cler zero scale")
    inp, _, dh, dST = case("channel", 128, "bf16", seed=530)
    t, h = dev_inputs(inp, "bf16")
    h0 = h.clone()
    z = torch.zeros(2 * 128, device="cuda")
    gpu_fwd(t, h0, z)
    assert torch.equal(h0, h)
    g0 = gpu_bwd(t, to_dev(dh, torch.bfloat16), z, to_dev(dST))
    gp = gpu_bwd(t, None, None, to_dev(dST))
    for n in ("dq", "dk", "dv", "dbeta", "dalpha", "dS0"):
        assert torch.equal(g0[n], gp[n]), n
    _, _, E = oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], inp["S0"], want_errors=True)
    _, dlam = oracle.cler_backward(dh, E, np.zeros(256))
    e = rel(g0["dclvr_scale"], dlam)
    report(dlam=e)
    assert e < 2e-3


def test_cler_unit_scale_when_scale_is_null():
    inp, _, dh, _ = case("scalar", 64, "bf16", seed=540, T=150)
    t, h = dev_inputs(inp, "bf16")
    h1, h2 = h.clone(), h.clone()
    gpu_fwd(t, h1, None)
    gpu_fwd(t, h2, torch.ones(2 * 64, device="cuda"))
    assert torch.equal(h1, h2)
    g1 = gpu_bwd(t, to_dev(dh, torch.bfloat16), None)
    g2 = gpu_bwd(t, to_dev(dh, torch.bfloat16), torch.ones(2 * 64, device="cuda"))
    for n in ("dq", "dk", "dv", "dbeta", "dalpha", "dS0", "dclvr_scale"):
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("T", [1, 64, 65])
def test_cler_ragged_lengths(T):
    announce("cler ragged T=%d" % T)
    inp, lam, dh, dST = case("channel", 128, "bf16", seed=550 + T, B=1, T=T, H=3)
    t, h = dev_inputs(inp, "bf16")
    gpu_fwd(t, h, to_dev(lam))
    g = gpu_bwd(t, to_dev(dh, torch.bfloat16), to_dev(lam), to_dev(dST))
    _, _, h_ref, ref = oracle_cler(inp, lam, dh, dST)
    errs = {"h": rel(h, h_ref)}
    for n in ("dq", "dk", "dv", "dbeta", "dalpha", "dS0", "dclvr_scale"):
        errs[n] = rel(g[n], ref[n])
    report(**errs)
    assert errs["h"] < tol("bf16", "bf16") and max(errs.values()) < tol("bf16", "bf16"), errs
    assert max(v for n, v in errs.items() if n != "h") < 2e-3, errs


def test_cler_training_pair_equals_separate_calls():
    announce("cler training pair")
    inp, lam, dh, dST = case("channel", 128, "bf16", seed=560)
    t, h = dev_inputs(inp, "bf16")
    lam_d, dh_d, dST_d = to_dev(lam), to_dev(dh, torch.bfloat16), to_dev(dST)
    ws = torch.empty(gdr.workspace_size(2, 200, 2, 128, gdr.GATE_CHANNEL, torch.bfloat16, torch.float32,
                                        backward=True, route="error"), dtype=torch.uint8, device="cuda")
    h1, h2 = h.clone(), h.clone()
    o1, S1 = gpu_fwd(t, h1, lam_d, workspace=ws, save_for_backward=True)
    g1 = gpu_bwd(t, dh_d, lam_d, dST_d, saved_workspace=ws)
    o2, S2 = gpu_fwd(t, h2, lam_d)
    g2 = gpu_bwd(t, dh_d, lam_d, dST_d)
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(h1, h2)
    for n in ("dq", "dk", "dv", "dbeta", "dalpha", "dS0", "dclvr_scale"):
        assert torch.equal(g1[n], g2[n]), n


def test_cler_full_layer_sampled_head():
    """The 350M-layer shape (B=8, T=4096, H=8, d=128, KDA, bf16) through the
    training pair; the oracle recomputes head 3 of every sequence (the scale
    gradient of a head sums over all sequences)."""
    announce("cler full layer c4")
    inp, cfg = gdr_inputs.make_config("c4")
    B, T, H, d = inp["q"].shape
    r = np.random.default_rng(570)
    lam = r.standard_normal(H * d).astype(np.float32)
    dh = gdr_inputs.round_bf16(r.standard_normal((B, T, H * d)))
    t, h = dev_inputs(inp, "bf16")
    ws = torch.empty(gdr.workspace_size(B, T, H, d, gdr.GATE_CHANNEL, torch.bfloat16, torch.bfloat16,
                                        backward=True, route="error"), dtype=torch.uint8, device="cuda")
    lam_d, dh_d = to_dev(lam), to_dev(dh, torch.bfloat16)
    o, _ = gpu_fwd(t, h, lam_d, out_dtype=torch.bfloat16, workspace=ws, save_for_backward=True)
    g = gpu_bwd(t, dh_d, lam_d, out_dtype=torch.bfloat16, saved_workspace=ws)
    hh = 3
    cols = slice(hh * d, (hh + 1) * d)
    sl = lambda a: None if a is None else a[:, :, hh:hh + 1]  # noqa: E731
    sub = {n: sl(inp[n]) for n in ("q", "k", "v", "beta", "alpha", "dO")}
    sub["S0"] = None
    sub["h"] = inp["h"][:, :, cols]
    o_ref, _, h_ref, ref = oracle_cler(sub, lam[cols], dh[:, :, cols], None)
    errs = {"o": rel(o[:, :, hh:hh + 1], o_ref), "h": rel(h[:, :, cols], h_ref),
            "dlam": rel(g["dclvr_scale"][cols], ref["dclvr_scale"])}
    for n in ("dq", "dk", "dv", "dbeta", "dalpha"):
        errs[n] = rel(g[n][:, :, hh:hh + 1], ref[n])
    report(**errs)
    assert max(errs.values()) < tol("bf16", "bf16"), errs
    assert errs["dbeta"] < 2e-3 and errs["dlam"] < 2e-3, errs
