"""GPU parity of the fused prologue (prologue="sigmoid" / "forget").

q and k arrive unnormalised and beta, alpha as logits; the library normalises
and activates them inside the chunked kernels and returns gradients with
respect to the raw inputs.  The oracle applies the same prologue in fp64
(``oracle.prologue_forward`` / ``prologue_backward``) around its token loop.
Tolerances as in gpu_util: 2e-3 for bf16 inputs, 1e-5 for fp32 inputs."""
import numpy as np
import pytest
import torch

import gated_delta_rule_37_amd as gdr
import gdr_inputs
import oracle
from gpu_util import TOL, announce, inputs_to_dev, rel, report, to_dev, tol

pytestmark = pytest.mark.gpu

MODES = {"sigmoid": oracle.PRO_ALPHA_SIGMOID, "forget": oracle.PRO_ALPHA_FORGET}
GRADS = ("dq", "dk", "dv", "dbeta", "dalpha", "dS0")


def oracle_pro(inp, mode, dST=None):
    m = MODES[mode]
    qh, kh, bt, al = oracle.prologue_forward(inp["q"], inp["k"], inp["beta"], inp["alpha"], m)
    o, ST = oracle.forward(qh, kh, inp["v"], bt, al, inp["S0"])
    g = oracle.backward(qh, kh, inp["v"], bt, al, inp["S0"], inp["dO"], dST)
    return o, ST, oracle.prologue_backward(inp["q"], inp["k"], inp["beta"], inp["alpha"], m, g)


def gpu_pro(t, mode, dST=None, out_dtype=torch.float32, **kw):
    fkw = {n: kw[n] for n in ("h", "clvr_scale", "workspace", "save_for_backward", "route") if n in kw}
    bkw = {n: kw[n] for n in ("dh", "clvr_scale", "want_dclvr_scale", "saved_workspace", "route") if n in kw}
    o, ST = gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], out_dtype=out_dtype,
                        prologue=mode, **fkw)
    g = gdr.backward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], t["dO"], dST, out_dtype=out_dtype,
                     prologue=mode, **bkw)
    torch.cuda.synchronize()
    return o, ST, g


def errors(o, ST, g, o_ref, ST_ref, ref):
    errs = {"o": rel(o, o_ref), "S": rel(ST, ST_ref)}
    for n in GRADS:
        if ref[n] is not None:
            errs[n] = rel(g[n], ref[n])
    return errs


@pytest.mark.parametrize("gate,d,in_dt,mode", [
    ("none", 128, "bf16", "forget"), ("scalar", 128, "bf16", "sigmoid"), ("scalar", 128, "bf16", "forget"),
    ("channel", 128, "bf16", "forget"), ("channel", 128, "bf16", "sigmoid"), ("channel", 64, "bf16", "forget"),
    ("scalar", 64, "fp32", "forget"), ("channel", 64, "fp32", "sigmoid"), ("channel", 64, "fp32", "forget"),
    ("scalar", 128, "fp32", "forget"), ("channel", 128, "fp32", "sigmoid"), ("none", 128, "fp32", "forget")])
def test_prologue_matches_oracle(gate, d, in_dt, mode):
    """At fp32 d = 128 the second gradient stage runs in two channel passes: the
    row-norm backward's row dots are carried across them and the first pass's
    channels are finished by the second."""
    announce("prologue gate=%s d=%d in=%s mode=%s" % (gate, d, in_dt, mode))
    inp = gdr_inputs.make(B=2, T=200, H=2, d=d, gate=gate, dtype=in_dt, seed=600 + d, s0=True, bwd=True,
                          prologue=mode)
    dST = (0.1 * np.random.default_rng(601).standard_normal((2, 2, d, d))).astype(np.float32)
    o, ST, g = gpu_pro(inputs_to_dev(inp, in_dt), mode, to_dev(dST))
    errs = errors(o, ST, g, *oracle_pro(inp, mode, dST))
    report(**errs)
    assert max(errs.values()) < TOL[in_dt], errs


@pytest.mark.parametrize("T", [1, 65])
def test_prologue_ragged_lengths(T):
    announce("prologue ragged T=%d" % T)
    inp = gdr_inputs.make(B=1, T=T, H=3, d=128, gate="channel", dtype="bf16", seed=610 + T, s0=True, bwd=True,
                          prologue="forget")
    o, ST, g = gpu_pro(inputs_to_dev(inp, "bf16"), "forget")
    errs = errors(o, ST, g, *oracle_pro(inp, "forget"))
    report(**errs)
    assert max(errs.values()) < 2e-3, errs


@pytest.mark.parametrize("d", [64, 128])
def test_prologue_zero_rows_take_the_clamped_norm(d):
    """A zero q row and a zero k row: their norms are clamped, the normalised
    rows are zero and the gradients are dx_hat / eps (no projection term)."""
    announce("prologue zero rows d=%d" % d)
    inp = gdr_inputs.make(B=1, T=70, H=2, d=d, gate="channel", dtype="fp32", seed=620, bwd=True,
                          prologue="forget")
    inp["q"][0, 5, 1] = 0.0
    inp["k"][0, 66, 0] = 0.0
    o, ST, g = gpu_pro(inputs_to_dev(inp, "fp32"), "forget")
    o_ref, ST_ref, ref = oracle_pro(inp, "forget")
    errs = errors(o, ST, g, o_ref, ST_ref, ref)
    report(**errs)
    assert np.abs(ref["dq"][0, 5, 1]).max() > 1e3  # the clamped branch is exercised
    assert max(errs.values()) < 1e-5, errs


def test_prologue_training_pair_and_clvr():
    """Training pair with the prologue and CLVR: bit for bit the separate
    calls; CLVR's dv and dlam terms as without the prologue."""
    announce("prologue training pair")
    inp = gdr_inputs.make(B=2, T=200, H=2, d=128, gate="channel", dtype="bf16", seed=630, bwd=True, clvr=True,
                          prologue="forget")
    r = np.random.default_rng(631)
    lam = to_dev(r.standard_normal(256).astype(np.float32))
    dh = to_dev(gdr_inputs.round_bf16(r.standard_normal((2, 200, 256))), torch.bfloat16)
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("h", "lam")}, "bf16")
    h0 = to_dev(inp["h"], torch.bfloat16)
    ws = torch.empty(gdr.workspace_size(2, 200, 2, 128, gdr.GATE_CHANNEL, torch.bfloat16, torch.float32,
                                        backward=True, prologue="forget"), dtype=torch.uint8, device="cuda")
    h1, h2 = h0.clone(), h0.clone()
    o1, S1, g1 = gpu_pro(t, "forget", h=h1, clvr_scale=lam, dh=dh, want_dclvr_scale=True, workspace=ws,
                         save_for_backward=True, saved_workspace=ws)
    o2, S2, g2 = gpu_pro(t, "forget", h=h2, clvr_scale=lam, dh=dh, want_dclvr_scale=True)
    assert torch.equal(o1, o2) and torch.equal(S1, S2) and torch.equal(h1, h2)
    for n in GRADS + ("dclvr_scale",):
        if g1[n] is not None:
            assert torch.equal(g1[n], g2[n]), n
    o_ref, ST_ref, ref = oracle_pro(inp, "forget")
    dv_c, dlam = oracle.clvr_backward(dh.float().cpu().numpy(), inp["v"], lam.cpu().numpy())
    ref["dv"] = ref["dv"] + dv_c
    errs = errors(o1, S1, g1, o_ref, ST_ref, ref)
    errs["h"] = rel(h1, oracle.clvr_forward(inp["h"], inp["v"], lam.cpu().numpy()))
    errs["dlam"] = rel(g1["dclvr_scale"], dlam)
    report(**errs)
    assert errs["h"] < tol("bf16", "bf16") and max(v for n, v in errs.items() if n != "h") < 2e-3, errs


def test_prologue_with_error_routing():
    announce("prologue + cler")
    inp = gdr_inputs.make(B=1, T=150, H=2, d=128, gate="scalar", dtype="bf16", seed=640, s0=True, bwd=True,
                          clvr=True, prologue="sigmoid")
    r = np.random.default_rng(641)
    lam = r.standard_normal(256).astype(np.float32)
    dh = gdr_inputs.round_bf16(r.standard_normal((1, 150, 256)))
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("h", "lam")}, "bf16")
    h = to_dev(inp["h"], torch.bfloat16)
    o, ST, g = gpu_pro(t, "sigmoid", h=h, clvr_scale=to_dev(lam), dh=to_dev(dh, torch.bfloat16),
                       want_dclvr_scale=True, route="error")
    m = MODES["sigmoid"]
    qh, kh, bt, al = oracle.prologue_forward(inp["q"], inp["k"], inp["beta"], inp["alpha"], m)
    o_ref, ST_ref, E = oracle.forward(qh, kh, inp["v"], bt, al, inp["S0"], want_errors=True)
    dE, dlam = oracle.cler_backward(dh, E, lam)
    ref = oracle.prologue_backward(inp["q"], inp["k"], inp["beta"], inp["alpha"], m,
                                   oracle.backward(qh, kh, inp["v"], bt, al, inp["S0"], inp["dO"], dE=dE))
    errs = errors(o, ST, g, o_ref, ST_ref, ref)
    errs["h"] = rel(h, oracle.cler_forward(inp["h"], E, lam))
    errs["dlam"] = rel(g["dclvr_scale"], dlam)
    report(**errs)
    assert errs["h"] < tol("bf16", "bf16") and max(v for n, v in errs.items() if n != "h") < 2e-3, errs


def test_prologue_full_layer_sampled_head():
    """The 350M-layer shape (B=8, T=4096, H=8, d=128, KDA, bf16) with the forget
    prologue through the training pair; the oracle recomputes (b, h) = (2, 5)."""
    announce("prologue full layer c4")
    cfg = dict(gdr_inputs.CONFIGS["c4"])
    cfg.update(prologue="forget", clvr=False)
    inp = gdr_inputs.make(**cfg)
    B, T, H, d = inp["q"].shape
    t = inputs_to_dev(inp, "bf16")
    ws = torch.empty(gdr.workspace_size(B, T, H, d, gdr.GATE_CHANNEL, torch.bfloat16, torch.bfloat16,
                                        backward=True, prologue="forget"), dtype=torch.uint8, device="cuda")
    o, _, g = gpu_pro(t, "forget", out_dtype=torch.bfloat16, workspace=ws, save_for_backward=True,
                      saved_workspace=ws)
    b, hh = 2, 5
    sub = {n: (None if inp[n] is None else inp[n][b:b + 1, :, hh:hh + 1])
           for n in ("q", "k", "v", "beta", "alpha", "dO")}
    sub["S0"] = None
    o_ref, _, ref = oracle_pro(sub, "forget")
    errs = {"o": rel(o[b:b + 1, :, hh:hh + 1], o_ref)}
    for n in ("dq", "dk", "dv", "dbeta", "dalpha"):
        errs[n] = rel(g[n][b:b + 1, :, hh:hh + 1], ref[n])
    report(**errs)
    assert max(errs.values()) < tol("bf16", "bf16"), errs
    assert errs["dbeta"] < 2e-3, errs
