"""GPU checks of the training pair (gdr_forward_train + gdr_backward_saved).

The training forward must give the plain forward's results bit for bit and
leave in its workspace what the saved backward needs; the saved backward must
give the recomputing backward's gradients bit for bit.  Parity with the fp64
oracle is also checked directly on the small cases."""
import numpy as np
import pytest
import torch

import gated_delta_rule_37_amd as gdr
import gdr_inputs
import oracle
from gpu_util import announce, inputs_to_dev, rel, report, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dbeta", "dalpha", "dS0", "dclvr_scale")


def run_pair(t, dtype, out_dtype, lam=None, dh=None, h=None, dST=None):
    B, T, H, d = t["q"].shape
    gate = gdr.GATE_NONE if t["alpha"] is None else (gdr.GATE_SCALAR if t["alpha"].dim() == 3
                                                      else gdr.GATE_CHANNEL)
    ws = torch.empty(gdr.workspace_size(B, T, H, d, gate, dtype, out_dtype, backward=True),
                     dtype=torch.uint8, device="cuda")
    h1 = None if h is None else h.clone()
    o, ST = gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], out_dtype=out_dtype, h=h1,
                        clvr_scale=lam, workspace=ws, save_for_backward=True)
    g = gdr.backward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], t["dO"], dST, out_dtype=out_dtype,
                     dh=dh, clvr_scale=lam, want_dclvr_scale=dh is not None, saved_workspace=ws)
    torch.cuda.synchronize()
    return o, ST, h1, g


def run_separate(t, out_dtype, lam=None, dh=None, h=None, dST=None):
    h2 = None if h is None else h.clone()
    o, ST = gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], out_dtype=out_dtype, h=h2,
                        clvr_scale=lam)
    g = gdr.backward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], t["dO"], dST, out_dtype=out_dtype,
                     dh=dh, clvr_scale=lam, want_dclvr_scale=dh is not None)
    torch.cuda.synchronize()
    return o, ST, h2, g


def assert_same(a, b):
    o1, S1, h1, g1 = a
    o2, S2, h2, g2 = b
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    if h1 is not None:
        assert torch.equal(h1, h2)
    for n in GRADS:
        if g1[n] is None:
            assert g2[n] is None, n
        else:
            assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_training_pair_bf16_equals_separate_calls_and_oracle(gate):
    announce("training pair bf16 gate=%s" % gate)
    inp = gdr_inputs.make(B=2, T=200, H=2, d=128, gate=gate, dtype="bf16", seed=400, s0=True, bwd=True,
                          clvr=True)
    r = np.random.default_rng(401)
    lam = to_dev(r.standard_normal(256).astype(np.float32))
    dh = to_dev(gdr_inputs.round_bf16(r.standard_normal((2, 200, 256))), torch.bfloat16)
    dST = (0.1 * r.standard_normal((2, 2, 128, 128))).astype(np.float32)
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("h", "lam")}, "bf16")
    h = to_dev(inp["h"], torch.bfloat16)
    pair = run_pair(t, torch.bfloat16, torch.float32, lam, dh, h, to_dev(dST))
    assert_same(pair, run_separate(t, torch.float32, lam, dh, h, to_dev(dST)))
    o, ST, _, g = pair
    o_ref, ST_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], inp["S0"])
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], inp["S0"], inp["dO"], dST)
    errs = {"o": rel(o, o_ref), "S": rel(ST, ST_ref)}
    for n in ("dq", "dk", "dbeta", "dalpha", "dS0"):
        if ref[n] is not None:
            errs[n] = rel(g[n], ref[n])
    dv_c, _ = oracle.clvr_backward(dh.float().cpu().numpy(), inp["v"], lam.cpu().numpy())
    errs["dv"] = rel(g["dv"], ref["dv"] + dv_c)
    report(**errs)
    assert max(errs.values()) < 2e-3, errs


@pytest.mark.parametrize("d", [64, 128])
def test_training_pair_fp32_equals_separate_calls(d):
    announce("training pair fp32 d=%d" % d)
    inp = gdr_inputs.make(B=1, T=150, H=2, d=d, gate="channel", dtype="fp32", seed=410, s0=True, bwd=True)
    t = inputs_to_dev(inp, "fp32")
    pair = run_pair(t, torch.float32, torch.float32)
    assert_same(pair, run_separate(t, torch.float32))
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], inp["S0"], inp["dO"])
    errs = {n: rel(pair[3][n], ref[n]) for n in ("dq", "dk", "dv", "dbeta", "dalpha", "dS0")}
    report(**errs)
    assert max(errs.values()) < 1e-5, errs


def test_training_pair_full_layer_equals_separate_calls():
    """350M-layer shape (B=8, T=4096, H=8, d=128, KDA, bf16, CLVR)."""
    announce("training pair full c4")
    inp, cfg = gdr_inputs.make_config("c4")
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("h", "lam")}, "bf16")
    lam = to_dev(inp["lam"])
    h = to_dev(inp["h"], torch.bfloat16)
    dh = to_dev(gdr_inputs.round_bf16(np.random.default_rng(420).standard_normal(inp["h"].shape)),
                torch.bfloat16)
    assert_same(run_pair(t, torch.bfloat16, torch.bfloat16, lam, dh, h),
                run_separate(t, torch.bfloat16, lam, dh, h))


@pytest.mark.parametrize("out_dt", ["fp32", "bf16"])
def test_training_pair_32k_prefill_sampled_heads(out_dt):
    """The timed training step itself: KDA, B=1 H=16 T=32768 d=128, bf16 inputs,
    CLVR with its scale gradient, through gdr_forward_train + gdr_backward_saved
    (the forward chain and the reverse pass cut into chunk ranges, the per-chunk
    kernels of each range on the second stream).  o, S_T and every gradient of
    heads 0 and 11 are compared with the oracle, element by element; h and
    dlam over the whole hidden stream.  fp32 outputs are held to 2e-3, bf16
    outputs (the timed configuration) to 2e-3 + 2^-8."""
    announce("training pair 32K prefill sampled heads, %s outputs" % out_dt)
    inp, cfg = gdr_inputs.make_config("c5b", bwd=True, clvr=True)
    B, T, H, d = cfg["B"], cfg["T"], cfg["H"], cfg["d"]
    r = np.random.default_rng(430)
    lam = r.standard_normal(H * d).astype(np.float32)
    dh = gdr_inputs.round_bf16(r.standard_normal((B, T, H * d)))
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("h", "lam")}, "bf16")
    od = torch.float32 if out_dt == "fp32" else torch.bfloat16
    h = to_dev(inp["h"], torch.bfloat16)
    ws = torch.empty(gdr.workspace_size(B, T, H, d, gdr.GATE_CHANNEL, torch.bfloat16, od, backward=True),
                     dtype=torch.uint8, device="cuda")
    o, ST = gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], None, out_dtype=od, h=h,
                        clvr_scale=to_dev(lam), workspace=ws, output_final_state=True, save_for_backward=True)
    g = gdr.backward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], None, t["dO"], out_dtype=od,
                     dh=to_dev(dh, torch.bfloat16), clvr_scale=to_dev(lam), want_dclvr_scale=True,
                     saved_workspace=ws)
    torch.cuda.synchronize()
    heads = [0, 11]
    sl = lambda a: np.ascontiguousarray(a[:, :, heads])  # noqa: E731
    o_ref, ST_ref = oracle.forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]), sl(inp["alpha"]),
                                   None, nthreads=len(heads))
    ref = oracle.backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]), sl(inp["alpha"]), None,
                          sl(inp["dO"]), nthreads=len(heads))
    dvc, dlam = oracle.clvr_backward(dh, inp["v"], lam)
    h_ref = oracle.clvr_forward(inp["h"], inp["v"], lam)
    ref["dv"] = ref["dv"] + sl(dvc.reshape(B, T, H, d))
    errs = {"o": rel(o[:, :, heads], o_ref), "S_T": rel(ST[:, heads], ST_ref)}
    for n in ("dq", "dk", "dv", "dbeta", "dalpha"):
        errs[n] = rel(g[n][:, :, heads], ref[n])
    errs["dlam"] = rel(g["dclvr_scale"], dlam)
    errs["h"] = rel(h, h_ref)
    report(**errs)
    bar = 2e-3 if out_dt == "fp32" else 2e-3 + 2.0 ** -8
    # o, dq, dk, dv are stored in the output dtype; S_T, dbeta, dalpha, dlam are
    # always fp32; h is the bf16 hidden stream
    for n, e in errs.items():
        b = bar if n in ("o", "dq", "dk", "dv") else (2e-3 + 2.0 ** -8 if n == "h" else 2e-3)
        assert e < b, (n, e, b)
