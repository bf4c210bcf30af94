"""GPU parity of the output-gate epilogue y = sigmoid(g) * w * RMSNorm(o) per
head (KDA blog 4.1), standalone and chained with the operator.

The gate is fp32 arithmetic on stored values, so with fp32 storage it is held
to 1e-5; bf16-stored results add bf16's unit roundoff 2^-8.  The chained
training test holds the operator's gradients to the usual 2e-3 (bf16 inputs)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_37_amd as gdr
import gdr_inputs
import oracle
from gpu_util import BF16_ULP, announce, inputs_to_dev, rel, report, to_dev

pytestmark = pytest.mark.gpu

TD = {"bf16": torch.bfloat16, "fp32": torch.float32}


def gate_inputs(B, T, H, d, o_dt, g_dt, seed):
    r = np.random.default_rng(seed)
    o = gdr_inputs.round_to(r.standard_normal((B, T, H, d)) * r.uniform(0.05, 3, (B, T, H, 1)), o_dt)
    g = gdr_inputs.round_to(r.standard_normal((B, T, H, d)) * 2, g_dt)
    w = (1 + 0.3 * r.standard_normal(H * d)).astype(np.float32)
    dy = gdr_inputs.round_to(r.standard_normal((B, T, H, d)), o_dt)
    return o, g, w, dy


@pytest.mark.parametrize("d,o_dt,g_dt", [(128, "fp32", "fp32"), (64, "fp32", "fp32"), (128, "bf16", "bf16"),
                                         (128, "fp32", "bf16"), (64, "bf16", "fp32")])
def test_output_gate_matches_oracle(d, o_dt, g_dt):
    announce("output gate d=%d o=%s g=%s" % (d, o_dt, g_dt))
    o, g, w, dy = gate_inputs(2, 300, 3, d, o_dt, g_dt, seed=700 + d)
    od, gd, wd, dyd = to_dev(o, TD[o_dt]), to_dev(g, TD[g_dt]), to_dev(w), to_dev(dy, TD[o_dt])
    y = gdr.output_gate(od, gd, wd)
    dO, dg, dw = gdr.output_gate_backward(od, gd, wd, dyd)
    torch.cuda.synchronize()
    y_ref, _ = oracle.output_gate_forward(o, g, w)
    do_ref, dg_ref, dw_ref = oracle.output_gate_backward(o, g, w, dy)
    errs = {"y": rel(y, y_ref), "dO": rel(dO, do_ref), "dg": rel(dg, dg_ref), "dw": rel(dw, dw_ref)}
    report(**errs)
    ty = 1e-5 + (BF16_ULP if o_dt == "bf16" else 0)
    tg = 1e-5 + (BF16_ULP if g_dt == "bf16" else 0)
    assert errs["y"] < ty and errs["dO"] < tg and errs["dg"] < tg and errs["dw"] < 1e-5, errs


def test_output_gate_in_place_and_unit_weight():
    o, g, _, dy = gate_inputs(1, 70, 2, 128, "fp32", "fp32", seed=710)
    od, gd = to_dev(o), to_dev(g)
    y1 = gdr.output_gate(od, gd, None)
    y2 = gdr.output_gate(od, gd, torch.ones(256, device="cuda"))
    o2 = od.clone()
    gdr.output_gate(o2, gd, None, out=o2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(y1, o2)
    assert rel(y1, oracle.output_gate_forward(o, g)[0]) < 1e-5


def test_output_gate_ragged_and_tiny():
    """Token counts that leave the last token range short, and a single row."""
    for B, T in ((1, 1), (3, 257), (1, 1000)):
        o, g, w, dy = gate_inputs(B, T, 2, 64, "fp32", "fp32", seed=720 + T)
        od, gd, wd, dyd = to_dev(o), to_dev(g), to_dev(w), to_dev(dy)
        y = gdr.output_gate(od, gd, wd)
        dO, dg, dw = gdr.output_gate_backward(od, gd, wd, dyd)
        torch.cuda.synchronize()
        do_ref, dg_ref, dw_ref = oracle.output_gate_backward(o, g, w, dy)
        errs = {"y": rel(y, oracle.output_gate_forward(o, g, w)[0]), "dO": rel(dO, do_ref), "dg": rel(dg, dg_ref),
                "dw": rel(dw, dw_ref)}
        report(**errs)
        assert max(errs.values()) < 1e-5, (B, T, errs)


def test_output_gate_full_size():
    """The 32K-token KDA prefill shape (B=1, T=32768, H=16, dv=128, bf16), the
    whole tensor against the oracle."""
    announce("output gate full size")
    o, g, w, dy = gate_inputs(1, 32768, 16, 128, "bf16", "bf16", seed=730)
    od, gd, wd, dyd = to_dev(o, torch.bfloat16), to_dev(g, torch.bfloat16), to_dev(w), to_dev(dy, torch.bfloat16)
    y = gdr.output_gate(od, gd, wd)
    dO, dg, dw = gdr.output_gate_backward(od, gd, wd, dyd)
    torch.cuda.synchronize()
    do_ref, dg_ref, dw_ref = oracle.output_gate_backward(o, g, w, dy)
    errs = {"y": rel(y, oracle.output_gate_forward(o, g, w)[0]), "dO": rel(dO, do_ref), "dg": rel(dg, dg_ref),
            "dw": rel(dw, dw_ref)}
    report(**errs)
    assert errs["dw"] < 1e-5 and max(errs.values()) < 1e-5 + BF16_ULP, errs


def test_output_gate_chained_with_the_operator():
    """Training step of a gated KDA layer: o = forward(...), y = gate(o, g);
    from dy the gate gives dO (bf16, the operator's dO) and the operator's
    backward the input gradients.  The oracle runs the same chain in fp64 from
    the GPU's own dO, so the comparison isolates each stage."""
    announce("output gate chained")
    inp = gdr_inputs.make(B=2, T=200, H=2, d=128, gate="channel", dtype="bf16", seed=740, s0=True, bwd=True)
    t = inputs_to_dev(inp, "bf16")
    r = np.random.default_rng(741)
    g = gdr_inputs.round_bf16(r.standard_normal((2, 200, 2, 128)))
    w = (1 + 0.3 * r.standard_normal(256)).astype(np.float32)
    dy = r.standard_normal((2, 200, 2, 128)).astype(np.float32)
    o, _ = gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], out_dtype=torch.float32)
    y = gdr.output_gate(o, to_dev(g, torch.bfloat16), to_dev(w))
    dO, dg, dw = gdr.output_gate_backward(o, to_dev(g, torch.bfloat16), to_dev(w), to_dev(dy))
    gr = gdr.backward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], dO, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], inp["S0"])
    y_ref, _ = oracle.output_gate_forward(o_ref, g, w)
    do_ref, dg_ref, dw_ref = oracle.output_gate_backward(o_ref, g, w, dy)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], inp["S0"],
                          dO.float().cpu().numpy())
    errs = {"y": rel(y, y_ref), "dO": rel(dO, do_ref), "dg": rel(dg, dg_ref), "dw": rel(dw, dw_ref)}
    for n in ("dq", "dk", "dv", "dbeta", "dalpha", "dS0"):
        errs[n] = rel(gr[n], ref[n])
    report(**errs)
    assert errs["y"] < 2e-3 and errs["dw"] < 2e-3, errs
    assert errs["dO"] < 2e-3 + BF16_ULP and errs["dg"] < 2e-3 + BF16_ULP, errs
    assert max(errs[n] for n in ("dq", "dk", "dv", "dbeta", "dalpha", "dS0")) < 2e-3, errs
