"""GPU parity of gdr_decode_step against the fp64 oracle (one recurrence step)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_37_amd as gdr
import gdr_inputs
import oracle
from gpu_util import TORCH, report, announce, rel, to_dev

pytestmark = pytest.mark.gpu


def run(N, H, d, gate, in_dt, out_dt, seed):
    inp = gdr_inputs.make_decode(N=N, H=H, d=d, gate=gate, dtype=in_dt, seed=seed)
    announce("decode N=%d H=%d d=%d gate=%s in=%s out=%s seed=%d" % (N, H, d, gate, in_dt, out_dt, seed))
    t = {n: (None if inp[n] is None else to_dev(inp[n], TORCH[in_dt] if n in "qkv" else torch.float32))
         for n in ("q", "k", "v", "beta", "alpha")}
    S = to_dev(inp["S"][0])
    o = gdr.decode_step(t["q"], t["k"], t["v"], t["beta"], t["alpha"], S, scale=0.75,
                        out_dtype=TORCH[out_dt])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.decode(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], inp["S"][0],
                                 scale=0.75)
    return rel(o, o_ref), rel(S, S_ref)


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("in_dt,out_dt", [("bf16", "fp32"), ("fp32", "fp32"), ("bf16", "bf16")])
def test_decode_parity(gate, d, in_dt, out_dt):
    eo, es = run(5, 3, d, gate, in_dt, out_dt, seed=40 + d)
    # all arithmetic is fp32 on exact inputs: fp32-level agreement, plus the
    # output rounding when o is stored in bf16
    report(o=eo, S=es)
    assert es < 1e-5
    assert eo < (1e-5 if out_dt == "fp32" else 2.0 ** -8 + 1e-5)


def test_decode_full_size_256_sequences():
    """The 256-sequence, 16-head KDA decode step (256 MiB of fp32 state), every
    slab compared."""
    cfg = gdr_inputs.DECODE_CONFIG
    eo, es = run(cfg["N"], cfg["H"], cfg["d"], cfg["gate"], "bf16", "fp32", seed=cfg["seed"])
    report(o=eo, S=es)
    assert eo < 1e-5 and es < 1e-5


def test_decode_steps_compose():
    """Two steps in a row equal two oracle steps (state handed over in place)."""
    inp = gdr_inputs.make_decode(N=4, H=2, d=128, seed=50)
    inp2 = gdr_inputs.make_decode(N=4, H=2, d=128, seed=51)
    S = to_dev(inp["S"][0])
    S_ref = inp["S"][0].astype(np.float64)
    for x in (inp, inp2):
        t = {n: to_dev(x[n], torch.bfloat16 if n in "qkv" else torch.float32)
             for n in ("q", "k", "v", "beta", "alpha")}
        o = gdr.decode_step(t["q"], t["k"], t["v"], t["beta"], t["alpha"], S, out_dtype=torch.float32)
        o_ref, S_ref = oracle.decode(x["q"], x["k"], x["v"], x["beta"], x["alpha"], S_ref)
        torch.cuda.synchronize()
        assert rel(o, o_ref) < 1e-5
    assert rel(S, S_ref) < 1e-5


def test_decode_rejects_cpu_tensors():
    inp = gdr_inputs.make_decode(N=2, H=1, d=64, seed=52)
    t = {n: torch.from_numpy(inp[n]) for n in ("q", "k", "v", "beta", "alpha")}
    with pytest.raises(ValueError):
        gdr.decode_step(t["q"], t["k"], t["v"], t["beta"], t["alpha"], torch.from_numpy(inp["S"][0]))
