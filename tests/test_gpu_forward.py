"""GPU parity of gdr_forward_chunked against the fp64 oracle.

Small cases span several chunks and a ragged tail (T = 200 = 3 * 64 + 8); the
full-size workloads are checked on sampled heads, which the oracle computes
completely (heads are independent).  Tolerances: see gpu_util.TOL."""
import numpy as np
import pytest
import torch

import gated_delta_rule_37_amd as gdr
import gdr_inputs
import oracle
from gpu_util import TORCH, announce, inputs_to_dev, rel, report, tol

pytestmark = pytest.mark.gpu


def gpu_forward(t, out_dt="fp32", scale=1.0, h=None, lam=None):
    o, ST = gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], scale=scale,
                        out_dtype=TORCH[out_dt], h=h, clvr_scale=lam)
    torch.cuda.synchronize()
    return o, ST


def check(inp, in_dt, out_dt="fp32", scale=1.0, heads=None):
    t = inputs_to_dev(inp, in_dt)
    o, ST = gpu_forward(t, out_dt, scale)
    if heads is None:
        o_ref, ST_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"],
                                       inp["S0"], scale=scale)
        return rel(o, o_ref), rel(ST, ST_ref)
    eo = es = 0.0
    for (b, h) in heads:
        sl = lambda a: None if a is None else a[b:b + 1, :, h:h + 1]  # noqa: E731
        S0 = None if inp["S0"] is None else inp["S0"][b:b + 1, h:h + 1]
        o_ref, ST_ref = oracle.forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]),
                                       sl(inp["alpha"]), S0, scale=scale)
        eo = max(eo, rel(o[b:b + 1, :, h:h + 1], o_ref))
        es = max(es, rel(ST[b:b + 1, h:h + 1], ST_ref))
    return eo, es


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("in_dt", ["bf16", "fp32"])
@pytest.mark.parametrize("s0", [False, True])
def test_forward_parity_small(gate, d, in_dt, s0):
    announce("forward small gate=%s d=%d in=%s s0=%s" % (gate, d, in_dt, s0))
    inp = gdr_inputs.make(B=2, T=200, H=2, d=d, gate=gate, dtype=in_dt, seed=100 + d, s0=s0)
    eo, es = check(inp, in_dt)
    report(o=eo, S=es)
    assert eo < tol(in_dt, "fp32") and es < tol(in_dt, "fp32"), (eo, es)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_forward_ragged_lengths(T):
    announce("forward ragged T=%d" % T)
    inp = gdr_inputs.make(B=1, T=T, H=3, d=128, gate="channel", dtype="bf16", seed=200 + T, s0=True)
    eo, es = check(inp, "bf16")
    report(o=eo, S=es)
    assert eo < 2e-3 and es < 2e-3, (eo, es)


@pytest.mark.parametrize("d,B,H", [(64, 5, 14), (128, 3, 11)])
def test_forward_more_state_slices_than_cus(d, B, H):
    """More 16-column state slices (B*H*d/16 = 280 and 264) than the chip has
    CUs (256): the chain pass then carries two slices per workgroup.  Ragged
    T = 130, with an initial state."""
    announce("forward two-slice chain d=%d B=%d H=%d" % (d, B, H))
    inp = gdr_inputs.make(B=B, T=130, H=H, d=d, gate="channel", dtype="bf16", seed=250 + d, s0=True)
    eo, es = check(inp, "bf16")
    report(o=eo, S=es)
    assert eo < 2e-3 and es < 2e-3, (eo, es)


def test_forward_empty_sequence_copies_state():
    announce("forward T=0")
    inp = gdr_inputs.make(B=2, T=0, H=2, d=64, gate="channel", dtype="bf16", seed=210, s0=True)
    t = inputs_to_dev(inp, "bf16")
    o, ST = gpu_forward(t)
    assert o.numel() == 0
    assert torch.equal(ST.cpu(), torch.from_numpy(inp["S0"]))


def test_forward_deltanet_fp32_config():
    """DeltaNet, fp32, B=1 H=2 T=256 d=64, zero start (tolerance 1e-5)."""
    announce("forward c1")
    inp, cfg = gdr_inputs.make_config("c1")
    eo, es = check(inp, "fp32")
    report(o=eo, S=es)
    assert eo < 1e-5 and es < 1e-5, (eo, es)


def test_forward_bf16_output():
    announce("forward bf16 out")
    inp = gdr_inputs.make(B=1, T=300, H=2, d=128, gate="channel", dtype="bf16", seed=220, s0=True)
    eo, es = check(inp, "bf16", out_dt="bf16", scale=0.5)
    report(o=eo, S=es)
    assert eo < tol("bf16", "bf16") and es < 2e-3, (eo, es)


@pytest.mark.parametrize("gate", ["channel", "scalar"])
@pytest.mark.parametrize("recipe", ["sigmoid(N(-1,1))", "uniform[1e-6,1e-3]"])
def test_forward_strong_gates(recipe, gate):
    """Gates far stronger than the workloads': the in-block decay range exceeds
    what fp16 operands can carry, so the exact diagonal-block path runs; with
    alpha <= 1e-3 a chunk's total decay (below 2^-600) leaves the fp32 range, for
    the scalar gate as for the channel gate."""
    announce("forward strong gates %s %s" % (gate, recipe))
    inp = gdr_inputs.make(B=1, T=2048, H=2, d=128, gate=gate, dtype="bf16", seed=230,
                          s0=True, alpha_recipe=recipe)
    eo, es = check(inp, "bf16")
    report(o=eo, S=es)
    assert eo < 2e-3 and es < 2e-3, (eo, es)


@pytest.mark.parametrize("gate", ["channel", "scalar"])
def test_forward_strong_gates_fp32(gate):
    announce("forward strong gates fp32 %s" % gate)
    inp = gdr_inputs.make(B=1, T=300, H=2, d=64, gate=gate, dtype="fp32", seed=231,
                          s0=True, alpha_recipe="uniform[1e-6,1e-3]")
    eo, es = check(inp, "fp32")
    report(o=eo, S=es)
    assert eo < 1e-5 and es < 1e-5, (eo, es)


@pytest.mark.parametrize("beta", ["const:0", "const:1", "choice{0,1,2}"])
def test_forward_beta_edge_values(beta):
    announce("forward beta %s" % beta)
    inp = gdr_inputs.make(B=1, T=256, H=2, d=128, gate="channel", dtype="bf16", seed=240, s0=True,
                          beta_recipe=beta)
    eo, es = check(inp, "bf16")
    report(o=eo, S=es)
    assert eo < 2e-3 and es < 2e-3, (eo, es)


def test_forward_exact_retrieval_on_gpu():
    """Unit keys, beta = 1, q = k: every read returns the value just written."""
    announce("forward exact retrieval")
    inp = gdr_inputs.make(B=1, T=192, H=2, d=128, gate="channel", dtype="fp32", seed=250, s0=True,
                          beta_recipe="const:1")
    inp["q"] = inp["k"]
    t = inputs_to_dev(inp, "fp32")
    o, _ = gpu_forward(t)
    assert rel(o, inp["v"]) < 1e-5


# ------------------------------------------------------------------ CLVR


def test_clvr_epilogue_matches_oracle():
    announce("clvr")
    inp = gdr_inputs.make(B=2, T=130, H=2, d=128, gate="channel", dtype="bf16", seed=260, clvr=True)
    r = np.random.default_rng(261)
    lam = r.standard_normal(2 * 128).astype(np.float32)
    t = inputs_to_dev(inp, "bf16")
    h = t["h"].clone()
    gpu_forward(t, h=h, lam=torch.from_numpy(lam).cuda())
    h_ref = oracle.clvr_forward(inp["h"], inp["v"], lam)
    h_ref_bf16 = gdr_inputs.round_bf16(h_ref)
    # one fused multiply-add in fp32, then one rounding to bf16
    diff = np.abs(h.float().cpu().numpy() - h_ref_bf16)
    ulp = np.abs(h_ref_bf16) * 2.0 ** -7 + 1e-30
    assert np.all(diff <= ulp)


def test_clvr_zero_scale_is_bitwise_no_op_and_unit_scale_adds_v():
    """CLVR's projection is zero-initialised: with lam = 0 the hidden stream is
    unchanged; with lam = 1 it gains exactly v (one rounding)."""
    announce("clvr zero/unit")
    inp = gdr_inputs.make(B=1, T=100, H=2, d=64, gate="scalar", dtype="bf16", seed=262, clvr=True)
    t = inputs_to_dev(inp, "bf16")
    h0 = t["h"].clone()
    gpu_forward(t, h=h0, lam=torch.zeros(128, device="cuda"))
    assert torch.equal(h0, t["h"])
    h1 = t["h"].clone()
    gpu_forward(t, h=h1)  # lam NULL means 1
    ref = gdr_inputs.round_bf16(inp["h"].astype(np.float64) + inp["v"].reshape(1, 100, 128))
    assert np.array_equal(h1.float().cpu().numpy(), ref)


# ------------------------------------------------------------------ invariants (GPU vs GPU)


def test_split_call_state_handoff():
    """Running T = T1 + T2 as two calls with S_T handed over equals one call."""
    announce("split call")
    inp = gdr_inputs.make(B=2, T=256, H=2, d=128, gate="channel", dtype="bf16", seed=270, s0=True)
    t = inputs_to_dev(inp, "bf16")
    o, ST = gpu_forward(t)
    a = {n: (None if v is None or n == "S0" else v[:, :128].contiguous()) for n, v in t.items()}
    bb = {n: (None if v is None or n == "S0" else v[:, 128:].contiguous()) for n, v in t.items()}
    a["S0"] = t["S0"]
    o1, S1 = gpu_forward(a)
    bb["S0"] = S1
    o2, S2 = gpu_forward(bb)
    scale_o = o.abs().max().item()
    assert (torch.cat([o1, o2], 1) - o).abs().max().item() / scale_o < 1e-3
    assert (S2 - ST).abs().max().item() / ST.abs().max().item() < 1e-3


def test_decode_steps_equal_chunked_forward():
    announce("decode vs forward")
    inp = gdr_inputs.make(B=2, T=70, H=2, d=64, gate="channel", dtype="fp32", seed=271, s0=True)
    t = inputs_to_dev(inp, "fp32")
    o, ST = gpu_forward(t)
    S = t["S0"].clone()
    for s in range(70):
        ot = gdr.decode_step(t["q"][:, s].contiguous(), t["k"][:, s].contiguous(),
                             t["v"][:, s].contiguous(), t["beta"][:, s].contiguous(),
                             t["alpha"][:, s].contiguous(), S)
        assert (ot - o[:, s]).abs().max().item() < 1e-4
    torch.cuda.synchronize()
    assert (S - ST).abs().max().item() < 1e-4


def test_forward_is_deterministic():
    announce("determinism")
    inp = gdr_inputs.make(B=1, T=500, H=4, d=128, gate="channel", dtype="bf16", seed=272, s0=True)
    t = inputs_to_dev(inp, "bf16")
    o1, S1 = gpu_forward(t)
    o2, S2 = gpu_forward(t)
    assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_state_may_alias_initial_state():
    announce("ST aliases S0")
    inp = gdr_inputs.make(B=1, T=100, H=2, d=64, gate="scalar", dtype="bf16", seed=273, s0=True)
    t = inputs_to_dev(inp, "bf16")
    o, ST = gpu_forward(t)
    S = t["S0"].clone()
    desc_o = torch.empty_like(o)
    import ctypes
    from gated_delta_rule_37_amd import _lib
    lib = _lib.load_library()
    d = _lib._desc(t["q"], t["v"], t["alpha"], torch.float32, 1.0)
    need = lib.gdr_workspace_size(ctypes.byref(d), 0)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    rc = lib.gdr_forward_chunked(ctypes.byref(d), _lib._ptr(t["q"]), _lib._ptr(t["k"]),
                                 _lib._ptr(t["v"]), _lib._ptr(t["beta"]), _lib._ptr(t["alpha"]),
                                 _lib._ptr(S), _lib._ptr(desc_o), _lib._ptr(S), None, None,
                                 _lib._ptr(ws), need, _lib._stream(S.device))
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(S, ST) and torch.equal(desc_o, o)


# ------------------------------------------------------------------ full-size workloads, sampled heads


@pytest.mark.parametrize("name,heads", [
    ("c2", [(0, 0), (3, 15)]),
    ("c3", [(0, 5)]),
    ("c5b", [(0, 0), (0, 11)]),
])
def test_forward_full_size_sampled_heads(name, heads):
    """The full workload runs on the GPU in the configuration the benchmark
    times; the oracle recomputes the listed (batch, head) slabs completely."""
    announce("forward full size %s" % name)
    inp, cfg = gdr_inputs.make_config(name)
    eo, es = check(inp, cfg["dtype"], heads=heads)
    report(o=eo, S=es)
    assert eo < 2e-3 and es < 2e-3, (eo, es)
