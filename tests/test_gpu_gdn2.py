"""GPU parity of the Gated DeltaNet-2 path (separate erase and write gates)
against the oracle's token loop (popular article on the study, its Gated
DeltaNet-2 paragraph; the reading implemented is
S_t = (I - (e_t*k_t) k_t^T) Diag(alpha_t) S_{t-1} + (w_t*k_t) v_t^T).

Chunked forward and decode step, every gate kind, d = 64 and 128, bf16 inputs
(fp32 outputs, bar 2e-3) and fp32 inputs (bar 1e-5; the two input types run
different intra-chunk kernels), ragged and empty
sequences, strong gates (the exact diagonal-block path), the equal-gate
reduction to the KDA path, T decode steps against the chunked forward, and a
16-head 16K-token run checked on sampled heads."""
import numpy as np
import pytest
import torch

import gated_delta_rule_37_amd as gdr
import gdr_inputs
import oracle
from gpu_util import TORCH, announce, inputs_to_dev, rel, report, to_dev

pytestmark = pytest.mark.gpu


def gates(shape, seed, kind="uniform"):
    """Erase and write gates [..., dk]: independent U(0, 1) draws (fp32)."""
    r = np.random.default_rng(seed)
    if kind == "uniform":
        return r.uniform(0, 1, shape).astype(np.float32), r.uniform(0, 1, shape).astype(np.float32)
    raise ValueError(kind)


def make(B, T, H, d, gate, dtype, seed, s0=True, alpha_recipe="sigmoid(N(3,1))"):
    inp = gdr_inputs.make(B=B, T=T, H=H, d=d, gate=gate, dtype=dtype, seed=seed, s0=s0, alpha_recipe=alpha_recipe)
    inp["erase"], inp["write"] = gates((B, T, H, d), seed + 1)
    return inp


def run(inp, dtype, out_dtype=torch.float32):
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("erase", "write", "beta")}, dtype)
    o, ST = gdr.gdn2_forward(t["q"], t["k"], t["v"], to_dev(inp["erase"]), to_dev(inp["write"]), t["alpha"], t["S0"],
                             out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, ST


def ref(inp, heads=None):
    if heads is None:
        return oracle.gdn2_forward(inp["q"], inp["k"], inp["v"], inp["erase"], inp["write"], inp["alpha"], inp["S0"])
    sl = lambda a: None if a is None else np.ascontiguousarray(a[:, :, heads])  # noqa: E731
    S0 = None if inp["S0"] is None else np.ascontiguousarray(inp["S0"][:, heads])
    return oracle.gdn2_forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["erase"]), sl(inp["write"]),
                               sl(inp["alpha"]), S0, nthreads=len(heads))


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("d", [64, 128])
def test_gdn2_forward_bf16(gate, d):
    announce("gdn2 forward bf16 gate=%s d=%d" % (gate, d))
    inp = make(2, 200, 2, d, gate, "bf16", 1000 + d)
    o, ST = run(inp, "bf16")
    o_ref, S_ref = ref(inp)
    errs = {"o": rel(o, o_ref), "S_T": rel(ST, S_ref)}
    report(**errs)
    assert max(errs.values()) < 2e-3, errs


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("d", [64, 128])
def test_gdn2_forward_fp32(gate, d):
    announce("gdn2 forward fp32 gate=%s d=%d" % (gate, d))
    inp = make(1, 150, 2, d, gate, "fp32", 1010)
    o, ST = run(inp, "fp32")
    o_ref, S_ref = ref(inp)
    errs = {"o": rel(o, o_ref), "S_T": rel(ST, S_ref)}
    report(**errs)
    assert max(errs.values()) < 1e-5, errs


@pytest.mark.parametrize("T", [0, 1, 63, 64, 65, 130])
def test_gdn2_forward_ragged(T):
    announce("gdn2 forward ragged T=%d" % T)
    inp = make(1, T, 2, 128, "channel", "bf16", 1020 + T)
    o, ST = run(inp, "bf16")
    o_ref, S_ref = ref(inp)
    if T == 0:
        assert torch.equal(ST.cpu(), torch.from_numpy(inp["S0"]))
        return
    errs = {"o": rel(o, o_ref), "S_T": rel(ST, S_ref)}
    report(**errs)
    assert max(errs.values()) < 2e-3, errs


@pytest.mark.parametrize("gate", ["channel", "scalar"])
@pytest.mark.parametrize("recipe", ["sigmoid(N(-1,1))", "uniform[1e-6,1e-3]"])
def test_gdn2_forward_strong_gates(recipe, gate):
    """Decay ranges above 60 (log2) inside a 16-token block take the pair-by-pair
    path of the diagonal blocks."""
    announce("gdn2 forward strong gates %s %s" % (gate, recipe))
    inp = make(1, 300, 2, 128, gate, "bf16", 1030, alpha_recipe=recipe)
    o, ST = run(inp, "bf16")
    o_ref, S_ref = ref(inp)
    errs = {"o": rel(o, o_ref), "S_T": rel(ST, S_ref)}
    report(**errs)
    assert max(errs.values()) < 2e-3, errs


def test_gdn2_equal_gates_is_the_kda_path():
    """e = w = beta (broadcast): the GDN-2 kernels and the KDA kernels both
    match the KDA oracle (the page's reduction)."""
    announce("gdn2 equal gates vs KDA")
    inp = gdr_inputs.make(B=1, T=300, H=2, d=128, gate="channel", dtype="bf16", seed=1040, s0=True)
    g = np.repeat(inp["beta"][..., None], 128, -1).astype(np.float32)
    inp["erase"], inp["write"] = g, g
    o2, S2 = run(inp, "bf16")
    o_ref, S_ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], inp["S0"])
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("erase", "write")}, "bf16")
    o1, S1 = gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], out_dtype=torch.float32)
    torch.cuda.synchronize()
    errs = {"gdn2_o": rel(o2, o_ref), "gdn2_S": rel(S2, S_ref), "kda_o": rel(o1, o_ref), "kda_S": rel(S1, S_ref)}
    report(**errs)
    assert max(errs.values()) < 2e-3, errs


def test_gdn2_forward_16_heads_16k_tokens_sampled_heads():
    """B=1 H=16 T=16384 d=128 bf16 (256 chunks per sequence), heads 0 and 9
    recomputed by the oracle."""
    announce("gdn2 forward B=1 H=16 T=16384, sampled heads")
    inp = make(1, 16384, 16, 128, "channel", "bf16", 1050)
    o, ST = run(inp, "bf16")
    heads = [0, 9]
    o_ref, S_ref = ref(inp, heads)
    errs = {"o": rel(o[:, :, heads], o_ref), "S_T": rel(ST[:, heads], S_ref)}
    report(**errs)
    assert max(errs.values()) < 2e-3, errs


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_gdn2_decode(gate, dtype, d):
    announce("gdn2 decode gate=%s %s d=%d" % (gate, dtype, d))
    dec = gdr_inputs.make_decode(N=16, H=4, d=d, gate=gate, dtype=dtype, seed=1060)
    e, w = gates((16, 4, d), 1061)
    td = {n: to_dev(dec[n], TORCH[dtype]) for n in ("q", "k", "v")}
    al = None if dec["alpha"] is None else to_dev(dec["alpha"])
    S = to_dev(dec["S"][0])
    o = gdr.gdn2_decode_step(td["q"], td["k"], td["v"], to_dev(e), to_dev(w), al, S, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn2_decode(dec["q"], dec["k"], dec["v"], e, w, dec["alpha"], dec["S"][0])
    errs = {"o": rel(o, o_ref), "S": rel(S, S_ref)}
    report(**errs)
    assert max(errs.values()) < 1e-5, errs


def test_gdn2_decode_steps_equal_chunked_forward():
    announce("gdn2 decode steps vs chunked forward")
    inp = make(1, 70, 2, 128, "channel", "bf16", 1070)
    o, ST = run(inp, "bf16")
    S = to_dev(inp["S0"][:, :, :, :].copy())
    outs = []
    for t_ in range(70):
        x = {n: to_dev(np.ascontiguousarray(inp[n][:, t_]), torch.bfloat16) for n in ("q", "k", "v")}
        ot = gdr.gdn2_decode_step(x["q"], x["k"], x["v"], to_dev(np.ascontiguousarray(inp["erase"][:, t_])),
                                  to_dev(np.ascontiguousarray(inp["write"][:, t_])),
                                  to_dev(np.ascontiguousarray(inp["alpha"][:, t_])), S, out_dtype=torch.float32)
        outs.append(ot)
    torch.cuda.synchronize()
    od = torch.stack(outs, dim=1)
    errs = {"o": rel(od, o.cpu().double().numpy()), "S": rel(S, ST.cpu().double().numpy())}
    report(**errs)
    assert max(errs.values()) < 2e-3, errs


@pytest.mark.parametrize("which", ["no erase", "no write", "neither"])
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_gdn2_degenerate_gates(which, dt):
    """Gates at zero: e = 0 writes without erasing, w = 0 erases without writing,
    and with both zero the state only decays (S_T = prod Diag(alpha) S0)."""
    announce("gdn2 degenerate gates %s %s" % (which, dt))
    inp = make(1, 150, 2, 128, "channel", dt, 1080)
    if which in ("no erase", "neither"):
        inp["erase"] = np.zeros_like(inp["erase"])
    if which in ("no write", "neither"):
        inp["write"] = np.zeros_like(inp["write"])
    o, ST = run(inp, dt)
    o_ref, S_ref = ref(inp)
    if which == "neither":
        # pure decay of the initial state, independent of k and v
        decay = np.prod(inp["alpha"][0].astype(np.float64), axis=0)  # [H, dk]
        np.testing.assert_allclose(S_ref[0], decay[:, :, None] * inp["S0"][0], rtol=1e-12, atol=1e-14)
    errs = {"o": rel(o, o_ref), "S_T": rel(ST, S_ref)}
    report(**errs)
    assert max(errs.values()) < (2e-3 if dt == "bf16" else 1e-5), errs
