"""GPU parity of the cut reverse state pass.

When the reverse state pass leaves compute units idle (few batch x head
slices), the library runs it in up to four chunk ranges and overlaps the
gradient kernels of each finished range on a second stream.  These shapes
take that path (one or two heads, 2K-4K tokens); the results must match the
oracle like every other backward, and the training pair must still equal the
separate calls bit for bit."""
import numpy as np
import pytest
import torch

import gated_delta_rule_37_amd as gdr
import gdr_inputs
import oracle
from gpu_util import TOL, announce, inputs_to_dev, rel, report, to_dev

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "dbeta", "dalpha", "dS0")


@pytest.mark.parametrize("T,H,d,in_dt,gate", [(4096, 1, 128, "bf16", "channel"), (2100, 2, 128, "bf16", "scalar"),
                                              (3000, 1, 64, "fp32", "channel")])
def test_cut_reverse_pass_matches_oracle(T, H, d, in_dt, gate):
    announce("cut reverse pass T=%d H=%d d=%d %s %s" % (T, H, d, in_dt, gate))
    inp = gdr_inputs.make(B=1, T=T, H=H, d=d, gate=gate, dtype=in_dt, seed=800 + T, s0=True, bwd=True, clvr=True)
    r = np.random.default_rng(801)
    dST = (0.1 * r.standard_normal((1, H, d, d))).astype(np.float32)
    lam = r.standard_normal(H * d).astype(np.float32)
    dh = gdr_inputs.round_to(r.standard_normal((1, T, H * d)), in_dt)
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("h", "lam")}, in_dt)
    td = torch.bfloat16 if in_dt == "bf16" else torch.float32
    g = gdr.backward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], t["dO"], to_dev(dST),
                     out_dtype=torch.float32, dh=to_dev(dh, td), clvr_scale=to_dev(lam), want_dclvr_scale=True)
    torch.cuda.synchronize()
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], inp["S0"], inp["dO"], dST)
    dv_c, dlam = oracle.clvr_backward(dh, inp["v"], lam)
    ref["dv"] = ref["dv"] + dv_c
    errs = {n: rel(g[n], ref[n]) for n in GRADS if ref[n] is not None}
    errs["dlam"] = rel(g["dclvr_scale"], dlam)
    report(**errs)
    assert max(errs.values()) < TOL[in_dt], errs


def test_cut_reverse_pass_training_pair_and_error_route():
    announce("cut reverse pass, training pair, error route")
    inp = gdr_inputs.make(B=1, T=4096, H=1, d=128, gate="channel", dtype="bf16", seed=810, bwd=True, clvr=True)
    r = np.random.default_rng(811)
    lam = to_dev(r.standard_normal(128).astype(np.float32))
    dh = to_dev(gdr_inputs.round_bf16(r.standard_normal((1, 4096, 128))), torch.bfloat16)
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("h", "lam")}, "bf16")
    h0 = to_dev(inp["h"], torch.bfloat16)
    for route in ("value", "error"):
        ws = torch.empty(gdr.workspace_size(1, 4096, 1, 128, gdr.GATE_CHANNEL, torch.bfloat16, torch.float32,
                                            backward=True, route=route), dtype=torch.uint8, device="cuda")
        h1, h2 = h0.clone(), h0.clone()
        gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], None, out_dtype=torch.float32, h=h1,
                    clvr_scale=lam, workspace=ws, save_for_backward=True, route=route)
        g1 = gdr.backward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], None, t["dO"], out_dtype=torch.float32,
                          dh=dh, clvr_scale=lam, want_dclvr_scale=True, saved_workspace=ws, route=route)
        g2 = gdr.backward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], None, t["dO"], out_dtype=torch.float32,
                          dh=dh, clvr_scale=lam, want_dclvr_scale=True, route=route)
        torch.cuda.synchronize()
        for n in GRADS + ("dclvr_scale",):
            if g1[n] is not None:
                assert torch.equal(g1[n], g2[n]), (route, n)
    # the error route against the oracle
    _, _, E = oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], None, want_errors=True)
    dE, dlam = oracle.cler_backward(dh.float().cpu().numpy(), E, lam.cpu().numpy())
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], None, inp["dO"], dE=dE)
    errs = {n: rel(g1[n], ref[n]) for n in GRADS if ref[n] is not None}
    errs["dlam"] = rel(g1["dclvr_scale"], dlam)
    report(**errs)
    assert max(errs.values()) < 2e-3, errs


@pytest.mark.parametrize("route", ["value", "error"])
def test_cut_forward_chain_matches_oracle(route):
    """The forward state pass cut into ranges (state handed through the
    workspace) with the outputs of finished ranges on the second stream."""
    announce("cut forward chain route=%s" % route)
    inp = gdr_inputs.make(B=1, T=4000, H=2, d=128, gate="channel", dtype="bf16", seed=820, s0=True, clvr=True)
    r = np.random.default_rng(821)
    lam = r.standard_normal(256).astype(np.float32)
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("h", "lam")}, "bf16")
    h = to_dev(inp["h"], torch.bfloat16)
    o, ST = gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], out_dtype=torch.float32, h=h,
                        clvr_scale=to_dev(lam), route=route)
    torch.cuda.synchronize()
    o_ref, ST_ref, E = oracle.forward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["alpha"], inp["S0"],
                                      want_errors=True)
    h_ref = (oracle.cler_forward(inp["h"], E, lam) if route == "error"
             else oracle.clvr_forward(inp["h"], inp["v"], lam))
    errs = {"o": rel(o, o_ref), "S": rel(ST, ST_ref), "h": rel(h, h_ref)}
    report(**errs)
    assert errs["o"] < 2e-3 and errs["S"] < 2e-3 and errs["h"] < 2e-3 + 2.0 ** -8, errs


def test_training_pair_replays_from_a_hip_graph():
    """The cut passes fork work onto the library's second stream and join it
    back with events, which a graph capture on the caller's stream records as
    well.  The captured training pair is replayed three times, with eager work
    and synchronisations in between, and every replay must equal the eager
    results bit for bit."""
    announce("graph replay of the training pair")
    inp = gdr_inputs.make(B=1, T=4096, H=1, d=128, gate="channel", dtype="bf16", seed=830, bwd=True, clvr=True)
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("h", "lam")}, "bf16")
    lam = to_dev(inp["lam"])
    h0 = to_dev(inp["h"], torch.bfloat16)
    dh = to_dev(gdr_inputs.round_bf16(np.random.default_rng(831).standard_normal((1, 4096, 128))), torch.bfloat16)
    ws = torch.empty(gdr.workspace_size(1, 4096, 1, 128, gdr.GATE_CHANNEL, torch.bfloat16, torch.bfloat16,
                                        backward=True), dtype=torch.uint8, device="cuda")
    h = h0.clone()

    def pair():
        h.copy_(h0)
        o, ST = gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], None, h=h, clvr_scale=lam,
                            workspace=ws, save_for_backward=True)
        g = gdr.backward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], None, t["dO"], dh=dh, clvr_scale=lam,
                         want_dclvr_scale=True, saved_workspace=ws)
        return [o, ST, h] + [g[n] for n in ("dq", "dk", "dv", "dbeta", "dalpha", "dclvr_scale")]

    eager = [x.clone() for x in pair()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        pair()  # warm the caching allocator on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = pair()
    for rep in range(3):
        scratch = torch.randn(1 << 20, device="cuda") * 2  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), (rep, i)
        del scratch
