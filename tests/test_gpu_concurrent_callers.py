"""Two host threads on their own streams calling the library at once.

A cut state pass forks work onto the library's second and third streams and
joins it back with events; those streams and events are shared by every
caller on the device, and a mutex orders the enqueueing.  Each thread runs the
training pair (forward keeping its intermediates, then the saved backward)
several times on its own inputs, workspace and stream while the other does the
same, and every result must equal that of the same pair run alone, bit for bit.
"""
import threading

import pytest
import torch

import gated_delta_rule_37_amd as gdr
import gdr_inputs
from gpu_util import announce, inputs_to_dev, to_dev

pytestmark = pytest.mark.gpu

# 64 chunks per sequence and 16 state slices: the passes are cut into ranges
B, T, H, D = 1, 4096, 2, 128
REPS = 4


def make_case(seed):
    inp = gdr_inputs.make(B=B, T=T, H=H, d=D, gate="channel", dtype="bf16", seed=seed, s0=True, bwd=True,
                          clvr=True)
    t = inputs_to_dev({n: a for n, a in inp.items() if n not in ("h", "lam")}, "bf16")
    t["h0"] = to_dev(inp["h"], torch.bfloat16)
    t["lam"] = to_dev(inp["lam"])
    t["ws"] = torch.empty(gdr.workspace_size(B, T, H, D, gdr.GATE_CHANNEL, torch.bfloat16, torch.float32,
                                             backward=True), dtype=torch.uint8, device="cuda")
    return t


def pair(t):
    h = t["h0"].clone()
    o, ST = gdr.forward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], out_dtype=torch.float32, h=h,
                        clvr_scale=t["lam"], workspace=t["ws"], save_for_backward=True)
    g = gdr.backward(t["q"], t["k"], t["v"], t["beta"], t["alpha"], t["S0"], t["dO"], out_dtype=torch.float32,
                     dh=h, clvr_scale=t["lam"], want_dclvr_scale=True, saved_workspace=t["ws"])
    return [o, ST, h] + [g[n] for n in ("dq", "dk", "dv", "dbeta", "dalpha", "dS0", "dclvr_scale")]


def test_two_threads_share_the_library_streams():
    announce("two host threads, training pairs with cut passes at once")
    cases = [make_case(950), make_case(951)]
    alone = []
    for t in cases:
        alone.append([x.clone() for x in pair(t)])
        torch.cuda.synchronize()

    results = [[None] * REPS for _ in cases]
    errors = []
    start = threading.Barrier(len(cases))

    def worker(i):
        try:
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                start.wait(timeout=60)
                for r in range(REPS):
                    results[i][r] = [x.clone() for x in pair(cases[i])]
            stream.synchronize()
        except Exception as exc:  # reported by the main thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(i,), daemon=True) for i in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not any(th.is_alive() for th in threads), "a caller did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(len(cases)):
        for r in range(REPS):
            for j, (a, b) in enumerate(zip(results[i][r], alone[i])):
                assert torch.equal(a, b), (i, r, j)
