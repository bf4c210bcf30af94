"""Benchmark of the gated delta-rule hot path on one MI355X.

One step = one pass of the whole chunked path over the 32K-token Kimi Delta
Attention prefill (B=1, H=16, T=32768, dk=dv=128, bf16 inputs, fp32 state):
gate prep + intra-chunk transform + state pass + output + CLVR epilogue, then
the chunked backward (including the CLVR scale gradient).  Inputs are resident in
HBM before the timed region starts.  The decode step (256 sequences x 16 heads,
256 MiB fp32 state, rotating over independent state sets so the 256 MB
Infinity Cache cannot serve it) is timed in the same run and reported beside.

Prints ONE JSON line: metric, value (tokens/s), timing, config, plus `roofline`
(the dominant kernel's algorithmic GB/s against the 8 TB/s HBM peak, with its
measured traffic from the stored counter summary), `cpu_baseline` (the fp64
oracle on a bounded sample), and per-kernel, forward, decode, error-route,
prologue and output-gate figures.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, published
MFMA_F16_PEAK_TFS = 2500.0  # dense fp16/bf16 matrix peak, published
METRIC = "tokens/s of KDA/GDN chunked fwd(+bwd) at T=32K; % MFMA peak; decode % HBM BW"


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=10)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--decode-steps", type=int, default=30)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-backward", action="store_true")
    p.add_argument("--cpu-sample-tokens", type=int, default=2048)
    p.add_argument("--no-other-configs", action="store_true",
                   help="skip the GDN forward, KDA-with-S0, 350M-layer and sequence-length-sweep workloads")
    p.add_argument("--no-peaks", action="store_true", help="skip the measured copy and matrix peaks")
    p.add_argument("--no-gdn2", action="store_true", help="skip the Gated DeltaNet-2 forward and decode")
    p.add_argument("--copy-calibration", action="store_true",
                   help="end with three 1 GiB device copies (reference kernel for HBM counters)")
    return p.parse_args()


class KernelTimer:
    """Live per-kernel HIP event timing through gdr_profile_begin/end."""

    class Rec(ctypes.Structure):
        _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int64),
                    ("total_ms", ctypes.c_double)]

    def __init__(self, lib):
        self.lib = lib
        lib.gdr_profile_begin.restype = ctypes.c_int32
        lib.gdr_profile_end.restype = ctypes.c_int32
        lib.gdr_profile_end.argtypes = [ctypes.c_void_p, ctypes.c_int32]

    def begin(self):
        self.lib.gdr_profile_begin()

    def end(self):
        buf = (self.Rec * 32)()
        n = self.lib.gdr_profile_end(ctypes.cast(buf, ctypes.c_void_p), 32)
        if n < 0:
            raise RuntimeError("gdr_profile_end failed")
        return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(n)}


# Path tensors each kernel must touch at least once (bytes per token-head, KDA,
# bf16 q/k/v/dO/h and bf16 outputs, fp32 beta/alpha and their gradients).  Each
# distinct tensor counts once per launch, however many times the kernel reads
# it; a tensor read by two kernels counts for both; workspace intermediates
# never count.
BT16, F32, AK = 256, 4, 512        # a bf16 row of d = 128, one fp32 scalar, an fp32 alpha row
PER_TH_BYTES = {
    "intra_fwd": 3 * BT16 + F32 + AK + 2 * BT16,   # q,k,v,beta,alpha read; h read+write (CLVR)
    "intra_train": 3 * BT16 + F32 + AK + 2 * BT16,  # the same, training forward
    "state_fwd": 0,                                 # intermediates only (+ S_T)
    "state_train": 0,                               # intermediates only (+ S_T)
    "output": BT16,                                 # o written
    "intra_bwd": 3 * BT16 + F32 + AK,               # q,k,v,beta,alpha read
    "state_fwd_save": 0,                            # intermediates only
    "state_bwd": BT16,                              # dO read
    # both gradient stages in one launch: q,k,v,beta,alpha,dO,dh read; dq,dk,dv,dbeta,dalpha
    # written (the backward's 2824 B of the path tensors plus dh's 256)
    "grads": (5 * BT16 + F32 + AK) + (3 * BT16 + F32 + AK),
    "clvr_dlam": 2 * BT16,                          # dh, v read
    # error-routing epilogue (CLER-H) training step
    "output_cler": BT16 + 2 * BT16 + F32,           # o written; h read+write; beta read
    "cler_mt": BT16,                                # dh read
    "state_bwd_cler": 2 * BT16 + F32,               # dO, dh, beta read
    # the error route's gradient kernel touches the same tensors as "grads"
    "grads_cler": (5 * BT16 + F32 + AK) + (3 * BT16 + F32 + AK),
    # output-gate epilogue (bf16 o, g, y, dy, dO, dg)
    "gate_fwd": 3 * BT16,                           # o, g read; y written
    "gate_bwd": 5 * BT16,                           # o, g, dy read; dO, dg written
}
# The whole training step's compulsory bytes per token-head: the forward's
# q,k,v,beta,alpha reads and o write (1540) with CLVR's h read+write (512), and
# the backward's reads of q,k,v,beta,alpha,dO,dh and writes of dq,dk,dv,dbeta,
# dalpha (3080); plus S_T once per (b,h).
STEP_TH_BYTES = 1540 + 512 + 3080
# Per (b,h) state tensors (fp32 d x d): S_T written by the forward state pass.
PER_BH_STATE = {"state_fwd": 1, "state_train": 1}

# Kernel -> HIP sources whose text defines it (for matching stored counter runs).
KERNEL_SOURCES = {
    "intra_fwd": ["gdr_intra.hip"], "intra_bwd": ["gdr_intra.hip"], "intra_train": ["gdr_intra.hip"],
    "state_fwd": ["gdr_state.hip"], "state_fwd_save": ["gdr_state.hip"], "state_train": ["gdr_state.hip"],
    "output": ["gdr_output.hip", "gdr_gate.hpp", "gdr_gate_rows.hpp"], "output_cler": ["gdr_output.hip", "gdr_cler.hpp", "gdr_gate.hpp", "gdr_gate_rows.hpp"],
    "cler_mt": ["gdr_cler.hip", "gdr_cler.hpp"],
    "state_bwd_cler": ["gdr_bwd_state.hip"],
    "gate_fwd": ["gdr_gate.hip", "gdr_gate.hpp", "gdr_gate_rows.hpp"], "gate_bwd": ["gdr_gate.hip", "gdr_gate.hpp", "gdr_gate_rows.hpp"],
    "intra_train_pro": ["gdr_intra.hip"],
    "state_bwd": ["gdr_bwd_state.hip"],
    "clvr_dlam": ["gdr_bwd_grad.hip"],
    "grads": ["gdr_bwd_grad.hip"], "grads_pro": ["gdr_bwd_grad.hip"],
    "grads_cler": ["gdr_bwd_grad.hip", "gdr_cler.hpp"],
    "decode": ["gdr_decode.hip"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_kda_t32k.txt")


def kernel_alg_bytes(B, T, H, d):
    th = B * T * H
    out = {n: th * b * d // 128 for n, b in PER_TH_BYTES.items()}
    for n, k in PER_BH_STATE.items():
        out[n] += k * B * H * d * d * 4
    return out


def kernel_source_digest(name):
    import hashlib
    hsh = hashlib.sha256()
    csrc = os.path.join(ROOT, "gated_delta_rule_37_amd", "csrc")
    for f in KERNEL_SOURCES[name] + ["gdr_common.hpp", "gdr_launch.hpp"]:
        with open(os.path.join(csrc, f), "rb") as fh:
            hsh.update(fh.read())
    return hsh.hexdigest()[:16]


def measured_traffic(name):
    """HBM bytes per launch from the stored rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
    scaled by the same counters' reading for a copy of known size; None when no
    run is stored or the kernel's source has changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    digest = kernel_source_digest(name)
    with open(TRAFFIC_FILE) as fh:
        for line in fh:
            f = line.split()
            if len(f) >= 5 and f[0] == "traffic" and f[1] == name:
                return int(float(f[3]) + float(f[4])) if f[2] == digest else None
    return None


def cuda_time_ms(fn, steps, warmup=1):
    """Average milliseconds of fn() over `steps` calls between events on the
    current stream, after `warmup` untimed calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_call_ms(fn, n):
    """Milliseconds of each of n calls of fn(), each between its own pair of
    events on the current stream (the calls run back to back)."""
    import torch
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def host_cpu():
    """(cores available to this process, cores on the host, CPU model name)."""
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return avail, os.cpu_count() or avail, model


def fwd_flops_per_th(d, C=64):
    # five triangular C x C x d products, three d x d state products, the solve
    return 5 * C * d + 6 * d * d + C * C / 3


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (the operator shards over "
              "batch and heads with no communication between GPUs). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gated_delta_rule_37_amd as gdr
    import gdr_inputs

    dev = torch.device("cuda:0")
    lib = gdr.load_library()
    timer = KernelTimer(lib)
    bf = torch.bfloat16

    def to_dev(a, dt=torch.float32):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)

    # ---------------- chunked workload: KDA prefill at 32K tokens ----------------
    cfg = dict(gdr_inputs.CONFIGS["c5b"])
    B, T, H, d = cfg["B"], cfg["T"], cfg["H"], cfg["d"]
    log("generating inputs B=%d T=%d H=%d d=%d" % (B, T, H, d))
    inp = gdr_inputs.make(**dict(cfg, bwd=True, clvr=True))
    q, k, v, dO, h = (to_dev(inp[n], bf) for n in ("q", "k", "v", "dO", "h"))
    beta, alpha, lam = (to_dev(inp[n]) for n in ("beta", "alpha", "lam"))
    ws_f = torch.empty(gdr.workspace_size(B, T, H, d, gdr.GATE_CHANNEL, bf, bf), dtype=torch.uint8,
                       device=dev)
    do_bwd = not args.no_backward
    ws_b = None
    if do_bwd:
        nb = gdr.workspace_size(B, T, H, d, gdr.GATE_CHANNEL, bf, bf, backward=True)
        ws_b = torch.empty(nb, dtype=torch.uint8, device=dev)

    def step():
        # training step: the forward keeps its intermediates in ws_b, the
        # backward reads them instead of recomputing them
        if do_bwd:
            gdr.forward(q, k, v, beta, alpha, None, h=h, clvr_scale=lam, workspace=ws_b,
                        output_final_state=True, save_for_backward=True)
            gdr.backward(q, k, v, beta, alpha, None, dO, dh=h, clvr_scale=lam, want_dclvr_scale=True,
                         saved_workspace=ws_b)
        else:
            gdr.forward(q, k, v, beta, alpha, None, h=h, clvr_scale=lam, workspace=ws_f,
                        output_final_state=True)

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("timing %d steps" % args.steps)
    ms_step = cuda_time_ms(step, args.steps, warmup=0)
    tokens = B * T
    value = tokens / (ms_step / 1e3)

    # per-kernel durations, HIP events on the launch stream
    timer.begin()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = timer.end()
    kernels = {n: {"launches": c, "avg_us": 1e3 * ms / c} for n, (c, ms) in kt.items()}
    log("step %.3f ms; kernels %s" % (ms_step, json.dumps(kernels)))
    # the spread of single steps (each between its own events), beside the mean above
    per_step = per_call_ms(step, args.steps)

    # the inference forward alone (no intermediates kept), timed the same way
    def fwd():
        gdr.forward(q, k, v, beta, alpha, None, h=h, clvr_scale=lam, workspace=ws_f, output_final_state=True)

    fwd_us = 1e3 * cuda_time_ms(fwd, args.steps)
    per_fwd = per_call_ms(fwd, args.steps)
    timer.begin()
    for _ in range(args.steps):
        fwd()
    torch.cuda.synchronize()
    for n, (c, ms) in timer.end().items():
        kernels.setdefault(n, {"launches": c, "avg_us": 1e3 * ms / c})
    log("forward %.1f us" % fwd_us)

    th = B * T * H
    fwd_bytes = th * (1540 + 512)  # the whole forward: intra + state + output, CLVR's h read+write
    fwd_flops = th * fwd_flops_per_th(d)
    kbytes = kernel_alg_bytes(B, T, H, d)
    for n, kr in kernels.items():
        # a kernel may run as several launches per step (a state pass cut into
        # chunk ranges and the per-chunk kernels of each range): bytes per launch
        nb = kbytes.get(n)
        if nb:
            nb = nb * args.steps // kr["launches"]
        kr["alg_bytes"] = nb
        kr["alg_GBs"] = None if not nb else round(nb / (kr["avg_us"] * 1e-6) / 1e9, 1)
        kr["hbm_frac"] = None if not nb else round(nb / (kr["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    # dominant kernel: the largest share of the step's time
    dom = max(kt, key=lambda n: kernels[n]["avg_us"] * kernels[n]["launches"])
    achieved = kernels[dom]["alg_GBs"]
    roofline = {"kernel": dom, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom), "alg_bytes_per_launch": kernels[dom]["alg_bytes"],
                "avg_us": round(kernels[dom]["avg_us"], 2)}
    # the whole step against both roofs, in algorithmic bytes and flops
    step_bytes = th * (STEP_TH_BYTES if do_bwd else 1540 + 512) + B * H * d * d * 4
    step_flops = th * fwd_flops_per_th(d) * (3 if do_bwd else 1)
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    step_tfs = step_flops / (ms_step * 1e-3) / 1e12
    step_roof = {"alg_bytes": step_bytes, "alg_GBs": round(step_gbs, 1), "hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
                 "alg_flops": int(step_flops), "alg_TFLOPs": round(step_tfs, 2),
                 "mfma_frac": round(step_tfs / MFMA_F16_PEAK_TFS, 4),
                 "note": "algorithmic bytes (%d B per token-head + S_T) and flops (3 x %.0f per token-head) of the "
                         "training step over its measured time" % (STEP_TH_BYTES, fwd_flops_per_th(d))}
    log("step roofline %s" % json.dumps(step_roof))

    # ---------------- the same training step with the error-routing epilogue ----------------
    cler = None
    if do_bwd:
        nbc = gdr.workspace_size(B, T, H, d, gdr.GATE_CHANNEL, bf, bf, backward=True, route="error")
        del ws_b
        ws_c = torch.empty(nbc, dtype=torch.uint8, device=dev)

        def cler_step():
            gdr.forward(q, k, v, beta, alpha, None, h=h, clvr_scale=lam, workspace=ws_c, output_final_state=True,
                        save_for_backward=True, route="error")
            gdr.backward(q, k, v, beta, alpha, None, dO, dh=h, clvr_scale=lam, want_dclvr_scale=True,
                         saved_workspace=ws_c, route="error")

        cler_ms = cuda_time_ms(cler_step, args.steps, args.warmup)
        timer.begin()
        for _ in range(args.steps):
            cler_step()
        torch.cuda.synchronize()
        ck = {}
        for n, (c, ms) in timer.end().items():
            if n in ("output_cler", "cler_mt", "state_bwd_cler", "grads_cler"):
                us = 1e3 * ms / c
                gbs = kbytes[n] * args.steps / c / (us * 1e-6) / 1e9
                ck[n] = {"avg_us": round(us, 2), "alg_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        cler = {"workload": "the same step with route=error (CLER-H: h += lam * write error)",
                "ms_per_step": round(cler_ms, 4), "tokens_per_s": round(tokens / (cler_ms * 1e-3), 1),
                "kernels": ck}
        log("cler step %.3f ms; kernels %s" % (cler_ms, json.dumps(ck)))
        del ws_c

    # ---------------- the same training step with the fused prologue ----------------
    prologue = None
    if do_bwd:
        pinp = gdr_inputs.make(**dict(cfg, bwd=True, prologue="forget"))
        pq, pk = to_dev(pinp["q"], bf), to_dev(pinp["k"], bf)
        pb, pa = to_dev(pinp["beta"]), to_dev(pinp["alpha"])
        del pinp
        nbp = gdr.workspace_size(B, T, H, d, gdr.GATE_CHANNEL, bf, bf, backward=True, prologue="forget")
        ws_p = torch.empty(nbp, dtype=torch.uint8, device=dev)

        def pro_step():
            gdr.forward(pq, pk, v, pb, pa, None, h=h, clvr_scale=lam, workspace=ws_p, output_final_state=True,
                        save_for_backward=True, prologue="forget")
            gdr.backward(pq, pk, v, pb, pa, None, dO, dh=h, clvr_scale=lam, want_dclvr_scale=True,
                         saved_workspace=ws_p, prologue="forget")

        def separate_pass():
            # what the prologue replaces: a pass that normalises q, k and
            # activates the gates before the operator (torch ops, for comparison)
            qn = torch.nn.functional.normalize(pq.float(), dim=-1, eps=1e-6).to(bf)
            kn = torch.nn.functional.normalize(pk.float(), dim=-1, eps=1e-6).to(bf)
            return qn, kn, torch.sigmoid(pb), torch.sigmoid(-pa)

        pro_ms = cuda_time_ms(pro_step, args.steps, args.warmup)
        sep_ms = cuda_time_ms(separate_pass, args.steps, args.warmup)
        timer.begin()
        for _ in range(args.steps):
            pro_step()
        torch.cuda.synchronize()
        pk_t = {n: round(1e3 * ms / c, 2) for n, (c, ms) in timer.end().items()}
        prologue = {"workload": "the same step with prologue=forget: raw q, k and gate logits, normalised and "
                                "activated inside the kernels",
                    "ms_per_step": round(pro_ms, 4), "tokens_per_s": round(tokens / (pro_ms * 1e-3), 1),
                    "separate_pass_ms": round(sep_ms, 4), "kernels_avg_us": pk_t}
        log("prologue step %.3f ms (separate torch pass it replaces: %.3f ms); kernels %s" % (
            pro_ms, sep_ms, json.dumps(pk_t)))
        del ws_p, pq, pk, pb, pa

    # ---------------- output-gate epilogue on the step's output shape ----------------
    og = torch.randn((B, T, H, d), device=dev).to(bf)
    ow = torch.ones(H * d, device=dev)
    oo = torch.randn((B, T, H, d), device=dev).to(bf)
    ody = torch.randn((B, T, H, d), device=dev).to(bf)

    def gate_pass():
        gdr.output_gate(oo, og, ow)
        gdr.output_gate_backward(oo, og, ow, ody)

    for _ in range(args.warmup):
        gate_pass()
    torch.cuda.synchronize()
    timer.begin()
    for _ in range(args.steps):
        gate_pass()
    torch.cuda.synchronize()
    gk = {}
    for n, (c, ms) in timer.end().items():
        if n in ("gate_fwd", "gate_bwd"):
            us = 1e3 * ms / c
            gbs = kbytes[n] * args.steps / c / (us * 1e-6) / 1e9
            gk[n] = {"avg_us": round(us, 2), "alg_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    # the inference forward with the gate fused into its output kernel
    # (gdr_forward_chunked_gated), against the forward and then the gate launch
    yg = torch.empty((B, T, H, d), device=dev, dtype=bf)

    def fwd_gated():
        gdr.forward_gated(q, k, v, beta, alpha, og, ow, workspace=ws_f, output_final_state=True)

    def fwd_then_gate():
        o_, _ = gdr.forward(q, k, v, beta, alpha, None, workspace=ws_f, output_final_state=True)
        gdr.output_gate(o_, og, ow, out=yg)

    fused_ms = cuda_time_ms(fwd_gated, args.steps, args.warmup)
    sep_ms = cuda_time_ms(fwd_then_gate, args.steps, args.warmup)
    gk["forward_gated"] = {"us": round(1e3 * fused_ms, 2), "separate_us": round(1e3 * sep_ms, 2),
                           "tokens_per_s": round(tokens / (fused_ms * 1e-3), 1)}
    del yg
    output_gate = {"workload": "sigmoid(g) * RMSNorm(o) per head on [B=%d, T=%d, H=%d, dv=%d] bf16" % (B, T, H, d),
                   "kernels": gk}
    log("output gate %s" % json.dumps(gk))
    del og, oo, ody, q, k, v, dO, h, beta, alpha, ws_f

    # ---------------- the other workloads: one set of 262,144 token-heads per gate ----------------
    # GDN forward (B=4 H=16 T=4096), KDA forward with S0 (B=1 H=16 T=16384), the
    # 350M training layer (B=8 H=8 T=4096, KDA fwd+bwd+CLVR) and the sequence-length
    # sweep of the 350M layer (B*T = 32768, H = 8) all hold 262,144 token-heads:
    # one draw per gate kind, viewed in each shape (rows stay unit-norm and iid).
    others = {}
    if not args.no_other_configs:
        n_th, dd = 262144, 128
        sets = {}
        for gname, seed in (("channel", 4), ("scalar", 2)):
            gi = gdr_inputs.make(B=1, T=n_th // 8, H=8, d=dd, gate=gname, dtype="bf16", seed=seed, bwd=True)
            sets[gname] = {n: (to_dev(a, bf) if n in ("q", "k", "v", "dO") else to_dev(a))
                           for n, a in gi.items() if a is not None}
            del gi
        S0c3 = to_dev((0.02 * np.random.default_rng(3).standard_normal((1, 16, dd, dd))).astype(np.float32))

        def view(gname, Bv, Tv, Hv):
            src = sets[gname]
            out = {n: t.view(Bv, Tv, Hv, *t.shape[3:]) for n, t in src.items()}
            return out

        def run_fwd(x, S0=None):
            gdr.forward(x["q"], x["k"], x["v"], x["beta"], x.get("alpha"), S0, output_final_state=True)

        def fwd_entry(name, gname, Bv, Tv, Hv, S0=None, desc=""):
            x = view(gname, Bv, Tv, Hv)
            wsz = gdr.workspace_size(Bv, Tv, Hv, dd, gdr.GATE_CHANNEL if gname == "channel" else gdr.GATE_SCALAR,
                                     bf, bf)
            ws = torch.empty(wsz, dtype=torch.uint8, device=dev)

            def f():
                gdr.forward(x["q"], x["k"], x["v"], x["beta"], x["alpha"], S0, workspace=ws, output_final_state=True)

            us = 1e3 * cuda_time_ms(f, args.steps, args.warmup)
            nth = Bv * Tv * Hv
            nbytes = nth * (1540 if gname == "channel" else 1032) + Bv * Hv * dd * dd * 4 * (2 if S0 is not None else 1)
            gbs = nbytes / (us * 1e-6) / 1e9
            tfs = nth * fwd_flops_per_th(dd) / (us * 1e-6) / 1e12
            return {"workload": desc, "us": round(us, 2), "tokens_per_s": round(Bv * Tv / (us * 1e-6), 1),
                    "alg_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                    "alg_TFLOPs": round(tfs, 2), "mfma_frac": round(tfs / MFMA_F16_PEAK_TFS, 4)}

        def train_entry(gname, Bv, Tv, Hv, clvr, desc=""):
            x = view(gname, Bv, Tv, Hv)
            gate = gdr.GATE_CHANNEL if gname == "channel" else gdr.GATE_SCALAR
            ws = torch.empty(gdr.workspace_size(Bv, Tv, Hv, dd, gate, bf, bf, backward=True), dtype=torch.uint8,
                             device=dev)
            hh = torch.randn((Bv, Tv, Hv * dd), device=dev).to(bf) if clvr else None
            ll = torch.ones(Hv * dd, device=dev) if clvr else None

            def f():
                gdr.forward(x["q"], x["k"], x["v"], x["beta"], x["alpha"], None, h=hh, clvr_scale=ll, workspace=ws,
                            output_final_state=True, save_for_backward=True)
                gdr.backward(x["q"], x["k"], x["v"], x["beta"], x["alpha"], None, x["dO"], dh=hh, clvr_scale=ll,
                             want_dclvr_scale=clvr, saved_workspace=ws)

            ms = cuda_time_ms(f, args.steps, args.warmup)
            nth = Bv * Tv * Hv
            per = (1540 + 2824) if gname == "channel" else (1032 + 2824 - 2 * 508)
            if clvr:
                per += 512 + 256
            nbytes = nth * per + Bv * Hv * dd * dd * 4
            gbs = nbytes / (ms * 1e-3) / 1e9
            tfs = 3 * nth * fwd_flops_per_th(dd) / (ms * 1e-3) / 1e12
            return {"workload": desc, "ms_per_step": round(ms, 4), "tokens_per_s": round(Bv * Tv / (ms * 1e-3), 1),
                    "alg_GBs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                    "alg_TFLOPs": round(tfs, 2), "mfma_frac": round(tfs / MFMA_F16_PEAK_TFS, 4)}

        others["gdn_fwd_B4_H16_T4096"] = fwd_entry("c2", "scalar", 4, 4096, 16,
                                                   desc="Gated DeltaNet forward, B=4 H=16 T=4096 d=128 bf16")
        others["kda_fwd_s0_B1_H16_T16384"] = fwd_entry("c3", "channel", 1, 16384, 16, S0=S0c3,
                                                       desc="KDA forward with initial state, B=1 H=16 T=16384")
        if do_bwd:
            others["kda_train_350m_layer_B8_H8_T4096"] = train_entry(
                "channel", 8, 4096, 8, True, desc="KDA fwd+bwd+CLVR (h [8,4096,1024]), B=8 H=8 T=4096")
        sweep = []
        for gname in ("channel", "scalar"):
            for Tv in (4096, 16384, 32768):
                Bv = 32768 // Tv
                e = {"gate": "KDA" if gname == "channel" else "GDN", "B": Bv, "T": Tv, "H": 8}
                e["fwd_us"] = fwd_entry("", gname, Bv, Tv, 8)["us"]
                if do_bwd:
                    e["train_ms"] = train_entry(gname, Bv, Tv, 8, False)["ms_per_step"]
                sweep.append(e)
        for gname in ("KDA", "GDN"):
            pts = [e for e in sweep if e["gate"] == gname]
            key = "train_ms" if do_bwd else "fwd_us"
            growth = pts[-1][key] / pts[0][key] - 1.0
            for e in pts:
                e["growth_vs_T4096"] = round(e[key] / pts[0][key] - 1.0, 4)
            log("T-sweep %s: %s (4K -> 32K growth %+.1f %%)" % (gname, json.dumps(pts), 100 * growth))
        others["t_sweep_350m_layer"] = {"workload": "B*T = 32768 tokens, H=8, d=128, bf16; forward (fwd_us) and "
                                                    "training step (train_ms) per sequence length",
                                        "points": sweep}
        log("other workloads %s" % json.dumps({n: e for n, e in others.items() if n != "t_sweep_350m_layer"}))
        del sets

    # ---------------- Gated DeltaNet-2 (separate erase and write gates) ----------------
    gdn2 = None
    if not args.no_gdn2:
        g = gdr_inputs.make(**dict(cfg))  # the 32K-token KDA prefill inputs
        gq, gk, gv = (to_dev(g[n], bf) for n in ("q", "k", "v"))
        ga = to_dev(g["alpha"])
        del g
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        ge = torch.rand((B, T, H, d), generator=gen, device=dev)
        gw = torch.rand((B, T, H, d), generator=gen, device=dev)
        gws = torch.empty(gdr.gdn2_workspace_size(B, T, H, d, gdr.GATE_CHANNEL, bf, bf), dtype=torch.uint8, device=dev)

        def gdn2_fwd():
            gdr.gdn2_forward(gq, gk, gv, ge, gw, ga, None, workspace=gws)

        g_ms = cuda_time_ms(gdn2_fwd, args.steps, args.warmup)
        timer.begin()
        for _ in range(args.steps):
            gdn2_fwd()
        torch.cuda.synchronize()
        g_k = {n: {"avg_us": round(1e3 * ms / c, 2)} for n, (c, ms) in timer.end().items()}
        g_bytes = th * (3 * 256 + 2 * 512 + 512 + 256) + B * H * d * d * 4  # q,k,v, e,w, alpha, o; S_T
        g_flops = th * (9 * 64 * d + 8 * d * d)
        g_gbs = g_bytes / (g_ms * 1e-3) / 1e9
        g_tfs = g_flops / (g_ms * 1e-3) / 1e12
        del gq, gk, gv, ga, ge, gw, gws
        # decode step at the decode shape (256 sequences x 16 heads), rotating state sets
        dc2 = gdr_inputs.DECODE_CONFIG
        di = gdr_inputs.make_decode(N=dc2["N"], H=dc2["H"], d=dc2["d"], seed=dc2["seed"], nstates=3)
        xq, xk, xv = (to_dev(di[n], bf) for n in ("q", "k", "v"))
        xa = to_dev(di["alpha"])
        xst = [to_dev(sx) for sx in di["S"]]
        del di
        xe = torch.rand((dc2["N"], dc2["H"], dc2["d"]), generator=gen, device=dev)
        xw = torch.rand((dc2["N"], dc2["H"], dc2["d"]), generator=gen, device=dev)
        xo = torch.empty((dc2["N"], dc2["H"], dc2["d"]), dtype=bf, device=dev)
        rot2 = [0]

        def gdn2_dec():
            gdr.gdn2_decode_step(xq, xk, xv, xe, xw, xa, xst[rot2[0] % 3], out=xo)
            rot2[0] += 1

        gd_us = 1e3 * cuda_time_ms(gdn2_dec, args.decode_steps, 3)
        nsl = dc2["N"] * dc2["H"]
        gd_bytes = nsl * (2 * dc2["d"] * dc2["d"] * 4 + 3 * dc2["d"] * 2 + 3 * dc2["d"] * 4 + dc2["d"] * 2)
        del xq, xk, xv, xa, xst, xe, xw, xo
        gdn2 = {"workload": "Gated DeltaNet-2 forward (erase, write gates U(0,1) per channel; KDA gates), "
                            "B=%d H=%d T=%d d=%d bf16" % (B, H, T, d),
                "us": round(g_ms * 1e3, 2), "tokens_per_s": round(tokens / (g_ms * 1e-3), 1),
                "alg_GBs": round(g_gbs, 1), "hbm_frac": round(g_gbs / HBM_PEAK_GBS, 4),
                "alg_TFLOPs": round(g_tfs, 2), "mfma_frac": round(g_tfs / MFMA_F16_PEAK_TFS, 4),
                "kernels": g_k,
                "decode": {"workload": "one step, N=256 H=16 d=128, 3 rotating fp32 state sets",
                           "us_per_step": round(gd_us, 2),
                           "achieved_GBs": round(gd_bytes / (gd_us * 1e-6) / 1e9, 1),
                           "hbm_frac": round(gd_bytes / (gd_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}}
        log("gdn2 %s" % json.dumps(gdn2))

    # ---------------- decode: 256 sequences x 16 heads ----------------
    dc = gdr_inputs.DECODE_CONFIG
    nsets = 3
    dinp = gdr_inputs.make_decode(N=dc["N"], H=dc["H"], d=dc["d"], seed=dc["seed"], nstates=nsets)
    dq, dk_, dv_ = (to_dev(dinp[n], bf) for n in ("q", "k", "v"))
    db, da = to_dev(dinp["beta"]), to_dev(dinp["alpha"])
    states = [to_dev(s) for s in dinp["S"]]
    del dinp
    od = torch.empty((dc["N"], dc["H"], dc["d"]), dtype=bf, device=dev)
    rot = [0]

    def dec_rot():
        # rotating over independent state sets (768 MiB) so the Infinity Cache cannot serve it
        gdr.decode_step(dq, dk_, dv_, db, da, states[rot[0] % nsets], out=od)
        rot[0] += 1

    def dec_inplace():
        gdr.decode_step(dq, dk_, dv_, db, da, states[0], out=od)

    dec_us = 1e3 * cuda_time_ms(dec_rot, args.decode_steps, 3)
    dec_ip_us = 1e3 * cuda_time_ms(dec_inplace, args.decode_steps, 3)
    slabs = dc["N"] * dc["H"]
    dec_bytes = slabs * (2 * dc["d"] * dc["d"] * 4 + 3 * dc["d"] * 2 + dc["d"] * 4 + 4 + dc["d"] * 2)
    dec_gbs = dec_bytes / (dec_us * 1e-6) / 1e9
    decode = {"workload": "KDA decode step, N=256 H=16 d=128, fp32 state 256 MiB, %d rotating sets" % nsets,
              "us_per_step": round(dec_us, 2), "tokens_per_s": round(dc["N"] / (dec_us * 1e-6), 1),
              "achieved_GBs": round(dec_gbs, 1), "hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
              "in_place_us_per_step": round(dec_ip_us, 2),
              "in_place_GBs": round(dec_bytes / (dec_ip_us * 1e-6) / 1e9, 1),
              "in_place_note": "one state set updated in place: 256 MiB fits the 256 MB Infinity Cache in part, "
                               "so this rate is not a DRAM rate"}
    del states, dq, dk_, dv_, db, da, od

    # ---------------- measured peaks on this GPU ----------------
    peaks = {}
    if not args.no_peaks:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        cp_ms = cuda_time_ms(lambda: dst.copy_(src), 10, 2)
        peaks["copy_GBs"] = round(2 * src.numel() * 4 / (cp_ms * 1e-3) / 1e9, 1)
        del src, dst
        n = 8192
        a16 = torch.randn((n, n), device=dev, dtype=torch.float16)
        b16 = torch.randn((n, n), device=dev, dtype=torch.float16)
        mm_ms = cuda_time_ms(lambda: torch.mm(a16, b16), 10, 3)
        peaks["fp16_gemm_TFLOPs"] = round(2 * n ** 3 / (mm_ms * 1e-3) / 1e12, 1)
        peaks["note"] = ("copy: a 1 GiB device-to-device copy (read + write); matrix: an 8192^3 fp16 torch.mm "
                         "(hipBLASLt), as the attainable rates beside the published 8 TB/s and 2.5 PFLOP/s")
        del a16, b16
        log("measured peaks %s" % json.dumps(peaks))

    # ---------------- CPU baseline: the fp64 oracle on a bounded sample ----------------
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        ts = min(args.cpu_sample_tokens, T)
        avail, host_cores, model = host_cpu()
        threads = min(avail, B * H)
        sl = lambda a: np.ascontiguousarray(a[:, :ts])  # noqa: E731
        t0 = time.perf_counter()
        oracle.forward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]), sl(inp["alpha"]),
                       None, nthreads=threads)
        if do_bwd:
            oracle.backward(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["beta"]),
                            sl(inp["alpha"]), None, sl(inp["dO"]), nthreads=threads)
        cpu_s = time.perf_counter() - t0
        cpu = {"value": round(B * ts / cpu_s, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
               "sample": "first %d of %d tokens, all %d heads, %s, fp64 token-by-token, one thread per head" % (
                   ts, T, H, "forward+backward" if do_bwd else "forward"),
               "host_cores_available": avail, "host_cores": host_cores, "cpu_model": model}

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms_median": round(float(np.median(per_step)), 4),
        "step_ms_min": round(float(np.min(per_step)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-in/fp16-mfma/fp32-state",
        "data": "synthetic",
        "config": {"workload": "KDA chunked %s + CLVR, B=%d H=%d T=%d dk=dv=%d, chunk 64" % (
            "fwd+bwd" if do_bwd else "fwd", B, H, T, d), "global_batch": B, "seq_len": T,
            "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "step_roofline": step_roof,
        "cpu_baseline": cpu,
        "forward": {"us": round(fwd_us, 2), "us_median": round(1e3 * float(np.median(per_fwd)), 2),
                    "us_min": round(1e3 * float(np.min(per_fwd)), 2),
                    "tokens_per_s": round(tokens / (fwd_us * 1e-6), 1),
                    "alg_GBs": round(fwd_bytes / (fwd_us * 1e-6) / 1e9, 1),
                    "alg_TFLOPs": round(fwd_flops / (fwd_us * 1e-6) / 1e12, 2),
                    "hbm_frac": round(fwd_bytes / (fwd_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                    "mfma_frac": round(fwd_flops / (fwd_us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFS, 4)},
        "kernels": {n: {"avg_us": round(kr["avg_us"], 2), "launches_per_step": round(kr["launches"] / args.steps, 2),
                        "alg_GBs": kr["alg_GBs"], "hbm_frac": kr["hbm_frac"]}
                    for n, kr in kernels.items()},
        "decode": decode,
        "other_workloads": others,
        "measured_peaks": peaks,
        "cler": cler,
        "prologue": prologue,
        "output_gate": output_gate,
        "gdn2": gdn2,
    }
    print(json.dumps(out), flush=True)

    if args.copy_calibration:
        # A plain copy of known size: 1 GiB read + 1 GiB written per launch.
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy calibration: 3 x 1 GiB copies done")


if __name__ == "__main__":
    main()
