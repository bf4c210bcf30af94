"""The byte and flop accounting bench.py reports its roofline fractions with.

Each figure is recomputed here from the tensors a kernel must touch (bf16
q, k, v, dO, dh and outputs, fp32 beta, alpha and their gradients, d = 128,
chunk 64), so a tensor counted twice or left out fails a test.  CPU only.
"""
import importlib.util
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


ROW16 = 128 * 2     # one bf16 row of d = 128
ROW32 = 128 * 4     # one fp32 alpha row (channel gate)
SCALAR = 4          # one fp32 beta (or d beta)


def test_forward_and_clvr_bytes(bench):
    # reads q, k, v, beta, alpha; CLVR reads and writes h
    assert bench.PER_TH_BYTES["intra_fwd"] == 3 * ROW16 + SCALAR + ROW32 + 2 * ROW16
    assert bench.PER_TH_BYTES["intra_train"] == bench.PER_TH_BYTES["intra_fwd"]
    assert bench.PER_TH_BYTES["output"] == ROW16  # o written
    assert bench.PER_TH_BYTES["state_fwd"] == 0  # intermediates only (S_T per head separately)


def test_gradient_kernel_counts_each_tensor_once(bench):
    # reads q, k, v, dO, dh, beta, alpha; writes dq, dk, dv, dbeta, dalpha
    reads = 5 * ROW16 + SCALAR + ROW32
    writes = 3 * ROW16 + SCALAR + ROW32
    assert bench.PER_TH_BYTES["grads"] == reads + writes == 3080
    assert bench.PER_TH_BYTES["grads_cler"] == bench.PER_TH_BYTES["grads"]


def test_step_bytes_are_forward_clvr_and_backward(bench):
    fwd = 3 * ROW16 + SCALAR + ROW32 + ROW16  # q, k, v, beta, alpha read; o written
    assert fwd == 1540
    assert bench.STEP_TH_BYTES == fwd + 2 * ROW16 + 3080


def test_per_launch_bytes_scale_with_token_heads(bench):
    B, T, H, d = 1, 32768, 16, 128
    b = bench.kernel_alg_bytes(B, T, H, d)
    th = B * T * H
    assert b["grads"] == 3080 * th
    # the state pass writes S_T once per (batch, head)
    assert b["state_fwd"] == B * H * d * d * 4
    # d = 64 halves every row
    assert bench.kernel_alg_bytes(B, T, H, 64)["grads"] == 3080 * th // 2


def test_forward_flops_per_token_head(bench):
    # five C x C x d products, three d x d products, the C x C solve (C = 64, d = 128)
    assert bench.fwd_flops_per_th(128) == pytest.approx(5 * 64 * 128 + 6 * 128 * 128 + 64 * 64 / 3)
    assert round(bench.fwd_flops_per_th(128)) == 140629


def test_stored_traffic_is_ignored_once_the_source_changes(bench, tmp_path, monkeypatch):
    digest = bench.kernel_source_digest("grads")
    f = tmp_path / "traffic.txt"
    f.write_text("# header\ntraffic grads %s 1000 24\ntraffic intra_fwd 0000000000000000 5 5\n" % digest)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic("grads") == 1024
    assert bench.measured_traffic("intra_fwd") is None  # digest of other sources
    assert bench.measured_traffic("output") is None     # no line stored
