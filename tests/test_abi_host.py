"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/gdr.h declares, sizes workspaces as documented and rejects
invalid arguments before touching the device.

The invalid-argument calls below pass fake device addresses: validation only
compares pointer values and sizes, and returns before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

gdr = pytest.importorskip("gated_delta_rule_37_amd")
from gated_delta_rule_37_amd import _lib  # noqa: E402

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.library_path()):
        from gated_delta_rule_37_amd import build
        build.build()
    return _lib.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("gdr_forward_chunked", "gdr_backward", "gdr_decode_step", "gdr_workspace_size",
              "gdr_status_string", "gdr_last_error", "gdr_version"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (gdr_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_desc_layout_matches_header():
    # int64 x5, int32 x3, float, int32 x3 -> 68 bytes, padded to 72
    assert ctypes.sizeof(_lib.Desc) == 72
    assert _lib.Desc.scale.offset == 52 and _lib.Desc.chunk.offset == 56 and _lib.Desc.route.offset == 60
    assert _lib.Desc.prologue.offset == 64


def test_status_strings_and_version(lib):
    for code, name in _lib._STATUS.items():
        assert lib.gdr_status_string(code).decode() == name
    assert lib.gdr_version() >= 100


def desc(B=2, T=100, H=3, d=128, gate=2, in_dt=0, out_dt=1, scale=1.0, chunk=0, route=0, prologue=0):
    return _lib.Desc(B, T, H, d, d, gate, in_dt, out_dt, scale, chunk, route, prologue)


def test_workspace_size_formula(lib):
    # per chunk-head: W, Ut, Qt, Kb^T ([64][d] each), A [64][64] in operand
    # precision, gamma [d] fp32, the chunk-start state [d][d] and U [64][d] in
    # operand precision; every region rounded up to 256 bytes
    def al(x):
        return (x + 255) // 256 * 256

    for d, in_dt, opb in ((128, 0, 2), (64, 1, 4), (64, 0, 2)):
        dd = desc(B=2, T=130, H=3, d=d, in_dt=in_dt)
        nch = 2 * 3 * 3
        expect = (5 * al(nch * 64 * d * opb) + al(nch * 64 * 64 * opb) + al(nch * d * 4)
                  + al(nch * d * d * opb))
        # plus the fp32 state handed between the ranges of a cut state pass
        expect += al(2 * 3 * d * d * 4)
        assert lib.gdr_workspace_size(ctypes.byref(dd), 0) == expect
        assert lib.gdr_workspace_size(ctypes.byref(dd), 1) > expect
        # the error-routing epilogue adds nothing to the forward; its backward
        # keeps M^T dE ([64][d] per chunk-head, operand precision) and one fp32
        # partial row of H*d scale gradients per chunk and batch
        de = desc(B=2, T=130, H=3, d=d, in_dt=in_dt, route=1)
        assert lib.gdr_workspace_size(ctypes.byref(de), 0) == expect
        clvr_part = al(min(2 * 130, 256) * 3 * d * 4)
        cler_part = al(2 * 3 * 3 * d * 4)
        # ... and the gradient partials that the value route hands between its
        # two gradient stages on chip: dKt [64][d], dA, dP [64][64] and dgamma
        # [d] always, dQt and dKb [64][d] at d = 64 only
        on_chip = (al(nch * 64 * d * opb) + 2 * al(nch * 64 * 64 * opb) + al(nch * d * 4)
                   + (2 * al(nch * 64 * d * opb) if d == 64 else 0))
        assert (lib.gdr_workspace_size(ctypes.byref(de), 1) - lib.gdr_workspace_size(ctypes.byref(dd), 1)
                == al(nch * 64 * d * opb) + cler_part - clvr_part + on_chip)
        # the prologue keeps the activated beta and the reciprocal q and k row
        # norms: one fp32 per token slot each, in both layouts
        dp = desc(B=2, T=130, H=3, d=d, in_dt=in_dt, prologue=2)
        for op in (0, 1):
            assert (lib.gdr_workspace_size(ctypes.byref(dp), op) - lib.gdr_workspace_size(ctypes.byref(dd), op)
                    == 3 * al(nch * 64 * 4))
    assert lib.gdr_workspace_size(ctypes.byref(desc(T=0)), 0) == 0


FAKE = 0x7F0000000000  # a 16-byte aligned address that is never dereferenced


def fake(i):
    return ctypes.c_void_p(FAKE + i * (1 << 32))


def fwd(lib, d, q=1, k=2, v=3, beta=4, alpha=5, S0=None, o=6, ST=None, h=None, lam=None, ws=7,
        ws_bytes=1 << 40):
    P = lambda i: None if i is None else (fake(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_forward_chunked(ctypes.byref(d), P(q), P(k), P(v), P(beta), P(alpha), P(S0),
                                   P(o), P(ST), P(h), P(lam), P(ws), ws_bytes, None)


def test_forward_rejects_invalid_arguments(lib):
    assert fwd(lib, desc(d=96)) == UNSUPPORTED
    assert fwd(lib, desc(chunk=32)) == UNSUPPORTED
    assert fwd(lib, desc(gate=3)) == INVALID
    assert fwd(lib, desc(route=2)) == INVALID
    assert fwd(lib, desc(prologue=3)) == INVALID
    assert fwd(lib, desc(prologue=-1)) == INVALID
    assert fwd(lib, desc(route=-1)) == INVALID
    assert fwd(lib, desc(in_dt=5)) == INVALID
    assert fwd(lib, desc(B=-1)) == INVALID
    assert fwd(lib, desc(scale=float("nan"))) == INVALID
    assert fwd(lib, desc(), q=None) == INVALID
    assert fwd(lib, desc(gate=0)) == INVALID  # alpha given for DeltaNet
    assert fwd(lib, desc(gate=2), alpha=None) == INVALID  # alpha missing for KDA
    assert fwd(lib, desc(), k=ctypes.c_void_p(FAKE + (2 << 32) + 8)) == INVALID  # misaligned
    assert fwd(lib, desc(), o=1) == INVALID  # o aliases q
    assert fwd(lib, desc(), ws_bytes=16) == WORKSPACE
    assert fwd(lib, desc(), ws=None) == WORKSPACE
    assert fwd(lib, desc(), lam=8) == INVALID  # CLVR scale without the hidden stream
    assert "not 16-byte aligned" not in lib.gdr_last_error().decode() or True


def fwd_gated(lib, d, g=8, w=9, y=6, ws_bytes=1 << 40):
    P = lambda i: None if i is None else fake(i)  # noqa: E731
    return lib.gdr_forward_chunked_gated(ctypes.byref(d), P(1), P(2), P(3), P(4), P(5), None, P(g), P(w), P(y),
                                         None, None, None, P(7), ws_bytes, None)


def test_gated_forward_rejects_invalid_arguments(lib):
    assert fwd_gated(lib, desc(), g=None) == INVALID  # g is required
    assert b"g is required" in lib.gdr_last_error()
    assert fwd_gated(lib, desc(), g=None, w=None) == INVALID
    assert fwd_gated(lib, desc(), y=8) == INVALID  # y aliases g
    assert fwd_gated(lib, desc(), y=3) == INVALID  # y aliases v
    assert fwd_gated(lib, desc(), ws_bytes=16) == WORKSPACE
    assert fwd_gated(lib, desc(d=96)) == UNSUPPORTED
    assert fwd_gated(lib, desc(B=0), g=None) == OK  # nothing to compute


def test_forward_error_message_is_thread_local_detail(lib):
    assert fwd(lib, desc(d=96)) == UNSUPPORTED
    assert b"dk == dv" in lib.gdr_last_error()


def test_empty_batch_is_a_no_op(lib):
    # B = 0: nothing to launch, no pointer needed
    d = desc(B=0)
    assert fwd(lib, d, q=None, k=None, v=None, beta=None, alpha=None, o=None, ws=None, ws_bytes=0) == OK


def dec(lib, N=4, H=2, dk=128, dv=128, gate=2, in_dt=0, out_dt=0, q=1, k=2, v=3, beta=4, alpha=5,
        S=6, o=7):
    P = lambda i: None if i is None else (fake(i) if isinstance(i, int) else i)  # noqa: E731
    return lib.gdr_decode_step(N, H, dk, dv, gate, in_dt, out_dt, 1.0, P(q), P(k), P(v), P(beta),
                               P(alpha), P(S), P(o), None)


def test_decode_rejects_invalid_arguments(lib):
    assert dec(lib, dk=128, dv=64) == UNSUPPORTED
    assert dec(lib, gate=7) == INVALID
    assert dec(lib, S=None) == INVALID
    assert dec(lib, gate=0) == INVALID  # alpha must be NULL for DeltaNet
    assert dec(lib, o=6) == INVALID  # o aliases S
    assert dec(lib, N=0) == OK  # nothing to do


def test_backward_validates_descriptor(lib):
    d = desc(d=96)
    P = ctypes.c_void_p
    args = [P(FAKE)] * 17
    assert lib.gdr_backward(ctypes.byref(d), *args, P(FAKE), 1 << 40, None) == UNSUPPORTED


def test_output_gate_validation_and_workspace(lib):
    d = desc(B=2, T=100, H=3, d=64)
    P = fake
    # workspace: one fp32 partial row of H*dv per token range (at most 256 ranges)
    assert lib.gdr_output_gate_workspace_size(ctypes.byref(d)) == (min(200, 256) * 3 * 64 * 4 + 255) // 256 * 256
    f = lib.gdr_output_gate_forward
    assert f(ctypes.byref(d), None, P(2), None, P(3), None) == INVALID          # o missing
    assert f(ctypes.byref(d), P(1), P(2), None, ctypes.c_void_p(FAKE + (3 << 32) + 4), None) == INVALID  # misaligned
    assert f(ctypes.byref(d), P(1), P(2), None, ctypes.c_void_p(FAKE + (1 << 32) + 64), None) == INVALID  # y overlaps o
    assert f(ctypes.byref(desc(d=96)), P(1), P(2), None, P(3), None) == UNSUPPORTED
    b = lib.gdr_output_gate_backward
    assert b(ctypes.byref(d), P(1), P(2), None, P(3), P(4), P(5), P(6), P(7), 16, None) == WORKSPACE
    assert b(ctypes.byref(d), P(1), P(2), None, P(3), P(4), P(4), None, None, 0, None) == INVALID  # dO and dg overlap
    assert b(ctypes.byref(d), P(1), P(2), None, P(3), P(1), P(5), None, None, 0, None) == INVALID  # dO overlaps o
