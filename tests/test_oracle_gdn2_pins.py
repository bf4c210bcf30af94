"""Pins for the oracle's Gated DeltaNet-2 recurrence (CPU only).

The pages describe Gated DeltaNet-2 in words only (popular article on the
study, its Gated DeltaNet-2 paragraph): erasing and writing are decoupled and
steered by two gates computed independently from the token, the erase gate
choosing which regions of the memory to clear and the write gate which regions
to write; with the two gates equal the mechanism falls back to Kimi Delta
Attention and further to Gated DeltaNet.  The reading under test (gates are
key-channel vectors e_t, w_t):

    S_t = (I - (e_t * k_t) k_t^T) Diag(alpha_t) S_{t-1} + (w_t * k_t) v_t^T
    o_t = scale * S_t^T q_t

What pins it, with no second implementation of the chunked operator: the
reduction the page states (equal gates -> KDA), closed forms (no erase: gated
linear attention written as explicit sums; no erase and no write: pure decay;
unit keys with full gates: exact retrieval and exact erasure), channel
selectivity (a channel with a zero gate is neither erased nor written), and an
independent formulation by explicit dk x dk transition matrices.  Beyond the
reduction to KDA the reading itself is not fixed by the pages (parity
unpinned in that sense); these pins fix that the oracle computes the reading.
Planted mistakes (mutants) show each class of error fails a pin.
"""
import numpy as np
import pytest

import oracle


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def case(B=1, T=9, H=2, dk=6, dv=5, gate="channel", s0=True, seed=0):
    r = np.random.default_rng(seed)
    q = unit(r.standard_normal((B, T, H, dk)))
    k = unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    e = r.uniform(0.0, 1.0, (B, T, H, dk))
    w = r.uniform(0.0, 1.0, (B, T, H, dk))
    if gate == "none":
        a = None
    elif gate == "scalar":
        a = r.uniform(0.3, 1.0, (B, T, H))
    else:
        a = r.uniform(0.3, 1.0, (B, T, H, dk))
    S0 = 0.3 * r.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, e, w, a, S0


def avec(a, b, t, h, dk):
    if a is None:
        return np.ones(dk)
    if a.ndim == 3:
        return np.full(dk, a[b, t, h])
    return a[b, t, h]


def relerr(x, y):
    den = np.abs(y).max()
    return float(np.abs(x - y).max() / (den if den > 0 else 1.0))


# --------------------------------------------------------------------------
# mutants: NumPy recurrences with one plausible mistake each
# --------------------------------------------------------------------------
def mutant(kind):
    def fwd(q, k, v, e, w, a, S0, scale=1.0):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        o = np.zeros((B, T, H, dv))
        ST = np.zeros((B, H, dk, dv))
        for b in range(B):
            for h in range(H):
                S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
                for t in range(T):
                    al, kt, vt, et, wt = avec(a, b, t, h, dk), k[b, t, h], v[b, t, h], e[b, t, h], w[b, t, h]
                    if kind == "gates_swapped":
                        et, wt = wt, et
                    Sd = al[:, None] * S
                    if kind == "erase_gate_on_read_side":
                        p = Sd.T @ (et * kt)
                        S = Sd - np.outer(kt, p) + np.outer(wt * kt, vt)
                    elif kind == "write_not_decayed":
                        p = S.T @ kt
                        S = al[:, None] * (S - np.outer(et * kt, p)) + np.outer(wt * kt, vt)
                    elif kind == "prediction_before_decay":
                        p = S.T @ kt
                        S = Sd - np.outer(et * kt, p) + np.outer(wt * kt, vt)
                    else:  # the reading itself (used to check the harness)
                        p = Sd.T @ kt
                        S = Sd - np.outer(et * kt, p) + np.outer(wt * kt, vt)
                    o[b, t, h] = scale * (S.T @ q[b, t, h])
                ST[b, h] = S
        return o, ST
    return fwd


MUTANTS = ["gates_swapped", "erase_gate_on_read_side", "write_not_decayed", "prediction_before_decay"]


def oracle_fwd(q, k, v, e, w, a, S0, scale=1.0):
    return oracle.gdn2_forward(q, k, v, e, w, a, S0, scale=scale, nthreads=2)


# --------------------------------------------------------------------------
# pins (each a function of a forward implementation)
# --------------------------------------------------------------------------
def pin_equal_gates_is_kda(fwd):
    """e = w = beta (broadcast over channels) is the KDA step (the page: equal
    gates fall back to Kimi Delta Attention); uniform alpha then gives GDN."""
    q, k, v, e, w, a, S0 = case(seed=1)
    beta = np.random.default_rng(2).uniform(0.1, 1.0, q.shape[:3])
    g = np.repeat(beta[..., None], q.shape[-1], -1)
    o1, S1 = fwd(q, k, v, g, g, a, S0)
    o2, S2 = oracle.forward(q, k, v, beta, a, S0)
    return max(relerr(o1, o2), relerr(S1, S2)) < 1e-13


def pin_no_erase_is_gated_linear_attention(fwd):
    """e = 0: S_t = Diag(prod alpha) S0 + sum_i Diag(prod_{s=i+1..t} alpha_s)(w_i*k_i) v_i^T,
    written as explicit sums (no recurrence)."""
    q, k, v, e, w, a, S0 = case(seed=3)
    e = np.zeros_like(e)
    o, ST = fwd(q, k, v, e, w, a, S0)
    B, T, H, dk = q.shape
    ok = True
    for b in range(B):
        for h in range(H):
            for t in range(T):
                dec0 = np.prod([avec(a, b, s, h, dk) for s in range(t + 1)], axis=0)
                St = dec0[:, None] * S0[b, h]
                for i in range(t + 1):
                    dec = np.prod([avec(a, b, s, h, dk) for s in range(i + 1, t + 1)], axis=0) if i < t \
                        else np.ones(dk)
                    St = St + np.outer(dec * w[b, i, h] * k[b, i, h], v[b, i, h])
                ok &= relerr(o[b, t, h], St.T @ q[b, t, h]) < 1e-12
                if t == T - 1:
                    ok &= relerr(ST[b, h], St) < 1e-12
    return bool(ok)


def pin_pure_decay(fwd):
    q, k, v, e, w, a, S0 = case(seed=4)
    o, ST = fwd(q, k, v, np.zeros_like(e), np.zeros_like(w), a, S0)
    dec = np.prod(a, axis=1)  # [B, H, dk]
    return relerr(ST, dec[..., None] * S0) < 1e-13


def pin_full_gates_unit_keys_retrieve(fwd):
    """|k| = 1, e = w = 1, any alpha: S_t^T k_t = v_t, so q_t = k_t reads v_t."""
    q, k, v, e, w, a, S0 = case(seed=5)
    o, _ = fwd(k, k, v, np.ones_like(e), np.ones_like(w), a, S0)
    return relerr(o, v) < 1e-13


def pin_full_erase_clears_the_key_direction(fwd):
    """|k| = 1, e = 1, w = 0: the step projects the decayed state off k_t, so the
    read-out with q_t = k_t is exactly zero."""
    q, k, v, e, w, a, S0 = case(seed=6)
    o, _ = fwd(k, k, v, np.ones_like(e), np.zeros_like(w), a, S0)
    return np.abs(o).max() < 1e-13


def pin_channel_selectivity(fwd):
    """A key channel whose erase gate is 0 is not erased, and one whose write gate
    is 0 is not written: with e[c] = w[c] = 0 (other channels gated as drawn) the
    row c of S only decays."""
    q, k, v, e, w, a, S0 = case(T=7, seed=7)
    c = 2
    e[..., c] = 0.0
    w[..., c] = 0.0
    _, ST = fwd(q, k, v, e, w, a, S0)
    dec = np.prod(a, axis=1)  # [B, H, dk]
    return relerr(ST[:, :, c], dec[:, :, c, None] * S0[:, :, c]) < 1e-13


def unrolled(q, k, v, e, w, a, S0):
    """S_T = Phi_T S0 + sum_t Phi_{T<-t} (w_t*k_t) v_t^T with explicit dk x dk
    transitions A_s = (I - (e_s*k_s) k_s^T) Diag(alpha_s); o_t from S_t."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            A = [(np.eye(dk) - np.outer(e[b, s, h] * k[b, s, h], k[b, s, h])) @ np.diag(avec(a, b, s, h, dk))
                 for s in range(T)]
            for t in range(T):
                Phi = np.eye(dk)
                for s in range(t, -1, -1):
                    Phi = Phi @ A[s]
                St = Phi @ S0[b, h]
                for i in range(t + 1):
                    P = np.eye(dk)
                    for s in range(t, i, -1):
                        P = P @ A[s]
                    St = St + P @ np.outer(w[b, i, h] * k[b, i, h], v[b, i, h])
                o[b, t, h] = St.T @ q[b, t, h]
                if t == T - 1:
                    ST[b, h] = St
    return o, ST


def pin_unrolled(fwd):
    q, k, v, e, w, a, S0 = case(T=6, seed=9)
    o1, S1 = fwd(q, k, v, e, w, a, S0)
    o2, S2 = unrolled(q, k, v, e, w, a, S0)
    return max(relerr(o1, o2), relerr(S1, S2)) < 1e-12


PINS = {f.__name__: f for f in (pin_equal_gates_is_kda, pin_no_erase_is_gated_linear_attention, pin_pure_decay,
                                pin_full_gates_unit_keys_retrieve, pin_full_erase_clears_the_key_direction,
                                pin_channel_selectivity, pin_unrolled)}


@pytest.mark.parametrize("name", sorted(PINS))
def test_gdn2_oracle_pin(name):
    assert PINS[name](oracle_fwd)


@pytest.mark.parametrize("kind", MUTANTS)
def test_gdn2_pins_catch_mutant(kind):
    failed = [n for n, f in PINS.items() if not f(mutant(kind))]
    assert failed, "no pin catches the mutant %s" % kind


def test_gdn2_mutant_harness_is_faithful():
    """The NumPy harness without a planted mistake passes every pin."""
    assert all(f(mutant("none")) for f in PINS.values())


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_gdn2_decode_steps_equal_forward(gate):
    q, k, v, e, w, a, S0 = case(T=5, seed=10, gate=gate)
    o_ref, S_ref = oracle.gdn2_forward(q, k, v, e, w, a, S0)
    S = S0.copy()
    for t in range(q.shape[1]):
        at = None if a is None else a[:, t]
        ot, S = oracle.gdn2_decode(q[:, t], k[:, t], v[:, t], e[:, t], w[:, t], at, S)
        assert relerr(ot, o_ref[:, t]) < 1e-14
    assert relerr(S, S_ref) < 1e-14


def test_gdn2_scale_and_empty_sequence():
    q, k, v, e, w, a, S0 = case(seed=11)
    o1, _ = oracle.gdn2_forward(q, k, v, e, w, a, S0)
    o2, _ = oracle.gdn2_forward(q, k, v, e, w, a, S0, scale=0.25)
    assert relerr(o2, 0.25 * o1) < 1e-15
    z = lambda x: x[:, :0]  # noqa: E731
    _, ST = oracle.gdn2_forward(z(q), z(k), z(v), z(e), z(w), z(a), S0)
    assert np.array_equal(ST, S0)
