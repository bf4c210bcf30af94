"""Pins for the fp64 oracle: facts the pages and the mathematics fix, checked
without any second implementation of the operator.

The recurrence under test (KDA blog, section 2.1):
    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
    o_t = S_t^T q_t.

Each pin is written as a function of a forward implementation, so the same
checks also run against deliberately broken NumPy variants ("mutants") to show
that a plausible mistake -- decay after the write, read before the write,
S q instead of S^T q, the channel gate on the value axis, a dropped beta on the
erase term -- fails at least one pin.
"""
import json
import os

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
RNG = np.random.default_rng(1234)


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_case(B=1, T=10, H=2, dk=6, dv=5, gate="channel", s0=True, seed=0):
    r = np.random.default_rng(seed)
    q = unit(r.standard_normal((B, T, H, dk)))
    k = unit(r.standard_normal((B, T, H, dk)))
    v = r.standard_normal((B, T, H, dv))
    beta = 1 / (1 + np.exp(-r.standard_normal((B, T, H))))
    if gate == "none":
        alpha = None
    elif gate == "scalar":
        alpha = r.uniform(0.3, 1.0, (B, T, H))
    else:
        alpha = r.uniform(0.3, 1.0, (B, T, H, dk))
    S0 = 0.3 * r.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, beta, alpha, S0


def oracle_fwd(q, k, v, beta, alpha, S0, scale=1.0):
    return oracle.forward(q, k, v, beta, alpha, S0, scale=scale, nthreads=2)


def gate_vec(alpha, b, t, h, dk):
    if alpha is None:
        return np.ones(dk)
    if alpha.ndim == 3:
        return np.full(dk, alpha[b, t, h])
    return alpha[b, t, h]


# --------------------------------------------------------------------------
# mutants: small NumPy recurrences with one plausible mistake each
# --------------------------------------------------------------------------

def mutant_fwd(kind):
    def f(q, k, v, beta, alpha, S0, scale=1.0):
        B, T, H, dk = q.shape
        dv = v.shape[-1]
        o = np.zeros((B, T, H, dv))
        ST = np.zeros((B, H, dk, dv))
        for b in range(B):
            for h in range(H):
                S = np.zeros((dk, dv)) if S0 is None else S0[b, h].copy()
                for t in range(T):
                    a = gate_vec(alpha, b, t, h, dk)
                    kt, vt, bt, qt = k[b, t, h], v[b, t, h], beta[b, t, h], q[b, t, h]
                    if kind == "gate_on_value_axis":
                        ag = np.resize(a, dv)
                        Sd = S * ag[None, :]
                    elif kind == "decay_after_write":
                        Sd = S
                    else:
                        Sd = a[:, None] * S
                    if kind == "no_beta_on_erase":
                        Sn = Sd - np.outer(kt, Sd.T @ kt) + bt * np.outer(kt, vt)
                    else:
                        Sn = Sd + np.outer(kt, bt * (vt - Sd.T @ kt))
                    if kind == "decay_after_write":
                        Sn = a[:, None] * Sn
                    if kind == "read_before_write":
                        o[b, t, h] = scale * (S.T @ qt)
                    elif kind == "S_q_not_St_q" and dk == dv:
                        o[b, t, h] = scale * (Sn @ qt)
                    else:
                        o[b, t, h] = scale * (Sn.T @ qt)
                    S = Sn
                ST[b, h] = S
        return o, ST
    return f


MUTANTS = ["decay_after_write", "read_before_write", "S_q_not_St_q", "gate_on_value_axis",
           "no_beta_on_erase"]

# --------------------------------------------------------------------------
# pins, each returning the max abs error against what the pages fix
# --------------------------------------------------------------------------


def pin_exact_retrieval(fwd):
    """P1: unit k, beta = 1, any alpha and any S0: S_t^T k_t = v_t, so
    reading with q_t = k_t returns v_t (KDA blog 2.1; the DeltaNet section of the
    popular article: the delta rule stores exactly the value it writes)."""
    err = 0.0
    for gate in ("none", "scalar", "channel"):
        q, k, v, beta, alpha, S0 = rand_case(T=12, dk=6, dv=6, gate=gate, seed=11)
        beta = np.ones_like(beta)
        o, _ = fwd(k, k, v, beta, alpha, S0)
        err = max(err, np.abs(o - v).max())
    return err


def pin_zero_difference(fwd):
    """P2: writing (k, v) again with beta = 1, alpha = 1 and unit k leaves the
    state unchanged (the article: the delta rule records a zero difference when
    the memory already knows the pair)."""
    q, k, v, beta, alpha, S0 = rand_case(T=6, dk=5, dv=4, gate="none", seed=12)
    k[:, 5] = k[:, 4]
    v[:, 5] = v[:, 4]
    beta = np.ones_like(beta)
    _, S5 = fwd(q[:, :5], k[:, :5], v[:, :5], beta[:, :5], None, S0)
    _, S6 = fwd(q, k, v, beta, None, S0)
    return np.abs(S6 - S5).max()


def pin_pure_decay(fwd):
    """P5: beta = 0 means no writes, S_t = Diag(prod_{s<=t} alpha_s) S0 and
    o_t = S_t^T q_t; with alpha = 1 too, o = S0^T q (a library matmul)."""
    q, k, v, beta, alpha, S0 = rand_case(T=9, dk=5, dv=7, gate="channel", seed=13)
    beta = np.zeros_like(beta)
    o, ST = fwd(q, k, v, beta, alpha, S0)
    cum = np.cumprod(alpha, axis=1)  # [B,T,H,dk]
    o_ref = np.einsum("bthi,bhij->bthj", q * cum, S0)
    ST_ref = cum[:, -1][..., None] * S0
    o1, _ = fwd(q, k, v, beta, None, S0)
    o1_ref = np.einsum("bthi,bhij->bthj", q, S0)
    return max(np.abs(o - o_ref).max(), np.abs(ST - ST_ref).max(), np.abs(o1 - o1_ref).max())


def pin_one_hot_keys(fwd):
    """P6: distinct one-hot keys e_pi(t), S0 = 0, T <= dk:
    o_t = sum_{i<=t} beta_i (prod_{s=i+1..t} alpha_s[pi(i)]) q_t[pi(i)] v_i.
    This fixes which channel of alpha decays which row of S."""
    B, T, H, dk, dv = 1, 7, 2, 8, 3
    r = np.random.default_rng(14)
    q = r.standard_normal((B, T, H, dk))
    v = r.standard_normal((B, T, H, dv))
    beta = r.uniform(0.2, 1.5, (B, T, H))
    alpha = r.uniform(0.2, 1.0, (B, T, H, dk))
    k = np.zeros((B, T, H, dk))
    perm = [r.permutation(dk)[:T] for _ in range(H)]
    for h in range(H):
        for t in range(T):
            k[0, t, h, perm[h][t]] = 1.0
    o, _ = fwd(q, k, v, beta, alpha, None)
    o_ref = np.zeros_like(o)
    for h in range(H):
        for t in range(T):
            for i in range(t + 1):
                c = perm[h][i]
                dec = np.prod(alpha[0, i + 1:t + 1, h, c])
                o_ref[0, t, h] += beta[0, i, h] * dec * q[0, t, h, c] * v[0, i, h]
    return np.abs(o - o_ref).max()


def pin_linear_attention(fwd):
    """P6b: alpha = 1, orthonormal keys, S0 = 0 reduce the rule to causal linear
    attention, o = tril(Q K^T) diag(beta) V (KDA blog, section 1)."""
    B, T, H, d = 1, 6, 1, 8
    r = np.random.default_rng(15)
    Qm, _ = np.linalg.qr(r.standard_normal((d, d)))
    k = Qm[:T][None, :, None, :]
    q = r.standard_normal((B, T, H, d))
    v = r.standard_normal((B, T, H, d))
    beta = r.uniform(0.1, 1.0, (B, T, H))
    o, _ = fwd(q, k, v, beta, None, None)
    att = np.tril(q[0, :, 0] @ k[0, :, 0].T) * beta[0, :, 0][None, :]
    return np.abs(o[0, :, 0] - att @ v[0, :, 0]).max()


def unrolled(q, k, v, beta, alpha, S0):
    """P7: the same recurrence written as explicit dk x dk transition matrices
    M_t = (I - beta_t k_t k_t^T) Diag(alpha_t), S_t = M_t S_{t-1} + beta_t k_t v_t^T,
    expanded into S_t = Phi_t S0 + sum_i Phi_{t<-i} beta_i k_i v_i^T."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            M = [(np.eye(dk) - beta[b, t, h] * np.outer(k[b, t, h], k[b, t, h]))
                 @ np.diag(gate_vec(alpha, b, t, h, dk)) for t in range(T)]
            s0 = np.zeros((dk, dv)) if S0 is None else S0[b, h]
            for t in range(T):
                Phi = np.eye(dk)
                for s in range(t, -1, -1):
                    Phi = Phi @ M[s]
                St = Phi @ s0
                for i in range(t + 1):
                    P = np.eye(dk)
                    for s in range(t, i, -1):
                        P = P @ M[s]
                    St = St + P @ (beta[b, i, h] * np.outer(k[b, i, h], v[b, i, h]))
                o[b, t, h] = St.T @ q[b, t, h]
                if t == T - 1:
                    ST[b, h] = St
    return o, ST


def pin_unrolled(fwd):
    err = 0.0
    for gate in ("none", "scalar", "channel"):
        case = rand_case(B=2, T=8, H=2, dk=5, dv=4, gate=gate, seed=16)
        o, ST = fwd(*case)
        o_ref, ST_ref = unrolled(*case)
        err = max(err, np.abs(o - o_ref).max(), np.abs(ST - ST_ref).max())
    return err


PINS = {
    "exact_retrieval": pin_exact_retrieval,
    "zero_difference": pin_zero_difference,
    "pure_decay": pin_pure_decay,
    "one_hot_keys": pin_one_hot_keys,
    "linear_attention": pin_linear_attention,
    "unrolled": pin_unrolled,
}


@pytest.mark.parametrize("name", sorted(PINS))
def test_oracle_pin(name):
    assert PINS[name](oracle_fwd) < 1e-12


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_mutant(kind):
    """Every mutant must fail at least one pin by a wide margin."""
    errs = {n: p(mutant_fwd(kind)) for n, p in PINS.items()}
    assert max(errs.values()) > 1e-3, errs


def test_mutant_harness_is_faithful():
    """The unmutated NumPy recurrence passes every pin (so a failing mutant fails
    because of its mistake, not because of the harness)."""
    for n, p in PINS.items():
        assert p(mutant_fwd("none")) < 1e-12, n


def test_hand_worked_examples():
    with open(os.path.join(HERE, "golden", "hand_worked_examples.json")) as f:
        data = json.load(f)
    for ex in data["examples"]:
        T, dk, dv = len(ex["q"]), ex["dk"], ex["dv"]
        q = np.array(ex["q"], float).reshape(1, T, 1, dk)
        k = np.array(ex["k"], float).reshape(1, T, 1, dk)
        v = np.array(ex["v"], float).reshape(1, T, 1, dv)
        beta = np.array(ex["beta"], float).reshape(1, T, 1)
        alpha = None if ex["alpha"] is None else np.array(ex["alpha"], float).reshape(1, T, 1, dk)
        o, ST = oracle_fwd(q, k, v, beta, alpha, None)
        assert np.abs(o.reshape(T, dv) - np.array(ex["o"], float)).max() < 1e-12, ex["name"]
        assert np.abs(ST.reshape(dk, dv) - np.array(ex["ST"], float)).max() < 1e-12, ex["name"]


def test_channel_gate_reduces_to_scalar_gate_bit_exact():
    """P3: alpha_t[:] = a_t makes Kimi Delta Attention identical to Gated
    DeltaNet (the article's chain of reductions)."""
    q, k, v, beta, alpha, S0 = rand_case(T=11, dk=6, dv=5, gate="scalar", seed=17)
    alpha_c = np.repeat(alpha[..., None], 6, axis=-1)
    o1, S1 = oracle_fwd(q, k, v, beta, alpha, S0)
    o2, S2 = oracle_fwd(q, k, v, beta, alpha_c, S0)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)
    dO = RNG.standard_normal(o1.shape)
    g1 = oracle.backward(q, k, v, beta, alpha, S0, dO)
    g2 = oracle.backward(q, k, v, beta, alpha_c, S0, dO)
    for n in ("dq", "dk", "dv", "dbeta", "dS0"):
        assert np.array_equal(g1[n], g2[n]), n
    assert np.abs(g1["dalpha"] - g2["dalpha"].sum(-1)).max() < 1e-12


def test_scalar_gate_of_one_is_deltanet_bit_exact():
    """P4: alpha = 1 makes Gated DeltaNet identical to DeltaNet."""
    q, k, v, beta, alpha, S0 = rand_case(T=11, dk=6, dv=5, gate="scalar", seed=18)
    o1, S1 = oracle_fwd(q, k, v, beta, np.ones_like(alpha), S0)
    o2, S2 = oracle_fwd(q, k, v, beta, None, S0)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_scale_is_linear_in_output():
    case = rand_case(T=7, gate="channel", seed=19)
    o1, S1 = oracle_fwd(*case, scale=1.0)
    o2, S2 = oracle_fwd(*case, scale=0.125)
    assert np.abs(o2 - 0.125 * o1).max() < 1e-14 and np.array_equal(S1, S2)


def test_threads_do_not_change_results():
    case = rand_case(B=3, T=9, H=3, gate="channel", seed=20)
    a = oracle.forward(*case, nthreads=1)
    b = oracle.forward(*case, nthreads=5)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_empty_sequence_passes_state_through():
    q, k, v, beta, alpha, S0 = rand_case(T=0, gate="channel", seed=21)
    o, ST = oracle_fwd(q, k, v, beta, alpha, S0)
    assert o.shape[1] == 0 and np.array_equal(ST, S0)


# --------------------------------------------------------------------------
# backward: finite differences and closed forms
# --------------------------------------------------------------------------


def _loss(case, dO, dST, scale=1.0):
    o, ST = oracle_fwd(*case, scale=scale)
    return float((o * dO).sum() + (ST * dST).sum())


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_backward_matches_central_differences(gate):
    """P8: the adjoint agrees with central differences of the forward."""
    case = list(rand_case(B=1, T=5, H=2, dk=4, dv=3, gate=gate, seed=22))
    r = np.random.default_rng(23)
    dO = r.standard_normal((1, 5, 2, 3))
    dST = r.standard_normal((1, 2, 4, 3))
    g = oracle.backward(*case, dO, dST, scale=0.7)
    names = ["dq", "dk", "dv", "dbeta", "dalpha", "dS0"]
    eps = 1e-6
    for idx, name in enumerate(names):
        x = case[idx]
        if x is None:
            assert g[name] is None
            continue
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            old = x[mi]
            x[mi] = old + eps
            lp = _loss(case, dO, dST, 0.7)
            x[mi] = old - eps
            lm = _loss(case, dO, dST, 0.7)
            x[mi] = old
            num[mi] = (lp - lm) / (2 * eps)
        err = np.abs(num - g[name]).max() / max(1.0, np.abs(num).max())
        assert err < 1e-7, (name, err)


def test_backward_closed_form_under_pure_decay():
    """P8b: with beta = 0 and alpha = 1 the map is o = scale S0^T q, so
    dq_t = scale S0 do_t and dS0 = scale sum_t q_t do_t^T."""
    q, k, v, beta, alpha, S0 = rand_case(B=2, T=6, H=2, dk=5, dv=4, gate="none", seed=24)
    beta = np.zeros_like(beta)
    dO = np.random.default_rng(25).standard_normal((2, 6, 2, 4))
    g = oracle.backward(q, k, v, beta, None, S0, dO, scale=0.5)
    dq_ref = 0.5 * np.einsum("bhij,bthj->bthi", S0, dO)
    dS0_ref = 0.5 * np.einsum("bthi,bthj->bhij", q, dO)
    assert np.abs(g["dq"] - dq_ref).max() < 1e-13
    assert np.abs(g["dS0"] - dS0_ref).max() < 1e-13
    assert np.abs(g["dv"]).max() == 0.0


def test_backward_with_long_sequence_checkpoints():
    """T larger than the checkpoint stride: the recompute between checkpoints
    reproduces the states exactly, so results equal a T where stride = 1."""
    case = rand_case(B=1, T=30, H=1, dk=4, dv=4, gate="channel", seed=26)
    dO = np.random.default_rng(27).standard_normal((1, 30, 1, 4))
    g = oracle.backward(*case, dO)
    # compare against a direct linearisation through finite differences of S0
    eps = 1e-6
    S0 = case[5]
    num = np.zeros_like(S0)
    for idx in np.ndindex(S0.shape):
        old = S0[idx]
        S0[idx] = old + eps
        lp = _loss(case, dO, np.zeros((1, 1, 4, 4)))
        S0[idx] = old - eps
        lm = _loss(case, dO, np.zeros((1, 1, 4, 4)))
        S0[idx] = old
        num[idx] = (lp - lm) / (2 * eps)
    assert np.abs(num - g["dS0"]).max() < 1e-7


# --------------------------------------------------------------------------
# decode and CLVR
# --------------------------------------------------------------------------


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_decode_is_one_transition_matrix_step(gate):
    """One decode step equals S_new = (I - beta k k^T) Diag(alpha) S + beta k v^T,
    o = S_new^T q, written with explicit matrices."""
    r = np.random.default_rng(28)
    N, H, dk, dv = 3, 2, 6, 5
    q = unit(r.standard_normal((N, H, dk)))
    k = unit(r.standard_normal((N, H, dk)))
    v = r.standard_normal((N, H, dv))
    beta = r.uniform(0, 1, (N, H))
    alpha = None if gate == "none" else (r.uniform(0.2, 1, (N, H)) if gate == "scalar"
                                         else r.uniform(0.2, 1, (N, H, dk)))
    S = r.standard_normal((N, H, dk, dv))
    o, Sn = oracle.decode(q, k, v, beta, alpha, S, scale=0.9)
    for n in range(N):
        for h in range(H):
            a = np.ones(dk) if alpha is None else (np.full(dk, alpha[n, h]) if alpha.ndim == 2
                                                    else alpha[n, h])
            M = (np.eye(dk) - beta[n, h] * np.outer(k[n, h], k[n, h])) @ np.diag(a)
            ref = M @ S[n, h] + beta[n, h] * np.outer(k[n, h], v[n, h])
            assert np.abs(Sn[n, h] - ref).max() < 1e-13
            assert np.abs(o[n, h] - 0.9 * ref.T @ q[n, h]).max() < 1e-13


def test_decode_steps_equal_forward():
    case = rand_case(B=2, T=5, H=2, dk=4, dv=3, gate="channel", seed=29)
    q, k, v, beta, alpha, S0 = case
    o, ST = oracle_fwd(*case)
    S = S0.copy()
    for t in range(5):
        ot, S = oracle.decode(q[:, t], k[:, t], v[:, t], beta[:, t], alpha[:, t], S)
        assert np.abs(ot - o[:, t]).max() < 1e-13
    assert np.abs(S - ST).max() < 1e-13


def test_clvr_zero_init_is_a_no_op_and_unit_scale_adds_v():
    """CLVR's routing projection starts at zero, so at initialisation the layer
    equals the one without routing (article, cross-layer section)."""
    r = np.random.default_rng(30)
    B, T, H, dv = 2, 3, 2, 4
    v = r.standard_normal((B, T, H, dv))
    h = r.standard_normal((B, T, H * dv))
    assert np.array_equal(oracle.clvr_forward(h, v, np.zeros(H * dv)), h)
    assert np.array_equal(oracle.clvr_forward(h, v, None), h + v.reshape(B, T, H * dv))
    lam = r.standard_normal(H * dv)
    out = oracle.clvr_forward(h, v, lam)
    assert np.abs(out - (h + lam * v.reshape(B, T, H * dv))).max() < 1e-15
    dh = r.standard_normal(h.shape)
    dv_acc, dlam = oracle.clvr_backward(dh, v, lam)
    assert np.abs(dv_acc.reshape(B, T, H * dv) - lam * dh).max() < 1e-15
    assert np.abs(dlam - (dh * v.reshape(B, T, H * dv)).sum((0, 1))).max() < 1e-13


# --------------------------------------------------------------------------
# write errors (the quantity the CLER-H epilogue routes into the hidden stream)
# --------------------------------------------------------------------------


def _errors_from_states(case):
    """Recovers every write error from consecutive states of the (pinned)
    forward on prefixes: the update is S_t = D_t S_{t-1} + beta_t k_t e_t^T, so
    k_t^T (S_t - D_t S_{t-1}) = beta_t |k_t|^2 e_t^T."""
    q, k, v, beta, alpha, S0 = case
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    E = np.zeros((B, T, H, dv))
    prev = np.zeros((B, H, dk, dv)) if S0 is None else S0
    for t in range(T):
        sl = lambda x: None if x is None else x[:, :t + 1]
        _, St = oracle_fwd(sl(q), sl(k), sl(v), sl(beta), sl(alpha), S0)
        for b in range(B):
            for h in range(H):
                D = np.diag(gate_vec(alpha, b, t, h, dk))
                kk = k[b, t, h]
                E[b, t, h] = kk @ (St[b, h] - D @ prev[b, h]) / (beta[b, t, h] * (kk @ kk))
        prev = St
    return E


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_write_errors_match_state_increments(gate):
    case = rand_case(B=2, T=7, H=2, dk=5, dv=4, gate=gate, seed=40)
    o, ST, E = oracle.forward(*case, want_errors=True, nthreads=2)
    o2, ST2 = oracle_fwd(*case)
    assert np.array_equal(o, o2) and np.array_equal(ST, ST2)
    assert np.abs(E - _errors_from_states(case)).max() < 1e-12


def test_write_error_pin_catches_undecayed_read():
    """A mistake that reads the error against S_{t-1} instead of the decayed
    D_t S_{t-1} fails the increment pin."""
    case = rand_case(B=1, T=5, H=1, dk=4, dv=3, gate="channel", seed=41)
    q, k, v, beta, alpha, S0 = case
    E_ref = _errors_from_states(case)
    S = S0[0, 0].copy()
    bad = np.zeros_like(E_ref)
    for t in range(5):
        kk, a = k[0, t, 0], alpha[0, t, 0]
        bad[0, t, 0] = v[0, t, 0] - S.T @ kk
        Sd = np.diag(a) @ S
        S = Sd + beta[0, t, 0] * np.outer(kk, v[0, t, 0] - Sd.T @ kk)
    assert np.abs(bad - E_ref).max() > 1e-3


def test_write_error_special_cases():
    """From zero state the first error is the value itself; writing the same
    unit-norm pair again with beta = 1 and no decay leaves no error; after a
    write the residual at k_t shrinks to (1 - beta_t |k_t|^2) e_t."""
    q, k, v, beta, alpha, S0 = rand_case(B=1, T=6, H=2, dk=5, dv=4, gate="scalar", s0=False, seed=42)
    _, _, E = oracle.forward(q, k, v, beta, alpha, None, want_errors=True)
    assert np.array_equal(E[:, 0], v[:, 0])
    k2, v2, b2, a2 = k.copy(), v.copy(), beta.copy(), alpha.copy()
    k2[:, 3], v2[:, 3] = k2[:, 2], v2[:, 2]
    b2[:, 2:4], a2[:, 3] = 1.0, 1.0
    _, _, E2 = oracle.forward(q, k2, v2, b2, a2, None, want_errors=True)
    assert np.abs(E2[:, 3]).max() < 1e-14
    case = rand_case(B=1, T=6, H=2, dk=5, dv=4, gate="channel", seed=43)
    q, k, v, beta, alpha, S0 = case
    _, _, E = oracle.forward(*case, want_errors=True)
    for t in range(6):
        sl = lambda x: x[:, :t + 1]
        _, St = oracle_fwd(sl(q), sl(k), sl(v), sl(beta), sl(alpha), S0)
        for h in range(2):
            kk = k[0, t, h]
            resid = v[0, t, h] - St[0, h].T @ kk
            assert np.abs(resid - (1 - beta[0, t, h] * (kk @ kk)) * E[0, t, h]).max() < 1e-13


def _loss_e(case, dO, dST, dE, scale):
    o, ST, E = oracle.forward(*case, scale=scale, want_errors=True, nthreads=2)
    return float((o * dO).sum() + (ST * dST).sum() + (E * dE).sum())


@pytest.mark.parametrize("gate", ["none", "channel"])
def test_backward_with_error_gradient_matches_central_differences(gate):
    case = list(rand_case(B=1, T=5, H=2, dk=4, dv=3, gate=gate, seed=44))
    r = np.random.default_rng(45)
    dO = r.standard_normal((1, 5, 2, 3))
    dST = r.standard_normal((1, 2, 4, 3))
    dE = r.standard_normal((1, 5, 2, 3))
    g = oracle.backward(*case, dO, dST, scale=0.6, dE=dE)
    eps = 1e-6
    for idx, name in enumerate(["dq", "dk", "dv", "dbeta", "dalpha", "dS0"]):
        x = case[idx]
        if x is None:
            assert g[name] is None
            continue
        num = np.zeros_like(x)
        for mi in np.ndindex(x.shape):
            old = x[mi]
            x[mi] = old + eps
            lp = _loss_e(case, dO, dST, dE, 0.6)
            x[mi] = old - eps
            lm = _loss_e(case, dO, dST, dE, 0.6)
            x[mi] = old
            num[mi] = (lp - lm) / (2 * eps)
        err = np.abs(num - g[name]).max() / max(1.0, np.abs(num).max())
        assert err < 1e-7, (name, err)


def test_zero_error_gradient_is_the_plain_backward():
    case = rand_case(B=2, T=6, H=2, dk=4, dv=3, gate="channel", seed=46)
    r = np.random.default_rng(47)
    dO = r.standard_normal((2, 6, 2, 3))
    a = oracle.backward(*case, dO)
    b = oracle.backward(*case, dO, dE=np.zeros((2, 6, 2, 3)))
    assert all(np.array_equal(a[n], b[n]) for n in a)


def test_cler_routing_adds_scaled_errors():
    """CLER-H adds lam * e_t to the hidden stream per channel h*dv + j; lam = 0
    leaves it unchanged, and its adjoint sends lam * dh to the errors."""
    case = rand_case(B=1, T=4, H=2, dk=4, dv=3, gate="channel", seed=48)
    _, _, E = oracle.forward(*case, want_errors=True)
    r = np.random.default_rng(49)
    hid = r.standard_normal((1, 4, 6))
    assert np.array_equal(oracle.cler_forward(hid, E, np.zeros(6)), hid)
    lam = r.standard_normal(6)
    out = oracle.cler_forward(hid, E, lam)
    assert np.abs(out - hid - lam * E.reshape(1, 4, 6)).max() < 1e-15
    dh = r.standard_normal(hid.shape)
    dE, dlam = oracle.cler_backward(dh, E, lam)
    assert np.abs(dE.reshape(1, 4, 6) - lam * dh).max() < 1e-15
    assert np.abs(dlam - (dh * E.reshape(1, 4, 6)).sum((0, 1))).max() < 1e-13


# --------------------------------------------------------------------------
# prologue: L2-normalised q, k and activated gates
# --------------------------------------------------------------------------


def test_l2_normalise_gives_unit_rows_and_keeps_zero_rows():
    r = np.random.default_rng(60)
    x = r.standard_normal((4, 3, 7)) * r.uniform(0.01, 50, (4, 3, 1))
    n = np.linalg.norm(oracle.l2_normalise(x), axis=-1)
    assert np.abs(n - 1).max() < 1e-15
    z = np.zeros((2, 5))
    assert np.array_equal(oracle.l2_normalise(z), z)
    tiny = np.full((1, 4), 1e-9)
    assert np.allclose(oracle.l2_normalise(tiny), tiny / oracle.NORM_EPS, rtol=1e-15)


def test_gate_activations():
    """beta = sigmoid(b); the two alpha readings are mirror images
    (exp(-softplus(a)) = 1 - sigmoid(a)), checked against log1p/exp directly."""
    a = np.linspace(-30, 30, 61)
    _, _, b0, al_s = oracle.prologue_forward(np.ones((1, 2)), np.ones((1, 2)), np.zeros(1), a,
                                             oracle.PRO_ALPHA_SIGMOID)
    _, _, _, al_f = oracle.prologue_forward(np.ones((1, 2)), np.ones((1, 2)), np.zeros(1), a,
                                            oracle.PRO_ALPHA_FORGET)
    assert b0[0] == 0.5
    assert np.abs(al_s + al_f - 1).max() < 1e-15
    assert np.abs(al_f - np.exp(-np.log1p(np.exp(a)))).max() < 1e-15
    assert np.abs(al_s - 1 / (1 + np.exp(-a))).max() < 1e-15


def test_forget_gate_bias_from_the_page():
    with open(os.path.join(HERE, "golden", "forget_gate_bias.json")) as f:
        g = json.load(f)
    _, _, _, al = oracle.prologue_forward(np.ones((1, 2)), np.ones((1, 2)), np.zeros(1), np.array([g["bias"]]),
                                          oracle.PRO_ALPHA_FORGET)
    assert abs((1 - al[0]) - g["forget_fraction"]) < g["tolerance"]
    assert al[0] > 0.9  # the state keeps most of itself per token at initialisation


def test_prologue_exact_retrieval_with_unnormalised_keys():
    """q = k = c * u for any c > 0 and beta -> 1 (logit 40 rounds to 1.0 in
    fp64): after the prologue the read-out returns v exactly (KDA blog 2.1)."""
    r = np.random.default_rng(61)
    B, T, H, d = 1, 6, 2, 5
    u = unit(r.standard_normal((B, T, H, d)))
    c = r.uniform(0.1, 40, (B, T, H, 1))
    v = r.standard_normal((B, T, H, d))
    a = r.standard_normal((B, T, H, d))
    qh, kh, bt, al = oracle.prologue_forward(c * u, c * u, np.full((B, T, H), 40.0), a, oracle.PRO_ALPHA_FORGET)
    assert np.all(bt == 1.0)
    o, _ = oracle.forward(qh, kh, v, bt, al, None)
    assert np.abs(o - v).max() < 1e-12


@pytest.mark.parametrize("mode", [1, 2])
def test_prologue_backward_matches_central_differences(mode):
    r = np.random.default_rng(62 + mode)
    B, T, H, d = 1, 5, 2, 4
    q = r.standard_normal((B, T, H, d)) * 3
    k = r.standard_normal((B, T, H, d)) * 0.5
    v = r.standard_normal((B, T, H, d))
    b = r.standard_normal((B, T, H))
    a = r.standard_normal((B, T, H, d)) + 2
    dO = r.standard_normal((B, T, H, d))

    def loss(q_, k_, b_, a_):
        qh, kh, bt, al = oracle.prologue_forward(q_, k_, b_, a_, mode)
        o, _ = oracle.forward(qh, kh, v, bt, al, None)
        return float((o * dO).sum())

    qh, kh, bt, al = oracle.prologue_forward(q, k, b, a, mode)
    g = oracle.prologue_backward(q, k, b, a, mode, oracle.backward(qh, kh, v, bt, al, None, dO))
    eps = 1e-6
    for name, x in (("dq", q), ("dk", k), ("dbeta", b), ("dalpha", a)):
        num = np.zeros_like(x)
        for mi in np.ndindex(x.shape):
            old = x[mi]
            x[mi] = old + eps
            lp = loss(q, k, b, a)
            x[mi] = old - eps
            lm = loss(q, k, b, a)
            x[mi] = old
            num[mi] = (lp - lm) / (2 * eps)
        err = np.abs(num - g[name]).max() / max(1.0, np.abs(num).max())
        assert err < 1e-7, (name, err)


# --------------------------------------------------------------------------
# output gate: sigmoid(g) * RMSNorm(o) per head
# --------------------------------------------------------------------------


def test_output_gate_normalises_rows_and_gates_them():
    """With w = 1 and a saturated gate the rows come out with unit RMS; g = 0
    halves them; positive rescaling of o cancels; w scales channel by channel."""
    r = np.random.default_rng(70)
    o = r.standard_normal((2, 3, 2, 8)) * r.uniform(0.5, 20, (2, 3, 2, 1))
    y, _ = oracle.output_gate_forward(o, np.full(o.shape, 40.0))
    m = (o * o).mean(-1)
    assert np.abs(np.sqrt((y * y).mean(-1)) - np.sqrt(m / (m + oracle.GATE_EPS))).max() < 1e-13
    y0, _ = oracle.output_gate_forward(o, np.zeros(o.shape))
    assert np.abs(2 * y0 - y).max() < 1e-12
    g = r.standard_normal(o.shape)
    a, _ = oracle.output_gate_forward(o, g)
    b, _ = oracle.output_gate_forward(7.5 * o, g)
    ratio = np.sqrt((m + oracle.GATE_EPS) / (m + oracle.GATE_EPS / 7.5 ** 2))[..., None]
    assert np.abs(a * ratio - b).max() < 1e-13
    w = r.standard_normal(16)
    c, _ = oracle.output_gate_forward(o, g, w)
    assert np.abs(c - a * w.reshape(2, 8)).max() < 1e-12


def test_output_gate_backward_matches_central_differences():
    r = np.random.default_rng(71)
    o = r.standard_normal((1, 3, 2, 5))
    g = r.standard_normal(o.shape)
    w = r.standard_normal(10)
    dy = r.standard_normal(o.shape)
    do, dg, dw = oracle.output_gate_backward(o, g, w, dy)

    def loss(o_, g_, w_):
        return float((oracle.output_gate_forward(o_, g_, w_)[0] * dy).sum())

    eps = 1e-6
    for x, ref in ((o, do), (g, dg), (w, dw)):
        num = np.zeros_like(x)
        for mi in np.ndindex(x.shape):
            old = x[mi]
            x[mi] = old + eps
            lp = loss(o, g, w)
            x[mi] = old - eps
            lm = loss(o, g, w)
            x[mi] = old
            num[mi] = (lp - lm) / (2 * eps)
        assert np.abs(num - ref).max() / max(1.0, np.abs(num).max()) < 1e-8
