"""Pins for the float64 oracle, independent of the oracle's own formulas.

Each check compares the oracle with something fixed outside it: hand-worked
cases (tests/golden/hand_worked.json), closed forms written with plain numpy
(Toeplitz powers of a constant forget gate, causal linear attention),
invariances of the method (linearity in V, the stabiliser's gauge freedom,
chunk-size independence) and the agreement of three independently written
forms (recurrent, quadratic, chunkwise).  The mutation checks at the end feed
deliberately wrong inputs and confirm that these pins notice.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import chunkwise_fw, log_sigmoid, quadratic_fw, recurrent_fw, sigmoid

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _num(x):
    if isinstance(x, str):
        return {"ln2": math.log(2.0), "ln3": math.log(3.0)}[x]
    return x


def _arr(x):
    if isinstance(x, list):
        return np.array([_arr(e) for e in x], dtype=np.float64)
    return _num(x)


def _rand_inputs(rng, lead, S, DK, DV, i_scale=1.0, f_mean=1.0, init=True):
    d = dict(
        Q=rng.standard_normal(lead + (S, DK)),
        K=rng.standard_normal(lead + (S, DK)),
        V=rng.standard_normal(lead + (S, DV)),
        i_pre=i_scale * rng.standard_normal(lead + (S,)),
        f_pre=f_mean + rng.standard_normal(lead + (S,)),
    )
    if init:
        d["C0"] = 0.5 * rng.standard_normal(lead + (DK, DV))
        d["n0"] = rng.random(lead + (DK,))
        d["m0"] = 0.3 * rng.standard_normal(lead)
    return d


def _call(fn, d, gate="exp", **kw):
    args = (d["Q"], d["K"], d["V"], d["i_pre"], d["f_pre"])
    if gate == "exp":
        return fn(*args, d.get("C0"), d.get("n0"), d.get("m0"), gate=gate, **kw)
    return fn(*args, d.get("C0"), gate=gate, **kw)


# --------------------------------------------------------------------------
# hand-worked cases


def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
@pytest.mark.parametrize("form", ["recurrent", "quadratic", "chunk1", "chunk2"])
def test_hand_worked(case, form):
    Q, K, V = _arr(case["q"]), _arr(case["k"]), _arr(case["v"])
    i_pre, f_pre = _arr(case["i_pre"]), _arr(case["f_pre"])
    gate = case["gate"]
    C0 = _arr(case["C0"]) if "C0" in case else None
    n0 = _arr(case["n0"]) if "n0" in case else None
    m0 = np.array(_num(case["m0"])) if "m0" in case else None
    kw = dict(gate=gate, qk_scale=1.0)
    if form == "recurrent":
        out = recurrent_fw(Q, K, V, i_pre, f_pre, C0, n0, m0, **kw)
    elif form == "quadratic":
        out = quadratic_fw(Q, K, V, i_pre, f_pre, C0, n0, m0, **kw)
    else:
        L = 1 if form == "chunk1" else 2
        out = chunkwise_fw(Q, K, V, i_pre, f_pre, C0, n0, m0, chunk_size=L, **kw)
    H, C, n, m = out
    np.testing.assert_allclose(H, _arr(case["H"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(C, _arr(case["C"]), rtol=0, atol=1e-12)
    if gate == "exp":
        np.testing.assert_allclose(n, _arr(case["n"]), rtol=0, atol=1e-12)
        np.testing.assert_allclose(m, _num(case["m"]), rtol=0, atol=1e-12)
    else:
        assert n is None and m is None


def test_log_sigmoid_against_direct_formula():
    x = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(log_sigmoid(x), np.log(1.0 / (1.0 + np.exp(-x))), rtol=1e-12, atol=1e-12)
    # no overflow far out, and the asymptotes
    assert log_sigmoid(np.array(-1000.0)) == -1000.0
    assert log_sigmoid(np.array(1000.0)) == 0.0
    np.testing.assert_allclose(sigmoid(np.array([0.0, math.log(3.0)])), [0.5, 0.75], rtol=1e-15)


# --------------------------------------------------------------------------
# three independently written forms agree


@pytest.mark.parametrize("gate", ["exp", "sig"])
@pytest.mark.parametrize("init", [False, True])
def test_recurrent_equals_quadratic(gate, init):
    rng = np.random.default_rng(11 + init)
    d = _rand_inputs(rng, (2, 2), 29, 5, 7, i_scale=2.0, init=init)
    if gate == "sig":
        d.pop("n0", None)
        d.pop("m0", None)
    r = _call(recurrent_fw, d, gate)
    q = _call(quadratic_fw, d, gate)
    for a, b in zip(r, q):
        if a is None:
            assert b is None
            continue
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("gate", ["exp", "sig"])
@pytest.mark.parametrize("L", [1, 2, 3, 7, 8, 16, 31, 40])
def test_chunk_size_invariance(gate, L):
    """H and the final state do not depend on the chunk length (ragged tails included)."""
    rng = np.random.default_rng(5)
    d = _rand_inputs(rng, (1, 2), 31, 6, 4, i_scale=1.5)
    if gate == "sig":
        d.pop("n0")
        d.pop("m0")
    r = _call(recurrent_fw, d, gate)
    c = _call(chunkwise_fw, d, gate, chunk_size=L)
    for a, b in zip(r, c):
        if a is None:
            continue
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-11)


def test_chunk_states_match_recurrent_prefix():
    """The state entering chunk c equals the recurrent state after c*L steps."""
    rng = np.random.default_rng(9)
    d = _rand_inputs(rng, (1,), 24, 4, 3)
    L = 8
    *_, (Cst, nst, Mst) = chunkwise_fw(d["Q"], d["K"], d["V"], d["i_pre"], d["f_pre"],
                                       d["C0"], d["n0"], d["m0"], chunk_size=L,
                                       return_states=True)
    for c in range(3):
        t = c * L
        pre = {k: (v[:, :t] if k in ("Q", "K", "V", "i_pre", "f_pre") else v) for k, v in d.items()}
        _, C, n, m = _call(recurrent_fw, pre)
        np.testing.assert_allclose(Cst[:, c], C, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(nst[:, c], n, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(Mst[:, c], m, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------
# closed forms


def _toeplitz_decay(f_gate, S):
    idx = np.arange(S)
    expo = idx[:, None] - idx[None, :]
    return np.where(expo >= 0, np.power(f_gate, np.maximum(expo, 0)), 0.0)


@pytest.mark.parametrize("eps", [0.0, 0.25])
def test_closed_form_constant_forget_gate(eps):
    """Constant forget gate f: key j reaches row t with weight f^(t-j) exp(i_j);
    the initial state reaches row t with weight f^t (forget gate at every step)."""
    rng = np.random.default_rng(3)
    S, DK, DV = 23, 4, 5
    Q, K, V = rng.standard_normal((S, DK)), rng.standard_normal((S, DK)), rng.standard_normal((S, DV))
    i_pre = rng.standard_normal(S)
    f_pre = np.full(S, 0.7)
    C0 = rng.standard_normal((DK, DV))
    n0 = rng.random(DK)
    fg = 1.0 / (1.0 + math.exp(-0.7))
    s = 1.0 / math.sqrt(DK)
    W = _toeplitz_decay(fg, S) * np.exp(i_pre)[None, :] * (s * Q @ K.T)
    w0 = np.power(fg, np.arange(1, S + 1))
    num = W @ V + w0[:, None] * (s * Q @ C0)
    den = W.sum(axis=1) + w0 * (s * Q @ n0)
    # with m0 = 0, the stabilised readout equals num / (max(|den|, 1) + eps*exp(m_t))
    H, C, n, m = recurrent_fw(Q, K, V, i_pre, f_pre, C0, n0, np.array(0.0), eps=eps)
    if eps == 0.0:
        np.testing.assert_allclose(H, num / np.maximum(np.abs(den), 1.0)[:, None], rtol=1e-11, atol=1e-11)
    Ctrue = np.power(fg, S) * C0 + (K * (np.power(fg, S - 1 - np.arange(S)) * np.exp(i_pre))[:, None]).T @ V
    np.testing.assert_allclose(C * math.exp(m), Ctrue, rtol=1e-11, atol=1e-11)


def test_closed_form_open_forget_gate():
    """Forget gate open (f_pre = 40) and i = 0: causal linear attention with the
    normaliser max(|row sum|, 1)."""
    rng = np.random.default_rng(4)
    S, DK, DV = 19, 8, 3
    Q, K, V = rng.standard_normal((S, DK)), rng.standard_normal((S, DK)), rng.standard_normal((S, DV))
    A = np.tril((Q @ K.T) / math.sqrt(DK))
    expect = (A @ V) / np.maximum(np.abs(A.sum(axis=1)), 1.0)[:, None]
    H, *_ = recurrent_fw(Q, K, V, np.zeros(S), np.full(S, 40.0))
    np.testing.assert_allclose(H, expect, rtol=1e-9, atol=1e-9)


def test_closed_form_single_step():
    rng = np.random.default_rng(8)
    DK, DV = 6, 4
    q, k, v = rng.standard_normal((1, DK)), rng.standard_normal((1, DK)), rng.standard_normal((1, DV))
    for i0 in (-3.0, 0.4, 5.0):
        s = 1.0 / math.sqrt(DK)
        a = math.exp(i0) * s * float(q[0] @ k[0])
        expect = a * v[0] / max(abs(a), 1.0)
        H, C, n, m = recurrent_fw(q, k, v, np.array([i0]), np.array([-2.0]))
        np.testing.assert_allclose(H[0], expect, rtol=1e-12, atol=1e-12)


def test_closed_form_sigmoid_variant():
    """Sigmoid input gate, constant forget gate: gated causal linear attention."""
    rng = np.random.default_rng(6)
    S, DK, DV = 21, 5, 6
    Q, K, V = rng.standard_normal((S, DK)), rng.standard_normal((S, DK)), rng.standard_normal((S, DV))
    i_pre = 2.0 * rng.standard_normal(S)
    f_pre = np.full(S, 1.3)
    C0 = rng.standard_normal((DK, DV))
    fg = 1.0 / (1.0 + math.exp(-1.3))
    ig = 1.0 / (1.0 + np.exp(-i_pre))
    s = 1.0 / math.sqrt(DK)
    W = _toeplitz_decay(fg, S) * ig[None, :] * (s * Q @ K.T)
    expect = W @ V + np.power(fg, np.arange(1, S + 1))[:, None] * (s * Q @ C0)
    H, C, n, m = recurrent_fw(Q, K, V, i_pre, f_pre, C0, gate="sig")
    np.testing.assert_allclose(H, expect, rtol=1e-11, atol=1e-11)
    assert n is None and m is None
    # fully open gates: plain causal linear attention
    H2, *_ = recurrent_fw(Q, K, V, np.full(S, 40.0), np.full(S, 40.0), gate="sig")
    np.testing.assert_allclose(H2, np.tril(s * Q @ K.T) @ V, rtol=1e-9, atol=1e-9)


# --------------------------------------------------------------------------
# invariants


def test_linear_in_values():
    rng = np.random.default_rng(12)
    d = _rand_inputs(rng, (2,), 17, 4, 5, init=False)
    H1, C1, n1, m1 = _call(recurrent_fw, d)
    d2 = dict(d, V=-2.5 * d["V"])
    H2, C2, n2, m2 = _call(recurrent_fw, d2)
    np.testing.assert_allclose(H2, -2.5 * H1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(C2, -2.5 * C1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(n2, n1, rtol=0, atol=0)


def test_stabiliser_gauge_freedom():
    """(C0, n0, m0) and (C0 e^d, n0 e^d, m0 - d) are the same state: H and the
    unscaled final state C e^m agree (eps = 0)."""
    rng = np.random.default_rng(13)
    d = _rand_inputs(rng, (1,), 20, 4, 3)
    H1, C1, n1, m1 = _call(recurrent_fw, d)
    delta = 1.7
    d2 = dict(d, C0=d["C0"] * math.exp(delta), n0=d["n0"] * math.exp(delta), m0=d["m0"] - delta)
    H2, C2, n2, m2 = _call(recurrent_fw, d2)
    np.testing.assert_allclose(H2, H1, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(C2 * np.exp(m2)[:, None, None], C1 * np.exp(m1)[:, None, None], rtol=1e-11)
    np.testing.assert_allclose(n2 * np.exp(m2)[:, None], n1 * np.exp(m1)[:, None], rtol=1e-11)


def test_zero_state_m0_invariance():
    rng = np.random.default_rng(14)
    d = _rand_inputs(rng, (1,), 15, 3, 3, init=False)
    H0, *_ = recurrent_fw(d["Q"], d["K"], d["V"], d["i_pre"], d["f_pre"], m0=np.array([0.0]))
    H1, *_ = recurrent_fw(d["Q"], d["K"], d["V"], d["i_pre"], d["f_pre"], m0=np.array([-4.0]))
    np.testing.assert_allclose(H0, H1, rtol=1e-11, atol=1e-11)


def test_split_sequence_state_carry():
    rng = np.random.default_rng(15)
    d = _rand_inputs(rng, (2,), 26, 4, 5)
    H, C, n, m = _call(recurrent_fw, d)
    cut = 11
    a = {k: (v[:, :cut] if k in ("Q", "K", "V", "i_pre", "f_pre") else v) for k, v in d.items()}
    Ha, Ca, na, ma = _call(recurrent_fw, a)
    b = {k: v[:, cut:] for k, v in d.items() if k in ("Q", "K", "V", "i_pre", "f_pre")}
    b.update(C0=Ca, n0=na, m0=ma)
    Hb, Cb, nb, mb = _call(recurrent_fw, b)
    np.testing.assert_allclose(np.concatenate([Ha, Hb], axis=1), H, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Cb, C, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mb, m, rtol=0, atol=1e-14)


def test_sigmoid_variant_from_exp_variant_rows():
    """The sigmoid-gate output equals the exp-gate output computed with the
    input gate log sigmoid(i), times max(|den| e^m, 1), where den and m are
    that run's stabilised normaliser and max-state."""
    rng = np.random.default_rng(16)
    d = _rand_inputs(rng, (1,), 18, 4, 4, init=False)
    Hs, Cs, _, _ = recurrent_fw(d["Q"], d["K"], d["V"], d["i_pre"], d["f_pre"], gate="sig")
    He, Ce, ne, me, rm, rden = recurrent_fw(d["Q"], d["K"], d["V"], log_sigmoid(d["i_pre"]),
                                           d["f_pre"], return_rows=True)
    scale = np.maximum(np.abs(rden) * np.exp(rm), 1.0)
    np.testing.assert_allclose(Hs, He * scale[..., None], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(Cs, Ce * np.exp(me)[:, None, None], rtol=1e-10)


def test_empty_sequence_returns_initial_state():
    rng = np.random.default_rng(17)
    d = _rand_inputs(rng, (2,), 0, 3, 2)
    for fn in (recurrent_fw, quadratic_fw):
        H, C, n, m = _call(fn, d)
        assert H.shape == (2, 0, 2)
        np.testing.assert_array_equal(C, d["C0"])
        np.testing.assert_array_equal(n, d["n0"])
        np.testing.assert_array_equal(m, d["m0"])
    H, C, n, m = _call(chunkwise_fw, d, chunk_size=4)
    np.testing.assert_array_equal(C, d["C0"])


# --------------------------------------------------------------------------
# mutation checks: plausible mistakes must trip at least one pin


def _closed_form_error(f_sign=1.0, swap_qk=False, drop_init=False, shift_i=0.0):
    rng = np.random.default_rng(3)
    S, DK, DV = 12, 4, 3
    Q, K, V = rng.standard_normal((S, DK)), rng.standard_normal((S, DK)), rng.standard_normal((S, DV))
    i_pre = rng.standard_normal(S)
    f_pre = np.full(S, 0.7)
    C0 = rng.standard_normal((DK, DV))
    n0 = rng.random(DK)
    fg = 1.0 / (1.0 + math.exp(-0.7))
    s = 1.0 / math.sqrt(DK)
    W = _toeplitz_decay(fg, S) * np.exp(i_pre)[None, :] * (s * Q @ K.T)
    w0 = np.power(fg, np.arange(1, S + 1))
    num = W @ V + w0[:, None] * (s * Q @ C0)
    den = W.sum(axis=1) + w0 * (s * Q @ n0)
    expect = num / np.maximum(np.abs(den), 1.0)[:, None]
    q_in, k_in = (K, Q) if swap_qk else (Q, K)
    H, *_ = recurrent_fw(q_in, k_in, V, i_pre + shift_i, f_sign * f_pre,
                         None if drop_init else C0, None if drop_init else n0, np.array(0.0))
    return float(np.abs(H - expect).max())


def test_mutations_are_detected():
    assert _closed_form_error() < 1e-10
    assert _closed_form_error(f_sign=-1.0) > 1e-3      # wrong forget-gate sign
    assert _closed_form_error(swap_qk=True) > 1e-3     # transposed q/k roles
    assert _closed_form_error(drop_init=True) > 1e-3   # dropped initial-state term
    assert _closed_form_error(shift_i=1.0) > 1e-3      # input gate off by a factor e
