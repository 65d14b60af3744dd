"""Pins for the float64 gradient oracle (oracle/mlstm_grad.py).

The gradient oracle is torch autograd over the quadratic form of the forward
pass.  Each check below compares it with something fixed outside it:
  * central finite differences of <dH, H> where H comes from the per-step
    recurrence `recurrent_fw` (the numpy definition, pinned on its own in
    test_oracle.py), for every input entry of small cases;
  * the textbook gradients of causal linear attention, which the sig
    variant becomes when both gates are fully open;
  * the stabiliser gauge: (C0 e^d, n0 e^d, m0 - d) leaves H and every input
    gradient unchanged and scales dC0, dn0 by e^{-d};
  * two identities of the exact gradient that the chunkwise backward uses:
    the input-gate gradient is k . dk, and the forget-gate gradient is
    sigmoid(-f) times the reverse cumulative sum of q . dq - k . dk.
A mutation check shows that the finite-difference pin does see the one
reading taken (m held constant) once eps > 0.
"""
import math

import numpy as np
import pytest

from oracle import grad_fw, recurrent_fw, sigmoid


def _inputs(rng, lead, S, DK, DV, init=True, f_mean=1.0):
    d = dict(
        Q=rng.standard_normal(lead + (S, DK)),
        K=rng.standard_normal(lead + (S, DK)),
        V=rng.standard_normal(lead + (S, DV)),
        i_pre=rng.standard_normal(lead + (S,)),
        f_pre=f_mean + rng.standard_normal(lead + (S,)),
        dH=rng.standard_normal(lead + (S, DV)),
    )
    if init:
        d["C0"] = 0.5 * rng.standard_normal(lead + (DK, DV))
        d["n0"] = rng.random(lead + (DK,)) + 0.5
        d["m0"] = 0.3 * rng.standard_normal(lead)
    return d


def _loss(d, gate, eps):
    kw = dict(gate=gate, eps=eps)
    if gate == "exp":
        H = recurrent_fw(d["Q"], d["K"], d["V"], d["i_pre"], d["f_pre"], d.get("C0"), d.get("n0"), d.get("m0"), **kw)[0]
    else:
        H = recurrent_fw(d["Q"], d["K"], d["V"], d["i_pre"], d["f_pre"], d.get("C0"), **kw)[0]
    return float((H * d["dH"]).sum())


def _grads(d, gate, eps=0.0):
    extra = dict(C0=d.get("C0"))
    if gate == "exp":
        extra.update(n0=d.get("n0"), m0=d.get("m0"))
    return grad_fw(d["Q"], d["K"], d["V"], d["i_pre"], d["f_pre"], d["dH"], **extra, gate=gate, eps=eps)


FD_KEYS = {"Q": "dQ", "K": "dK", "V": "dV", "i_pre": "d_i", "f_pre": "d_f", "C0": "dC0", "n0": "dn0", "m0": "dm0"}


def _fd(d, gate, eps, h=1e-6):
    out = {}
    for name, gname in FD_KEYS.items():
        if name not in d or (gate == "sig" and name in ("n0", "m0")):
            continue
        x = d[name] = np.array(d[name], dtype=np.float64)
        g = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            keep = x[idx]
            x[idx] = keep + h
            up = _loss(d, gate, eps)
            x[idx] = keep - h
            dn = _loss(d, gate, eps)
            x[idx] = keep
            g[idx] = (up - dn) / (2 * h)
        out[gname] = g
    return out


@pytest.mark.parametrize("gate", ["exp", "sig"])
@pytest.mark.parametrize("init", [False, True])
def test_gradient_matches_finite_differences_of_the_recurrence(gate, init):
    rng = np.random.default_rng(100 + init + 2 * (gate == "sig"))
    d = _inputs(rng, (2,), 6, 3, 2, init=init)
    g = _grads(d, gate)
    fd = _fd(d, gate, 0.0)
    for k, ref in fd.items():
        err = np.abs(g[k] - ref).max()
        assert err <= 1e-6 * max(1.0, np.abs(ref).max()), (k, err)


def test_gradient_with_a_strong_input_gate_spike_and_closed_forget_gates():
    """Input-gate spikes move the max-state; small forget-gate values make
    the decay steep.  Still the derivative of the recurrence."""
    rng = np.random.default_rng(7)
    d = _inputs(rng, (1,), 7, 2, 3, init=True, f_mean=-2.0)
    d["i_pre"][0, 2] += 8.0
    d["i_pre"][0, 5] -= 6.0
    g = _grads(d, "exp")
    fd = _fd(d, "exp", 0.0)
    for k, ref in fd.items():
        assert np.abs(g[k] - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max()), k


def test_open_gates_give_causal_linear_attention_gradients():
    """sig gate with f, i -> +inf: h_t = s sum_{j<=t} (q_t . k_j) v_j + s C0^T q_t."""
    rng = np.random.default_rng(3)
    S, DK, DV = 9, 4, 3
    d = _inputs(rng, (1,), S, DK, DV, init=True)
    d["f_pre"] = np.full((1, S), 60.0)
    d["i_pre"] = np.full((1, S), 60.0)
    g = _grads(d, "sig")
    s = 1.0 / math.sqrt(DK)
    Q, K, V, dH, C0 = d["Q"][0], d["K"][0], d["V"][0], d["dH"][0], d["C0"][0]
    A = s * np.tril(Q @ K.T)
    dA = np.tril(dH @ V.T)
    np.testing.assert_allclose(g["dV"][0], A.T @ dH, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dQ"][0], s * dA @ K + s * dH @ C0.T, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dK"][0], s * dA.T @ Q, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(g["dC0"][0], s * Q.T @ dH, rtol=1e-12, atol=1e-12)
    assert np.abs(g["d_f"]).max() < 1e-20 and np.abs(g["d_i"]).max() < 1e-20


def test_stabiliser_gauge():
    rng = np.random.default_rng(5)
    d = _inputs(rng, (2,), 8, 3, 4, init=True)
    a = _grads(d, "exp")
    dd = 1.7
    e = dict(d, C0=d["C0"] * math.exp(dd), n0=d["n0"] * math.exp(dd), m0=d["m0"] - dd)
    b = _grads(e, "exp")
    for k in ("dQ", "dK", "dV", "d_i", "d_f"):
        np.testing.assert_allclose(b[k], a[k], rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(b["dC0"], a["dC0"] * math.exp(-dd), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(b["dn0"], a["dn0"] * math.exp(-dd), rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("gate", ["exp", "sig"])
def test_gate_gradient_identities(gate):
    rng = np.random.default_rng(11)
    d = _inputs(rng, (2,), 10, 4, 3, init=True)
    g = _grads(d, gate)
    kdk = (d["K"] * g["dK"]).sum(-1)
    qdq = (d["Q"] * g["dQ"]).sum(-1)
    di = kdk if gate == "exp" else kdk * sigmoid(-d["i_pre"])
    np.testing.assert_allclose(g["d_i"], di, rtol=1e-9, atol=1e-11)
    dF = qdq - kdk
    dlf = np.flip(np.cumsum(np.flip(dF, -1), -1), -1)
    np.testing.assert_allclose(g["d_f"], dlf * sigmoid(-d["f_pre"]), rtol=1e-9, atol=1e-11)
    if gate == "exp":
        dm0 = (g["dC0"] * d["C0"]).sum((-1, -2)) + (g["dn0"] * d["n0"]).sum(-1)
        np.testing.assert_allclose(g["dm0"], dm0, rtol=1e-9, atol=1e-11)


def test_held_max_state_is_visible_once_eps_is_positive():
    """With eps > 0 the output depends on m, so the held-m gradient and the
    finite differences part ways; with eps = 0 they agree (tests above)."""
    rng = np.random.default_rng(13)
    d = _inputs(rng, (1,), 5, 2, 2, init=True)
    g = _grads(d, "exp", eps=0.5)
    fd = _fd(d, "exp", 0.5)
    worst = max(np.abs(g[k] - fd[k]).max() for k in ("d_i", "d_f", "dm0"))
    assert worst > 1e-4


def test_empty_sequence():
    rng = np.random.default_rng(1)
    d = _inputs(rng, (1,), 0, 2, 2, init=True)
    g = _grads(d, "exp")
    assert g["dQ"].shape == (1, 0, 2) and np.all(g["dC0"] == 0)
