"""Plain float64 CPU oracle of the mLSTM cell forward pass (test infrastructure).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  It shares no code with the HIP library.

Sources.  The pages describe the mLSTM in words: a matrix memory C updated by
an outer product, an exponential input gate, and normalisation plus
stabilisation of the exponential gates ("xLSTM: the NX-AI repository behind
the extended LSTM architecture", section "Exponential gating, matrix memory,
and why the kernels decide everything").  The TFLA abstract ("Tiled Flash
Linear Attention: More Efficient Linear RNN and xLSTM Kernels") adds the
chunkwise-parallel formulation and the sigmoid-input-gate variant with
reduced computation.  The quantities named for the forward pass (log-sigmoid
forget gate, max-state m, normaliser n, per-chunk C_k, n_k, m_k, in-chunk
cumulative log-forget sums, causal decay matrix D and the readout
normalisation max(|q.n|, exp(-m))) are written out below.

Readings taken where the pages leave a step open:
  * the 1/sqrt(DHQK) scale multiplies the query at readout; the states are
    built from raw k and v;
  * eps (added to the normaliser after the max) defaults to 0;
  * the forget gate applies at every step including the first, so chunk-local
    log-forget sums are inclusive;
  * the max-state m follows m_t = max(lf_t + m_{t-1}, i_t) from m_0 = m0
    (0 when absent); this fixes which (C, n, m) triple is returned;
  * the sigmoid-input-gate variant keeps only C: h_t = s C_t^T q_t, with
    C_t = sigmoid(f_t) C_{t-1} + sigmoid(i_t) k_t v_t^T, no n, no m, no
    division.

Array layout: Q, K (B, NH, S, DHQK); V (B, NH, S, DHV); i_pre, f_pre
(B, NH, S); C0 (B, NH, DHQK, DHV); n0 (B, NH, DHQK); m0 (B, NH).  Any leading
batch shape works as long as it is the same for every array.  Everything is
computed in float64.

Three forms are given; each is pinned in the tests against the others and
against closed forms:
  recurrent_fw  - the per-timestep recurrence (the definition);
  quadratic_fw  - the parallel (attention-like) form, O(S^2), tiny inputs;
  chunkwise_fw  - the chunkwise-parallel form for any chunk length L.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def log_sigmoid(x):
    """log(sigmoid(x)) = -log(1 + exp(-x)), written to avoid overflow."""
    x = np.asarray(x, dtype=np.float64)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def sigmoid(x):
    x = np.asarray(x, dtype=np.float64)
    return np.exp(log_sigmoid(x))


def _prep(Q, K, V, i_pre, f_pre, C0, n0, m0, gate):
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    i_pre = np.asarray(i_pre, dtype=np.float64)
    f_pre = np.asarray(f_pre, dtype=np.float64)
    lead = Q.shape[:-2]
    S, DK = Q.shape[-2:]
    DV = V.shape[-1]
    assert K.shape == Q.shape and V.shape == lead + (S, DV)
    assert i_pre.shape == lead + (S,) and f_pre.shape == lead + (S,)
    C0 = np.zeros(lead + (DK, DV)) if C0 is None else np.asarray(C0, dtype=np.float64)
    if gate == "exp":
        n0 = np.zeros(lead + (DK,)) if n0 is None else np.asarray(n0, dtype=np.float64)
        m0 = np.zeros(lead) if m0 is None else np.asarray(m0, dtype=np.float64)
        m0 = np.broadcast_to(m0, lead)
    elif gate == "sig":
        assert n0 is None and m0 is None, "the sigmoid-gate variant carries no n or m"
    else:
        raise ValueError(f"gate must be 'exp' or 'sig', not {gate!r}")
    return Q, K, V, i_pre, f_pre, C0, n0, m0, lead, S, DK, DV


def _scale(qk_scale, DK):
    return 1.0 / math.sqrt(DK) if qk_scale is None else float(qk_scale)


def recurrent_fw(Q, K, V, i_pre, f_pre, C0=None, n0=None, m0=None, *,
                 gate: str = "exp", qk_scale: Optional[float] = None,
                 eps: float = 0.0, return_rows: bool = False):
    """Per-timestep mLSTM recurrence (the definition of the forward pass).

    Exponential input gate, log-sigmoid forget gate, max-state stabiliser m
    and normaliser n, with s = qk_scale (default 1/sqrt(DHQK)):

        lf_t  = log sigmoid(f_t)
        m_t   = max(lf_t + m_{t-1}, i_t)
        a_t   = exp(lf_t + m_{t-1} - m_t),   b_t = exp(i_t - m_t)
        C_t   = a_t C_{t-1} + b_t k_t v_t^T
        n_t   = a_t n_{t-1} + b_t k_t
        h_t   = (s C_t^T q_t) / (max(|s n_t . q_t|, exp(-m_t)) + eps)

    Sigmoid-input-gate variant: C_t = sigmoid(f_t) C_{t-1} + sigmoid(i_t)
    k_t v_t^T and h_t = s C_t^T q_t.

    Returns (H, C_S, n_S, m_S); n_S and m_S are None for gate="sig".  With
    return_rows=True (exp variant only) also returns the per-row m_t and the
    stabilised normaliser sum s n_t . q_t.
    """
    Q, K, V, i_pre, f_pre, C0, n0, m0, lead, S, DK, DV = _prep(
        Q, K, V, i_pre, f_pre, C0, n0, m0, gate)
    s = _scale(qk_scale, DK)
    H = np.zeros(lead + (S, DV))
    C_out = np.zeros(lead + (DK, DV))
    n_out = np.zeros(lead + (DK,)) if gate == "exp" else None
    m_out = np.zeros(lead) if gate == "exp" else None
    rows_m = np.zeros(lead + (S,)) if return_rows else None
    rows_den = np.zeros(lead + (S,)) if return_rows else None
    for idx in np.ndindex(*lead):
        C = C0[idx].copy()
        if gate == "exp":
            n = n0[idx].copy()
            m = float(m0[idx])
        for t in range(S):
            lf = float(log_sigmoid(f_pre[idx + (t,)]))
            it = float(i_pre[idx + (t,)])
            k = K[idx + (t,)]
            v = V[idx + (t,)]
            q = s * Q[idx + (t,)]
            if gate == "exp":
                m_new = max(lf + m, it)
                a = math.exp(lf + m - m_new)
                b = math.exp(it - m_new)
                C = a * C + b * np.outer(k, v)
                n = a * n + b * k
                m = m_new
                num = C.T @ q
                den = float(n @ q)
                H[idx + (t,)] = num / (max(abs(den), math.exp(-m)) + eps)
                if return_rows:
                    rows_m[idx + (t,)] = m
                    rows_den[idx + (t,)] = den
            else:
                C = math.exp(lf) * C + float(sigmoid(it)) * np.outer(k, v)
                H[idx + (t,)] = C.T @ q
        C_out[idx] = C
        if gate == "exp":
            n_out[idx] = n
            m_out[idx] = m
    if return_rows:
        return H, C_out, n_out, m_out, rows_m, rows_den
    return H, C_out, n_out, m_out


def quadratic_fw(Q, K, V, i_pre, f_pre, C0=None, n0=None, m0=None, *,
                 gate: str = "exp", qk_scale: Optional[float] = None,
                 eps: float = 0.0):
    """Parallel (quadratic) form of the same forward pass, brute force.

    With F_t the inclusive sum of log-forget gates up to t (F_0 = 0), every
    output row t weighs key j <= t by the log-weight
        L[t, j] = F_t - F_j + i_j            (exp variant)
        L[t, j] = F_t - F_j + log sigmoid(i_j)   (sigmoid variant)
    and the initial state by L0[t] = F_t + m0 (exp) or F_t (sigmoid).  For
    the exp variant m_t = max(L0[t], max_j L[t, j]) and every weight is taken
    relative to it; the row is (weighted scores) V plus the initial-state
    readout, divided by max(|normaliser|, exp(-m_t)) + eps.
    O(S^2 * (DHQK + DHV)); meant for small inputs.
    Returns (H, C_S, n_S, m_S) like recurrent_fw.
    """
    Q, K, V, i_pre, f_pre, C0, n0, m0, lead, S, DK, DV = _prep(
        Q, K, V, i_pre, f_pre, C0, n0, m0, gate)
    s = _scale(qk_scale, DK)
    H = np.zeros(lead + (S, DV))
    if S == 0:
        return (H, C0.copy(), None if n0 is None else n0.copy(),
                None if m0 is None else np.array(m0, dtype=np.float64))
    C_out = np.zeros(lead + (DK, DV))
    n_out = np.zeros(lead + (DK,)) if gate == "exp" else None
    m_out = np.zeros(lead) if gate == "exp" else None
    causal = np.tril(np.ones((S, S), dtype=bool))
    for idx in np.ndindex(*lead):
        F = np.cumsum(log_sigmoid(f_pre[idx]))          # F[t] for t = 1..S
        if gate == "exp":
            src = i_pre[idx]
        else:
            src = log_sigmoid(i_pre[idx])
        Lw = F[:, None] - F[None, :] + src[None, :]
        Lw = np.where(causal, Lw, -np.inf)
        scores = s * (Q[idx] @ K[idx].T)
        if gate == "exp":
            L0 = F + m0[idx]
            mrow = np.maximum(L0, Lw.max(axis=1))
            W = np.exp(Lw - mrow[:, None])
            w0 = np.exp(L0 - mrow)
            num = (W * scores) @ V[idx] + w0[:, None] * (s * Q[idx] @ C0[idx])
            den = (W * scores).sum(axis=1) + w0 * (s * Q[idx] @ n0[idx])
            H[idx] = num / (np.maximum(np.abs(den), np.exp(-mrow)) + eps)[:, None]
            mS = mrow[-1]
            wS = np.exp(Lw[-1] - mS)
            C_out[idx] = np.exp(L0[-1] - mS) * C0[idx] + (K[idx] * wS[:, None]).T @ V[idx]
            n_out[idx] = np.exp(L0[-1] - mS) * n0[idx] + (K[idx] * wS[:, None]).sum(axis=0)
            m_out[idx] = mS
        else:
            W = np.exp(Lw)
            w0 = np.exp(F)
            H[idx] = (W * scores) @ V[idx] + w0[:, None] * (s * Q[idx] @ C0[idx])
            wS = np.exp(Lw[-1])
            C_out[idx] = np.exp(F[-1]) * C0[idx] + (K[idx] * wS[:, None]).T @ V[idx]
    return H, C_out, n_out, m_out


def chunkwise_fw(Q, K, V, i_pre, f_pre, C0=None, n0=None, m0=None, *,
                 chunk_size: int, gate: str = "exp",
                 qk_scale: Optional[float] = None, eps: float = 0.0,
                 return_states: bool = False):
    """Chunkwise-parallel form: states at chunk boundaries, parallel inside.

    The sequence is cut into chunks of chunk_size steps (the last one may be
    shorter).  Inside chunk c, with b_tau the inclusive chunk-local sum of
    log-forget gates (g = b at the chunk's last step) and (C, n, M) the
    stabilised state entering the chunk:

      exp variant
        a_tau    = g - b_tau + i_tau
        M_new    = max(g + M, max_tau a_tau)
        C_new    = exp(g + M - M_new) C + sum_tau exp(a_tau - M_new) k_tau v_tau^T
        n_new    = exp(g + M - M_new) n + sum_tau exp(a_tau - M_new) k_tau
        logD     = b_tau - b_sigma + i_sigma for sigma <= tau (else -inf)
        m_tau    = max(b_tau + M, max_sigma logD[tau, sigma])
        num_tau  = sum_sigma exp(logD - m_tau) s (q_tau.k_sigma) v_sigma
                   + exp(b_tau + M - m_tau) s C^T q_tau
        den_tau  = same with 1 in place of v_sigma and n in place of C
        h_tau    = num_tau / (max(|den_tau|, exp(-m_tau)) + eps)

      sigmoid variant (iota = log sigmoid(i))
        C_new    = exp(g) C + sum_tau exp(g - b_tau + iota_tau) k_tau v_tau^T
        h_tau    = sum_sigma exp(b_tau - b_sigma + iota_sigma) s (q_tau.k_sigma) v_sigma
                   + exp(b_tau) s C^T q_tau

    Returns (H, C_S, n_S, m_S).  With return_states=True also returns the
    list of states entering every chunk: arrays of shape lead + (N_c, ...)
    for C, n, M (n and M None for the sigmoid variant).
    """
    Q, K, V, i_pre, f_pre, C0, n0, m0, lead, S, DK, DV = _prep(
        Q, K, V, i_pre, f_pre, C0, n0, m0, gate)
    L = int(chunk_size)
    assert L >= 1
    s = _scale(qk_scale, DK)
    Nc = (S + L - 1) // L
    H = np.zeros(lead + (S, DV))
    C_out = np.zeros(lead + (DK, DV))
    n_out = np.zeros(lead + (DK,)) if gate == "exp" else None
    m_out = np.zeros(lead) if gate == "exp" else None
    Cst = np.zeros(lead + (Nc, DK, DV)) if return_states else None
    nst = np.zeros(lead + (Nc, DK)) if (return_states and gate == "exp") else None
    Mst = np.zeros(lead + (Nc,)) if (return_states and gate == "exp") else None
    for idx in np.ndindex(*lead):
        C = C0[idx].copy()
        if gate == "exp":
            n = n0[idx].copy()
            M = float(m0[idx])
        for c in range(Nc):
            t0, t1 = c * L, min(S, (c + 1) * L)
            if return_states:
                Cst[idx + (c,)] = C
                if gate == "exp":
                    nst[idx + (c,)] = n
                    Mst[idx + (c,)] = M
            q = Q[idx][t0:t1]
            k = K[idx][t0:t1]
            v = V[idx][t0:t1]
            b = np.cumsum(log_sigmoid(f_pre[idx][t0:t1]))
            g = b[-1]
            Lc = t1 - t0
            causal = np.tril(np.ones((Lc, Lc), dtype=bool))
            scores = s * (q @ k.T)
            if gate == "exp":
                it = i_pre[idx][t0:t1]
                logD = np.where(causal, b[:, None] - b[None, :] + it[None, :], -np.inf)
                mrow = np.maximum(b + M, logD.max(axis=1))
                P = scores * np.exp(logD - mrow[:, None])
                w_inter = np.exp(b + M - mrow)
                num = P @ v + w_inter[:, None] * (s * q @ C)
                den = P.sum(axis=1) + w_inter * (s * q @ n)
                H[idx][t0:t1] = num / (np.maximum(np.abs(den), np.exp(-mrow)) + eps)[:, None]
                a = g - b + it
                M_new = max(g + M, float(a.max()))
                wk = np.exp(a - M_new)
                decay = math.exp(g + M - M_new)
                C = decay * C + (k * wk[:, None]).T @ v
                n = decay * n + (k * wk[:, None]).sum(axis=0)
                M = M_new
            else:
                io = log_sigmoid(i_pre[idx][t0:t1])
                logD = np.where(causal, b[:, None] - b[None, :] + io[None, :], -np.inf)
                P = scores * np.exp(logD)
                H[idx][t0:t1] = P @ v + np.exp(b)[:, None] * (s * q @ C)
                wk = np.exp(g - b + io)
                C = math.exp(g) * C + (k * wk[:, None]).T @ v
        C_out[idx] = C
        if gate == "exp":
            n_out[idx] = n
            m_out[idx] = M
    if return_states:
        return H, C_out, n_out, m_out, (Cst, nst, Mst)
    return H, C_out, n_out, m_out
