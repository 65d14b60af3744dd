"""A float32 evaluation of the chunkwise mLSTM forward pass, for tests only.

It takes the steps of the chunkwise form in the order the GPU kernels take
them (in-chunk cumulative log-forget sums, the stabilised chunk state, the
intra-chunk scores with the running-max stabiliser, the inter-chunk term,
the normaliser) with every value and every accumulation in float32.  It is
not an oracle: it measures what float32 accumulation alone can reach on a
workload, which bounds what any float32-accumulating kernel can reach.
Readings as in the oracle: scale on the query, inclusive forget sums, m
from m0, eps added after the max.
"""
from __future__ import annotations

import numpy as np

f32 = np.float32


def _log_sigmoid(x):
    x = x.astype(f32)
    return (np.minimum(x, f32(0)) - np.log1p(np.exp(-np.abs(x)))).astype(f32)


def chunkwise_f32(q, k, v, i_pre, f_pre, C0=None, n0=None, m0=None, *, chunk_size: int, gate: str = "exp",
                  eps: float = 0.0):
    """H (S, DHV) and the final (C, n, m) of one head, all in float32."""
    q, k, v = (np.asarray(a, dtype=f32) for a in (q, k, v))
    S, DK = q.shape
    DV = v.shape[1]
    s = f32(1.0 / np.sqrt(DK))
    C = np.zeros((DK, DV), f32) if C0 is None else np.asarray(C0, f32).copy()
    n = np.zeros(DK, f32) if n0 is None else np.asarray(n0, f32).copy()
    M = f32(0.0) if m0 is None else f32(m0)
    src = np.asarray(i_pre, f32) if gate == "exp" else _log_sigmoid(np.asarray(i_pre, f32))
    lf = _log_sigmoid(np.asarray(f_pre, f32))
    H = np.zeros((S, DV), f32)
    L = chunk_size
    for t0 in range(0, S, L):
        sl = slice(t0, min(S, t0 + L))
        Lc = sl.stop - t0
        b = np.cumsum(lf[sl], dtype=f32)
        u = (src[sl] - b).astype(f32)
        Q, Kc, Vc = q[sl], k[sl], v[sl]
        scores = (Q @ Kc.T).astype(f32) * s
        causal = np.tril(np.ones((Lc, Lc), bool))
        if gate == "exp":
            pm = np.maximum.accumulate(u)
            mx = np.maximum(M, pm).astype(f32)             # m_t - b_t
            logd = (u[None, :] - mx[:, None]).astype(f32)
            P = np.where(causal, scores * np.exp(np.where(causal, logd, f32(0))), f32(0)).astype(f32)
            w0 = np.exp(M - mx).astype(f32)
            num = (P @ Vc + (w0 * s)[:, None] * (Q @ C)).astype(f32)
            den = (P.sum(axis=1, dtype=f32) + w0 * s * (Q @ n)).astype(f32)
            m_rows = (b + mx).astype(f32)
            H[sl] = num / (np.maximum(np.abs(den), np.exp(-m_rows)) + f32(eps))[:, None]
            g = b[-1]
            Mn = f32(max(g + M, (g + u).max()))
            wk = np.exp(g + u - Mn).astype(f32)
            dec = f32(np.exp(g + M - Mn))
            C = (dec * C + (Kc * wk[:, None]).T @ Vc).astype(f32)
            n = (dec * n + (Kc * wk[:, None]).sum(axis=0, dtype=f32)).astype(f32)
            M = Mn
        else:
            logd = (b[:, None] - b[None, :] + src[sl][None, :]).astype(f32)
            P = np.where(causal, scores * np.exp(np.where(causal, logd, f32(0))), f32(0)).astype(f32)
            H[sl] = (P @ Vc + (np.exp(b) * s)[:, None] * (Q @ C)).astype(f32)
            g = b[-1]
            wk = np.exp(g - b + src[sl]).astype(f32)
            C = (np.exp(g) * C + (Kc * wk[:, None]).T @ Vc).astype(f32)
    return H, C, (n if gate == "exp" else None), (M if gate == "exp" else None)


U32 = 2.0 ** -24   # unit roundoff of float32


def rounding_chain(DK: int, L: int, n_chunks: int) -> int:
    """Sequential float32 roundings one term of an output row can pass through
    in the chunkwise form: its score's dot product over DHQK and its share of
    P.V over the chunk's keys, both accumulated four products per matrix-core
    step; one decay per later chunk while it sits in the carried state; and
    16 for the exponentials, scalings, the inter-chunk product's own
    accumulation steps and the division (a worst-case count, linear in the
    chain length)."""
    return (DK + L) // 4 + n_chunks + 16


def accumulation_bound(q, k, v, i_pre, f_pre, C0=None, n0=None, m0=None, *, chunk_size: int,
                       gate: str = "exp", H_ref=None, m_rows=None, den_rows=None):
    """Per-element bound on |H_fp32 - H| (S, DHV) and on |den_fp32 - den| (S,)
    for float32 accumulation of one head, from the conditioning of each row.

    With w_tj <= 1 the stabilised weight of key j in row t (the oracle's
    m_t and den_t), g_tj = s sum_k |q_tk||k_jk| and the initial state's
    share w_t0 s |q_t|.|C0| (|q_t|.|n0| for the normaliser), a chain of c
    float32 roundings perturbs
        num_t by at most  c u A_t,   A_t = sum_{j<=t} w_tj g_tj |v_j| + w_t0 s |q_t|.|C0|
        den_t by at most  c u B_t,   B_t = sum_{j<=t} w_tj g_tj + w_t0 s |q_t|.|n0|
    and h = num / z with z = max(|den|, e^-m) by at most
        c u (A_t + |h_t| B_t) / z_t     (sig gate: c u A_t, no division).
    The absolute values make the bound cover every order of summation; it
    grows where a row's terms cancel (|A_t| >> |num_t| or B_t >> |den_t|),
    which is exactly where float32 accumulation loses digits.  H_ref,
    m_rows and den_rows are the oracle's H, per-row max-state and normaliser
    (the last two for the exp gate).  Returns (bound on H, bound on den);
    the second is None for the sig gate.
    """
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    S, DK = q.shape
    DV = v.shape[1]
    s = 1.0 / np.sqrt(DK)
    ls = lambda x: np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))
    F = np.cumsum(ls(np.asarray(f_pre, np.float64)))
    src = np.asarray(i_pre, np.float64) if gate == "exp" else ls(np.asarray(i_pre, np.float64))
    lam = F[:, None] - F[None, :] + src[None, :]
    causal = np.tril(np.ones((S, S), bool))
    M0 = 0.0 if (gate != "exp" or m0 is None) else float(m0)
    mt = np.asarray(m_rows, np.float64) if gate == "exp" else np.zeros(S)
    w = np.where(causal, np.exp(np.where(causal, lam - mt[:, None], -np.inf)), 0.0)
    w0 = np.exp(F + M0 - mt)
    g = s * (np.abs(q) @ np.abs(k).T)
    A = (w * g) @ np.abs(v)
    if C0 is not None:
        A += (w0 * s)[:, None] * (np.abs(q) @ np.abs(np.asarray(C0, np.float64)))
    c = rounding_chain(DK, chunk_size, (S + chunk_size - 1) // chunk_size)
    if gate != "exp":
        return c * U32 * A, None
    B = (w * g).sum(axis=1)
    if n0 is not None:
        B += w0 * s * (np.abs(q) @ np.abs(np.asarray(n0, np.float64)))
    z = np.maximum(np.abs(np.asarray(den_rows, np.float64)), np.exp(-mt))
    h = np.abs(np.asarray(H_ref, np.float64))
    return c * U32 * (A + h * B[:, None]) / z[:, None], c * U32 * B
