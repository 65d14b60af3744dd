"""Float64 CPU oracle of the gradients of the mLSTM forward pass (test
infrastructure).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  It shares no code with the HIP library.

What is differentiated.  The forward pass of the mLSTM cell as the pages
describe it ("xLSTM: the NX-AI repository behind the extended LSTM
architecture", section "Exponential gating, matrix memory, and why the
kernels decide everything": exponential gating with normalisation and
stabilisation, matrix memory; "Tiled Flash Linear Attention: More Efficient
Linear RNN and xLSTM Kernels", abstract: the chunkwise form is used for
training, and the sigmoid-input-gate variant).  The pages print no backward
pass; the gradient is the derivative of that forward pass, taken here by
torch autograd in float64 over the parallel (quadratic) form, with every
other step written out below:

    F_t      = sum_{u <= t} log sigmoid(f_u)
    L[t, j]  = F_t - F_j + i_j          (exp gate; log sigmoid(i_j) for sig)
    L0[t]    = F_t + m0                 (exp gate; F_t for sig)
    m_t      = max(L0[t], max_{j <= t} L[t, j])            (exp gate)
    P[t, j]  = e^{L[t, j] - m_t} s q_t . k_j,   w0_t = e^{L0[t] - m_t}
    num_t    = sum_j P[t, j] v_j + w0_t s C0^T q_t
    den_t    = sum_j P[t, j] + w0_t s n0 . q_t
    h_t      = num_t / (max(|den_t|, e^{-m_t}) + eps)
    sig gate: h_t = sum_j e^{L[t, j]} s (q_t . k_j) v_j + e^{F_t} s C0^T q_t

Reading taken where the pages are silent: the max-state m_t is a
stabiliser and is held constant under differentiation.  With eps = 0 the
output does not depend on m at all (numerator and normaliser scale together),
so this is the exact gradient; with eps > 0 it is the gradient at fixed m.
m0 still receives the gradient of its explicit appearance in L0 (the true
initial memory is e^{m0} C0, e^{m0} n0).

The loss is <dH, H>, so the returned arrays are the vector-Jacobian products
of the forward pass with dH: dQ, dK, dV, d_i (for i_pre), d_f (for f_pre) and
the initial-state gradients dC0, dn0, dm0 (with respect to the zero state
when none is given).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch


def _t(x, shape=None):
    if x is None:
        return torch.zeros(shape, dtype=torch.float64)
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


def quadratic_fw_torch(Q, K, V, i_pre, f_pre, C0, n0, m0, *, gate: str, s: float, eps: float,
                       hold_m: bool = True):
    """The forward pass above as float64 torch ops on (..., S, D) tensors."""
    S = Q.shape[-2]
    lf = torch.nn.functional.logsigmoid(f_pre)
    F = torch.cumsum(lf, dim=-1)
    src = i_pre if gate == "exp" else torch.nn.functional.logsigmoid(i_pre)
    causal = torch.tril(torch.ones(S, S, dtype=torch.bool))
    Lw = (F[..., :, None] - F[..., None, :] + src[..., None, :]).masked_fill(~causal, -math.inf)
    scores = s * (Q @ K.transpose(-1, -2))
    q_c0 = s * (Q @ C0)                                     # (..., S, DV)
    if gate == "exp":
        L0 = F + m0[..., None]
        mrow = torch.maximum(L0, Lw.max(dim=-1).values)
        if hold_m:
            mrow = mrow.detach()
        W = torch.exp(Lw - mrow[..., None])
        w0 = torch.exp(L0 - mrow)
        P = W * scores
        num = P @ V + w0[..., None] * q_c0
        den = P.sum(dim=-1) + w0 * s * (Q @ n0[..., :, None])[..., 0]
        return num / (torch.maximum(den.abs(), torch.exp(-mrow)) + eps)[..., None]
    W = torch.exp(Lw)
    return (W * scores) @ V + torch.exp(F)[..., None] * q_c0


def grad_fw(Q, K, V, i_pre, f_pre, dH, C0=None, n0=None, m0=None, *,
            gate: str = "exp", qk_scale: Optional[float] = None, eps: float = 0.0):
    """Vector-Jacobian product of the forward pass with dH (float64).

    Arrays as in the forward oracle: Q, K (..., S, DHQK); V, dH (..., S, DHV);
    i_pre, f_pre (..., S); C0 (..., DHQK, DHV); n0 (..., DHQK); m0 (...).
    Returns a dict with dQ, dK, dV, d_i, d_f, dC0 and, for the exp gate, dn0
    and dm0 (numpy float64)."""
    Qt, Kt, Vt = _t(Q), _t(K), _t(V)
    lead, S, DK = tuple(Qt.shape[:-2]), Qt.shape[-2], Qt.shape[-1]
    DV = Vt.shape[-1]
    it, ft, dHt = _t(i_pre), _t(f_pre), _t(dH)
    C0t = _t(C0, lead + (DK, DV))
    n0t = _t(n0, lead + (DK,))
    m0t = _t(m0, lead)
    leaves = [Qt, Kt, Vt, it, ft, C0t] + ([n0t, m0t] if gate == "exp" else [])
    for x in leaves:
        x.requires_grad_(True)
    s = 1.0 / math.sqrt(DK) if qk_scale is None else float(qk_scale)
    names = ["dQ", "dK", "dV", "d_i", "d_f", "dC0"] + (["dn0", "dm0"] if gate == "exp" else [])
    if S == 0:
        return {n: np.zeros(tuple(x.shape)) for n, x in zip(names, leaves)}
    H = quadratic_fw_torch(Qt, Kt, Vt, it, ft, C0t, n0t, m0t, gate=gate, s=s, eps=eps)
    grads = torch.autograd.grad((H * dHt).sum(), leaves, allow_unused=True)
    out = {}
    for n, x, g in zip(names, leaves, grads):
        out[n] = np.zeros(tuple(x.shape)) if g is None else g.detach().numpy()
    return out
