"""Float64 CPU oracle of the int8 block-quantised memory state of the
recurrent (decode) step (test infrastructure).

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this module.  It shares no code with the HIP library.

Source.  The "flash-xlstm-exp 0.1.0" page (section "Upgrade roadmap") lists a
quantised fp8/int8 memory state for long-context inference and says nothing
more.  Readings taken here, the plainest ones the rest supports:
  * only the matrix memory C is quantised; n and m stay float32;
  * int8 codes with one scale per block of 64 consecutive values of a row of
    C (row = key index, DHQK rows of DHV values, DHV a multiple of 64);
  * encoding of a block x: amax = max |x_i|; if amax = 0 every code is 0 and
    the scale is 0; otherwise code_i = round-half-even(x_i * (127 / amax)),
    which lies in [-127, 127], and scale = amax / 127; the block represents
    code_i * scale;
  * a step decodes the state, applies one step of the float recurrence
    (`recurrent_fw` over one token), reads h from the updated state before
    it is encoded again, and encodes the updated C.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .mlstm_oracle import recurrent_fw

BLOCK = 64


def q8_encode(C):
    """Encode (..., DHQK, DHV) float values: (codes int8, scales float64 of
    shape (..., DHQK, DHV // 64))."""
    C = np.asarray(C, dtype=np.float64)
    DV = C.shape[-1]
    if DV % BLOCK:
        raise ValueError("DHV must be a multiple of 64")
    x = C.reshape(C.shape[:-1] + (DV // BLOCK, BLOCK))
    amax = np.abs(x).max(axis=-1)
    safe = np.where(amax > 0, amax, 1.0)
    scaled = x * (127.0 / safe)[..., None]
    codes = np.where(amax[..., None] > 0, np.rint(scaled), 0.0)
    scales = np.where(amax > 0, amax / 127.0, 0.0)
    return codes.reshape(C.shape).astype(np.int8), scales


def q8_scaled(C):
    """The values x_i * 127 / amax before rounding (0 in all-zero blocks):
    what the encoding rounds, for judging how close a value sits to a tie."""
    C = np.asarray(C, dtype=np.float64)
    DV = C.shape[-1]
    x = C.reshape(C.shape[:-1] + (DV // BLOCK, BLOCK))
    amax = np.abs(x).max(axis=-1)
    safe = np.where(amax > 0, amax, 1.0)
    return (x * (127.0 / safe)[..., None]).reshape(C.shape)


def q8_decode(codes, scales):
    """(..., DHQK, DHV) float64 values of an encoded state."""
    codes = np.asarray(codes, dtype=np.float64)
    scales = np.asarray(scales, dtype=np.float64)
    DV = codes.shape[-1]
    x = codes.reshape(codes.shape[:-1] + (DV // BLOCK, BLOCK)) * scales[..., None]
    return x.reshape(codes.shape)


def recurrent_step_q8(q, k, v, i_pre, f_pre, codes=None, scales=None, n=None, m=None, *,
                      gate: str = "exp", qk_scale: Optional[float] = None, eps: float = 0.0):
    """One decode step from an encoded state.  q, k (..., DHQK); v (...,
    DHV); i_pre, f_pre (...); codes, scales as q8_encode returns them (None =
    zero state).  Returns (h, C_float, codes', scales', n', m'): C_float is
    the updated state before encoding (what h is read from)."""
    q = np.asarray(q, dtype=np.float64)
    DK, DV = q.shape[-1], np.asarray(v).shape[-1]
    lead = q.shape[:-1]
    C0 = np.zeros(lead + (DK, DV)) if codes is None else q8_decode(codes, scales)
    args = [np.asarray(a, dtype=np.float64)[..., None, :] for a in (q, k, v)]
    args += [np.asarray(a, dtype=np.float64)[..., None] for a in (i_pre, f_pre)]
    if gate == "exp":
        H, C1, n1, m1 = recurrent_fw(*args, C0, n, m, gate=gate, qk_scale=qk_scale, eps=eps)
    else:
        H, C1, n1, m1 = recurrent_fw(*args, C0, gate=gate, qk_scale=qk_scale, eps=eps)
    c1, s1 = q8_encode(C1)
    return H[..., 0, :], C1, c1, s1, n1, m1
