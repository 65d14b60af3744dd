"""Seeded synthetic inputs for the mLSTM chunkwise forward pass.

This module is shared by the tests, the benchmark and the oracle-side checks.
It draws random numbers and rounds them to the storage dtype; it holds none of
the mLSTM arithmetic (no gates, no cumulative sums, no state updates).

Workloads (all tensors contiguous (B, NH, S, D); gates (B, NH, S)):

  fp32_s256_d64     fp32, B=1 NH=1 S=256 DHQK=DHV=64 chunk=64
                    Q,K,V ~ N(0,1); i ~ N(0,1); f ~ N(3,1); zero C0/n0/m0
  bf16_s2048_d128   bf16 in / fp32 accumulate, B=8 NH=8 S=2048 DHQK=DHV=128
                    chunk=128 (Lq=Lkv=64); i ~ N(0, std 2) plus +8 spikes with
                    probability 1%; f ~ N(3,1); zero initial state
  bf16_7b_s8192     7B-shaped heads, bf16, B=8 NH=8 S=8192 DHQK=256 DHV=512
                    chunk=256; i ~ N(0,1); f ~ U(2,6); zero initial state
  bf16_7b_s65536    long context, bf16, B=1 NH=8 S=65536 DHQK=256 DHV=512
                    chunk=1024 (Lq=Lkv=128); C0 ~ N(0, std 0.1), n0 ~ U(0,1),
                    m0 = 0; gates as bf16_7b_s8192
  sig_7b_s8192      sigmoid-input-gate variant, shapes and gates as
                    bf16_7b_s8192, zero initial C (no n, no m)

Every (b, h) head draws from its own PCG64 stream seeded with
SeedSequence([seed, b, h]), in the fixed order Q, K, V, i, spike mask, f, C0,
n0.  That lets a check regenerate a few heads of a large workload without
drawing the rest.  Values are drawn in float32; for bf16 workloads Q, K and V
are rounded to bf16 with round-to-nearest-even, and the float32 copy holds the
rounded values exactly, so the GPU path and the oracle read identical numbers.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    NH: int
    S: int
    DHQK: int
    DHV: int
    chunk: int
    qkv_dtype: str            # "f32" or "bf16"
    gate: str                 # "exp" or "sig"
    i_dist: tuple             # ("normal", mean, std) with optional spikes
    f_dist: tuple             # ("normal", mean, std) or ("uniform", lo, hi)
    i_spike_prob: float = 0.0
    i_spike_value: float = 0.0
    init_state: bool = False  # C0 ~ N(0, c0_std), n0 ~ U(0,1), m0 = 0
    c0_std: float = 0.1
    tile_lq: int = 0          # 0: library chooses
    tile_lkv: int = 0
    seed: int = 0

    @property
    def BH(self) -> int:
        return self.B * self.NH

    @property
    def tokens(self) -> int:
        return self.B * self.S

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "fp32_s256_d64": Workload(
        "fp32_s256_d64", 1, 1, 256, 64, 64, 64, "f32", "exp",
        ("normal", 0.0, 1.0), ("normal", 3.0, 1.0), seed=1001),
    "bf16_s2048_d128": Workload(
        "bf16_s2048_d128", 8, 8, 2048, 128, 128, 128, "bf16", "exp",
        ("normal", 0.0, 2.0), ("normal", 3.0, 1.0),
        i_spike_prob=0.01, i_spike_value=8.0, tile_lq=64, tile_lkv=64,
        seed=1002),
    "bf16_7b_s8192": Workload(
        "bf16_7b_s8192", 8, 8, 8192, 256, 512, 256, "bf16", "exp",
        ("normal", 0.0, 1.0), ("uniform", 2.0, 6.0), seed=1003),
    "bf16_7b_s65536": Workload(
        "bf16_7b_s65536", 1, 8, 65536, 256, 512, 1024, "bf16", "exp",
        ("normal", 0.0, 1.0), ("uniform", 2.0, 6.0), init_state=True,
        c0_std=0.1, tile_lq=128, tile_lkv=128, seed=1004),
    "sig_7b_s8192": Workload(
        "sig_7b_s8192", 8, 8, 8192, 256, 512, 256, "bf16", "sig",
        ("normal", 0.0, 1.0), ("uniform", 2.0, 6.0), seed=1005),
}

WORKLOAD_ORDER = ["fp32_s256_d64", "bf16_s2048_d128", "bf16_7b_s8192",
                  "bf16_7b_s65536", "sig_7b_s8192"]


def round_to_bf16(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Round float32 values to bfloat16, nearest-even.

    Returns (values as float32, raw bf16 bit patterns as uint16).  Inputs are
    finite; NaN handling is not needed for drawn data.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32), (r >> np.uint32(16)).astype(np.uint16)


def _draw(rng: np.random.Generator, dist: tuple, n: int) -> np.ndarray:
    kind = dist[0]
    if kind == "normal":
        return (dist[1] + dist[2] * rng.standard_normal(n, dtype=np.float32)
                ).astype(np.float32)
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], n).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def head_inputs(w: Workload, b: int, h: int, S: Optional[int] = None) -> dict:
    """Draw the inputs of one (b, h) head as float32 numpy arrays.

    S overrides the sequence length (a prefix-stable draw is not promised:
    a different S gives different numbers)."""
    S = w.S if S is None else S
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, b, h])))
    q = rng.standard_normal((S, w.DHQK), dtype=np.float32)
    k = rng.standard_normal((S, w.DHQK), dtype=np.float32)
    v = rng.standard_normal((S, w.DHV), dtype=np.float32)
    i_pre = _draw(rng, w.i_dist, S)
    if w.i_spike_prob > 0:
        spikes = rng.random(S) < w.i_spike_prob
        i_pre = (i_pre + np.float32(w.i_spike_value) * spikes).astype(np.float32)
    f_pre = _draw(rng, w.f_dist, S)
    out = {"q": q, "k": k, "v": v, "i": i_pre, "f": f_pre}
    if w.init_state:
        out["C0"] = (w.c0_std * rng.standard_normal((w.DHQK, w.DHV), dtype=np.float32)
                     ).astype(np.float32)
        out["n0"] = rng.uniform(0.0, 1.0, w.DHQK).astype(np.float32)
        out["m0"] = np.zeros((), dtype=np.float32)
    if w.qkv_dtype == "bf16":
        for key in ("q", "k", "v"):
            out[key] = round_to_bf16(out[key])[0]
    return out


def make_inputs(w: Workload, heads: Optional[Sequence[tuple[int, int]]] = None) -> dict:
    """Draw the full (B, NH, ...) inputs, or only the listed (b, h) heads.

    With `heads`, arrays have a leading axis of len(heads) in place of
    (B, NH); the caller slices the GPU output the same way.
    Returns float32 arrays: q, k, v (values already bf16-rounded for bf16
    workloads), i, f and, if the workload has an initial state, C0, n0, m0.
    """
    if heads is None:
        heads = [(b, h) for b in range(w.B) for h in range(w.NH)]
        lead = (w.B, w.NH)
    else:
        heads = list(heads)
        lead = (len(heads),)
    per = [head_inputs(w, b, h) for (b, h) in heads]
    out = {}
    for key in per[0]:
        out[key] = np.stack([p[key] for p in per]).reshape(lead + per[0][key].shape)
    return out


def sha256_of(arr: np.ndarray) -> str:
    import hashlib
    return hashlib.sha256(np.ascontiguousarray(arr).tobytes()).hexdigest()
