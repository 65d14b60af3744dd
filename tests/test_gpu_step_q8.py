"""Parity of the int8 block-quantised decode state (mlstm_recurrent_step_q8,
mlstm_state_q8_encode / _decode) against the float64 oracle (needs an MI355X).

The codes are integers that a float value decides: the GPU forms that value
in float32 and the oracle in float64, so they may round differently where
the value sits next to a tie.  The check is exact everywhere else: codes equal
wherever the oracle's pre-rounding value (x * 127 / amax) lies more than 1e-3
from a half-integer, and within +-1 where it does.  Scales: relative 1e-5.
h: max abs error 2e-2 (bf16 inputs) / 1e-4 (float32 inputs), the forward
pass's bounds (h is read from the float32 update, before encoding); n, m as
for the float step.  Inputs are seeded draws; Q, K, V rounded to bf16 for the
bf16 cases.  The library keeps the scales block-major, (B, NH, DHV/64,
DHQK); the oracle's are (B, NH, DHQK, DHV/64), and the tests swap the last
two axes between them.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import q8_decode, q8_encode, q8_scaled, recurrent_step_q8, recurrent_fw  # noqa: E402
from workloads import round_to_bf16  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_H = {"bf16": 2e-2, "f32": 1e-4}
NEAR_TIE = 1e-3


@pytest.fixture(scope="module")
def mt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import xlstm_mlstm_chunkwise_amd as m
    m.lib()
    return m


def _dev(a, dtype=torch.float32):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def _np(t):
    return None if t is None else t.cpu().numpy()


def to_lib(scales):
    return np.ascontiguousarray(np.swapaxes(scales, -1, -2))


def from_lib(scales):
    return np.swapaxes(scales, -1, -2)


def check_codes(tag, codes_gpu, scales_lib, C_ref):
    """GPU encoding of the state whose float64 value is C_ref."""
    scales_gpu = from_lib(scales_lib)
    codes_ref, scales_ref = q8_encode(C_ref)
    scaled = q8_scaled(C_ref)
    near = np.abs(np.abs(scaled - np.trunc(scaled)) - 0.5) < NEAR_TIE
    d = codes_gpu.astype(np.int32) - codes_ref.astype(np.int32)
    assert np.all(d[~near] == 0), f"{tag}: {np.count_nonzero(d[~near])} codes differ away from ties"
    assert np.all(np.abs(d[near]) <= 1), f"{tag}: a code near a tie is off by more than one"
    rel = np.abs(scales_gpu.astype(np.float64) - scales_ref) / np.maximum(scales_ref, 1e-30)
    assert rel.max() <= 1e-5, f"{tag}: scale rel err {rel.max():.3g}"
    return int(np.count_nonzero(d))


def _draw(seed, B, NH, DK, DV, kind, gate, zero=False):
    rng = np.random.default_rng(seed)
    x = dict(q=rng.standard_normal((B, NH, DK)), k=rng.standard_normal((B, NH, DK)),
             v=rng.standard_normal((B, NH, DV)), i=rng.standard_normal((B, NH)),
             f=2.0 + 4.0 * rng.random((B, NH)))
    x = {n: a.astype(np.float32) for n, a in x.items()}
    if kind == "bf16":
        for n in ("q", "k", "v"):
            x[n] = round_to_bf16(x[n])[0]
    st = {}
    if not zero:
        st["Cq"] = rng.integers(-127, 128, (B, NH, DK, DV)).astype(np.int8)
        st["Cs"] = (0.1 * rng.random((B, NH, DK, DV // 64)) / 127).astype(np.float32)   # oracle layout
        if gate == "exp":
            st["n"] = rng.random((B, NH, DK)).astype(np.float32)
            st["m"] = rng.standard_normal((B, NH)).astype(np.float32)
    return x, st


def _step(mt, x, st, gate, kind, inplace=False):
    qd = torch.bfloat16 if kind == "bf16" else torch.float32
    Cq = _dev(st.get("Cq"), torch.int8)
    Cs = None if "Cs" not in st else _dev(to_lib(st["Cs"]))
    out = mt.mlstm_recurrent_step_q8(_dev(x["q"], qd), _dev(x["k"], qd), _dev(x["v"], qd), _dev(x["i"]),
                                     _dev(x["f"]), Cq, Cs, _dev(st.get("n")), _dev(st.get("m")), gate=gate,
                                     Cq_out=Cq if inplace else None, Cs_out=Cs if inplace else None)
    torch.cuda.synchronize()
    return [_np(o) for o in out]


def _check_step(tag, x, st, gate, kind, gpu):
    h, Cq, Cs, n, m = gpu
    ref = recurrent_step_q8(x["q"], x["k"], x["v"], x["i"], x["f"], st.get("Cq"),
                            None if "Cs" not in st else st["Cs"].astype(np.float64),
                            st.get("n"), st.get("m"), gate=gate)
    herr = np.abs(h.astype(np.float64) - ref[0]).max()
    assert herr <= TOL_H[kind], f"{tag}: max|dh| {herr:.3g}"
    flips = check_codes(tag, Cq, Cs, ref[1])
    if gate == "exp":
        assert np.abs(n - ref[4]).max() / max(1.0, np.abs(ref[4]).max()) <= 1e-5
        assert np.abs(m - ref[5]).max() <= 1e-5
    return herr, flips


CASES = [
    ("exp_bf16_d256x512", dict(B=2, NH=3, DK=256, DV=512, kind="bf16", gate="exp")),
    ("sig_bf16_d256x512", dict(B=2, NH=3, DK=256, DV=512, kind="bf16", gate="sig")),
    ("exp_f32_d64x64", dict(B=1, NH=5, DK=64, DV=64, kind="f32", gate="exp")),
    ("exp_f32_d128x192", dict(B=3, NH=1, DK=128, DV=192, kind="f32", gate="exp")),
    ("exp_bf16_d512x320", dict(B=1, NH=2, DK=512, DV=320, kind="bf16", gate="exp")),
]


@pytest.mark.parametrize("name,c", CASES, ids=[s[0] for s in CASES])
def test_q8_step_against_oracle(mt, name, c):
    x, st = _draw(50 + CASES.index((name, c)), c["B"], c["NH"], c["DK"], c["DV"], c["kind"], c["gate"])
    herr, flips = _check_step(name, x, st, c["gate"], c["kind"], _step(mt, x, st, c["gate"], c["kind"]))
    print(f"\n[{name}] max|dh|={herr:.3g} codes at ties={flips}", flush=True)


def test_q8_zero_state_and_in_place(mt):
    x, st = _draw(60, 2, 2, 128, 256, "bf16", "exp", zero=True)
    _check_step("zero state", x, st, "exp", "bf16", _step(mt, x, st, "exp", "bf16"))
    x, st = _draw(61, 2, 2, 256, 128, "bf16", "exp")
    a = _step(mt, x, st, "exp", "bf16")
    b = _step(mt, x, st, "exp", "bf16", inplace=True)
    for u, w in zip(a, b):
        np.testing.assert_array_equal(u, w)


def test_q8_encode_decode(mt):
    rng = np.random.default_rng(62)
    C = (rng.standard_normal((2, 3, 64, 192)) * rng.uniform(1e-3, 1e2, (2, 3, 64, 1))).astype(np.float32)
    C[0, 0, 5] = 0.0                                         # an all-zero row
    Cq, Cs = mt.state_q8_encode(_dev(C))
    flips = check_codes("encode", _np(Cq), _np(Cs), C.astype(np.float64))
    back = _np(mt.state_q8_decode(Cq, Cs)).astype(np.float64)
    np.testing.assert_allclose(back, q8_decode(_np(Cq), from_lib(_np(Cs)).astype(np.float64)), rtol=1e-7, atol=0)
    assert np.all(back[0, 0, 5] == 0)
    print(f"\n[encode] codes at ties={flips}", flush=True)


@pytest.mark.parametrize("gate", ["exp", "sig"])
def test_q8_decode_continues_a_forward_pass(mt, gate):
    """Prefill with mlstm_chunkwise_fw, encode its final state, decode K
    tokens on the quantised state.  Each step is checked against the oracle
    step from the state the GPU held (so a tie decided differently does not
    carry over).  The drift of h from the unquantised float decode is the
    quantisation error itself, not a parity error: an element of a block is
    off by at most half a scale (amax / 254), about 0.7 % of a typical
    value's size as noise, and h sums such noise over DHQK rows much as it
    sums the signal, so the drift is bounded relative to the size of h: 5 %
    of max |h|."""
    B, NH, DK, DV, S0, K = 1, 2, 256, 256, 200, 6
    rng = np.random.default_rng(63)
    S = S0 + K
    q = round_to_bf16(rng.standard_normal((B, NH, S, DK)).astype(np.float32))[0]
    k = round_to_bf16(rng.standard_normal((B, NH, S, DK)).astype(np.float32))[0]
    v = round_to_bf16(rng.standard_normal((B, NH, S, DV)).astype(np.float32))[0]
    i_pre = rng.standard_normal((B, NH, S)).astype(np.float32)
    f_pre = (2.0 + 4.0 * rng.random((B, NH, S))).astype(np.float32)
    qd = torch.bfloat16
    H0, C, n, m = mt.mlstm_chunkwise_fw(_dev(q[:, :, :S0], qd), _dev(k[:, :, :S0], qd), _dev(v[:, :, :S0], qd),
                                        _dev(i_pre[:, :, :S0]), _dev(f_pre[:, :, :S0]), chunk_size=64, gate=gate)
    Cq, Cs = mt.state_q8_encode(C)
    full = recurrent_fw(*[a.astype(np.float64) for a in (q, k, v, i_pre, f_pre)], gate=gate)[0]
    worst, drift, hmax = 0.0, 0.0, 0.0
    for t in range(S0, S):
        x = dict(q=q[:, :, t], k=k[:, :, t], v=v[:, :, t], i=i_pre[:, :, t], f=f_pre[:, :, t])
        st = {"Cq": _np(Cq), "Cs": from_lib(_np(Cs))}
        if gate == "exp":
            st.update(n=_np(n), m=_np(m))
        h, Cq, Cs, n, m = mt.mlstm_recurrent_step_q8(*(_dev(x[a], qd) for a in ("q", "k", "v")), _dev(x["i"]),
                                                     _dev(x["f"]), Cq, Cs, n, m, gate=gate)
        torch.cuda.synchronize()
        herr, _ = _check_step(f"decode token {t}", x, st, gate, "bf16", [_np(h), _np(Cq), _np(Cs), _np(n), _np(m)])
        worst = max(worst, herr)
        drift = max(drift, np.abs(_np(h).astype(np.float64) - full[:, :, t]).max())
        hmax = max(hmax, np.abs(full[:, :, t]).max())
    print(f"\n[q8 decode {gate}] max|dh| vs oracle step={worst:.3g}, vs float decode={drift:.3g} "
          f"(max|h|={hmax:.3g}, relative {drift / hmax:.3g})", flush=True)
    assert drift <= 0.05 * hmax, f"quantised decode drifts {drift:.3g} from the float decode (max|h| {hmax:.3g})"


@pytest.mark.parametrize("gate", ["exp", "sig"])
def test_q8_step_full_size_sampled_heads(mt, gate):
    """7B-shaped heads (B=8, NH=8, DHQK=256, DHV=512): all heads on the GPU,
    the oracle on two of them."""
    B, NH, DK, DV = 8, 8, 256, 512
    x, st = _draw(64, B, NH, DK, DV, "bf16", gate)
    gpu = _step(mt, x, st, gate, "bf16")
    for (b, hd) in [(0, 0), (B - 1, NH - 1)]:
        xs = {n: a[b:b + 1, hd:hd + 1] for n, a in x.items()}
        ss = {n: a[b:b + 1, hd:hd + 1] for n, a in st.items()}
        g = [None if o is None else o[b:b + 1, hd:hd + 1] for o in gpu]
        _check_step(f"7B head {(b, hd)}", xs, ss, gate, "bf16", g)
