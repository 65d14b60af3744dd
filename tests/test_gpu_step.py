"""Parity of the recurrent step (decode) kernel against the float64 oracle
(needs an MI355X).

The reference for one step is the oracle's per-timestep recurrence run over a
one-token sequence from the given state; a decode run is the same recurrence
over the prefill plus the decoded tokens.  Inputs are seeded draws; Q, K, V
are rounded to bf16 (RNE) for the bf16 cases and both sides read the same
values.  Tolerances (max abs error): h 2e-2 (bf16 inputs) / 1e-4 (float32
inputs), the bounds of the forward pass; state C and n relative to
max(1, max|ref|) 1e-5, m 1e-5 (the step computes in float32 throughout).
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import recurrent_fw  # noqa: E402
from workloads import round_to_bf16  # noqa: E402

pytestmark = pytest.mark.gpu

TOL_H = {"bf16": 2e-2, "f32": 1e-4}
TOL_STATE = 1e-5


@pytest.fixture(scope="module")
def mt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import xlstm_mlstm_chunkwise_amd as m
    m.lib()
    return m


def _draw(seed, B, NH, DK, DV, kind, gate, with_state=True, S=1):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, NH, S, DK)).astype(np.float32)
    k = rng.standard_normal((B, NH, S, DK)).astype(np.float32)
    v = rng.standard_normal((B, NH, S, DV)).astype(np.float32)
    if kind == "bf16":
        q, k, v = (round_to_bf16(x)[0] for x in (q, k, v))
    i_pre = rng.standard_normal((B, NH, S)).astype(np.float32)
    f_pre = (2.0 + 4.0 * rng.random((B, NH, S))).astype(np.float32)
    st = {}
    if with_state:
        st["C"] = (0.1 * rng.standard_normal((B, NH, DK, DV))).astype(np.float32)
        if gate == "exp":
            st["n"] = rng.random((B, NH, DK)).astype(np.float32)
            st["m"] = rng.standard_normal((B, NH)).astype(np.float32)
    return dict(q=q, k=k, v=v, i=i_pre, f=f_pre), st


def _dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(device="cuda", dtype=dtype)


def _oracle(x, st, gate, t0=0, t1=None):
    """Recurrence over tokens t0..t1-1 from state st: (H, C, n, m)."""
    sl = slice(t0, t1)
    args = [x[n][:, :, sl].astype(np.float64) for n in ("q", "k", "v")]
    args += [x[n][:, :, sl].astype(np.float64) for n in ("i", "f")]
    C0 = st.get("C")
    n0 = st.get("n") if gate == "exp" else None
    m0 = st.get("m") if gate == "exp" else None
    return recurrent_fw(*args, C0, n0, m0, gate=gate)


def _step_gpu(mt, x, st, gate, t, kind, h_dtype=None, inplace=False):
    qd = torch.bfloat16 if kind == "bf16" else torch.float32
    q, k, v = (_dev(x[n][:, :, t], qd) for n in ("q", "k", "v"))
    i_pre, f_pre = _dev(x["i"][:, :, t], torch.float32), _dev(x["f"][:, :, t], torch.float32)
    C = _dev(st["C"], torch.float32) if "C" in st else None
    n = _dev(st["n"], torch.float32) if "n" in st else None
    m = _dev(st["m"], torch.float32) if "m" in st else None
    out = mt.mlstm_recurrent_step(q, k, v, i_pre, f_pre, C, n, m, gate=gate, h_dtype=h_dtype,
                                  C_out=C if (inplace and C is not None) else None)
    torch.cuda.synchronize()
    return [None if o is None else o.float().cpu().numpy().astype(np.float64) for o in out]


def _check(tag, kind, gate, gpu, ref, h_tol=None):
    h, C, n, m = gpu
    H, Cr, nr, mr = ref
    herr = np.abs(h - H[:, :, -1]).max()
    tol = TOL_H[kind] if h_tol is None else h_tol
    assert herr <= tol, f"{tag}: max|dh| = {herr:.3g} > {tol}"
    cerr = np.abs(C - Cr).max() / max(1.0, np.abs(Cr).max())
    assert cerr <= TOL_STATE, f"{tag}: C rel err {cerr:.3g}"
    if gate == "exp":
        nerr = np.abs(n - nr).max() / max(1.0, np.abs(nr).max())
        assert nerr <= TOL_STATE, f"{tag}: n rel err {nerr:.3g}"
        merr = np.abs(m - mr).max()
        assert merr <= TOL_STATE, f"{tag}: m err {merr:.3g}"
    return herr


STEP_CASES = [
    ("exp_bf16_d256x512", dict(B=2, NH=3, DK=256, DV=512, kind="bf16", gate="exp")),
    ("sig_bf16_d256x512", dict(B=2, NH=3, DK=256, DV=512, kind="bf16", gate="sig")),
    ("exp_f32_d64x64", dict(B=1, NH=5, DK=64, DV=64, kind="f32", gate="exp")),
    ("exp_f32_d128x192", dict(B=3, NH=1, DK=128, DV=192, kind="f32", gate="exp")),
    ("sig_f32_d256x128", dict(B=1, NH=2, DK=256, DV=128, kind="f32", gate="sig")),
    ("exp_bf16_d512x320", dict(B=1, NH=2, DK=512, DV=320, kind="bf16", gate="exp")),
]


@pytest.mark.parametrize("name,c", STEP_CASES, ids=[s[0] for s in STEP_CASES])
def test_step_against_oracle(mt, name, c):
    x, st = _draw(11, c["B"], c["NH"], c["DK"], c["DV"], c["kind"], c["gate"])
    gpu = _step_gpu(mt, x, st, c["gate"], 0, c["kind"])
    ref = _oracle(x, st, c["gate"])
    e = _check(name, c["kind"], c["gate"], gpu, ref)
    print(f"\n[{name}] max|dh|={e:.3g}", flush=True)


def test_step_with_eps(mt):
    x, st = _draw(16, 2, 2, 128, 128, "f32", "exp")
    qd = torch.float32
    out = mt.mlstm_recurrent_step(*(_dev(x[n][:, :, 0], qd) for n in ("q", "k", "v")), _dev(x["i"][:, :, 0], qd),
                                  _dev(x["f"][:, :, 0], qd), _dev(st["C"], qd), _dev(st["n"], qd),
                                  _dev(st["m"], qd), gate="exp", eps=0.25)
    torch.cuda.synchronize()
    gpu = [o.float().cpu().numpy().astype(np.float64) for o in out]
    args = [x[n][:, :, :1].astype(np.float64) for n in ("q", "k", "v", "i", "f")]
    ref = recurrent_fw(*args, st["C"], st["n"], st["m"], gate="exp", eps=0.25)
    _check("eps 0.25", "f32", "exp", gpu, ref)


def test_step_zero_state_in_place_and_bf16_h(mt):
    x, st = _draw(12, 2, 2, 128, 256, "bf16", "exp", with_state=False)
    gpu = _step_gpu(mt, x, st, "exp", 0, "bf16")
    _check("zero state", "bf16", "exp", gpu, _oracle(x, st, "exp"))
    # in place: C_out is the C_in buffer
    x, st = _draw(13, 2, 2, 256, 128, "bf16", "exp")
    a = _step_gpu(mt, x, st, "exp", 0, "bf16")
    b = _step_gpu(mt, x, st, "exp", 0, "bf16", inplace=True)
    for u, w in zip(a, b):
        np.testing.assert_array_equal(u, w)
    # bf16 h: the bound plus half a bf16 ulp of |h|
    h16 = _step_gpu(mt, x, st, "exp", 0, "bf16", h_dtype=torch.bfloat16)
    H = _oracle(x, st, "exp")[0][:, :, -1]
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(H), 1e-30))) - 8)
    assert np.all(np.abs(h16[0] - H) <= 2e-2 + ulp)


@pytest.mark.parametrize("gate", ["exp", "sig"])
def test_decode_continues_a_forward_pass(mt, gate):
    """Prefill S0 tokens with mlstm_chunkwise_fw, then decode K tokens with the
    step kernel from its final state: every decoded h and the final state
    match the oracle's recurrence over all S0 + K tokens."""
    B, NH, DK, DV, S0, K = 1, 2, 256, 256, 200, 6
    x, _ = _draw(14, B, NH, DK, DV, "bf16", gate, with_state=False, S=S0 + K)
    qd = torch.bfloat16
    q, k, v = (_dev(x[n][:, :, :S0], qd) for n in ("q", "k", "v"))
    i_pre, f_pre = _dev(x["i"][:, :, :S0], torch.float32), _dev(x["f"][:, :, :S0], torch.float32)
    H0, C, n, m = mt.mlstm_chunkwise_fw(q, k, v, i_pre, f_pre, chunk_size=64, gate=gate)
    ref_all = _oracle(x, {}, gate)
    worst = 0.0
    for t in range(S0, S0 + K):
        qt, kt, vt = (_dev(x[nm][:, :, t], qd) for nm in ("q", "k", "v"))
        it, ft = _dev(x["i"][:, :, t], torch.float32), _dev(x["f"][:, :, t], torch.float32)
        h, C, n, m = mt.mlstm_recurrent_step(qt, kt, vt, it, ft, C, n, m, gate=gate)
        torch.cuda.synchronize()
        err = np.abs(h.cpu().numpy().astype(np.float64) - ref_all[0][:, :, t]).max()
        worst = max(worst, err)
        assert err <= TOL_H["bf16"], f"decode token {t}: max|dh| = {err:.3g}"
    Cr = ref_all[1]
    cerr = np.abs(C.cpu().numpy().astype(np.float64) - Cr).max() / max(1.0, np.abs(Cr).max())
    assert cerr <= 1e-3, f"final C rel err {cerr:.3g}"
    if gate == "exp":
        assert np.abs(m.cpu().numpy() - ref_all[3]).max() <= 1e-3
    print(f"\n[decode {gate}] max|dh|={worst:.3g}", flush=True)


@pytest.mark.parametrize("gate", ["exp", "sig"])
def test_step_full_size_sampled_heads(mt, gate):
    """The 7B-shaped heads (B=8, NH=8, DHQK=256, DHV=512), all heads on the
    GPU, the oracle on two of them."""
    B, NH, DK, DV = 8, 8, 256, 512
    x, st = _draw(15, B, NH, DK, DV, "bf16", gate)
    gpu = _step_gpu(mt, x, st, gate, 0, "bf16")
    worst = 0.0
    for (b, hd) in [(0, 0), (B - 1, NH - 1)]:
        xs = {n: a[b:b + 1, hd:hd + 1] for n, a in x.items()}
        ss = {n: a[b:b + 1, hd:hd + 1] for n, a in st.items()}
        ref = _oracle(xs, ss, gate)
        g = [None if o is None else o[b:b + 1, hd:hd + 1] for o in gpu]
        worst = max(worst, _check(f"full size head {(b, hd)}", "bf16", gate, g, ref))
    print(f"\n[step 7B {gate}] max|dh|={worst:.3g}", flush=True)
