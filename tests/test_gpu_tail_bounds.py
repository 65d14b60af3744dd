"""Reads and writes stay inside each head's rows on a ragged last chunk (needs
an MI355X).

Every input tensor is passed as a contiguous view at the start of a larger
allocation whose elements after the last head's S rows are NaN, so a kernel
that read a row past the sequence end would read NaN from memory it owns
(and carry it into H or the states: a zero weight does not clear a NaN).
H is written into a view of a larger buffer pre-filled with a sentinel; the
sentinel must survive, so no store landed past the last row.  The outputs
are compared with the float64 oracle at the usual bounds.

The kernels covered are the ones that address their rows through buffer
resources: the wide states and intra-chunk kernels (both tile heights), the
fused walker, and the backward's state-gradient kernel (Q and dH); the
generic and float64 kernels, which check every row explicitly, run too.
bf16 H, which the walker and the wide intra-chunk kernel store as pairs of
adjacent columns after a lane exchange, is checked the same way and value for
value against the float32 H of the same call, rounded to bf16.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import grad_fw, recurrent_fw  # noqa: E402
from workloads import WORKLOADS, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu

PAD_ROWS = 1024          # at least one chunk of rows past the last head
SENTINEL = 12345.0


@pytest.fixture(scope="module")
def mt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import xlstm_mlstm_chunkwise_amd as m
    m.lib()
    return m


def _nan_tail(a, dtype, row_elems):
    """`a` on the GPU as the first elements of an allocation continued by NaN."""
    flat = torch.full((a.size + PAD_ROWS * row_elems,), float("nan"), dtype=dtype, device="cuda")
    flat[:a.size] = torch.from_numpy(np.ascontiguousarray(a).reshape(-1)).to(device="cuda", dtype=dtype)
    return flat[:a.size].view(a.shape)


def _sentinel_out(shape, dtype, row_elems):
    n = int(np.prod(shape))
    flat = torch.full((n + PAD_ROWS * row_elems,), SENTINEL, dtype=dtype, device="cuda")
    return flat, flat[:n].view(shape)


def _workload(**over):
    base = WORKLOADS["bf16_s2048_d128"].replace(i_spike_prob=0.0, i_dist=("normal", 0.0, 1.0),
                                                 tile_lq=0, tile_lkv=0, seed=91)
    return base.replace(**over)


FORWARD = [
    # name, workload overrides, schedule
    ("wide_exp_tq64", dict(B=1, NH=2, S=300, DHQK=256, DHV=512, chunk=256), "two_stage"),
    ("wide_sig_tq64", dict(gate="sig", B=1, NH=2, S=300, DHQK=256, DHV=512, chunk=256), "two_stage"),
    ("wide_exp_tq128", dict(B=1, NH=2, S=700, DHQK=256, DHV=512, chunk=256, tile_lq=128, tile_lkv=128),
     "two_stage"),
    ("wide_exp_d128_v256_init", dict(B=1, NH=2, S=333, DHQK=128, DHV=256, chunk=128, init_state=True),
     "two_stage"),
    ("rows_exp_many_heads", dict(B=4, NH=8, S=300, DHQK=256, DHV=512, chunk=128), "two_stage"),
    ("segments_exp", dict(B=2, NH=4, S=620, DHQK=256, DHV=512, chunk=64, init_state=True), "two_stage"),
    ("fused_exp", dict(B=1, NH=2, S=300, DHQK=256, DHV=512, chunk=256), "fused"),
    ("fused_sig_init", dict(gate="sig", B=1, NH=2, S=333, DHQK=256, DHV=256, chunk=128, init_state=True),
     "fused"),
    ("generic_bf16", dict(B=1, NH=2, S=200, DHQK=64, DHV=128, chunk=64), "two_stage"),
    ("generic_f32", dict(qkv_dtype="f32", B=1, NH=2, S=200, DHQK=64, DHV=128, chunk=64), "two_stage"),
]


@pytest.mark.parametrize("name,over,schedule", FORWARD, ids=[c[0] for c in FORWARD])
def test_forward_ragged_tail_reads_nothing_past_the_rows(mt, name, over, schedule):
    w = _workload(**over)
    x = make_inputs(w)
    qd = torch.bfloat16 if w.qkv_dtype == "bf16" else torch.float32
    DK, DV = w.DHQK, w.DHV
    q, k = _nan_tail(x["q"], qd, DK), _nan_tail(x["k"], qd, DK)
    v = _nan_tail(x["v"], qd, DV)
    i_pre, f_pre = _nan_tail(x["i"], torch.float32, 1), _nan_tail(x["f"], torch.float32, 1)
    st = {}
    if w.init_state:
        st["C0"] = _nan_tail(x["C0"], torch.float32, DV)
        if w.gate == "exp":
            st["n0"] = _nan_tail(x["n0"], torch.float32, 1)
            st["m0"] = _nan_tail(x["m0"], torch.float32, 1)
    Hflat, H = _sentinel_out((w.B, w.NH, w.S, DV), torch.float32, DV)
    print(f"\n[{name}] schedule {schedule}", flush=True)
    _, C, n, m = mt.mlstm_chunkwise_fw(q, k, v, i_pre, f_pre, st.get("C0"), st.get("n0"), st.get("m0"),
                                       chunk_size=w.chunk, gate=w.gate, tile_lq=w.tile_lq, tile_lkv=w.tile_lkv,
                                       schedule=schedule, out=H)
    torch.cuda.synchronize()
    tail = Hflat[H.numel():].cpu().numpy()
    assert np.all(tail == SENTINEL), f"{name}: H stores past the last row ({np.sum(tail != SENTINEL)} values)"
    Hg = H.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(Hg)), f"{name}: non-finite H"
    tol = 2e-2 if w.qkv_dtype == "bf16" else 1e-4
    for b in range(w.B):
        for h in range(w.NH):
            args = [x[nm][b, h].astype(np.float64) for nm in ("q", "k", "v", "i", "f")]
            r = recurrent_fw(*args, x["C0"][b, h] if w.init_state else None,
                             x["n0"][b, h] if (w.init_state and w.gate == "exp") else None,
                             x["m0"][b, h] if (w.init_state and w.gate == "exp") else None, gate=w.gate)
            err = np.abs(Hg[b, h] - r[0]).max()
            assert err <= tol, f"{name} head {(b, h)}: max|dH| {err:.3g}"
            Cg = C.cpu().numpy()[b, h]
            assert np.all(np.isfinite(Cg))
            assert np.abs(Cg - r[1]).max() / max(1.0, np.abs(r[1]).max()) <= 1e-3
            if w.gate == "exp":
                assert np.isfinite(m.cpu().numpy()[b, h]) and abs(m.cpu().numpy()[b, h] - r[3]) <= 1e-3
                assert np.abs(n.cpu().numpy()[b, h] - r[2]).max() / max(1.0, np.abs(r[2]).max()) <= 1e-3


BF16_H = [
    # name, workload overrides, schedule
    ("fused_exp_bf16h", dict(B=1, NH=2, S=300, DHQK=256, DHV=512, chunk=256), "fused"),
    ("fused_sig_bf16h_init", dict(gate="sig", B=1, NH=2, S=333, DHQK=256, DHV=256, chunk=128, init_state=True),
     "fused"),
    ("wide_exp_tq64_bf16h", dict(B=1, NH=2, S=300, DHQK=256, DHV=512, chunk=256), "two_stage"),
    ("wide_exp_tq128_bf16h", dict(B=1, NH=2, S=700, DHQK=256, DHV=512, chunk=256, tile_lq=128, tile_lkv=128),
     "two_stage"),
    ("generic_bf16h", dict(B=1, NH=2, S=200, DHQK=64, DHV=128, chunk=64), "two_stage"),
]


@pytest.mark.parametrize("name,over,schedule", BF16_H, ids=[c[0] for c in BF16_H])
def test_bf16_h_is_the_rounded_float32_h_and_stays_in_the_rows(mt, name, over, schedule):
    """bf16 H (lane pairs swap values and store two adjacent columns of a
    row as one word in the walker and the wide intra-chunk kernel) is, value
    for value, the round-to-nearest-even bf16 of the float32 H of the same
    call, and no store lands past the last row."""
    w = _workload(**over)
    x = make_inputs(w)
    DK, DV = w.DHQK, w.DHV
    q, k = _nan_tail(x["q"], torch.bfloat16, DK), _nan_tail(x["k"], torch.bfloat16, DK)
    v = _nan_tail(x["v"], torch.bfloat16, DV)
    i_pre, f_pre = _nan_tail(x["i"], torch.float32, 1), _nan_tail(x["f"], torch.float32, 1)
    st = {}
    if w.init_state:
        st["C0"] = _nan_tail(x["C0"], torch.float32, DV)
        if w.gate == "exp":
            st["n0"] = _nan_tail(x["n0"], torch.float32, 1)
            st["m0"] = _nan_tail(x["m0"], torch.float32, 1)
    shape = (w.B, w.NH, w.S, DV)
    outs = {}
    for dt in (torch.float32, torch.bfloat16):
        flat, H = _sentinel_out(shape, dt, DV)
        print(f"\n[{name}] schedule {schedule}, H {dt}", flush=True)
        mt.mlstm_chunkwise_fw(q, k, v, i_pre, f_pre, st.get("C0"), st.get("n0"), st.get("m0"),
                              chunk_size=w.chunk, gate=w.gate, tile_lq=w.tile_lq, tile_lkv=w.tile_lkv,
                              schedule=schedule, h_dtype=dt, out=H)
        torch.cuda.synchronize()
        tail = flat[H.numel():].cpu()
        sent = torch.full_like(tail, SENTINEL)
        assert torch.equal(tail, sent), f"{name}: {dt} H stores past the last row"
        outs[dt] = H.cpu()
    want = outs[torch.float32].to(torch.bfloat16).view(torch.int16)
    got = outs[torch.bfloat16].view(torch.int16)
    bad = int((want != got).sum())
    assert bad == 0, f"{name}: {bad} bf16 H values differ from the rounded float32 H"
    r = recurrent_fw(*[x[nm][0, 0].astype(np.float64) for nm in ("q", "k", "v", "i", "f")],
                     x["C0"][0, 0] if w.init_state else None,
                     x["n0"][0, 0] if (w.init_state and w.gate == "exp") else None,
                     x["m0"][0, 0] if (w.init_state and w.gate == "exp") else None, gate=w.gate)
    err = np.abs(outs[torch.float32].numpy()[0, 0].astype(np.float64) - r[0]).max()
    assert err <= 2e-2, f"{name}: float32 H max|dH| {err:.3g}"


BACKWARD = [
    # name, B, NH, S, DK, DV, L, gate, dH dtype
    ("bw_exp_d256x512_f32dh", 1, 2, 300, 256, 512, 256, "exp", torch.float32),
    ("bw_exp_d256x512_bf16dh", 1, 2, 300, 256, 512, 128, "exp", torch.bfloat16),
    ("bw_sig_d128x256_f32dh", 1, 2, 200, 128, 256, 64, "sig", torch.float32),
]


@pytest.mark.parametrize("c", BACKWARD, ids=[c[0] for c in BACKWARD])
def test_backward_ragged_tail_reads_nothing_past_the_rows(mt, c):
    name, B, NH, S, DK, DV, L, gate, dhd = c
    rng = np.random.default_rng(1234 + BACKWARD.index(c))
    from workloads import round_to_bf16
    x = dict(q=round_to_bf16(rng.standard_normal((B, NH, S, DK)).astype(np.float32))[0],
             k=round_to_bf16(rng.standard_normal((B, NH, S, DK)).astype(np.float32))[0],
             v=round_to_bf16(rng.standard_normal((B, NH, S, DV)).astype(np.float32))[0],
             i=rng.standard_normal((B, NH, S)).astype(np.float32),
             f=(2.0 + 4.0 * rng.random((B, NH, S))).astype(np.float32),
             dH=rng.standard_normal((B, NH, S, DV)).astype(np.float32))
    if dhd == torch.bfloat16:
        x["dH"] = round_to_bf16(x["dH"])[0]
    print(f"\n[{name}]", flush=True)
    g = mt.mlstm_chunkwise_bw(_nan_tail(x["q"], torch.bfloat16, DK), _nan_tail(x["k"], torch.bfloat16, DK),
                              _nan_tail(x["v"], torch.bfloat16, DV), _nan_tail(x["i"], torch.float32, 1),
                              _nan_tail(x["f"], torch.float32, 1), _nan_tail(x["dH"], dhd, DV),
                              chunk_size=L, gate=gate, state_grads=True)
    torch.cuda.synchronize()
    f64 = {n: a.astype(np.float64) for n, a in x.items()}
    r = grad_fw(f64["q"], f64["k"], f64["v"], f64["i"], f64["f"], f64["dH"], gate=gate)
    for key in ("dQ", "dK", "dV", "d_i", "d_f", "dC0"):
        gk = g[key].cpu().numpy().astype(np.float64)
        assert np.all(np.isfinite(gk)), f"{name}: non-finite {key}"
        err = np.abs(gk - r[key]).max() / max(1.0, np.abs(r[key]).max())
        assert err <= 1e-3, f"{name}: {key} rel err {err:.3g}"
