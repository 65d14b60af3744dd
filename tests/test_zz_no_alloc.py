"""The allocation-free forward entry point (mlstm_chunkwise_fw_noalloc, its
workspace a static device array of the library) against the workspace entry
point mlstm_chunkwise_fw on the same inputs (needs an MI355X).

Both run the same kernels on the same inputs, so their outputs must be
bitwise equal; the oracle bounds of the forward parity tests apply as well.
Each case makes two calls in a row on the static array, the second with a
smaller problem, so a result that depended on what the first call left there
would show.  Outputs are allocated before the calls; torch's allocator must
not grow during them.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from f32_chunkwise import accumulation_bound  # noqa: E402
from oracle import recurrent_fw  # noqa: E402
from workloads import WORKLOADS, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mt():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import xlstm_mlstm_chunkwise_amd as m
    m.lib()
    return m


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device="cuda", dtype=dtype)


def _inputs(w):
    x = make_inputs(w)
    qd = torch.bfloat16 if w.qkv_dtype == "bf16" else torch.float32
    d = dict(q=_dev(x["q"], qd), k=_dev(x["k"], qd), v=_dev(x["v"], qd), i=_dev(x["i"], torch.float32),
             f=_dev(x["f"], torch.float32))
    if w.init_state:
        d["C0"] = _dev(x["C0"], torch.float32)
        if w.gate == "exp":
            d["n0"], d["m0"] = _dev(x["n0"], torch.float32), _dev(x["m0"], torch.float32)
    return x, d


def _outputs(w):
    f32 = dict(dtype=torch.float32, device="cuda")
    o = dict(H=torch.empty((w.B, w.NH, w.S, w.DHV), **f32), C=torch.empty((w.B, w.NH, w.DHQK, w.DHV), **f32))
    if w.gate == "exp":
        o["n"], o["m"] = torch.empty((w.B, w.NH, w.DHQK), **f32), torch.empty((w.B, w.NH), **f32)
    return o


def _workload(**over):
    return WORKLOADS["bf16_s2048_d128"].replace(i_spike_prob=0.0, i_dist=("normal", 0.0, 1.0), tile_lq=0,
                                                tile_lkv=0, seed=23).replace(**over)


PAIRS = [
    # name, first call, second (smaller) call, schedule
    ("walker_exp", dict(B=2, NH=4, S=1000, DHQK=256, DHV=512, chunk=256, init_state=True),
     dict(B=1, NH=2, S=300, DHQK=256, DHV=256, chunk=128), "auto"),
    ("walker_sig", dict(gate="sig", B=2, NH=2, S=700, DHQK=256, DHV=512, chunk=256),
     dict(gate="sig", B=1, NH=1, S=130, DHQK=256, DHV=128, chunk=64, init_state=True), "auto"),
    ("two_stage_wide", dict(B=1, NH=4, S=600, DHQK=256, DHV=512, chunk=128, init_state=True),
     dict(B=1, NH=2, S=200, DHQK=128, DHV=256, chunk=64), "two_stage"),
    ("two_stage_generic_f32", dict(qkv_dtype="f32", B=2, NH=2, S=400, DHQK=128, DHV=128, chunk=128),
     dict(qkv_dtype="f32", B=1, NH=1, S=90, DHQK=64, DHV=64, chunk=64, init_state=True), "two_stage"),
    # int16-coded chunk states on the static array
    ("two_stage_int16", dict(B=1, NH=4, S=600, DHQK=256, DHV=512, chunk=128, init_state=True),
     dict(gate="sig", B=1, NH=2, S=200, DHQK=128, DHV=256, chunk=64), "two_stage:int16"),
]


def _check_against_oracle(w, x, o, tag):
    tol = 2e-2 if w.qkv_dtype == "bf16" else 1e-4
    H = o["H"].cpu().numpy().astype(np.float64)
    for b in range(w.B):
        for h in range(w.NH):
            args = [x[nm][b, h].astype(np.float64) for nm in ("q", "k", "v", "i", "f")]
            init = [x[nm][b, h] if (w.init_state and (nm == "C0" or w.gate == "exp")) else None
                    for nm in ("C0", "n0", "m0")]
            r = recurrent_fw(*args, *init, gate=w.gate, return_rows=w.gate == "exp")
            err = np.abs(H[b, h] - r[0])
            bound = tol
            if w.qkv_dtype == "f32":
                # float32 accumulation bound from the row's conditioning
                bound = accumulation_bound(*[x[nm][b, h] for nm in ("q", "k", "v", "i", "f")], *init,
                                           chunk_size=w.chunk, gate=w.gate, H_ref=r[0],
                                           m_rows=r[4] if w.gate == "exp" else None,
                                           den_rows=r[5] if w.gate == "exp" else None)[0]
            assert np.all(err <= bound), f"{tag} head {(b, h)}: max|dH| {err.max():.3g}"


@pytest.mark.parametrize("name,first,second,schedule", PAIRS, ids=[p[0] for p in PAIRS])
def test_noalloc_matches_workspace_entry_point(mt, name, first, second, schedule):
    schedule, _, codes = schedule.partition(":")
    codes = codes or "split"
    runs = []
    for over in (first, second):
        w = _workload(**over)
        x, d = _inputs(w)
        o, o_ref = _outputs(w), _outputs(w)
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        print(f"\n[{name}] noalloc call B={w.B} NH={w.NH} S={w.S} DHQK={w.DHQK} DHV={w.DHV} L={w.chunk}",
              flush=True)
        mt.mlstm_chunkwise_fw_noalloc(d["q"], d["k"], d["v"], d["i"], d["f"], d.get("C0"), d.get("n0"),
                                      d.get("m0"), chunk_size=w.chunk, gate=w.gate, schedule=schedule,
                                      state_codes=codes, out=o["H"], C_out=o["C"], n_out=o.get("n"),
                                      m_out=o.get("m"))
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        runs.append((w, x, d, o, o_ref))
    for w, x, d, o, o_ref in runs:
        H, C, n, m = mt.mlstm_chunkwise_fw(d["q"], d["k"], d["v"], d["i"], d["f"], d.get("C0"), d.get("n0"),
                                           d.get("m0"), chunk_size=w.chunk, gate=w.gate, schedule=schedule,
                                           state_codes=codes)
        torch.cuda.synchronize()
        assert torch.equal(o["H"], H), f"{name}: H differs from the workspace entry point"
        assert torch.equal(o["C"], C)
        if w.gate == "exp":
            assert torch.equal(o["n"], n) and torch.equal(o["m"], m)
        _check_against_oracle(w, x, o, name)


def test_noalloc_refuses_a_workspace_beyond_the_static_array(mt):
    # the two-stage kernels at the 7B-shaped heads need 1.1 GB of chunk states
    w = WORKLOADS["bf16_7b_s8192"].replace(B=1, NH=8)
    d = mt.make_desc(w.B, w.NH, w.S, w.DHQK, w.DHV, w.chunk, schedule="two_stage")
    assert mt.workspace_bytes(d) > mt.NOALLOC_WORKSPACE_BYTES
    q = torch.zeros((w.B, w.NH, w.S, w.DHQK), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((w.B, w.NH, w.S, w.DHV), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((w.B, w.NH, w.S), dtype=torch.float32, device="cuda")
    H = torch.full((w.B, w.NH, w.S, w.DHV), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(mt.MlstmError) as e:
        mt.mlstm_chunkwise_fw_noalloc(q, q, v, g, g, chunk_size=w.chunk, schedule="two_stage", out=H)
    assert e.value.status == 6
    torch.cuda.synchronize()
    assert bool(torch.all(H == 7.0))      # nothing was launched
    # the automatic schedule runs the walker there, which needs no workspace
    mt.mlstm_chunkwise_fw_noalloc(q, q, v, g, g, chunk_size=w.chunk, out=H)
    torch.cuda.synchronize()
    assert bool(torch.all(H == 0.0))      # zero keys and values give zero H
