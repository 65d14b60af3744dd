"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects invalid arguments before any device work.

No test here launches a kernel: every call is one that validation refuses,
so these run on a machine without a GPU.
"""
import ctypes
import os
import re
import subprocess

import pytest

import xlstm_mlstm_chunkwise_amd as mt

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlstm_tfla.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlstm_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    for n in ("mlstm_chunkwise_fw", "mlstm_fw_states", "mlstm_fw_hintra", "mlstm_fw_unpack_states"):
        assert n in names
    out = subprocess.run(["nm", "-D", "--defined-only", mt.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    lib = mt.lib()
    for n in names:
        assert getattr(lib, n) is not None


def _declared_prototypes():
    """name -> list of parameter declarations, from the header's prototypes."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = {}
    for m in re.finditer(r"\b(mlstm_[a-z0-9_]+)\s*\(([^;{]*?)\)\s*;", text):
        params = [p.strip() for p in m.group(2).replace("\n", " ").split(",")]
        protos[m.group(1)] = [] if params == ["void"] or params == [""] else params
    return protos


def test_binding_signatures_match_the_header():
    """Every binding's argument count equals the prototype's, pointer
    parameters are passed as pointers and size_t as size_t."""
    protos = _declared_prototypes()
    assert set(protos) == set(_declared_functions())
    for name, (restype, argtypes) in mt._SYMBOLS.items():
        params = protos[name]
        assert len(argtypes) == len(params), (name, len(argtypes), len(params))
        for decl, at in zip(params, argtypes):
            if "*" in decl:
                assert at in (ctypes.c_void_p, ctypes.c_char_p) or issubclass(at, ctypes._Pointer), (name, decl)
            elif decl.startswith("size_t"):
                assert at is ctypes.c_size_t, (name, decl)
            else:
                assert at in (ctypes.c_int, ctypes.c_int32), (name, decl)
    assert set(mt._SYMBOLS) == set(protos), set(protos) ^ set(mt._SYMBOLS)


def test_abi_version_and_status_strings():
    assert mt.abi_version() == 11
    assert mt.status_str(0) == "ok"
    for code in range(1, 10):
        assert mt.status_str(code) not in ("ok", "unknown status")
    assert mt.status_str(999) == "unknown status"


def test_desc_layout_matches_header():
    # 17 int/float fields plus reserved, all 4 bytes
    assert ctypes.sizeof(mt.FwDesc) == 18 * 4
    assert mt.FwDesc.schedule.offset == 14 * 4
    assert mt.FwDesc.block_chunks.offset == 15 * 4
    assert mt.FwDesc.state_codes.offset == 16 * 4


def _desc(**kw):
    base = dict(B=2, NH=3, S=1000, DHQK=128, DHV=64, chunk_size=128)
    base.update({k: kw.pop(k) for k in list(kw) if k in base})
    return mt.make_desc(base["B"], base["NH"], base["S"], base["DHQK"], base["DHV"],
                        base["chunk_size"], **kw)


def test_valid_descriptor_and_workspace_size():
    d = _desc()
    assert mt.validate(d) == 0
    Nc = (1000 + 127) // 128
    assert mt.num_chunks(d) == Nc
    def r256(x):
        return (x + 255) // 256 * 256
    BH = 6
    expect = r256(BH * (Nc + 1) * 128 * 64 * 4) + r256(BH * (Nc + 1) * 128 * 4) + r256(BH * (Nc + 1) * 4)
    assert mt.workspace_bytes(d) == expect
    ds = _desc(gate="sig")
    assert mt.workspace_bytes(ds) == r256(BH * (Nc + 1) * 128 * 64 * 4)
    # wide-tile family: regions of per-position gate terms and of the
    # stabilisers of segment-local state runs
    dw = _desc(DHQK=256, DHV=512, chunk_size=256)
    Ncw = (1000 + 255) // 256
    expect_w = (r256(BH * (Ncw + 1) * 256 * 512 * 4) + r256(BH * (Ncw + 1) * 256 * 4) + r256(BH * (Ncw + 1) * 4)
                + r256(BH * 1000 * 4 * 3) + r256(BH * (Ncw + 1) * 4))
    assert mt.workspace_bytes(dw) == expect_w
    dws = _desc(DHQK=256, DHV=512, chunk_size=256, gate="sig")
    assert mt.workspace_bytes(dws) == (r256(BH * (Ncw + 1) * 256 * 512 * 4) + r256(BH * 1000 * 4 * 2)
                                       + r256(BH * (Ncw + 1) * 4))
    assert mt.validate(_desc(S=0)) == 0
    assert mt.num_chunks(_desc(S=0)) == 0
    # the longest head the 32-bit buffer offsets allow
    assert mt.validate(_desc(S=(1 << 20) - 1, DHQK=64, DHV=512)) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 2), (dict(NH=-1), 2), (dict(S=-5), 2),
    (dict(S=1 << 20, DHQK=64, DHV=512), 2), (dict(S=1 << 21, DHQK=256, DHV=256), 2),
    (dict(DHQK=96), 2), (dict(DHQK=1024), 2), (dict(DHV=32), 2), (dict(DHV=576), 2),
    (dict(chunk_size=96), 3), (dict(chunk_size=8), 3), (dict(chunk_size=2048), 3),
    (dict(tile_lq=48), 3), (dict(tile_lkv=256), 3),
    (dict(qkv_dtype=7), 4), (dict(h_dtype=-1), 4),
    (dict(gate=2), 9), (dict(precision=5), 9), (dict(eps=-1.0), 9), (dict(eps=float("nan")), 9),
    (dict(qk_scale=float("inf")), 9),
    (dict(qkv_dtype=mt.MLSTM_F32, DHQK=512), 5),
])
def test_validation_errors(kw, code):
    d = _desc(**kw)
    assert mt.validate(d) == code
    assert mt.workspace_bytes(d) == 0
    assert mt.num_chunks(d) == -1


def test_reserved_fields_must_be_zero():
    d = _desc()
    d.reserved = 1
    assert mt.validate(d) == 9
    d = _desc()
    d.state_codes = 2
    assert mt.validate(d) == 9
    d = _desc()
    d.block_chunks = -1
    assert mt.validate(d) == 9


def _fw(desc, **ptrs):
    names = ["Q", "K", "V", "i", "f", "C0", "n0", "m0", "H", "C_out", "n_out", "m_out"]
    vals = [ptrs.get(n, 4096) for n in names]
    ws = ptrs.get("ws", 1 << 20)
    ws_bytes = ptrs.get("ws_bytes", mt.workspace_bytes(desc) if desc is not None else 0)
    return mt.lib().mlstm_chunkwise_fw(ctypes.byref(desc) if desc is not None else None, *vals, ws, ws_bytes, None)


def test_entry_points_refuse_before_launch():
    lib = mt.lib()
    d = _desc()
    assert _fw(None) == 1
    assert _fw(d, Q=None) == 1
    assert _fw(d, H=None) == 1
    assert _fw(d, K=4096 + 8) == 8           # Q/K/V/H need 16-byte alignment
    assert _fw(d, i=4096 + 2) == 8
    assert _fw(d, ws=None) == 6
    assert _fw(d, ws_bytes=mt.workspace_bytes(d) - 1) == 6
    assert _fw(d, ws=(1 << 20) + 64) == 6    # workspace needs 256-byte alignment
    ds = _desc(gate="sig")
    assert _fw(ds, C0=None, n0=4096, m0=None, n_out=None, m_out=None) == 5
    assert _fw(ds, C0=None, n0=None, m0=None, n_out=None, m_out=4096) == 5
    bad = _desc(DHQK=100)
    assert _fw(bad) == 2
    # stage calls
    wsb = mt.workspace_bytes(d)
    assert lib.mlstm_fw_states(ctypes.byref(d), *([4096] * 7), None, wsb, None, None, None, None) == 6
    assert lib.mlstm_fw_states(ctypes.byref(d), None, *([4096] * 6), 1 << 20, wsb, None, None, None, None) == 1
    assert lib.mlstm_fw_states(ctypes.byref(ds), *([4096] * 5), 4096, None, 1 << 20, wsb, None, None, None,
                               None) == 5
    assert lib.mlstm_fw_hintra(ctypes.byref(d), *([4096] * 5), 1 << 20, wsb, None, None, None, None) == 1
    assert lib.mlstm_fw_hintra(ctypes.byref(ds), *([4096] * 5), 1 << 20, wsb, 4096, 4096, None, None) == 5
    assert lib.mlstm_fw_hintra(ctypes.byref(d), *([4096] * 5), 1 << 20, wsb - 1, 4096, None, None, None) == 6
    assert lib.mlstm_fw_unpack_states(ctypes.byref(ds), 1 << 20, wsb, None, 4096, None, None) == 5
    assert lib.mlstm_fw_unpack_states(ctypes.byref(d), None, wsb, 4096, None, None, None) == 6


def test_kernel_family_query():
    # the automatic schedule takes the fused walker where it covers the shape
    assert mt.kernel_family(_desc(DHQK=256, DHV=512, chunk_size=256)) == mt.MLSTM_FAMILY_FUSED
    assert mt.kernel_family(_desc(DHQK=256, DHV=512, chunk_size=256, schedule="two_stage")) == mt.MLSTM_FAMILY_WIDE
    assert mt.kernel_family(_desc(DHQK=128, DHV=256, chunk_size=128)) == mt.MLSTM_FAMILY_WIDE
    assert mt.kernel_family(_desc(DHQK=256, DHV=512, chunk_size=1024, tile_lq=128)) == mt.MLSTM_FAMILY_WIDE
    assert mt.kernel_family(_desc(DHQK=128, DHV=128, chunk_size=128)) == mt.MLSTM_FAMILY_GENERIC
    assert mt.kernel_family(_desc(DHQK=64, DHV=64, chunk_size=64, qkv_dtype=mt.MLSTM_F32)) == mt.MLSTM_FAMILY_GENERIC
    assert mt.kernel_family(_desc(DHQK=256, DHV=512, chunk_size=256, qkv_dtype=mt.MLSTM_F32)) == mt.MLSTM_FAMILY_GENERIC
    assert mt.kernel_family(_desc(DHQK=256, DHV=512, chunk_size=256, precision="f64")) == mt.MLSTM_FAMILY_F64
    assert mt.kernel_family(_desc(DHQK=100)) == -2


def test_schedule_field():
    # the fused walker covers bf16, DHQK 256, DHV a multiple of 128, chunk <=
    # 512; the automatic schedule takes it there unless tile sizes are given
    big = dict(B=8, NH=8, S=8192, DHQK=256, DHV=512, chunk_size=256)
    assert mt.kernel_family(_desc(**big)) == mt.MLSTM_FAMILY_FUSED
    assert mt.kernel_family(_desc(**big, tile_lq=64)) == mt.MLSTM_FAMILY_WIDE
    assert mt.kernel_family(_desc(**big, tile_lkv=64)) == mt.MLSTM_FAMILY_WIDE
    assert mt.kernel_family(_desc(**dict(big, chunk_size=1024))) == mt.MLSTM_FAMILY_WIDE
    assert mt.kernel_family(_desc(**dict(big, DHQK=128))) == mt.MLSTM_FAMILY_WIDE
    assert mt.kernel_family(_desc(**big, schedule="two_stage")) == mt.MLSTM_FAMILY_WIDE
    assert mt.kernel_family(_desc(**big, schedule="fused")) == mt.MLSTM_FAMILY_FUSED
    assert mt.kernel_family(_desc(**big, gate="sig", schedule="fused")) == mt.MLSTM_FAMILY_FUSED
    assert mt.kernel_family(_desc(**dict(big, B=1, NH=1, DHV=128), schedule="fused")) == mt.MLSTM_FAMILY_FUSED
    assert mt.kernel_family(_desc(**big, precision="f64")) == mt.MLSTM_FAMILY_F64
    # a forced fused schedule on a shape it does not cover, and unknown values
    assert mt.validate(_desc(**dict(big, DHQK=128), schedule="fused")) == 5
    assert mt.validate(_desc(**dict(big, chunk_size=1024), schedule="fused")) == 5
    assert mt.validate(_desc(**big, qkv_dtype=mt.MLSTM_F32, schedule="fused")) == 5
    assert mt.validate(_desc(**big, schedule=4)) == 9
    assert mt.validate(_desc(**big, schedule=-1)) == 9
    # workspace: the fused schedule needs none (the walker forms its own gate
    # terms); auto keeps room for the two-stage kernels, which the stage-wise
    # calls run for an auto descriptor
    fused = _desc(**big, schedule="fused")
    assert mt.workspace_bytes(fused) == 0
    assert mt.workspace_bytes(_desc(**big, gate="sig", schedule="fused")) == 0
    auto = mt.workspace_bytes(_desc(**big))
    assert auto == mt.workspace_bytes(_desc(**big, schedule="two_stage"))
    assert auto > 64 * 33 * 256 * 512 * 4
    # the stage-wise calls refuse a fused descriptor before touching pointers
    lib = mt.lib()
    wsb = mt.workspace_bytes(fused)
    assert lib.mlstm_fw_states(ctypes.byref(fused), *([4096] * 7), 1 << 20, wsb, None, None, None, None) == 5
    assert lib.mlstm_fw_hintra(ctypes.byref(fused), *([4096] * 5), 1 << 20, wsb, 4096, None, None, None) == 5
    assert lib.mlstm_fw_unpack_states(ctypes.byref(fused), 1 << 20, wsb, 4096, None, None, None) == 5


def test_recurrent_step_refuses_before_launch():
    lib = mt.lib()
    d1 = _desc(S=1, DHQK=256, DHV=512, chunk_size=64)

    def step(desc, **ptrs):
        names = ["q", "k", "v", "i", "f", "C_in", "n_in", "m_in", "h", "C_out", "n_out", "m_out"]
        vals = [ptrs.get(n, 4096 * (j + 1)) for j, n in enumerate(names)]
        return lib.mlstm_recurrent_step(ctypes.byref(desc) if desc is not None else None, *vals, None)

    assert step(None) == 1
    assert step(_desc(S=2, chunk_size=64)) == 2          # one token per call
    assert step(_desc(S=1, DHQK=100, chunk_size=64)) == 2
    assert step(d1, C_out=None) == 1
    assert step(d1, h=None) == 1
    assert step(d1, q=None) == 1
    assert step(d1, C_in=4096 + 8) == 8                   # the state is read in 16-byte pieces
    assert step(d1, h=4096 * 9 + 4) == 8
    assert step(d1, n_out=4096 * 7) == 9                  # n_out may not be n_in
    assert step(d1, m_out=4096 * 8) == 9                  # m_out may not be m_in
    ds = _desc(S=1, DHQK=256, DHV=512, chunk_size=64, gate="sig")
    assert step(ds, n_in=4096, m_in=None, n_out=None, m_out=None) == 5
    assert step(ds, n_in=None, m_in=None, n_out=4096, m_out=None) == 5


def test_backward_refuses_before_launch():
    lib = mt.lib()
    d = _desc(S=300, DHQK=128, DHV=128, chunk_size=64)
    need = lib.mlstm_bw_workspace_bytes(ctypes.byref(d))
    assert need > lib.mlstm_fw_workspace_bytes(ctypes.byref(d))

    def bw(desc, ws_bytes=need, **ptrs):
        names = ["q", "k", "v", "i", "f", "C0", "n0", "m0", "dH", "dQ", "dK", "dV", "d_i", "d_f",
                 "dC0", "dn0", "dm0", "ws"]
        vals = [ptrs.get(n, 4096 * (j + 1)) for j, n in enumerate(names)]
        return lib.mlstm_chunkwise_bw(ctypes.byref(desc) if desc is not None else None, *vals, ws_bytes, None)

    assert bw(None) == 1
    assert bw(_desc(S=300, DHQK=100, chunk_size=64)) == 2
    assert bw(d, dH=None) == 1
    assert bw(d, dQ=None) == 1
    assert bw(d, d_f=None) == 1
    assert bw(d, dV=4096 * 12 + 4) == 8                   # gradients are written in 16-byte pieces
    assert bw(d, dH=4096 * 9 + 8) == 8
    assert bw(d, d_i=4096 * 13 + 2) == 8
    assert bw(d, ws=None) == 6
    assert bw(d, ws_bytes=need - 1) == 6
    assert bw(d, ws=4096 * 18 + 64) == 6                  # 256-byte aligned workspace
    ds = _desc(S=300, DHQK=128, DHV=128, chunk_size=64, gate="sig")
    assert bw(ds, n0=None, m0=None, dm0=None) == 5         # sig gate: no dn0
    assert bw(ds, n0=None, m0=None, dn0=None) == 5         # sig gate: no dm0
    assert lib.mlstm_bw_workspace_bytes(None) == 0
    # the stage calls check the same way
    rc = lambda desc, **kw: lib.mlstm_bw_recompute(
        ctypes.byref(desc), *[kw.get(n, 4096 * (j + 1)) for j, n in enumerate(
            ["q", "k", "v", "i", "f", "C0", "n0", "m0", "dH", "ws"])], kw.get("ws_bytes", need), None)
    assert rc(d, q=None) == 1
    assert rc(d, dH=None) == 1
    assert rc(d, dH=4096 * 9 + 4) == 8
    assert rc(d, ws_bytes=need - 1) == 6
    assert rc(ds, n0=4096) == 5
    gr = lambda desc, **kw: lib.mlstm_bw_grads(
        ctypes.byref(desc), *[kw.get(n, 4096 * (j + 1)) for j, n in enumerate(
            ["q", "k", "v", "i", "f", "C0", "n0", "dH", "dQ", "dK", "dV", "d_i", "d_f", "dC0", "dn0", "dm0",
             "ws"])], kw.get("ws_bytes", need), None)
    assert gr(d, dK=None) == 1
    assert gr(d, dQ=4096 * 9 + 4) == 8
    assert gr(d, ws=None) == 6
    assert gr(ds, n0=None, dn0=None) == 5                 # sig gate: no dm0


def test_saved_forward_entry_points_refuse_before_launch():
    """mlstm_chunkwise_fw_rows and mlstm_chunkwise_bw_saved check their extra
    arguments (the forward's H and per-row m and normaliser) before any
    launch, besides those of mlstm_chunkwise_fw and mlstm_chunkwise_bw."""
    lib = mt.lib()
    d = _desc(S=300, DHQK=128, DHV=128, chunk_size=64)
    need = lib.mlstm_bw_workspace_bytes(ctypes.byref(d))

    def sb(desc, ws_bytes=need, **ptrs):
        names = ["q", "k", "v", "i", "f", "C0", "n0", "m0", "H", "m_rows", "den_rows", "dH", "dQ", "dK", "dV",
                 "d_i", "d_f", "dC0", "dn0", "dm0", "ws"]
        vals = [ptrs.get(n, 4096 * (j + 1)) for j, n in enumerate(names)]
        return lib.mlstm_chunkwise_bw_saved(ctypes.byref(desc), *vals, ws_bytes, None)

    assert sb(d, H=None) == 1                             # exp gate: H, m_rows, den_rows required
    assert sb(d, m_rows=None) == 1
    assert sb(d, den_rows=None) == 1
    assert sb(d, H=4096 * 9 + 4) == 8                     # H in 16-byte pieces
    assert sb(d, den_rows=4096 * 11 + 2) == 8
    assert sb(d, dQ=None) == 1                            # the checks of mlstm_chunkwise_bw
    assert sb(d, ws_bytes=need - 1) == 6
    assert sb(_desc(S=300, DHQK=128, DHV=128, chunk_size=64, h_dtype=mt.MLSTM_BF16)) == 5  # H is float32
    ds = _desc(S=300, DHQK=128, DHV=128, chunk_size=64, gate="sig")
    assert sb(ds, n0=None, m0=None, dn0=None, dm0=None) == 5            # sig gate: no row terms
    assert sb(ds, n0=None, m0=None, dn0=None, dm0=None, H=None, m_rows=None) == 5

    wsb = mt.workspace_bytes(d)

    def fr(desc, **ptrs):
        names = ["q", "k", "v", "i", "f", "C0", "n0", "m0", "H", "C_out", "n_out", "m_out", "m_rows", "den_rows"]
        vals = [ptrs.get(n, 4096 * (j + 1)) for j, n in enumerate(names)]
        return lib.mlstm_chunkwise_fw_rows(ctypes.byref(desc), *vals, ptrs.get("ws", 1 << 20),
                                           ptrs.get("ws_bytes", wsb), None)

    assert fr(d, q=None) == 1
    assert fr(d, m_rows=4096 * 13 + 2) == 8
    assert fr(d, ws_bytes=wsb - 1) == 6
    assert fr(ds, n0=None, m0=None, n_out=None, m_out=None) == 5       # sig gate: no rows
    assert fr(ds, n0=None, m0=None, n_out=None, m_out=None, m_rows=None) == 5


def test_backward_workspace_formula():
    """Workspace of the 7B-shaped backward: the forward's two-stage workspace
    plus float32 chunk states, six per-position arrays (the recompute forms
    1/z and delta in the intra-chunk kernel, so H is not kept on these
    shapes), the state gradients after each chunk, the initial-state
    gradients and (bf16 inputs) the weighted dS tiles that the dk pass hands
    to the dq pass, each region rounded up to 256 bytes.  The generic shapes
    (here DHQK 64) keep H.  (The 7B-shaped heads fill the CUs, so the
    backward cuts them into chunks of 128: two 64-row tiles, three tile
    pairs per chunk.)"""
    d = _desc(B=8, NH=8, S=8192, DHQK=256, DHV=512, chunk_size=128)
    lib = mt.lib()
    BH, S, DK, DV, Nc = 64, 8192, 256, 512, 64
    r = lambda x: (x + 255) // 256 * 256
    fw = r(lib.mlstm_fw_workspace_bytes(ctypes.byref(d)))
    rest = [BH * S * 4, BH * S * 4, BH * S * 4, BH * S * 4,                     # b, src, 1/z, delta
            BH * Nc * DK * DV * 4, BH * Nc * DK * 4,                            # state gradients
            BH * S * 4, BH * S * 4,                                             # q.dq, k.dk
            BH * (S // 1024 + 32) * 4,                                          # gate sums, dm0 partial sums
            BH * DK * DV * 4, BH * DK * 4]                                      # dC0, dn0
    expect = fw + sum(r(x) for x in [
        BH * (Nc + 1) * DK * DV * 4, BH * (Nc + 1) * DK * 4, BH * (Nc + 1) * 4,   # states
        0, BH * S * 4, BH * S * 4,                                               # (no H), m, den
        *rest,
        BH * Nc * 3 * 64 * 64 * 4])                   # weighted dS of the 3 tile pairs per chunk
    assert lib.mlstm_bw_workspace_bytes(ctypes.byref(d)) == expect
    # generic kernels (DHQK 64, one row tile per head: chunks of 256 stay):
    # H in float32 as well.  64 row tiles fill a quarter of the 256 CUs, so
    # the state-gradient recurrence runs as 4 sequence segments of 8 chunks,
    # each leaving its own gradient (and normaliser gradient) for the joins.
    DK, Nc = 64, 32
    dg = _desc(B=8, NH=8, S=8192, DHQK=DK, DHV=512, chunk_size=256)
    fw = r(lib.mlstm_fw_workspace_bytes(ctypes.byref(dg)))
    rest[4:6] = [BH * Nc * DK * DV * 4, BH * Nc * DK * 4]
    rest[9:11] = [BH * DK * DV * 4, BH * DK * 4]
    expect = fw + sum(r(x) for x in [
        BH * (Nc + 1) * DK * DV * 4, BH * (Nc + 1) * DK * 4, BH * (Nc + 1) * 4,
        BH * S * DV * 4, BH * S * 4, BH * S * 4,                                 # H, m, den
        *rest,
        BH * Nc * 10 * 64 * 64 * 4,
        BH * 4 * DK * DV * 4, BH * 4 * DK * 4])                                  # segments
    assert lib.mlstm_bw_workspace_bytes(ctypes.byref(dg)) == expect
    # the backward picks its own cut: chunks of at most 128 rows when the
    # heads fill the CUs (64 heads x 4 row tiles here), else 256
    for L in (256, 512, 1024):
        dl = _desc(B=8, NH=8, S=8192, DHQK=256, DHV=512, chunk_size=L, tile_lq=128, tile_lkv=128)
        assert lib.mlstm_bw_workspace_bytes(ctypes.byref(dl)) == lib.mlstm_bw_workspace_bytes(ctypes.byref(d))
    few = _desc(B=1, NH=8, S=8192, DHQK=256, DHV=512, chunk_size=256)
    for L in (512, 1024):
        dl = _desc(B=1, NH=8, S=8192, DHQK=256, DHV=512, chunk_size=L, tile_lq=128, tile_lkv=128)
        assert lib.mlstm_bw_workspace_bytes(ctypes.byref(dl)) == lib.mlstm_bw_workspace_bytes(ctypes.byref(few))


def test_q8_step_refuses_before_launch():
    lib = mt.lib()
    d1 = _desc(S=1, DHQK=256, DHV=512, chunk_size=64)

    def step(desc, **ptrs):
        names = ["q", "k", "v", "i", "f", "Cq_in", "Cs_in", "n_in", "m_in", "h", "Cq_out", "Cs_out", "n_out",
                 "m_out"]
        vals = [ptrs.get(n, 4096 * (j + 1)) for j, n in enumerate(names)]
        return lib.mlstm_recurrent_step_q8(ctypes.byref(desc), *vals, None)

    assert step(_desc(S=2, chunk_size=64)) == 2
    assert step(d1, Cq_out=None) == 1
    assert step(d1, Cs_out=None) == 1
    assert step(d1, Cs_in=None) == 1                        # codes without scales
    assert step(d1, Cq_in=4096 * 6 + 2) == 8                # codes are read in 4-byte pieces
    assert step(d1, Cs_in=4096 * 7 + 4) == 8                # scales in 16-byte pieces
    assert step(d1, n_out=4096 * 8) == 9                    # n_out may not be n_in
    ds = _desc(S=1, DHQK=256, DHV=512, chunk_size=64, gate="sig")
    assert step(ds, n_in=None, m_in=None, n_out=None) == 5
    assert lib.mlstm_state_q8_encode(ctypes.byref(d1), None, 4096, 8192, None) == 1
    assert lib.mlstm_state_q8_decode(ctypes.byref(d1), 4096, 8192 + 2, 4096 * 4, None) == 8


def test_flops_formula():
    # 7B-shaped heads, S=8192, chunk 256: 378.4 GFLOP
    f = mt.flops(8, 8, 8192, 256, 512, 256)
    assert abs(f / 1e9 - 378.4) < 0.1


def test_noalloc_entry_point_refuses_before_launch():
    """mlstm_chunkwise_fw_noalloc checks its arguments, then the size of the
    workspace the chosen kernels need against its static array, before any
    device call."""
    lib = mt.lib()
    names = ["Q", "K", "V", "i", "f", "C0", "n0", "m0", "H", "C_out", "n_out", "m_out"]

    def call(desc, **ptrs):
        vals = [ptrs.get(n, 4096) for n in names]
        return lib.mlstm_chunkwise_fw_noalloc(ctypes.byref(desc) if desc is not None else None, *vals, None)

    d = _desc()
    assert call(None) == 1
    assert call(d, Q=None) == 1
    assert call(d, H=4096 + 8) == 8
    assert call(_desc(DHQK=100)) == 2
    assert call(_desc(gate="sig"), n0=4096) == 5
    # two-stage kernels at the 7B-shaped heads: 1.1 GB of chunk states
    big = _desc(B=8, NH=8, S=8192, DHQK=256, DHV=512, chunk_size=256, schedule=mt.MLSTM_SCHED_TWO_STAGE)
    assert mt.workspace_bytes(big) > mt.NOALLOC_WORKSPACE_BYTES
    assert call(big) == 6
    # the walker uses no workspace, so any size it covers fits (not called
    # here: the pointers above are not device memory)
    huge = _desc(B=64, NH=1, S=1 << 17, DHQK=256, DHV=512, chunk_size=256, schedule=mt.MLSTM_SCHED_FUSED)
    assert mt.validate(huge) == 0 and mt.workspace_bytes(huge) == 0


def test_short_chunks_run_on_the_generic_kernels():
    """Chunks of 16 and 32 rows are valid: the generic (and float64) kernels
    take one tile per chunk; the backward runs its kernels on chunks of 64
    (its result does not depend on the chunking), so its workspace is that
    of chunk 64."""
    for L in (16, 32):
        for kw in (dict(), dict(DHQK=256, DHV=512), dict(qkv_dtype=mt.MLSTM_F32)):
            d = _desc(chunk_size=L, **kw)
            assert mt.validate(d) == 0
            assert mt.kernel_family(d) == mt.MLSTM_FAMILY_GENERIC
            assert mt.num_chunks(d) == (1000 + L - 1) // L
            assert mt.bw_workspace_bytes(d) == mt.bw_workspace_bytes(_desc(chunk_size=64, **kw))
        assert mt.validate(_desc(chunk_size=L, tile_lq=64)) == 3
        assert mt.kernel_family(_desc(chunk_size=L, precision="f64")) == mt.MLSTM_FAMILY_F64
        assert mt.validate(_desc(chunk_size=L, DHQK=256, DHV=512, schedule="fused")) == 5


def test_blocked_schedule():
    """The blocked schedule: the wide kernels with the row-tile states kernel,
    run per block of chunks; its workspace holds one block's chunk states
    (block_chunks + 1 per head) and the state passed between blocks, twice;
    the stage-wise calls refuse it."""
    big = dict(B=8, NH=8, S=8192, DHQK=256, DHV=512, chunk_size=256)
    d = _desc(**big, schedule="blocked")
    assert mt.validate(d) == 0
    assert mt.kernel_family(d) == mt.MLSTM_FAMILY_BLOCKED
    BH, DK, DV, S = 64, 256, 512, 8192
    r = lambda x: (x + 255) // 256 * 256
    for k in (0, 1, 3):
        dk = _desc(**big, schedule="blocked", block_chunks=k)
        kk = k or (128 << 20) // (BH * DK * DV * 4)       # half the Infinity Cache: 4 chunks here
        want = (r(BH * (kk + 1) * DK * DV * 4) + r(BH * (kk + 1) * DK * 4) + r(BH * (kk + 1) * 4)
                + r(BH * S * 12) + 2 * (r(BH * DK * DV * 4) + r(BH * DK * 4) + r(BH * 4)))
        assert mt.workspace_bytes(dk) == want, k
    # shapes outside the row-tile states kernel, fp64 and float32 inputs refuse it
    assert mt.validate(_desc(B=2, NH=2, S=1000, DHQK=128, DHV=128, chunk_size=128, schedule="blocked")) == 5
    assert mt.validate(_desc(**big, schedule="blocked", precision="f64")) == 5
    assert mt.validate(_desc(**big, schedule="blocked", qkv_dtype=mt.MLSTM_F32)) == 5
    lib = mt.lib()
    wsb = mt.workspace_bytes(d)
    assert lib.mlstm_fw_states(ctypes.byref(d), *([4096] * 7), 1 << 20, wsb, None, None, None, None) == 5
    assert lib.mlstm_fw_hintra(ctypes.byref(d), *([4096] * 5), 1 << 20, wsb, 4096, None, None, None) == 5


def test_int16_state_codes():
    """int16-coded chunk states: the wide family with split operands and a
    row-tile shape, on the two-stage schedule; the chunk states take 2 bytes
    a value plus one float32 scale per 16 x 32 block."""
    def r256(x):
        return (x + 255) // 256 * 256
    BH = 6
    for DK, DV in ((256, 512), (128, 512), (256, 256), (128, 256)):
        for sched in ("auto", "two_stage"):
            d = _desc(DHQK=DK, DHV=DV, chunk_size=256, schedule=sched, state_codes="int16")
            assert mt.validate(d) == 0, (DK, DV, sched)
            Nc = (1000 + 255) // 256
            expect = (r256(BH * (Nc + 1) * DK * DV * 2) + r256(BH * (Nc + 1) * DK * 4) + r256(BH * (Nc + 1) * 4)
                      + r256(BH * 1000 * 4 * 3) + r256(BH * (Nc + 1) * 4)
                      + r256(BH * (Nc + 1) * (DK // 16) * (DV // 32) * 4))
            assert mt.workspace_bytes(d) == expect, (DK, DV, sched)
    # sig gate: no normaliser or stabiliser regions
    ds = _desc(DHQK=256, DHV=512, chunk_size=256, schedule="two_stage", state_codes="int16", gate="sig")
    Nc = 4
    assert mt.workspace_bytes(ds) == (r256(BH * (Nc + 1) * 256 * 512 * 2) + r256(BH * 1000 * 4 * 2)
                                      + r256(BH * (Nc + 1) * 4) + r256(BH * (Nc + 1) * 16 * 16 * 4))
    for kw in (dict(DHQK=128, DHV=64),                                   # generic family
               dict(DHQK=256, DHV=512, chunk_size=256, precision="f16"),   # single-rounded operands
               dict(DHQK=256, DHV=512, chunk_size=256, precision="f64"),
               dict(DHQK=256, DHV=512, chunk_size=256, qkv_dtype=mt.MLSTM_F32),
               dict(DHQK=256, DHV=512, chunk_size=256, schedule="fused"),
               dict(DHQK=256, DHV=512, chunk_size=256, schedule="blocked")):
        d = _desc(state_codes="int16", **kw)
        assert mt.validate(d) == 5, kw
        assert mt.workspace_bytes(d) == 0
