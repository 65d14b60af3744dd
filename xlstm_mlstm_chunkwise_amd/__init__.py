"""MI355X (gfx950) chunkwise mLSTM: Python binding of libmlstm_tfla.so (forward
pass, backward pass and recurrent decode step).

The binding only marshals arguments: it allocates outputs and workspace with
PyTorch (device memory), passes raw device pointers and the current HIP
stream to the C ABI declared in include/mlstm_tfla.h, and turns a non-zero
status into an exception.  Every step of the computation runs in the HIP
kernels; there is no other code path.  If the shared library is missing the
import of the functions below fails with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmlstm_tfla.so")

MLSTM_F32, MLSTM_BF16 = 0, 1
MLSTM_GATE_EXP, MLSTM_GATE_SIG = 0, 1
MLSTM_PREC_SPLIT, MLSTM_PREC_F16, MLSTM_PREC_F64 = 0, 1, 2
MLSTM_FAMILY_GENERIC, MLSTM_FAMILY_WIDE, MLSTM_FAMILY_F64, MLSTM_FAMILY_FUSED, MLSTM_FAMILY_BLOCKED = 0, 1, 2, 3, 4
MLSTM_SCHED_AUTO, MLSTM_SCHED_TWO_STAGE, MLSTM_SCHED_FUSED, MLSTM_SCHED_BLOCKED = 0, 1, 2, 3
_PREC = {"split": MLSTM_PREC_SPLIT, "f16": MLSTM_PREC_F16, "f64": MLSTM_PREC_F64}
_GATE = {"exp": MLSTM_GATE_EXP, "sig": MLSTM_GATE_SIG}
_SCHED = {"auto": MLSTM_SCHED_AUTO, "two_stage": MLSTM_SCHED_TWO_STAGE, "fused": MLSTM_SCHED_FUSED,
          "blocked": MLSTM_SCHED_BLOCKED}
MLSTM_STATES_SPLIT, MLSTM_STATES_I16 = 0, 1
_CODES = {"split": MLSTM_STATES_SPLIT, "int16": MLSTM_STATES_I16}

STATUS_NAMES = {
    0: "MLSTM_OK", 1: "MLSTM_E_NULLPTR", 2: "MLSTM_E_SHAPE", 3: "MLSTM_E_CHUNK",
    4: "MLSTM_E_DTYPE", 5: "MLSTM_E_UNSUPPORTED", 6: "MLSTM_E_WORKSPACE",
    7: "MLSTM_E_HIP", 8: "MLSTM_E_ALIGN", 9: "MLSTM_E_ARG",
}


class MlstmError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_str(status)})")


class FwDesc(ctypes.Structure):
    """Mirror of mlstm_fw_desc_t."""
    _fields_ = [
        ("B", ctypes.c_int32), ("NH", ctypes.c_int32), ("S", ctypes.c_int32),
        ("DHQK", ctypes.c_int32), ("DHV", ctypes.c_int32), ("chunk_size", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32), ("h_dtype", ctypes.c_int32), ("gate", ctypes.c_int32),
        ("precision", ctypes.c_int32), ("qk_scale", ctypes.c_float), ("eps", ctypes.c_float),
        ("tile_lq", ctypes.c_int32), ("tile_lkv", ctypes.c_int32), ("schedule", ctypes.c_int32),
        ("block_chunks", ctypes.c_int32), ("state_codes", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


_lib = None
_SYMBOLS = {
    "mlstm_abi_version": (ctypes.c_int, []),
    "mlstm_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "mlstm_fw_validate": (ctypes.c_int, [ctypes.POINTER(FwDesc)]),
    "mlstm_fw_num_chunks": (ctypes.c_int64, [ctypes.POINTER(FwDesc)]),
    "mlstm_fw_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(FwDesc)]),
    "mlstm_fw_kernel_family": (ctypes.c_int, [ctypes.POINTER(FwDesc)]),
    "mlstm_chunkwise_fw": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 12
                           + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mlstm_chunkwise_fw_rows": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 14
                                + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mlstm_chunkwise_fw_noalloc": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 13),
    "mlstm_fw_states": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 8
                        + [ctypes.c_size_t] + [ctypes.c_void_p] * 4),
    "mlstm_fw_hintra": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 6
                        + [ctypes.c_size_t] + [ctypes.c_void_p] * 4),
    "mlstm_fw_unpack_states": (ctypes.c_int, [ctypes.POINTER(FwDesc), ctypes.c_void_p, ctypes.c_size_t]
                               + [ctypes.c_void_p] * 4),
    "mlstm_recurrent_step": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 13),
    "mlstm_recurrent_step_q8": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 15),
    "mlstm_state_q8_encode": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 4),
    "mlstm_state_q8_decode": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 4),
    "mlstm_bw_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(FwDesc)]),
    "mlstm_chunkwise_bw": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 18
                           + [ctypes.c_size_t, ctypes.c_void_p]),
    "mlstm_chunkwise_bw_saved": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 21
                                 + [ctypes.c_size_t, ctypes.c_void_p]),
    "mlstm_bw_recompute": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 10
                           + [ctypes.c_size_t, ctypes.c_void_p]),
    "mlstm_bw_grads": (ctypes.c_int, [ctypes.POINTER(FwDesc)] + [ctypes.c_void_p] * 17
                       + [ctypes.c_size_t, ctypes.c_void_p]),
}


def lib() -> ctypes.CDLL:
    """Load libmlstm_tfla.so (built in-tree by xlstm_mlstm_chunkwise_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing; build it with `python -m xlstm_mlstm_chunkwise_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (restype, argtypes) in _SYMBOLS.items():
            fn = getattr(handle, name)
            fn.restype = restype
            fn.argtypes = argtypes
        _lib = handle
    return _lib


def abi_version() -> int:
    return lib().mlstm_abi_version()


def status_str(status: int) -> str:
    return lib().mlstm_status_str(status).decode()


def make_desc(B, NH, S, DHQK, DHV, chunk_size, *, qkv_dtype=MLSTM_BF16, h_dtype=MLSTM_F32,
              gate="exp", precision="split", qk_scale=0.0, eps=0.0, tile_lq=0, tile_lkv=0,
              schedule="auto", block_chunks=0, state_codes="split") -> FwDesc:
    d = FwDesc()
    d.B, d.NH, d.S, d.DHQK, d.DHV, d.chunk_size = B, NH, S, DHQK, DHV, chunk_size
    d.qkv_dtype, d.h_dtype = qkv_dtype, h_dtype
    d.gate = _GATE[gate] if isinstance(gate, str) else gate
    d.precision = _PREC[precision] if isinstance(precision, str) else precision
    d.qk_scale, d.eps = qk_scale, eps
    d.tile_lq, d.tile_lkv = tile_lq, tile_lkv
    d.schedule = _SCHED[schedule] if isinstance(schedule, str) else schedule
    d.block_chunks = block_chunks
    d.state_codes = _CODES[state_codes] if isinstance(state_codes, str) else state_codes
    return d


def validate(desc: FwDesc) -> int:
    return lib().mlstm_fw_validate(ctypes.byref(desc))


def kernel_family(desc: FwDesc) -> int:
    """MLSTM_FAMILY_* of the kernels that run for `desc` (negated status if invalid)."""
    return lib().mlstm_fw_kernel_family(ctypes.byref(desc))


def workspace_bytes(desc: FwDesc) -> int:
    return lib().mlstm_fw_workspace_bytes(ctypes.byref(desc))


def num_chunks(desc: FwDesc) -> int:
    return lib().mlstm_fw_num_chunks(ctypes.byref(desc))


# ---------------------------------------------------------------------------
# torch-facing wrappers (device memory and streams only)

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MLSTM_BF16
    if t.dtype == torch.float32:
        return MLSTM_F32
    raise TypeError(f"Q/K/V must be bfloat16 or float32, got {t.dtype}")


def _check(t, name, shape, dtype=None):
    if t is None:
        return
    torch = _torch()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _desc_for(q, v, chunk_size, gate, h_dtype, precision, qk_scale, eps, tile_lq, tile_lkv, schedule="auto",
              block_chunks=0, state_codes="split"):
    torch = _torch()
    B, NH, S, DK = q.shape
    DV = v.shape[-1]
    hcode = MLSTM_BF16 if h_dtype == torch.bfloat16 else MLSTM_F32
    return make_desc(B, NH, S, DK, DV, chunk_size, qkv_dtype=_dtype_code(q), h_dtype=hcode,
                     gate=gate, precision=precision,
                     qk_scale=0.0 if qk_scale is None else float(qk_scale), eps=float(eps),
                     tile_lq=tile_lq, tile_lkv=tile_lkv, schedule=schedule, block_chunks=block_chunks,
                     state_codes=state_codes)


def _check_inputs(q, k, v, i_pre, f_pre):
    torch = _torch()
    if q.dim() != 4:
        raise ValueError("Q must be (B, NH, S, DHQK)")
    B, NH, S, DK = q.shape
    DV = v.shape[-1]
    _check(q, "Q", (B, NH, S, DK))
    _check(k, "K", (B, NH, S, DK), q.dtype)
    _check(v, "V", (B, NH, S, DV), q.dtype)
    _check(i_pre, "i_pre", (B, NH, S), torch.float32)
    _check(f_pre, "f_pre", (B, NH, S), torch.float32)
    return B, NH, S, DK, DV


def mlstm_chunkwise_fw(q, k, v, i_pre, f_pre, C0=None, n0=None, m0=None, *, chunk_size: int,
                       gate: str = "exp", h_dtype=None, precision: str = "split",
                       qk_scale: Optional[float] = None, eps: float = 0.0,
                       tile_lq: int = 0, tile_lkv: int = 0, schedule: str = "auto", workspace=None,
                       return_final_state: bool = True, out=None, block_chunks: int = 0,
                       state_codes: str = "split", return_rows: bool = False):
    """Chunkwise mLSTM forward pass on the GPU.

    q, k: (B, NH, S, DHQK); v: (B, NH, S, DHV), bfloat16 or float32;
    i_pre, f_pre: (B, NH, S) float32; C0 (B, NH, DHQK, DHV), n0 (B, NH, DHQK),
    m0 (B, NH) float32 or None (zero state).  Returns (H, C, n, m); n and m
    are None for gate="sig", and the final state is None when
    return_final_state is False.  H is float32 unless h_dtype says otherwise.
    schedule: "auto", "two_stage", "fused" or "blocked" (see
    mlstm_schedule_t); block_chunks: chunks per block of the blocked
    schedule (0: the library's choice); state_codes: "split" or "int16", how
    the two stages hand the chunk states over (see mlstm_state_codes_t).
    return_rows (exp gate): also return the per-row max-state m and
    normaliser, (B, NH, S) float32 each, as (H, C, n, m, m_rows, den_rows)
    (mlstm_chunkwise_fw_rows), for mlstm_chunkwise_bw(saved=...).
    """
    torch = _torch()
    B, NH, S, DK, DV = _check_inputs(q, k, v, i_pre, f_pre)
    h_dtype = torch.float32 if h_dtype is None else h_dtype
    _check(C0, "C0", (B, NH, DK, DV), torch.float32)
    _check(n0, "n0", (B, NH, DK), torch.float32)
    _check(m0, "m0", (B, NH), torch.float32)
    desc = _desc_for(q, v, chunk_size, gate, h_dtype, precision, qk_scale, eps, tile_lq, tile_lkv, schedule,
                     block_chunks, state_codes)
    st = validate(desc)
    if st:
        raise MlstmError(st, "mlstm_chunkwise_fw")
    dev = q.device
    H = out if out is not None else torch.empty((B, NH, S, DV), dtype=h_dtype, device=dev)
    _check(H, "H", (B, NH, S, DV), h_dtype)
    sig = gate == "sig"
    C_out = n_out = m_out = None
    if return_final_state:
        C_out = torch.empty((B, NH, DK, DV), dtype=torch.float32, device=dev)
        if not sig:
            n_out = torch.empty((B, NH, DK), dtype=torch.float32, device=dev)
            m_out = torch.empty((B, NH), dtype=torch.float32, device=dev)
    need = workspace_bytes(desc)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, need {need}")
    if return_rows:
        if sig:
            raise ValueError("return_rows: the sig gate has no per-row normaliser")
        m_rows = torch.empty((B, NH, S), dtype=torch.float32, device=dev)
        den_rows = torch.empty((B, NH, S), dtype=torch.float32, device=dev)
        st = lib().mlstm_chunkwise_fw_rows(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre),
            _ptr(C0), _ptr(n0), _ptr(m0), _ptr(H), _ptr(C_out), _ptr(n_out), _ptr(m_out), _ptr(m_rows),
            _ptr(den_rows), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
        if st:
            raise MlstmError(st, "mlstm_chunkwise_fw_rows")
        return H, C_out, n_out, m_out, m_rows, den_rows
    st = lib().mlstm_chunkwise_fw(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre),
        _ptr(C0), _ptr(n0), _ptr(m0), _ptr(H), _ptr(C_out), _ptr(n_out), _ptr(m_out),
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream())
    if st:
        raise MlstmError(st, "mlstm_chunkwise_fw")
    return H, C_out, n_out, m_out


NOALLOC_WORKSPACE_BYTES = 64 << 20   # MLSTM_NOALLOC_WORKSPACE_BYTES


def mlstm_chunkwise_fw_noalloc(q, k, v, i_pre, f_pre, C0=None, n0=None, m0=None, *, chunk_size: int,
                               gate: str = "exp", precision: str = "split", qk_scale: Optional[float] = None,
                               eps: float = 0.0, tile_lq: int = 0, tile_lkv: int = 0, schedule: str = "auto",
                               out=None, C_out=None, n_out=None, m_out=None, block_chunks: int = 0,
                               state_codes: str = "split"):
    """mlstm_chunkwise_fw on the library's static workspace
    (mlstm_chunkwise_fw_noalloc): no workspace argument, and nothing is
    allocated when every output is given (out = H, whose dtype is the H
    dtype; C_out, n_out, m_out may be None: not written).  Returns
    (H, C_out, n_out, m_out).  Calls that overlap on one GPU race."""
    torch = _torch()
    B, NH, S, DK, DV = _check_inputs(q, k, v, i_pre, f_pre)
    _check(C0, "C0", (B, NH, DK, DV), torch.float32)
    _check(n0, "n0", (B, NH, DK), torch.float32)
    _check(m0, "m0", (B, NH), torch.float32)
    H = out if out is not None else torch.empty((B, NH, S, DV), dtype=torch.float32, device=q.device)
    _check(H, "H", (B, NH, S, DV))
    _check(C_out, "C_out", (B, NH, DK, DV), torch.float32)
    _check(n_out, "n_out", (B, NH, DK), torch.float32)
    _check(m_out, "m_out", (B, NH), torch.float32)
    desc = _desc_for(q, v, chunk_size, gate, H.dtype, precision, qk_scale, eps, tile_lq, tile_lkv, schedule,
                     block_chunks, state_codes)
    st = lib().mlstm_chunkwise_fw_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(C0), _ptr(n0), _ptr(m0),
        _ptr(H), _ptr(C_out), _ptr(n_out), _ptr(m_out), _stream())
    if st:
        raise MlstmError(st, "mlstm_chunkwise_fw_noalloc")
    return H, C_out, n_out, m_out


def _workspace(desc, workspace, dev):
    torch = _torch()
    need = workspace_bytes(desc)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError(f"workspace holds {workspace.numel() * workspace.element_size()} bytes, need {need}")
    return workspace, workspace.numel() * workspace.element_size()


def mlstm_fw_states(k, v, i_pre, f_pre, C0=None, n0=None, m0=None, *, chunk_size: int,
                    gate: str = "exp", precision: str = "split", tile_lq: int = 0, tile_lkv: int = 0,
                    workspace=None, return_final_state: bool = True, state_codes: str = "split"):
    """Stage one alone.  Returns (workspace, C, n, m): the workspace now holds
    the chunk states (read them with unpack_states); C, n, m are the final
    state (None where not requested or not defined for the gate)."""
    torch = _torch()
    B, NH, S, DK, DV = _check_inputs(k, k, v, i_pre, f_pre)
    desc = _desc_for(k, v, chunk_size, gate, torch.float32, precision, None, 0.0, tile_lq, tile_lkv,
                     state_codes=state_codes)
    st = validate(desc)
    if st:
        raise MlstmError(st, "mlstm_fw_states")
    _check(C0, "C0", (B, NH, DK, DV), torch.float32)
    _check(n0, "n0", (B, NH, DK), torch.float32)
    _check(m0, "m0", (B, NH), torch.float32)
    dev = k.device
    sig = gate == "sig"
    workspace, ws_bytes = _workspace(desc, workspace, dev)
    C_out = n_out = m_out = None
    if return_final_state:
        C_out = torch.empty((B, NH, DK, DV), dtype=torch.float32, device=dev)
        if not sig:
            n_out = torch.empty((B, NH, DK), dtype=torch.float32, device=dev)
            m_out = torch.empty((B, NH), dtype=torch.float32, device=dev)
    st = lib().mlstm_fw_states(
        ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(C0), _ptr(n0), _ptr(m0),
        _ptr(workspace), ws_bytes, _ptr(C_out), _ptr(n_out), _ptr(m_out), _stream())
    if st:
        raise MlstmError(st, "mlstm_fw_states")
    return workspace, C_out, n_out, m_out


def mlstm_fw_hintra(q, k, v, i_pre, f_pre, workspace, *, chunk_size: int, gate: str = "exp",
                    h_dtype=None, precision: str = "split", qk_scale: Optional[float] = None,
                    eps: float = 0.0, tile_lq: int = 0, tile_lkv: int = 0, return_rows: bool = False,
                    state_codes: str = "split"):
    """Stage two alone: H (and, with return_rows, the per-row m and stabilised
    normaliser) from the chunk states that mlstm_fw_states left in workspace.
    The descriptor arguments must match the ones given to mlstm_fw_states."""
    torch = _torch()
    B, NH, S, DK, DV = _check_inputs(q, k, v, i_pre, f_pre)
    h_dtype = torch.float32 if h_dtype is None else h_dtype
    desc = _desc_for(q, v, chunk_size, gate, h_dtype, precision, qk_scale, eps, tile_lq, tile_lkv,
                     state_codes=state_codes)
    st = validate(desc)
    if st:
        raise MlstmError(st, "mlstm_fw_hintra")
    dev = q.device
    workspace, ws_bytes = _workspace(desc, workspace, dev)
    H = torch.empty((B, NH, S, DV), dtype=h_dtype, device=dev)
    m_rows = den_rows = None
    if return_rows and gate == "exp":
        m_rows = torch.empty((B, NH, S), dtype=torch.float32, device=dev)
        den_rows = torch.empty((B, NH, S), dtype=torch.float32, device=dev)
    st = lib().mlstm_fw_hintra(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(workspace), ws_bytes,
        _ptr(H), _ptr(m_rows), _ptr(den_rows), _stream())
    if st:
        raise MlstmError(st, "mlstm_fw_hintra")
    if return_rows:
        return H, m_rows, den_rows
    return H


def unpack_states(q_like, v_like, workspace, *, chunk_size: int, gate: str = "exp",
                  precision: str = "split", tile_lq: int = 0, tile_lkv: int = 0, state_codes: str = "split"):
    """The chunk states in workspace as float32 tensors (C_states, n_states,
    m_states) of shapes (B, NH, N_c+1, DHQK, DHV), (B, NH, N_c+1, DHQK),
    (B, NH, N_c+1); entry c is the state entering chunk c.  q_like / v_like
    only supply the shapes and the input dtype."""
    torch = _torch()
    desc = _desc_for(q_like, v_like, chunk_size, gate, torch.float32, precision, None, 0.0, tile_lq, tile_lkv,
                     state_codes=state_codes)
    st = validate(desc)
    if st:
        raise MlstmError(st, "mlstm_fw_unpack_states")
    B, NH, S, DK = q_like.shape
    DV = v_like.shape[-1]
    Nc = num_chunks(desc)
    dev = q_like.device
    sig = gate == "sig"
    Cst = torch.empty((B, NH, Nc + 1, DK, DV), dtype=torch.float32, device=dev)
    nst = None if sig else torch.empty((B, NH, Nc + 1, DK), dtype=torch.float32, device=dev)
    mst = None if sig else torch.empty((B, NH, Nc + 1), dtype=torch.float32, device=dev)
    st = lib().mlstm_fw_unpack_states(ctypes.byref(desc), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _ptr(Cst), _ptr(nst), _ptr(mst), _stream())
    if st:
        raise MlstmError(st, "mlstm_fw_unpack_states")
    return Cst, nst, mst


def flops(B, NH, S, DHQK, DHV, chunk_size) -> float:
    """Algorithmic matrix-core FLOPs of one forward pass, causal lower triangle
    only: per token 4*DHQK*DHV (Q.C and K^T.V) + (L+1)*(DHQK+DHV) (Q.K^T and P.V)."""
    return float(B) * NH * S * (4.0 * DHQK * DHV + (chunk_size + 1) * (DHQK + DHV))


def mlstm_recurrent_step(q, k, v, i_pre, f_pre, C=None, n=None, m=None, *, gate: str = "exp", h_dtype=None,
                         qk_scale: Optional[float] = None, eps: float = 0.0, C_out=None, n_out=None,
                         m_out=None):
    """One time step of the recurrence for every head (decode) on the GPU.

    q, k: (B, NH, DHQK); v: (B, NH, DHV), bfloat16 or float32; i_pre, f_pre:
    (B, NH) float32; C (B, NH, DHQK, DHV), n (B, NH, DHQK), m (B, NH) float32
    or None (zero state): the state entering the step, as returned by
    mlstm_chunkwise_fw.  Returns (h, C', n', m'); n' and m' are None for
    gate="sig".  C_out may be C itself (updated in place); n_out / m_out, when
    given, must be other buffers than n / m.
    """
    torch = _torch()
    if q.dim() != 3:
        raise ValueError("q must be (B, NH, DHQK)")
    B, NH, DK = q.shape
    DV = v.shape[-1]
    _check(q, "q", (B, NH, DK))
    _check(k, "k", (B, NH, DK), q.dtype)
    _check(v, "v", (B, NH, DV), q.dtype)
    _check(i_pre, "i_pre", (B, NH), torch.float32)
    _check(f_pre, "f_pre", (B, NH), torch.float32)
    _check(C, "C", (B, NH, DK, DV), torch.float32)
    _check(n, "n", (B, NH, DK), torch.float32)
    _check(m, "m", (B, NH), torch.float32)
    h_dtype = torch.float32 if h_dtype is None else h_dtype
    hcode = MLSTM_BF16 if h_dtype == torch.bfloat16 else MLSTM_F32
    desc = make_desc(B, NH, 1, DK, DV, 64, qkv_dtype=_dtype_code(q), h_dtype=hcode, gate=gate,
                     qk_scale=0.0 if qk_scale is None else float(qk_scale), eps=float(eps))
    dev = q.device
    h = torch.empty((B, NH, DV), dtype=h_dtype, device=dev)
    if C_out is None:
        C_out = torch.empty((B, NH, DK, DV), dtype=torch.float32, device=dev)
    _check(C_out, "C_out", (B, NH, DK, DV), torch.float32)
    if gate != "sig":
        if n_out is None:
            n_out = torch.empty((B, NH, DK), dtype=torch.float32, device=dev)
        if m_out is None:
            m_out = torch.empty((B, NH), dtype=torch.float32, device=dev)
    _check(n_out, "n_out", (B, NH, DK), torch.float32)
    _check(m_out, "m_out", (B, NH), torch.float32)
    st = lib().mlstm_recurrent_step(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(C), _ptr(n), _ptr(m),
        _ptr(h), _ptr(C_out), _ptr(n_out), _ptr(m_out), _stream())
    if st:
        raise MlstmError(st, "mlstm_recurrent_step")
    return h, C_out, n_out, m_out


def bw_workspace_bytes(desc: FwDesc) -> int:
    return lib().mlstm_bw_workspace_bytes(ctypes.byref(desc))


def mlstm_chunkwise_bw(q, k, v, i_pre, f_pre, dH, C0=None, n0=None, m0=None, *, chunk_size: int,
                       gate: str = "exp", precision: str = "split", qk_scale: Optional[float] = None,
                       eps: float = 0.0, tile_lq: int = 0, tile_lkv: int = 0, state_grads: bool = False,
                       workspace=None, saved=None):
    """Backward pass on the GPU: the gradients of sum(dH * H) for the forward
    pass mlstm_chunkwise_fw(q, k, v, i_pre, f_pre, C0, n0, m0, ...) with the
    same keyword arguments.  dH has H's shape; its dtype (bfloat16 or
    float32) is the h_dtype of the descriptor.  Returns a dict with dQ, dK,
    dV, d_i, d_f (float32) and, with state_grads, dC0 and for the exp gate
    dn0 and dm0.  saved (exp gate, float32 dH): the forward's (H, m_rows,
    den_rows) from mlstm_chunkwise_fw(return_rows=True), so that only the
    chunk states are recomputed (mlstm_chunkwise_bw_saved)."""
    torch = _torch()
    B, NH, S, DK, DV = _check_inputs(q, k, v, i_pre, f_pre)
    if dH.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"dH must be bfloat16 or float32, got {dH.dtype}")
    _check(dH, "dH", (B, NH, S, DV))
    _check(C0, "C0", (B, NH, DK, DV), torch.float32)
    _check(n0, "n0", (B, NH, DK), torch.float32)
    _check(m0, "m0", (B, NH), torch.float32)
    desc = _desc_for(q, v, chunk_size, gate, dH.dtype, precision, qk_scale, eps, tile_lq, tile_lkv)
    st = validate(desc)
    if st:
        raise MlstmError(st, "mlstm_chunkwise_bw")
    dev = q.device
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dQ=torch.empty((B, NH, S, DK), **f32), dK=torch.empty((B, NH, S, DK), **f32),
               dV=torch.empty((B, NH, S, DV), **f32), d_i=torch.empty((B, NH, S), **f32),
               d_f=torch.empty((B, NH, S), **f32))
    if state_grads:
        out["dC0"] = torch.empty((B, NH, DK, DV), **f32)
        if gate != "sig":
            out["dn0"] = torch.empty((B, NH, DK), **f32)
            out["dm0"] = torch.empty((B, NH), **f32)
    need = bw_workspace_bytes(desc)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    if ws_bytes < need:
        raise ValueError(f"workspace holds {ws_bytes} bytes, need {need}")
    if saved is not None:
        if gate == "sig":
            raise ValueError("saved: the sig gate has no per-row normaliser")
        H, m_rows, den_rows = saved
        _check(H, "H", (B, NH, S, DV), torch.float32)
        _check(m_rows, "m_rows", (B, NH, S), torch.float32)
        _check(den_rows, "den_rows", (B, NH, S), torch.float32)
        st = lib().mlstm_chunkwise_bw_saved(
            ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(C0), _ptr(n0),
            _ptr(m0), _ptr(H), _ptr(m_rows), _ptr(den_rows), _ptr(dH), _ptr(out["dQ"]), _ptr(out["dK"]),
            _ptr(out["dV"]), _ptr(out["d_i"]), _ptr(out["d_f"]), _ptr(out.get("dC0")), _ptr(out.get("dn0")),
            _ptr(out.get("dm0")), _ptr(workspace), ws_bytes, _stream())
        if st:
            raise MlstmError(st, "mlstm_chunkwise_bw_saved")
        return out
    st = lib().mlstm_chunkwise_bw(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(C0), _ptr(n0), _ptr(m0),
        _ptr(dH), _ptr(out["dQ"]), _ptr(out["dK"]), _ptr(out["dV"]), _ptr(out["d_i"]), _ptr(out["d_f"]),
        _ptr(out.get("dC0")), _ptr(out.get("dn0")), _ptr(out.get("dm0")), _ptr(workspace), ws_bytes, _stream())
    if st:
        raise MlstmError(st, "mlstm_chunkwise_bw")
    return out


def bw_flops(B, NH, S, DHQK, DHV, chunk_size) -> float:
    """Algorithmic matrix-core FLOPs of one backward pass, causal lower
    triangle only.  Per token: the five intra-chunk products (scores Q.K^T and
    dH.V^T, then dS.K, dS^T.Q and P^T.dH), (L+1)(3 DHQK + 2 DHV), plus the
    four products with a state (C.dn, G.v, G^T.k and the state-gradient
    update), 8 DHQK DHV."""
    return float(B) * NH * S * ((chunk_size + 1) * (3.0 * DHQK + 2.0 * DHV) + 8.0 * DHQK * DHV)


def _state_desc(C_like_shape):
    B, NH, DK, DV = C_like_shape
    return make_desc(B, NH, 1, DK, DV, 64)


def state_q8_encode(C):
    """float32 state (B, NH, DHQK, DHV) -> (codes int8, scales float32 of
    shape (B, NH, DHV // 64, DHQK), block-major); see mlstm_state_q8_encode."""
    torch = _torch()
    B, NH, DK, DV = C.shape
    _check(C, "C", (B, NH, DK, DV), torch.float32)
    Cq = torch.empty((B, NH, DK, DV), dtype=torch.int8, device=C.device)
    Cs = torch.empty((B, NH, DV // 64, DK), dtype=torch.float32, device=C.device)
    desc = _state_desc(C.shape)
    st = lib().mlstm_state_q8_encode(ctypes.byref(desc), _ptr(C), _ptr(Cq), _ptr(Cs), _stream())
    if st:
        raise MlstmError(st, "mlstm_state_q8_encode")
    return Cq, Cs


def state_q8_decode(Cq, Cs):
    """Encoded state -> float32 (B, NH, DHQK, DHV)."""
    torch = _torch()
    B, NH, DK, DV = Cq.shape
    _check(Cq, "Cq", (B, NH, DK, DV), torch.int8)
    _check(Cs, "Cs", (B, NH, DV // 64, DK), torch.float32)
    C = torch.empty((B, NH, DK, DV), dtype=torch.float32, device=Cq.device)
    desc = _state_desc(Cq.shape)
    st = lib().mlstm_state_q8_decode(ctypes.byref(desc), _ptr(Cq), _ptr(Cs), _ptr(C), _stream())
    if st:
        raise MlstmError(st, "mlstm_state_q8_decode")
    return C


def mlstm_recurrent_step_q8(q, k, v, i_pre, f_pre, Cq=None, Cs=None, n=None, m=None, *, gate: str = "exp",
                            h_dtype=None, qk_scale: Optional[float] = None, eps: float = 0.0, Cq_out=None,
                            Cs_out=None, n_out=None, m_out=None):
    """mlstm_recurrent_step on an int8 block-quantised state (Cq, Cs), as
    state_q8_encode returns it.  Returns (h, Cq', Cs', n', m').  Cq_out /
    Cs_out may be Cq / Cs (updated in place)."""
    torch = _torch()
    if q.dim() != 3:
        raise ValueError("q must be (B, NH, DHQK)")
    B, NH, DK = q.shape
    DV = v.shape[-1]
    _check(q, "q", (B, NH, DK))
    _check(k, "k", (B, NH, DK), q.dtype)
    _check(v, "v", (B, NH, DV), q.dtype)
    _check(i_pre, "i_pre", (B, NH), torch.float32)
    _check(f_pre, "f_pre", (B, NH), torch.float32)
    _check(Cq, "Cq", (B, NH, DK, DV), torch.int8)
    _check(Cs, "Cs", (B, NH, DV // 64, DK), torch.float32)
    _check(n, "n", (B, NH, DK), torch.float32)
    _check(m, "m", (B, NH), torch.float32)
    h_dtype = torch.float32 if h_dtype is None else h_dtype
    hcode = MLSTM_BF16 if h_dtype == torch.bfloat16 else MLSTM_F32
    desc = make_desc(B, NH, 1, DK, DV, 64, qkv_dtype=_dtype_code(q), h_dtype=hcode, gate=gate,
                     qk_scale=0.0 if qk_scale is None else float(qk_scale), eps=float(eps))
    dev = q.device
    h = torch.empty((B, NH, DV), dtype=h_dtype, device=dev)
    if Cq_out is None:
        Cq_out = torch.empty((B, NH, DK, DV), dtype=torch.int8, device=dev)
    if Cs_out is None:
        Cs_out = torch.empty((B, NH, DV // 64, DK), dtype=torch.float32, device=dev)
    _check(Cq_out, "Cq_out", (B, NH, DK, DV), torch.int8)
    _check(Cs_out, "Cs_out", (B, NH, DV // 64, DK), torch.float32)
    if gate != "sig":
        if n_out is None:
            n_out = torch.empty((B, NH, DK), dtype=torch.float32, device=dev)
        if m_out is None:
            m_out = torch.empty((B, NH), dtype=torch.float32, device=dev)
    st = lib().mlstm_recurrent_step_q8(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(i_pre), _ptr(f_pre), _ptr(Cq), _ptr(Cs), _ptr(n),
        _ptr(m), _ptr(h), _ptr(Cq_out), _ptr(Cs_out), _ptr(n_out), _ptr(m_out), _stream())
    if st:
        raise MlstmError(st, "mlstm_recurrent_step_q8")
    return h, Cq_out, Cs_out, n_out, m_out


def mlstm_chunkwise(q, k, v, i_pre, f_pre, C0=None, n0=None, m0=None, *, chunk_size: int, gate: str = "exp",
                    precision: str = "split", qk_scale: Optional[float] = None, eps: float = 0.0,
                    tile_lq: int = 0, tile_lkv: int = 0, schedule: str = "auto"):
    """H of the forward pass as a torch autograd function: the forward runs
    mlstm_chunkwise_fw, the backward mlstm_chunkwise_bw (gradients for q, k,
    v, i_pre, f_pre and, when given, C0, n0, m0).  H is float32.  The final
    state is not returned here: no gradient enters through it.  With the exp
    gate the forward also keeps the per-row m and normaliser, and the
    backward takes them with H instead of recomputing the intra-chunk pass
    (mlstm_chunkwise_bw_saved)."""
    torch = _torch()
    kw = dict(chunk_size=chunk_size, gate=gate, precision=precision, qk_scale=qk_scale, eps=eps,
              tile_lq=tile_lq, tile_lkv=tile_lkv)

    class _Fn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q_, k_, v_, i_, f_, C0_, n0_, m0_):
            if gate == "sig":
                H = mlstm_chunkwise_fw(q_, k_, v_, i_, f_, C0_, n0_, m0_, schedule=schedule,
                                       return_final_state=False, **kw)[0]
                ctx.save_for_backward(q_, k_, v_, i_, f_, C0_, n0_, m0_)
            else:
                H, _, _, _, m_rows, den_rows = mlstm_chunkwise_fw(q_, k_, v_, i_, f_, C0_, n0_, m0_,
                                                                  schedule=schedule, return_final_state=False,
                                                                  return_rows=True, **kw)
                ctx.save_for_backward(q_, k_, v_, i_, f_, C0_, n0_, m0_, H, m_rows, den_rows)
            return H

        @staticmethod
        def backward(ctx, dH):
            q_, k_, v_, i_, f_, C0_, n0_, m0_ = ctx.saved_tensors[:8]
            saved = tuple(ctx.saved_tensors[8:]) or None
            want_state = any(ctx.needs_input_grad[5:])
            g = mlstm_chunkwise_bw(q_, k_, v_, i_, f_, dH.contiguous().float(), C0_, n0_, m0_,
                                   state_grads=want_state, saved=saved, **kw)
            cast = lambda t, like: None if t is None else t.to(like.dtype)
            return (cast(g["dQ"], q_), cast(g["dK"], k_), cast(g["dV"], v_), g["d_i"], g["d_f"],
                    g.get("dC0") if C0_ is not None else None, g.get("dn0") if n0_ is not None else None,
                    g.get("dm0") if m0_ is not None else None)

    return _Fn.apply(q, k, v, i_pre, f_pre, C0, n0, m0)
