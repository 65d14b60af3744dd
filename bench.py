"""Benchmark of the chunkwise mLSTM forward pass on one MI355X.

A step is one full forward pass (inter-chunk states, then the intra-chunk
parallel stage) over one batch of synthetic inputs that are already resident
in GPU memory.  Default workload: 7B-shaped heads, bf16 inputs, B=8 NH=8
S=8192 DHQK=256 DHV=512 chunk=256, exponential input gate, fp32 H.

Prints ONE JSON line: throughput (tokens/s = B*S per step), the roofline
figures of the dominant kernel measured with HIP events on the launch stream,
and a CPU baseline: the float64 recurrent oracle timed on a bounded sample of
the same workload on this host.
"""
from __future__ import annotations

import argparse
import json
import multiprocessing as mp
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 matrix-core peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 matrix-core peak
PEAK_FP64_TFLOPS = 78.6     # MI355X dense fp64 matrix-core (and vector) peak
METRIC = "mLSTM chunkwise fwd tokens/s + TFLOP/s (% bf16 MFMA peak), 7B-shaped heads"
CSRC = os.path.join(ROOT, "xlstm_mlstm_chunkwise_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


# The source files whose bytes decide each profiled kernel's code: its own
# file (kernel and launch), the gate-terms kernel it reads from, and the
# shared device helpers.
KERNEL_SOURCES = {
    "walk": ("walk_kernel.hip", "gates_kernel.hip", "device_common.h", "pair_store.h"),
    "states": ("states2_kernel.hip", "gates_kernel.hip", "device_common.h"),
    "hintra": ("hintra2_kernel.hip", "device_common.h", "pair_store.h"),
    "blocked": ("states2_kernel.hip", "hintra2_kernel.hip", "gates_kernel.hip", "device_common.h", "pair_store.h"),
    "step": ("step_kernel.hip", "device_common.h"),
    "step_q8": ("step_kernel.hip", "device_common.h"),
    "states_int16": ("states2_kernel.hip", "gates_kernel.hip", "device_common.h"),
    "hintra_int16": ("hintra2_kernel.hip", "device_common.h", "pair_store.h"),
    "states_f64": ("f64_mfma_kernels.hip", "f64_common.h", "device_common.h"),
    "hintra_f64": ("f64_mfma_kernels.hip", "f64_common.h", "device_common.h"),
    "grads": ("bw_kernels.hip", "kernels.h", "tile_order.h", "device_common.h"),
}


def csrc_sha256(kernel: str = None) -> str:
    """Hash of the kernel's source files (name and bytes, in a fixed order),
    or of every source file when no kernel is named."""
    import hashlib
    names = KERNEL_SOURCES[kernel] if kernel else sorted(
        n for n in os.listdir(CSRC) if n.endswith((".hip", ".h")))
    h = hashlib.sha256()
    for name in names:
        h.update(name.encode())
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def algorithmic_bytes(w, h_bytes: int) -> dict:
    """HBM bytes each stage must move per launch, per token and head, times
    the B*NH*S units of one launch (the chunk states that pass between the
    stages are not counted: moving them is a property of the two-stage
    design, not of the method).

    states: reads K, V and both gate rows, plus the initial state when given;
            writes the final state.
    hintra: reads Q, K, V and the gate rows; writes H.
    walk:   the fused walker: hintra's bytes plus the initial and final state.
    blocked: the whole blocked-schedule call (both stages per block of
            chunks), the same algorithmic bytes as the walker."""
    el = 2 if w.qkv_dtype == "bf16" else 4
    per_state = (w.DHQK * w.DHV + (0 if w.gate == "sig" else w.DHQK + 1)) * 4
    units = w.BH * w.S
    init = w.BH * per_state if w.init_state else 0
    return {
        "states": units * ((w.DHQK + w.DHV) * el + 8) + init + w.BH * per_state,
        "hintra": units * ((2 * w.DHQK + w.DHV) * el + 8 + w.DHV * h_bytes),
        "walk": units * ((2 * w.DHQK + w.DHV) * el + 8 + w.DHV * h_bytes) + init + w.BH * per_state,
        "blocked": units * ((2 * w.DHQK + w.DHV) * el + 8 + w.DHV * h_bytes) + init + w.BH * per_state,
    }


def chunk_state_bytes(w, codes: str = "split") -> int:
    """Bytes of the chunk states the two stages pass through HBM (written by
    the states stage, read by the intra-chunk stage): 4 bytes a value, or
    with int16 codes 2 bytes a value plus a 4-byte scale per 512 values."""
    nc = -(-w.S // w.chunk)
    c_bytes = w.DHQK * w.DHV * 4 if codes == "split" else w.DHQK * w.DHV * 2 + (w.DHQK * w.DHV // 512) * 4
    per_state = c_bytes + (0 if w.gate == "sig" else (w.DHQK + 1) * 4)
    return w.BH * (nc + 1) * per_state


def recorded_traffic(workload: str, kernel: str, tile_lq, fname: str = None) -> tuple:
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current kernel sources; else (None, reason)."""
    path = os.path.join(PROFILES, fname or f"traffic_{workload}.md")
    if not os.path.exists(path):
        return None, "no counter summary"
    rec = {}
    for line in open(path):
        m = re.match(r"\s*traffic-record:\s*(.*)", line)
        if m:
            kv = dict(x.split("=", 1) for x in m.group(1).split())
            if kv.get("kernel") == kernel and kv.get("tile_lq", "default") == str(tile_lq or "default") \
                    and kv.get("workload", workload) == workload:
                rec = kv
    if not rec:
        return None, "kernel not in counter summary"
    if rec.get("source_sha256") != csrc_sha256(kernel):
        return None, "kernel sources changed since the counters were taken"
    b = float(rec["fetch_kib"]) * 1024 * float(rec["fetch_scale"]) + \
        float(rec["write_kib"]) * 1024 * float(rec["write_scale"])
    return b, os.path.relpath(path, ROOT)


def _oracle_head(args):
    """One head of the recurrent oracle on a sequence prefix (CPU baseline)."""
    name, b, h, S = args
    import numpy as np
    from oracle import recurrent_fw
    from workloads import WORKLOADS, head_inputs
    w = WORKLOADS[name]
    x = head_inputs(w, b, h)
    t0 = time.perf_counter()
    kw = {}
    if "C0" in x and w.gate == "exp":
        kw = dict(C0=x["C0"], n0=x["n0"], m0=x["m0"])
    elif "C0" in x:
        kw = dict(C0=x["C0"])
    recurrent_fw(*[x[k][:S].astype(np.float64) for k in ("q", "k", "v", "i", "f")], gate=w.gate, **kw)
    return time.perf_counter() - t0


# Worker processes of the CPU baseline: every core of this process's
# affinity set, up to 16 (the host cores that come with one GPU).
MAX_CPU_WORKERS = 16


def host_cpu() -> dict:
    """The host's CPU model (from /proc/cpuinfo) and its affinity core count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cores": len(os.sched_getaffinity(0))}


def cpu_baseline(name: str, budget_s: float) -> dict:
    """Time the float64 recurrent oracle on a bounded sample of the workload.

    Heads are spread over a process pool (one BLAS thread per worker).  The
    sample is n_heads full-length heads (or a prefix of one head when a
    single head exceeds the budget); tokens/s counts NH heads per token."""
    from workloads import WORKLOADS
    w = WORKLOADS[name]
    cores = max(1, min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS))
    # probe the per-step cost on a short prefix
    probe_steps = min(w.S, 256)
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    ctx = mp.get_context("spawn")
    with ctx.Pool(cores) as pool:
        dt = pool.map(_oracle_head, [(name, 0, 0, probe_steps)])[0]
        per_step = dt / probe_steps
        head_s = per_step * w.S
        if head_s * 1.0 <= budget_s * cores:
            n_heads = int(max(1, min(w.BH, (budget_s * cores) // head_s)))
            n_heads = max(1, (n_heads // cores) * cores) if n_heads >= cores else n_heads
            steps = w.S
        else:
            n_heads = 1
            steps = int(max(probe_steps, budget_s / per_step))
        heads = [(i // w.NH, i % w.NH) for i in range(n_heads)]
        t0 = time.perf_counter()
        pool.map(_oracle_head, [(name, b, h, steps) for (b, h) in heads])
        wall = time.perf_counter() - t0
    tokens = n_heads * steps / w.NH
    used = min(cores, n_heads)
    return {"value": tokens / wall, "unit": "tokens/s", "cores": used, "kind": "oracle",
            "sample": (f"float64 recurrent oracle, {n_heads} of {w.BH} heads x {steps} of {w.S} steps "
                       f"({w.name}), {used} worker processes with 1 BLAS thread each (affinity cores "
                       f"up to {MAX_CPU_WORKERS}); tokens/s counts {w.NH} heads per token; wall {wall:.1f} s"),
            **host_cpu()}


def w_dk(desc) -> int:
    return int(desc.DHQK)


def path_dtype(mt, desc, precision: str) -> str:
    """Arithmetic of the kernels that run for `desc`: the 16-bit type of the
    matrix-core operands (x2 when the computed operand is split hi + lo) and
    the accumulation type."""
    fam = mt.kernel_family(desc)
    if fam == mt.MLSTM_FAMILY_F64:
        # fp64 matrix cores for key widths up to 256, fp64 vector ALUs at 512
        return "f64-mfma/f64-acc" if w_dk(desc) <= 256 else "f64-valu/f64-acc"
    if desc.qkv_dtype == mt.MLSTM_F32:
        return "f32-mfma/f32-acc"
    return "bf16x2-mfma/f32-acc" if precision == "split" else "bf16-mfma/f32-acc"


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="bf16_7b_s8192")
    ap.add_argument("--precision", default="split", choices=["split", "f16", "f64"])
    ap.add_argument("--h-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--tile-lq", type=int, default=None, help="override the workload's intra-chunk row tile")
    ap.add_argument("--schedule", default="auto", choices=["auto", "two_stage", "fused", "blocked"],
                    help="kernels of the forward pass (see mlstm_schedule_t)")
    ap.add_argument("--state-codes", default="split", choices=["split", "int16"],
                    help="chunk-state hand-off of the two stages (see mlstm_state_codes_t)")
    ap.add_argument("--block-chunks", type=int, default=0,
                    help="chunks per block of the blocked schedule (0: the library's choice)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle wall time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode", action="store_true",
                    help="time the recurrent step (one token per head and call) on the workload's heads "
                         "instead of the forward pass")
    ap.add_argument("--state", default="f32", choices=["f32", "q8"],
                    help="with --decode: the state format (float32, or int8 codes with a float32 scale per "
                         "64-value block)")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (mlstm_chunkwise_bw) on the workload instead of the forward pass")
    ap.add_argument("--saved-forward", action="store_true",
                    help="with --backward (exp gate): time mlstm_chunkwise_bw_saved, which takes the forward's H "
                         "and per-row m and normaliser (from one untimed mlstm_chunkwise_fw_rows call) instead "
                         "of recomputing the intra-chunk pass")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, --steps times (the "
                         "reference reading for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch
    import xlstm_mlstm_chunkwise_amd as mt
    from workloads import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t = time.perf_counter()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t) / args.steps
        print(json.dumps({"copy_bytes": 4 * n, "steps": args.steps, "ms_per_copy": dt * 1e3,
                          "GB/s (read+write)": 8 * n / dt / 1e9}), flush=True)
        return 0
    mt.lib()  # fail loudly if the HIP library is missing
    w = WORKLOADS[args.workload]
    if args.decode:
        return bench_decode(args, w, mt, torch, np)
    if args.tile_lq is not None:
        w = w.replace(tile_lq=args.tile_lq)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t_gen = time.perf_counter()
    x = make_inputs(w)
    qd = torch.bfloat16 if w.qkv_dtype == "bf16" else torch.float32

    def up(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=dt)

    q, k, v = up(x["q"], qd), up(x["k"], qd), up(x["v"], qd)
    i_pre, f_pre = up(x["i"], torch.float32), up(x["f"], torch.float32)
    sig = w.gate == "sig"
    C0 = up(x["C0"], torch.float32) if "C0" in x else None
    n0 = up(x["n0"], torch.float32) if ("n0" in x and not sig) else None
    m0 = up(x["m0"], torch.float32) if ("m0" in x and not sig) else None
    del x
    print(f"# inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    if args.backward:
        return bench_backward(args, w, mt, torch, np, (q, k, v, i_pre, f_pre, C0, n0, m0))
    h_dtype = torch.bfloat16 if args.h_dtype == "bf16" else torch.float32
    H = torch.empty((w.B, w.NH, w.S, w.DHV), dtype=h_dtype, device=dev)
    desc = mt.make_desc(w.B, w.NH, w.S, w.DHQK, w.DHV, w.chunk,
                        qkv_dtype=mt.MLSTM_BF16 if w.qkv_dtype == "bf16" else mt.MLSTM_F32,
                        h_dtype=mt.MLSTM_BF16 if args.h_dtype == "bf16" else mt.MLSTM_F32,
                        gate=w.gate, precision=args.precision, tile_lq=w.tile_lq, tile_lkv=w.tile_lkv,
                        schedule=args.schedule, block_chunks=args.block_chunks, state_codes=args.state_codes)
    family = mt.kernel_family(desc)
    fused = family in (mt.MLSTM_FAMILY_FUSED, mt.MLSTM_FAMILY_BLOCKED)
    one_call = "blocked" if family == mt.MLSTM_FAMILY_BLOCKED else "walk"
    ws = torch.empty(max(1, mt.workspace_bytes(desc)), dtype=torch.uint8, device=dev)
    kw = dict(chunk_size=w.chunk, gate=w.gate, h_dtype=h_dtype, precision=args.precision,
              tile_lq=w.tile_lq, tile_lkv=w.tile_lkv, schedule=args.schedule, workspace=ws, out=H,
              block_chunks=args.block_chunks, state_codes=args.state_codes)

    def step():
        return mt.mlstm_chunkwise_fw(q, k, v, i_pre, f_pre, C0, n0, m0, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_wall) * 1e3 / args.steps
    ms = e0.elapsed_time(e1) / args.steps

    # Per-kernel durations with events on the launch stream.  Two-stage: the
    # same two launches, issued through the stage entry points (on the same
    # workspace) with events between them.  Fused: the walker call (its gate
    # terms pass, about half a percent of it, included).
    import ctypes
    L = mt.lib()
    ws_bytes = ws.numel()
    sptr = ctypes.c_void_p(stream.cuda_stream)

    def p(t):
        return None if t is None else t.data_ptr()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for it in range(args.steps):
        ev[it][0].record(stream)
        if fused:
            step()
            ev[it][1].record(stream)
            continue
        st = L.mlstm_fw_states(ctypes.byref(desc), p(k), p(v), p(i_pre), p(f_pre), p(C0), p(n0), p(m0),
                               p(ws), ws_bytes, None, None, None, sptr)
        ev[it][1].record(stream)
        st2 = L.mlstm_fw_hintra(ctypes.byref(desc), p(q), p(k), p(v), p(i_pre), p(f_pre), p(ws), ws_bytes,
                                p(H), None, None, sptr)
        ev[it][2].record(stream)
        if st or st2:
            raise mt.MlstmError(st or st2, "stage call")
    torch.cuda.synchronize()
    t_first = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    t_second = 0.0 if fused else sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps

    tokens = w.B * w.S
    flops = mt.flops(w.B, w.NH, w.S, w.DHQK, w.DHV, w.chunk)
    tflops = flops / (ms * 1e-3) / 1e12
    # The dominant kernel is priced against HBM: its algorithmic bytes per
    # launch over its mean launch time.  (Its FLOP/byte ratio sits far below
    # the bf16 matrix-core ridge point of 2500/8 flop per byte.)
    abytes = algorithmic_bytes(w, 2 if args.h_dtype == "bf16" else 4)
    # algorithmic FLOPs of each stage: states = K^T.V (2 DK DV per token-head);
    # intra = Q.C + causal Q.K^T and P.V
    f_stage = {"states": 2.0 * w.DHQK * w.DHV * w.BH * w.S,
               "hintra": (2.0 * w.DHQK * w.DHV + (w.chunk + 1) * (w.DHQK + w.DHV)) * w.BH * w.S}
    f_stage["walk"] = f_stage["blocked"] = f_stage["states"] + f_stage["hintra"]
    t_stage = {one_call: t_first} if fused else {"states": t_first, "hintra": t_second}
    f_stage = {k_: f_stage[k_] for k_ in t_stage}
    dominant = max(t_stage, key=t_stage.get)
    t_dom = t_stage[dominant]
    f64_mode = mt.kernel_family(desc) == mt.MLSTM_FAMILY_F64
    codes = args.state_codes if not fused else "split"
    traffic, traffic_src = recorded_traffic(
        w.name, dominant + ("_f64" if f64_mode else "") + ("_int16" if codes == "int16" else ""), args.tile_lq)
    if f64_mode:
        # The float64 kernels do about 50 FLOP per algorithmic byte, above the
        # fp64 ridge point (78.6 TFLOP/s over 8 TB/s, ~10 FLOP/byte): they are
        # priced against the fp64 peak with their algorithmic FLOPs.
        ach = f_stage[dominant] / (t_dom * 1e-3) / 1e12
        roof = {"kernel": dominant, "bound": "mfma", "achieved": ach, "peak": PEAK_FP64_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / PEAK_FP64_TFLOPS, "traffic": traffic,
                "algorithmic_flops": f_stage[dominant], "algorithmic_bytes": abytes[dominant],
                "traffic_source": traffic_src}
    else:
        ach = abytes[dominant] / (t_dom * 1e-3) / 1e9
        roof = {"kernel": dominant, "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ach / PEAK_HBM_GBS, "traffic": traffic,
                "algorithmic_bytes": abytes[dominant], "traffic_source": traffic_src}
    out = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": path_dtype(mt, desc, args.precision),
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "NH": w.NH, "S": w.S, "DHQK": w.DHQK, "DHV": w.DHV,
                   "chunk": w.chunk, "gate": w.gate, "qkv_dtype": w.qkv_dtype, "h_dtype": args.h_dtype,
                   "precision": args.precision, "tile_lq": w.tile_lq or 64,
                   "schedule": {"walk": "fused", "blocked": "blocked"}[one_call] if fused else "two_stage",
                   "state_codes": codes},
        "tflops": tflops,
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
        "wall_ms_per_step": wall_ms,
        "kernels_ms": t_stage,
        "kernels_GBps": {k: abytes[k] / (t_stage[k] * 1e-3) / 1e9 for k in t_stage},
        "chunk_state_bytes": chunk_state_bytes(w, codes),
        "kernels_TFLOPs": {k: f_stage[k] / (t_stage[k] * 1e-3) / 1e12 for k in t_stage},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w.name, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


def cpu_baseline_backward(name: str, budget_s: float, S: int = 2048) -> dict:
    """Time the float64 gradient oracle (torch autograd over the quadratic
    form) on a bounded sample: heads cut to their first S positions, run one
    after another in this process on torch's CPU threads (no worker
    processes: this one already holds the GPU); tokens/s counts NH heads per
    token.  The quadratic form's cost per token grows with S, so the figure
    holds for this prefix length only."""
    import numpy as np
    import torch
    from oracle import grad_fw
    from workloads import WORKLOADS, head_inputs
    w = WORKLOADS[name]
    cores = max(1, min(len(os.sched_getaffinity(0)), MAX_CPU_WORKERS))
    torch.set_num_threads(cores)
    dH = np.random.default_rng(7).standard_normal((1, S, w.DHV))
    n_heads, t_used = 0, 0.0
    while n_heads < w.BH and t_used < budget_s:
        x = head_inputs(w, n_heads // w.NH, n_heads % w.NH)
        t0 = time.perf_counter()
        grad_fw(*[x[k][None, :S].astype(np.float64) for k in ("q", "k", "v", "i", "f")], dH, gate=w.gate)
        t_used += time.perf_counter() - t0
        n_heads += 1
    return {"value": n_heads * S / w.NH / t_used, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": (f"float64 gradient oracle (autograd over the quadratic form), {n_heads} of {w.BH} heads "
                       f"x the first {S} of {w.S} positions ({w.name}), one process on {cores} torch threads; "
                       f"tokens/s counts {w.NH} heads per token; oracle time {t_used:.1f} s"), **host_cpu()}


def bench_backward(args, w, mt, torch, np, inputs) -> int:
    """The backward pass on the whole workload: mlstm_chunkwise_bw (forward
    quantities recomputed, then the gradient kernels) with a float32 dH drawn
    N(0, 1), timed with HIP events around back-to-back calls; then the two
    stages apart (mlstm_bw_recompute, mlstm_bw_grads) for the stage times.
    The roofline prices the gradient stage's algorithmic FLOPs against the
    dense peak of the matrix cores it runs on: bf16 for bf16 inputs (the
    computed operands go as hi + lo pairs, so 2-3 passes per product), fp32
    for float32 inputs."""
    import ctypes
    q, k, v, i_pre, f_pre, C0, n0, m0 = inputs
    dev = q.device
    sig = w.gate == "sig"
    dH = torch.randn((w.B, w.NH, w.S, w.DHV), generator=torch.Generator(device=dev).manual_seed(31),
                     device=dev, dtype=torch.float32)
    desc = mt.make_desc(w.B, w.NH, w.S, w.DHQK, w.DHV, w.chunk,
                        qkv_dtype=mt.MLSTM_BF16 if w.qkv_dtype == "bf16" else mt.MLSTM_F32,
                        h_dtype=mt.MLSTM_F32, gate=w.gate, precision=args.precision, tile_lq=w.tile_lq,
                        tile_lkv=w.tile_lkv, schedule="two_stage")
    f32 = dict(dtype=torch.float32, device=dev)
    dQ, dK = torch.empty((w.B, w.NH, w.S, w.DHQK), **f32), torch.empty((w.B, w.NH, w.S, w.DHQK), **f32)
    dV = torch.empty((w.B, w.NH, w.S, w.DHV), **f32)
    d_i, d_f = torch.empty((w.B, w.NH, w.S), **f32), torch.empty((w.B, w.NH, w.S), **f32)
    dC0 = torch.empty((w.B, w.NH, w.DHQK, w.DHV), **f32) if C0 is not None else None
    dn0 = torch.empty((w.B, w.NH, w.DHQK), **f32) if (C0 is not None and not sig) else None
    dm0 = torch.empty((w.B, w.NH), **f32) if (C0 is not None and not sig) else None
    ws_bytes = mt.bw_workspace_bytes(desc)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    L = mt.lib()
    P = lambda t: None if t is None else t.data_ptr()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    grads = (P(dH), P(dQ), P(dK), P(dV), P(d_i), P(d_f), P(dC0), P(dn0), P(dm0))

    saved = args.saved_forward and not sig
    if saved:
        # the forward's outputs, once, untimed (the automatic schedule: the
        # fused walker where it covers the shape)
        H, _, _, _, m_rows, den_rows = mt.mlstm_chunkwise_fw(
            q, k, v, i_pre, f_pre, C0, n0, m0, chunk_size=w.chunk, gate=w.gate, precision=args.precision,
            tile_lq=w.tile_lq or 0, tile_lkv=w.tile_lkv or 0, return_final_state=False, return_rows=True)
        torch.cuda.synchronize()

    def whole():
        if saved:
            st = L.mlstm_chunkwise_bw_saved(ctypes.byref(desc), P(q), P(k), P(v), P(i_pre), P(f_pre), P(C0), P(n0),
                                            P(m0), P(H), P(m_rows), P(den_rows), *grads, P(ws), ws_bytes, sp)
        else:
            st = L.mlstm_chunkwise_bw(ctypes.byref(desc), P(q), P(k), P(v), P(i_pre), P(f_pre), P(C0), P(n0),
                                      P(m0), *grads, P(ws), ws_bytes, sp)
        if st:
            raise mt.MlstmError(st, "mlstm_chunkwise_bw_saved" if saved else "mlstm_chunkwise_bw")

    for _ in range(args.warmup):
        whole()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        whole()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    t_rec = t_grads = None
    if not saved:
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
        for it in range(args.steps):
            ev[it][0].record(stream)
            st = L.mlstm_bw_recompute(ctypes.byref(desc), P(q), P(k), P(v), P(i_pre), P(f_pre), P(C0), P(n0), P(m0),
                                      P(dH), P(ws), ws_bytes, sp)
            ev[it][1].record(stream)
            st2 = L.mlstm_bw_grads(ctypes.byref(desc), P(q), P(k), P(v), P(i_pre), P(f_pre), P(C0), P(n0),
                                   *grads, P(ws), ws_bytes, sp)
            ev[it][2].record(stream)
            if st or st2:
                raise mt.MlstmError(st or st2, "backward stage call")
        torch.cuda.synchronize()
        t_rec = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
        t_grads = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    # the backward cuts the sequence into chunks of min(max(chunk, 64), Lmax)
    # rows, Lmax = 128 when B NH DHQK / 64 >= 256, else 256
    # (mlstm_chunkwise_bw): its algorithmic FLOPs are those of that cut
    bw_chunk = min(max(w.chunk, 64), 128 if w.B * w.NH * (w.DHQK // 64) >= 256 else 256)
    flops = mt.bw_flops(w.B, w.NH, w.S, w.DHQK, w.DHV, bw_chunk)
    # the gradient stage alone; from saved forward outputs there is no stage
    # call of its own, so the whole call is priced
    ach = flops / ((ms if saved else t_grads) * 1e-3) / 1e12
    # bf16 inputs: bf16 matrix cores (computed operands as hi + lo pairs);
    # float32 inputs: fp32 matrix cores.  Each is priced at its own peak.
    bf16_path = w.qkv_dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16_path else PEAK_FP32_TFLOPS
    # HBM bytes of the gradient stage per call, from the committed counter
    # summary while it matches the current sources (the saved call has no
    # stage of its own to price)
    traffic, traffic_src = (None, "no stage of its own") if saved else recorded_traffic(
        f"backward_{w.name}", "grads", None, fname="traffic_backward_7b.md")
    grads_dtype = "bf16x2-mfma/f32-acc" if bf16_path else "f32-mfma/f32-acc"
    out = {
        "metric": f"mLSTM chunkwise backward tokens/s, {w.gate} gate ({w.name})"
                  + (", from the forward's saved H and rows" if saved else ""),
        "value": w.B * w.S / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": grads_dtype + " (gradient kernels); recompute " + path_dtype(mt, desc, args.precision),
        "data": "synthetic",
        "config": {"workload": f"backward_{w.name}", "B": w.B, "NH": w.NH, "S": w.S, "DHQK": w.DHQK,
                   "DHV": w.DHV, "chunk": w.chunk, "backward_chunk": bw_chunk, "gate": w.gate,
                   "qkv_dtype": w.qkv_dtype, "dH": "float32", "precision": args.precision},
        # the stage calls of mlstm_chunkwise_bw (the saved call has none)
        "stages_ms": None if saved else {"recompute": t_rec, "grads": t_grads},
        "saved_forward": saved,
        "grads_TFLOPs": ach,
        "roofline": {"kernel": "whole backward from saved forward outputs (mlstm_chunkwise_bw_saved)" if saved
                     else "gradient stage (mlstm_bw_grads)", "bound": "mfma", "achieved": ach,
                     "peak": peak, "unit": "TFLOP/s", "frac": ach / peak, "traffic": traffic,
                     "algorithmic_flops": flops, "traffic_source": traffic_src},
    }
    if not args.no_cpu_baseline:
        print("# timing the CPU gradient oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_backward(w.name, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


def bench_decode(args, w, mt, torch, np) -> int:
    """The recurrent step on the workload's heads (B, NH, DHQK, DHV, dtype,
    gate): one token for each of the B sequences per call, each state updated
    in place, calls issued back to back through the C entry point with their
    arguments built once (so the host issues faster than the device runs).
    Cold (the headline): the calls cycle through 16 separate states, 540 MB at
    the 7B-shaped heads, more than the 256 MB Infinity Cache, so each call
    reads and writes its state in HBM -- one token through 16 layers.  Warm:
    one state, which can stay in the Infinity Cache between calls.  Isolated:
    one call after a 512 MiB read, bracketed by events alone (includes the
    dispatch latency of a lone kernel).  --state q8 runs the step on int8
    codes with a float32 scale per 64-value block (mlstm_recurrent_step_q8);
    its states are encoded from the same float32 draw."""
    import ctypes
    dev = torch.device("cuda", 0)
    rng = np.random.default_rng(2024)
    B, NH, DK, DV = w.B, w.NH, w.DHQK, w.DHV
    sig = w.gate == "sig"
    qd = torch.bfloat16 if w.qkv_dtype == "bf16" else torch.float32
    NSTATE = 16

    def up(a, dt):
        return torch.from_numpy(np.ascontiguousarray(a)).to(device=dev, dtype=dt)

    q = up(rng.standard_normal((B, NH, DK)), qd)
    k = up(rng.standard_normal((B, NH, DK)), qd)
    v = up(rng.standard_normal((B, NH, DV)), qd)
    i_pre = up(rng.standard_normal((B, NH)), torch.float32)
    f_pre = up(2.0 + 4.0 * rng.random((B, NH)), torch.float32)
    C0 = up(0.1 * rng.standard_normal((B, NH, DK, DV)), torch.float32)
    q8 = args.state == "q8"
    if q8:
        Cq0, Cs0 = mt.state_q8_encode(C0)
        Cs = [(Cq0.clone(), Cs0.clone()) for _ in range(NSTATE)]
    else:
        Cs = [C0.clone() for _ in range(NSTATE)]
    # n and m alternate between two buffers per state (outputs may not alias inputs)
    ns = [[None, None] if sig else [up(rng.random((B, NH, DK)), torch.float32), torch.empty(B, NH, DK, device=dev)]
          for _ in range(NSTATE)]
    ms = [[None, None] if sig else [up(rng.standard_normal((B, NH)), torch.float32), torch.empty(B, NH, device=dev)]
          for _ in range(NSTATE)]
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    h = torch.empty(B, NH, DV, dtype=torch.float32, device=dev)
    desc = mt.make_desc(B, NH, 1, DK, DV, 64, qkv_dtype=mt.MLSTM_BF16 if w.qkv_dtype == "bf16" else mt.MLSTM_F32,
                        gate=w.gate)
    fn = mt.lib().mlstm_recurrent_step_q8 if q8 else mt.lib().mlstm_recurrent_step
    P = lambda t: None if t is None else t.data_ptr()
    stream = torch.cuda.current_stream()
    sp = ctypes.c_void_p(stream.cuda_stream)
    st_in = (lambda j: [P(Cs[j][0]), P(Cs[j][1])]) if q8 else (lambda j: [P(Cs[j])])
    cargs = [[[ctypes.byref(desc), P(q), P(k), P(v), P(i_pre), P(f_pre)] + st_in(j) + [P(ns[j][a]), P(ms[j][a]),
               P(h)] + st_in(j) + [P(ns[j][1 - a]), P(ms[j][1 - a]), sp] for a in (0, 1)] for j in range(NSTATE)]
    it = [0] * NSTATE

    def call(j):
        st = fn(*cargs[j][it[j] & 1])
        if st:
            raise mt.MlstmError(st, "mlstm_recurrent_step")
        it[j] += 1

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(states):
        for r in range(args.warmup):
            call(states[r % len(states)])
        torch.cuda.synchronize()
        e0.record(stream)
        for r in range(args.steps):
            call(states[r % len(states)])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    cold_ms = timed(list(range(NSTATE)))
    warm_ms = timed([0])
    iso = []
    for _ in range(args.steps):
        flush.sum()
        e0.record(stream)
        call(0)
        e1.record(stream)
        torch.cuda.synchronize()
        iso.append(e0.elapsed_time(e1))
    iso_ms = float(np.median(iso))
    el = 2 if w.qkv_dtype == "bf16" else 4
    BH = B * NH
    state_bytes = BH * DK * DV * (1 + 4 / 64) if q8 else BH * DK * DV * 4
    abytes = (2 * state_bytes + (0 if sig else 2 * BH * (DK + 1) * 4) + BH * (2 * DK + DV) * el
              + BH * DV * 4 + 2 * BH * 4)
    ach = abytes / (cold_ms * 1e-3) / 1e9
    traffic, traffic_src = recorded_traffic(f"decode_{w.name}", "step_q8" if q8 else "step", None,
                                            "traffic_decode_7b.md")
    out = {
        "metric": f"mLSTM recurrent step (decode) tokens/s, {w.gate} gate, heads of {w.name}"
                  + (", int8 block-quantised state" if q8 else ""),
        "value": B / (cold_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": cold_ms,
        "warm_ms_per_step": warm_ms,
        "warm_tokens_per_s": B / (warm_ms * 1e-3),
        "isolated_ms_per_step": iso_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int8x64-state/f32-update" if q8 else "f32-state") + f"/{w.qkv_dtype}-qkv",
        "data": "synthetic",
        "config": {"workload": f"decode_{w.name}" + ("_q8" if q8 else ""), "B": B, "NH": NH, "DHQK": DK, "DHV": DV, "gate": w.gate,
                   "qkv_dtype": w.qkv_dtype,
                   "state": ("int8 codes + float32 scale per 64 values, updated in place" if q8
                             else "float32, updated in place"),
                   "states_cycled": NSTATE},
        "roofline": {"kernel": "step", "bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": ach / PEAK_HBM_GBS, "traffic": traffic, "algorithmic_bytes": abytes,
                     "traffic_source": traffic_src},
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
