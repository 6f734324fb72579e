#!/usr/bin/env python3
"""Throughput of the Falcon chunk-parallel forward pass on one MI355X.

A step is one falcon_fwd call over one batch of synthetic input (the whole
hot path: features, chunk operators, state carry and output).  The default
workload is Falcon-1, batch 8, 12 heads, T = 1024, d_k = d_v = 64, C = 64,
bf16 inputs and fp32 state.  Inputs are resident in HBM before timing.

Prints one JSON line (see the keys below).  `--gpus N` with N > 1 exits:
this build runs on one GPU only.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

METRIC = "Falcon chunk-parallel fwd tokens/s (B*H*T) + % of bf16 MFMA / HBM roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure


def algorithmic_bytes(w) -> int:
    """Unavoidable traffic of one forward call: q, k, v read once, o written
    once (io dtype), beta and lambda read once (fp32), final state written
    once (fp32)."""
    esz = 2 if w.dtype == "bf16" else 4
    n = w.batch * w.heads * w.seqlen
    beta_cols = w.dv if w.variant == "F2" else 1
    return (n * (2 * w.dk + 2 * w.dv) * esz + n * (beta_cols + 1) * 4
            + w.batch * w.heads * w.dk * w.dv * 4)


def algorithmic_flops(w) -> int:
    """Per-token work of the chunk form, triangle-aware: Falcon-1
    2C(dk+dv) + 6 dk dv (single residual solve); Falcon-2 2C dk + 3C dv +
    6 dk dv; Falcon-1A / 3A C dk + C dv + 4 dk dv (window terms are lower
    order)."""
    C = w.chunk or 64
    per = {"F1": 2 * C * (w.dk + w.dv) + 6 * w.dk * w.dv,
           "F2": 2 * C * w.dk + 3 * C * w.dv + 6 * w.dk * w.dv,
           "F3": 2 * C * (w.dk + w.dv) * w.window + 6 * w.dk * w.dv,
           "F1A": C * (w.dk + w.dv) + 4 * w.dk * w.dv,
           "F3A": C * (w.dk + w.dv) + 4 * w.dk * w.dv}[w.variant]
    return w.batch * w.heads * w.seqlen * per


def cpu_baseline(w, inp, min_seconds: float):
    """The fp64 oracle, as it is, on this host: the whole workload, repeated
    until at least `min_seconds` of CPU time, single-threaded."""
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        ctx = None
    import oracle
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.falcon_forward(w.variant, inp["q"], inp["k"], inp["v"], inp["beta"], inp["lam"],
                              window=w.window, eps=w.eps, eps_gamma=w.eps_gamma, eps_rms=w.eps_rms)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    if ctx is not None:
        ctx.unregister() if hasattr(ctx, "unregister") else None
    return {"value": w.tokens * reps / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"whole workload x{reps} ({dt:.1f} s), fp64 NumPy token recurrence, 1 thread"}


COPY_KERNEL = "__amd_rocclr_copyBuffer"   # the runtime's device copy (--copy-calibration)
COPY_BYTES = 256 << 20


def _db_rows(db, sql):
    import sqlite3
    con = sqlite3.connect(db)
    try:
        return list(con.execute(sql))
    finally:
        con.close()


def rocprof_summary(workload: str, kernels, stats_db: str, fetch_db: str, write_db: str,
                    command: str) -> str:
    """Markdown summary of three rocprofv3 runs of this script on one
    workload: kernel-trace statistics, then FETCH_SIZE and WRITE_SIZE per
    dispatch (KiB), each scaled by what the same counter reads for the plain
    device copy of COPY_BYTES that --copy-calibration adds."""
    from linear_recurrent_weight_amd.build import sources_digest
    top = _db_rows(stats_db, "select name, total_calls, average, total_duration from top_kernels")
    lines = [f"# rocprofv3 summary: workload {workload}", "",
             "Commands (run from the repository root on one MI355X; the .db files stay out of the tree):",
             "", "```", command.strip(), "```", "",
             "## Kernel trace (`--kernel-trace --stats`)", "",
             "| kernel | calls | average (us) |", "|---|---:|---:|"]
    for name, calls, avg, _ in top:
        lines.append(f"| `{name[:110]}` | {calls} | {avg:.3f} |")

    def counter(db, cname):
        rows = _db_rows(db, "select kernel_name, count(*), avg(value) from counters_collection "
                        f"where counter_name = '{cname}' group by kernel_name")
        return {k: (n, v) for k, n, v in rows}
    def copy_reading(db, cname):
        # the largest dispatch of the runtime's copy kernel is the calibration
        # copy (the inputs' uploads use the same kernel)
        rows = _db_rows(db, "select count(*), max(value) from counters_collection "
                        f"where counter_name = '{cname}' and kernel_name = '{COPY_KERNEL}'")
        return (rows[0][0], rows[0][1]) if rows and rows[0][0] else None
    fetch, write = counter(fetch_db, "FETCH_SIZE"), counter(write_db, "WRITE_SIZE")
    for table, db, cname in ((fetch, fetch_db, "FETCH_SIZE"), (write, write_db, "WRITE_SIZE")):
        r = copy_reading(db, cname)
        if r:
            table[COPY_KERNEL] = r
    f_copy = (COPY_BYTES / 1024) / fetch[COPY_KERNEL][1] if COPY_KERNEL in fetch else None
    w_copy = (COPY_BYTES / 1024) / write[COPY_KERNEL][1] if COPY_KERNEL in write else None
    lines += ["", "## HBM traffic (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`)", "",
              f"Calibration: a device copy of {COPY_BYTES >> 20} MiB reads "
              f"{fetch.get(COPY_KERNEL, (0, float('nan')))[1]:.0f} KiB by FETCH_SIZE and writes "
              f"{write.get(COPY_KERNEL, (0, float('nan')))[1]:.0f} KiB by WRITE_SIZE: scale factors "
              f"{f_copy if f_copy is None else round(f_copy, 3)} (fetch) and "
              f"{w_copy if w_copy is None else round(w_copy, 3)} (write).", "",
              "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | calibrated bytes / dispatch |",
              "|---|---:|---:|---:|---:|"]
    ours = {}
    for k in sorted(set(fetch) | set(write)):
        if "falcon::" not in k:
            continue
        fk, wk = fetch.get(k, (0, 0.0))[1], write.get(k, (0, 0.0))[1]
        b = (fk * (f_copy or 1.0) + wk * (w_copy or 1.0)) * 1024
        ours[k] = b
        lines.append(f"| `{k[:110]}` | {fetch.get(k, (0,))[0]} | {fk:.0f} | {wk:.0f} | {b:.4g} |")
    total = sum(ours.values())
    lines += ["", f"traffic_bytes_per_call: {total:.0f}",
              f"sources_digest: {sources_digest(kernels)}", ""]
    return "\n".join(lines)


def kernel_names(lib, w):
    """Names of the kernels one call of workload `w` launches (host-side plan)."""
    from linear_recurrent_weight_amd import falcon as fb
    a = fb.make_args(variant=w.variant, dtype=w.dtype, batch=w.batch, heads=w.heads, seqlen=w.seqlen,
                     dk=w.dk, dv=w.dv, chunk=w.chunk, window=w.window)
    names = []
    while True:
        nm = lib.falcon_kernel_name(ctypes.byref(a), len(names))
        if nm is None:
            return names
        names.append(nm.decode())


def profile_path(workload: str, kernels) -> str:
    """profiles/<kernel source(s)>_<workload>.md"""
    from linear_recurrent_weight_amd.build import KERNEL_SOURCES
    stems = []
    for k in kernels:
        stem = KERNEL_SOURCES[k].rsplit(".", 1)[0]
        if stem not in stems:
            stems.append(stem)
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                        "+".join(stems) + f"_{workload}.md")


def read_traffic(workload: str, kernels):
    """Calibrated HBM bytes per call from the committed summary, or None when
    it is missing or the kernel sources changed since the counters were read."""
    import re
    from linear_recurrent_weight_amd.build import sources_digest
    path = profile_path(workload, kernels)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^traffic_bytes_per_call: (\d+)$", text, re.M)
    d = re.search(r"^sources_digest: (\S+)$", text, re.M)
    if not m or not d or d.group(1) != sources_digest(kernels):
        return None
    return int(m.group(1))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--rocprof-summary", nargs=3, metavar=("STATS_DB", "FETCH_DB", "WRITE_DB"),
                    help="print a markdown summary of three rocprofv3 runs (no GPU needed)")
    ap.add_argument("--rocprof-command", default="", help="the commands that made the databases")
    args = ap.parse_args()
    if args.rocprof_summary:
        from linear_recurrent_weight_amd import falcon as fb
        from linear_recurrent_weight_amd.inputs import WORKLOADS
        names = kernel_names(fb.load_library(), WORKLOADS[args.workload])
        text = rocprof_summary(args.workload, names, *args.rocprof_summary, args.rocprof_command)
        path = profile_path(args.workload, names)
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as f:
            f.write(text)
        print(path)
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        return 2

    import numpy as np
    import torch

    from linear_recurrent_weight_amd import falcon as fb
    from linear_recurrent_weight_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(inp[n]).to(dev).to(dt).contiguous() for n in ("q", "k", "v"))
    beta = torch.from_numpy(inp["beta"]).to(dev).contiguous()
    lam = torch.from_numpy(inp["lam"]).to(dev).contiguous()
    o = torch.empty(w.batch, w.heads, w.seqlen, w.dv, dtype=dt, device=dev)
    st = fb.FalconState.empty(w.batch, w.heads, w.dk, w.dv, w.window, dev)
    st_c = st.to_c()
    lib = fb.load_library()
    cargs = fb.make_args(variant=w.variant, dtype=w.dtype, batch=w.batch, heads=w.heads,
                         seqlen=w.seqlen, dk=w.dk, dv=w.dv, chunk=w.chunk, window=w.window,
                         eps=w.eps, eps_gamma=w.eps_gamma, eps_rms=w.eps_rms, q=q, k=k, v=v,
                         beta=beta, lam=lam, o=o, state_out=st_c)
    nbytes = lib.falcon_fwd_workspace_size(ctypes.byref(cargs))
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    cargs.workspace = ws.data_ptr()
    cargs.workspace_bytes = ws.numel()
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    pargs = ctypes.byref(cargs)

    def step():
        rc = lib.falcon_fwd(pargs, sh)
        if rc != 0:
            raise fb.FalconError(rc, lib)

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K back-to-back calls, events on the library's stream
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = e0.elapsed_time(e1) / args.steps

    # per-kernel durations inside the call (events between the launches)
    names = []
    while True:
        nm = lib.falcon_kernel_name(pargs, len(names))
        if nm is None:
            break
        names.append(nm.decode())
    nk = len(names)
    reps = max(10, min(args.steps, 100))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(reps)]
    for row in evs:            # torch creates the HIP event at its first record
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for r in range(reps):
        arr = (ctypes.c_void_p * (nk + 1))(*[e.cuda_event for e in evs[r]])
        got = lib.falcon_fwd_profile(pargs, sh, arr, nk + 1)
        if got != nk:
            raise RuntimeError(f"falcon_fwd_profile launched {got} kernels, expected {nk}")
    torch.cuda.synchronize()
    per_kernel = {n: float(np.mean([evs[r][i].elapsed_time(evs[r][i + 1]) for r in range(reps)]))
                  for i, n in enumerate(names)}

    tokens = w.tokens
    alg_bytes = algorithmic_bytes(w)
    alg_flops = algorithmic_flops(w)
    achieved_gbs = alg_bytes / (ms * 1e-3) / 1e9
    traffic = read_traffic(args.workload, names)

    line = {
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
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: Falcon-{w.variant[1:]} chunk-parallel forward",
                   "variant": w.variant, "batch": w.batch, "heads": w.heads, "seq_len": w.seqlen,
                   "dk": w.dk, "dv": w.dv, "chunk": w.chunk, "window": w.window,
                   "io_dtype": w.dtype, "state_dtype": "f32", "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "falcon_fwd call (" + " + ".join(names) + ")",
                     "launch_ms": ms, "algorithmic_bytes": alg_bytes},
        "mfma": {"algorithmic_tflops": alg_flops / (ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                 "frac": alg_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS},
        "kernels_ms": per_kernel,
        "wall_s_timed": wall,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
