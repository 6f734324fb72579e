#!/usr/bin/env python3
"""Throughput of the Falcon chunk-parallel forward pass on one MI355X.

A step is one falcon_fwd call over one batch of synthetic input (the whole
hot path: features, chunk operators, state carry and output).  The default
workload is Falcon-1, batch 8, 12 heads, T = 1024, d_k = d_v = 64, C = 64,
bf16 inputs and fp32 state.  Inputs are resident in HBM before timing.

Prints one JSON line (see the keys below).  `--gpus N` with N > 1 exits:
this library runs on one GPU only.  `--backward` times the Falcon-1 backward
pass (falcon_bwd) on the workload instead, with its own metric.
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
F32_PEAK_TFLOPS = 157.3        # MI355X dense fp32 MFMA, vendor figure


def algorithmic_bytes(w) -> int:
    """Unavoidable traffic of one forward call: q, k, v read once, o written
    once (io dtype), beta and lambda read once (fp32), final state written
    once (fp32).  A single-token decode step continues a carried state, so
    it also reads the incoming state once (S, x_next, the tail pairs) and
    writes x_next and the tail."""
    esz = 2 if w.dtype == "bf16" else 4
    n = w.batch * w.heads * w.seqlen
    beta_cols = w.dv if w.variant in ("F2", "F2A") else 1
    total = (n * (2 * w.dk + 2 * w.dv) * esz + n * (beta_cols + 1) * 4
             + w.batch * w.heads * w.dk * w.dv * 4)
    if w.seqlen == 1:
        h = w.window - 1
        total += w.batch * w.heads * 4 * (w.dk * w.dv + 2 * w.dk + 2 * h * (w.dk + w.dv))
    return total


METRIC_BWD = "Falcon-1 backward tokens/s (B*H*T) + % of HBM roofline"


def algorithmic_bytes_bwd(w) -> int:
    """Unavoidable traffic of one backward call: q, k, v and d_o read once
    and d_q, d_k, d_v written once (io dtype); beta and lambda read and
    d_beta, d_lambda written once (fp32); per head the initial state and
    the final state's gradient read and the initial state's gradient written
    (fp32).  The forward's intermediates are recomputed, not counted."""
    esz = 2 if w.dtype == "bf16" else 4
    n = w.batch * w.heads * w.seqlen
    return (n * (2 * w.dk + 2 * w.dv + 2 * w.dk + w.dv) * esz + n * 4 * 4
            + w.batch * w.heads * w.dk * w.dv * 4 * 3)


def algorithmic_flops_bwd(w) -> int:
    """Matrix products of the chunk-parallel backward per head and 64-token
    chunk (C = 64, K = d_k, V = d_v; triangular products counted at half):
    the transfer records 3C^2 K + 3C^2 V + 2C K^2 + 6C K V, the two state
    carries 4 K^2 V, the token gradients 6C^2 K + 8C^2 V + 10 C K V; all in
    fp32."""
    C, K, V = 64, w.dk, w.dv
    per_chunk = 9 * C * C * K + 11 * C * C * V + 2 * C * K * K + 16 * C * K * V + 4 * K * K * V
    return w.batch * w.heads * (-(-w.seqlen // C)) * per_chunk


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
           "F2A": C * (w.dk + w.dv) + 4 * w.dk * w.dv,
           "F3A": C * (w.dk + w.dv) + 4 * w.dk * w.dv}[w.variant]
    return w.batch * w.heads * w.seqlen * per


_SHARED = {}   # inputs of the CPU baseline, inherited by its forked workers


def _limit_blas():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass


def _oracle_shard(heads, reps):
    import numpy as np
    """Run the oracle `reps` times on a subset of the flattened heads; returns
    the wall time."""
    import oracle
    w, flat = _SHARED["w"], _SHARED["flat"]
    part = {n: a[heads][None] for n, a in flat.items()}
    state = None
    if w.seqlen == 1:   # a decode step continues the same carried state as the GPU run
        from linear_recurrent_weight_amd.inputs import decode_state
        ds = decode_state(w)
        BH = w.batch * w.heads
        pick = lambda a: a.reshape(BH, *a.shape[2:])[heads].astype(np.float64)
        state = oracle.OracleState(S=pick(ds["S"]), fresh=False, x_next=pick(ds["x_next"]),
                                   tail_x=pick(ds["tail_x"]), tail_y=pick(ds["tail_y"]))
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.falcon_forward(w.variant, part["q"], part["k"], part["v"], part["beta"], part["lam"],
                              window=w.window, eps=w.eps, eps_gamma=w.eps_gamma, eps_rms=w.eps_rms,
                              state_in=state)
    return time.perf_counter() - t0


def _shard_worker(heads, reps, conn):
    _limit_blas()
    conn.send(_oracle_shard(heads, reps))
    conn.close()


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def cpu_baseline(w, inp, min_seconds: float):
    """The fp64 oracle, as it is, on this host's cores: P worker processes
    (P = the cores this process may run on), each with one BLAS thread, share
    the (batch, head) pairs of the workload and run them `reps` times; the
    single-core rate is one worker's share run alone.  Must run before the GPU
    is initialised (the workers are forked)."""
    import multiprocessing as mp
    import numpy as np
    P = len(os.sched_getaffinity(0))
    BH = w.batch * w.heads
    _SHARED["w"] = w
    _SHARED["flat"] = {n: a.reshape(BH, *a.shape[2:]) for n, a in inp.items()}
    shards = [s for s in np.array_split(np.arange(BH), min(P, BH)) if len(s)]
    # single core: the first share, repeated for at least a third of the budget
    _limit_blas()
    t1 = _oracle_shard(shards[0], 1)
    reps1 = max(1, int(np.ceil(min_seconds / 3 / max(t1, 1e-9))))
    if reps1 > 1:
        t1 = _oracle_shard(shards[0], reps1) / reps1
    one_core = len(shards[0]) * w.seqlen / t1
    # all cores: every share in its own process, repeated for about the budget
    reps = max(1, int(np.ceil(min_seconds / max(t1, 1e-9))))
    ctx = mp.get_context("fork")
    procs = []
    t0 = time.perf_counter()
    for sh in shards:
        r, wr = ctx.Pipe(duplex=False)
        pr = ctx.Process(target=_shard_worker, args=(sh, reps, wr))
        pr.start()
        procs.append((pr, r))
    for pr, r in procs:
        r.recv()
        pr.join()
    wall = time.perf_counter() - t0
    return {"value": w.tokens * reps / wall, "unit": "tokens/s", "cores": len(shards), "kind": "oracle",
            "sample": (f"whole workload x{reps}: {len(shards)} processes over the {BH} heads, "
                       f"1 BLAS thread each, {wall:.1f} s wall; fp64 NumPy token recurrence"),
            "single_core_value": one_core,
            "single_core_sample": f"{len(shards[0])} heads x {w.seqlen} tokens x{reps1}, one process",
            "cpu_model": cpu_model()}


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


def kernel_names(lib, w, backward=False):
    """Names of the kernels one call of workload `w` launches (host-side plan),
    of falcon_bwd with `backward`."""
    from linear_recurrent_weight_amd import falcon as fb
    if backward:
        a = fb.make_bwd_args(dtype=w.dtype, batch=w.batch, heads=w.heads, seqlen=w.seqlen, dk=w.dk, dv=w.dv)
        fn = lib.falcon_bwd_kernel_name
    else:
        a = fb.make_args(variant=w.variant, dtype=w.dtype, batch=w.batch, heads=w.heads, seqlen=w.seqlen,
                         dk=w.dk, dv=w.dv, chunk=w.chunk, window=w.window)
        fn = lib.falcon_kernel_name
    names = []
    while True:
        nm = fn(ctypes.byref(a), len(names))
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


def read_profile_value(workload: str, kernels, key: str):
    """A `key: value` line of the committed profile summary, or None when it
    is missing or the kernel sources changed since the counters were read."""
    import re
    from linear_recurrent_weight_amd.build import sources_digest
    path = profile_path(workload, kernels)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^%s: (\S+)$" % re.escape(key), text, re.M)
    d = re.search(r"^sources_digest: (\S+)$", text, re.M)
    if not m or not d or d.group(1) != sources_digest(kernels):
        return None
    return float(m.group(1))


def mfma_summary(mfma_db: str, stats_db: str, n_cu: int = 256, simd_per_cu: int = 4,
                 clock_mhz: float = 2400.0) -> str:
    """Markdown lines for one `--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA
    GRBM_GUI_ACTIVE` run: per kernel, the matrix-core busy fraction
    SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs x kernel cycles), with the kernel cycles
    from the kernel-trace average duration at the peak engine clock (a lower
    bound on the busy fraction when the clock runs below its peak)."""
    top = {name: avg for name, _, avg, _ in
           _db_rows(stats_db, "select name, total_calls, average, total_duration from top_kernels")}
    rows = _db_rows(mfma_db, "select kernel_name, counter_name, count(*), avg(value) from counters_collection "
                    "group by kernel_name, counter_name")
    per = {}
    for k, c, n, v in rows:
        per.setdefault(k, {})[c] = (n, v)
    lines = ["", "## Matrix-core use (`--pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA GRBM_GUI_ACTIVE`)", "",
             f"busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / ({n_cu} CUs x {simd_per_cu} SIMDs x average duration "
             f"x {clock_mhz:.0f} MHz)", "",
             "| kernel | dispatches | SQ_VALU_MFMA_BUSY_CYCLES | SQ_INSTS_MFMA | GRBM_GUI_ACTIVE | avg duration (us) | MFMA busy fraction |",
             "|---|---:|---:|---:|---:|---:|---:|"]
    fracs = {}
    for k in sorted(per):
        if "falcon::" not in k:
            continue
        busy = per[k].get("SQ_VALU_MFMA_BUSY_CYCLES", (0, float("nan")))
        insts = per[k].get("SQ_INSTS_MFMA", (0, float("nan")))[1]
        grbm = per[k].get("GRBM_GUI_ACTIVE", (0, float("nan")))[1]
        dur = top.get(k)
        frac = busy[1] / (n_cu * simd_per_cu * dur * clock_mhz) if dur else float("nan")
        fracs[k] = (frac, dur or 0.0)
        lines.append(f"| `{k[:110]}` | {busy[0]} | {busy[1]:.4g} | {insts:.4g} | {grbm:.4g} | "
                     f"{dur if dur else float('nan'):.3f} | {frac:.4f} |")
    tot = sum(d for _, d in fracs.values())
    call = sum(f * d for f, d in fracs.values()) / tot if tot else float("nan")
    lines += ["", f"mfma_busy_frac_per_call: {call:.6f}", ""]
    return "\n".join(lines)


def make_set(w, inp, dev, dt, fb, lib, ws=None):
    """One resident set of device inputs and outputs and the C arguments of a
    call on it; the workspace `ws` (scratch, not an input or output) is
    shared by the sets when given, as a caller reuses one scratch buffer."""
    import torch
    t = {n: torch.from_numpy(inp[n]).to(dev) for n in ("q", "k", "v", "beta", "lam")}
    for n in ("q", "k", "v"):
        t[n] = t[n].to(dt).contiguous()
    t["o"] = torch.empty(w.batch, w.heads, w.seqlen, w.dv, dtype=dt, device=dev)
    st = fb.FalconState.empty(w.batch, w.heads, w.dk, w.dv, w.window, dev)
    t["state"] = st
    t["st_c"] = st.to_c()
    st_in = None
    if w.seqlen == 1:   # a decode step continues a carried state
        from linear_recurrent_weight_amd.inputs import decode_state
        ds = decode_state(w)
        t["state_in"] = fb.FalconState(*(torch.from_numpy(ds[n]).to(dev) for n in
                                         ("S", "x_next", "tail_x", "tail_y")),
                                       n_tail=ds["n_tail"], fresh=False)
        t["st_in_c"] = st_in = t["state_in"].to_c()
    cargs = fb.make_args(variant=w.variant, dtype=w.dtype, batch=w.batch, heads=w.heads,
                         seqlen=w.seqlen, dk=w.dk, dv=w.dv, chunk=w.chunk, window=w.window,
                         eps=w.eps, eps_gamma=w.eps_gamma, eps_rms=w.eps_rms, q=t["q"], k=t["k"],
                         v=t["v"], beta=t["beta"], lam=t["lam"], o=t["o"], state_out=t["st_c"],
                         state_in=st_in)
    nbytes = lib.falcon_fwd_workspace_size(ctypes.byref(cargs))
    t["ws"] = ws if ws is not None else torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    cargs.workspace = t["ws"].data_ptr()
    cargs.workspace_bytes = t["ws"].numel()
    t["args"] = cargs
    t["bytes"] = sum(x.numel() * x.element_size() for n, x in t.items()
                     if n in ("q", "k", "v", "beta", "lam", "o"))
    t["bytes"] += sum(x.numel() * x.element_size() for x in (st.S, st.x_next, st.tail_x, st.tail_y))
    if "state_in" in t:
        t["bytes"] += sum(x.numel() * x.element_size() for x in
                          (t["state_in"].S, t["state_in"].x_next, t["state_in"].tail_x, t["state_in"].tail_y))
    return t


LLC_BYTES = 256 << 20   # MI355X last-level (Infinity) cache
MAX_SETS = 256          # at most this many resident input sets (a tiny workload stays in the cache)


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
    ap.add_argument("--rocprof-summary", nargs="+", metavar="DB",
                    help="STATS_DB FETCH_DB WRITE_DB [MFMA_DB]: write the markdown summary of "
                         "these rocprofv3 runs to profiles/ (no GPU needed)")
    ap.add_argument("--rocprof-command", default="", help="the commands that made the databases")
    ap.add_argument("--backward", action="store_true",
                    help="time the Falcon-1 backward pass (falcon_bwd) on the workload")
    args = ap.parse_args()
    prof_name = args.workload + ("_bwd" if args.backward else "")
    if args.rocprof_summary:
        from linear_recurrent_weight_amd import falcon as fb
        from linear_recurrent_weight_amd.inputs import WORKLOADS
        dbs = args.rocprof_summary
        if len(dbs) not in (3, 4):
            ap.error("--rocprof-summary takes 3 or 4 databases")
        names = kernel_names(fb.load_library(), WORKLOADS[args.workload], args.backward)
        text = rocprof_summary(prof_name, names, *dbs[:3], args.rocprof_command)
        if len(dbs) == 4:
            text += mfma_summary(dbs[3], dbs[0])
        path = profile_path(prof_name, names)
        os.makedirs(os.path.dirname(path), exist_ok=True)
        with open(path, "w") as f:
            f.write(text)
        print(path)
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; --gpus must be 1"}))
        return 2

    import numpy as np

    from linear_recurrent_weight_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    inp = make_inputs(w)
    if args.backward:
        return bwd_main(args, w, inp, prof_name)
    # the oracle's CPU baseline forks workers: it runs before the GPU is touched
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, inp, args.cpu_seconds)

    import torch

    from linear_recurrent_weight_amd import falcon as fb

    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    lib = fb.load_library()
    # enough resident sets of inputs and outputs that consecutive calls cannot
    # find them in the last-level cache (more than twice its size together);
    # one workspace serves every set
    sets = [make_set(w, inp, dev, dt, fb, lib)]
    while len(sets) * sets[0]["bytes"] <= 2 * LLC_BYTES and len(sets) < MAX_SETS:
        sets.append(make_set(w, inp, dev, dt, fb, lib, ws=sets[0]["ws"]))
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    pargs = [ctypes.byref(t["args"]) for t in sets]

    def step(i):
        rc = lib.falcon_fwd(pargs[i % len(pargs)], sh)
        if rc != 0:
            raise fb.FalconError(rc, lib)

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    def timed(rotate: bool):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        e0.record(stream)
        for i in range(args.steps):
            step(i if rotate else 0)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps, time.perf_counter() - w0

    # timed region: K back-to-back calls, events on the library's stream;
    # the headline rotates over the resident sets, the warm figure repeats
    # one set (its inputs then partly stay in the last-level cache)
    ms, wall = timed(True)
    ms_warm, _ = timed(False)

    # per-kernel durations inside the call (events between the launches)
    names = []
    while True:
        nm = lib.falcon_kernel_name(pargs[0], len(names))
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
        got = lib.falcon_fwd_profile(pargs[r % len(pargs)], sh, arr, nk + 1)
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
    mfma_busy = read_profile_value(args.workload, names, "mfma_busy_frac_per_call")
    form = ("single-token decode step" if w.seqlen == 1 else
            "token-recurrent" if w.chunk == 0 else f"chunk-parallel (C = {w.chunk})")
    win = f", window {w.window}" if w.window > 1 else ""
    dominant = max(per_kernel, key=per_kernel.get) if per_kernel else None

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
        "config": {"workload": f"{w.name}: Falcon-{w.variant[1:]} {form} forward{win}",
                   "variant": w.variant, "batch": w.batch, "heads": w.heads, "seq_len": w.seqlen,
                   "dk": w.dk, "dv": w.dv, "chunk": w.chunk, "window": w.window,
                   "io_dtype": w.dtype, "state_dtype": "f32", "parallelism": "none (1 GPU)",
                   "resident_sets": len(sets)},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "falcon_fwd call (" + " + ".join(names) + ")",
                     "dominant_kernel": dominant,
                     "launch_ms": ms, "algorithmic_bytes": alg_bytes},
        "mfma": {"algorithmic_tflops": alg_flops / (ms * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                 "frac": alg_flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                 "counter_busy_frac": mfma_busy},
        "kernels_ms": per_kernel,
        "warm_cache_ms_per_step": ms_warm,
        "wall_s_timed": wall,
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)
    return 0



def bwd_cpu_baseline(w, inp, min_seconds: float):
    """The fp64 backward oracle, as it is, on one core over a bounded sample
    of heads (whole sequences), scaled to head-tokens per second."""
    import numpy as np
    from oracle.falcon_backward import falcon1_backward
    _limit_blas()
    BH = w.batch * w.heads
    rng = np.random.default_rng(0)
    flat = {n: a.reshape(BH, *a.shape[2:]) for n, a in inp.items()}
    done, heads, t0 = 0, 0, time.perf_counter()
    while time.perf_counter() - t0 < min_seconds and heads < BH:
        part = {n: a[heads:heads + 1][None] for n, a in flat.items()}
        d_o = rng.standard_normal((1, 1, w.seqlen, w.dv))
        falcon1_backward(part["q"], part["k"], part["v"], part["beta"], part["lam"], d_o,
                         eps=w.eps, eps_gamma=w.eps_gamma, eps_rms=w.eps_rms)
        done += w.seqlen
        heads += 1
    wall = time.perf_counter() - t0
    return {"value": done / wall, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{heads} of {BH} heads x {w.seqlen} tokens, one process, {wall:.1f} s; "
                      "fp64 NumPy reverse token recurrence", "cpu_model": cpu_model()}


def bwd_main(args, w, inp, prof_name) -> int:
    """Time falcon_bwd (Falcon-1 backward) on workload w: K calls over
    resident input sets, events on the library's stream, per-kernel times
    from falcon_bwd_profile."""
    import numpy as np
    if w.variant != "F1" or w.window != 1:
        print(json.dumps({"error": "the backward pass covers Falcon-1 only"}))
        return 2
    cpu = None if args.no_cpu_baseline else bwd_cpu_baseline(w, inp, args.cpu_seconds)
    import torch
    from linear_recurrent_weight_amd import falcon as fb
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    lib = fb.load_library()
    gen = torch.Generator(device="cpu").manual_seed(5)
    ws = None

    def make_bwd_set():
        nonlocal ws
        t = {n: torch.from_numpy(inp[n]).to(dev) for n in ("q", "k", "v", "beta", "lam")}
        for n in ("q", "k", "v"):
            t[n] = t[n].to(dt).contiguous()
        B, H, T, dk, dv = w.batch, w.heads, w.seqlen, w.dk, w.dv
        t["d_o"] = torch.randn(B, H, T, dv, generator=gen).to(dev).to(dt)
        t["d_S_out"] = torch.randn(B, H, dk, dv, generator=gen).to(dev)
        for n, shape, d in (("d_q", (B, H, T, dk), dt), ("d_k", (B, H, T, dk), dt), ("d_v", (B, H, T, dv), dt),
                            ("d_beta", (B, H, T), torch.float32), ("d_lam", (B, H, T), torch.float32),
                            ("d_S_in", (B, H, dk, dv), torch.float32)):
            t[n] = torch.empty(*shape, dtype=d, device=dev)
        a = fb.make_bwd_args(dtype=w.dtype, batch=B, heads=H, seqlen=T, dk=dk, dv=dv, eps=w.eps,
                             eps_gamma=w.eps_gamma, eps_rms=w.eps_rms, q=t["q"], k=t["k"], v=t["v"],
                             beta=t["beta"], lam=t["lam"], d_o=t["d_o"], d_S_out=t["d_S_out"],
                             d_q=t["d_q"], d_k=t["d_k"], d_v=t["d_v"], d_beta=t["d_beta"],
                             d_lam=t["d_lam"], d_S_in=t["d_S_in"])
        nbytes = lib.falcon_bwd_workspace_size(ctypes.byref(a))
        if ws is None:
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel()
        t["args"] = a
        t["bytes"] = sum(x.numel() * x.element_size() for n, x in t.items() if n != "args")
        return t

    sets = [make_bwd_set()]
    while len(sets) * sets[0]["bytes"] <= 2 * LLC_BYTES and len(sets) < MAX_SETS:
        sets.append(make_bwd_set())
    stream = torch.cuda.current_stream(dev)
    sh = ctypes.c_void_p(stream.cuda_stream)
    pargs = [ctypes.byref(t["args"]) for t in sets]

    def step(i):
        rc = lib.falcon_bwd(pargs[i % len(pargs)], sh)
        if rc != 0:
            raise fb.FalconError(rc, lib)

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    wall = time.perf_counter() - w0

    names = kernel_names(lib, w, backward=True)
    nk = len(names)
    reps = max(5, min(args.steps, 50))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(reps)]
    for row in evs:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for r in range(reps):
        arr = (ctypes.c_void_p * (nk + 1))(*[e.cuda_event for e in evs[r]])
        got = lib.falcon_bwd_profile(pargs[r % len(pargs)], sh, arr, nk + 1)
        if got != nk:
            raise RuntimeError(f"falcon_bwd_profile launched {got} kernels, expected {nk}")
    torch.cuda.synchronize()
    per_kernel = {n: float(np.mean([evs[r][i].elapsed_time(evs[r][i + 1]) for r in range(reps)]))
                  for i, n in enumerate(names)}
    alg = algorithmic_bytes_bwd(w)
    gbs = alg / (ms * 1e-3) / 1e9
    chunked = names[0] == "bwd_ops"
    flops = algorithmic_flops_bwd(w)
    tfs = flops / (ms * 1e-3) / 1e12
    if chunked:   # fp32 products: the fp32 matrix-core peak binds before HBM
        roof = {"bound": "mfma", "achieved": tfs, "peak": F32_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": tfs / F32_PEAK_TFLOPS, "algorithmic_flops": flops,
                "hbm": {"achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}}
    else:
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": gbs / HBM_PEAK_GBS}
    roof.update({"traffic": read_traffic(prof_name, names),
                 "kernel": "falcon_bwd call (" + " + ".join(names) + ")",
                 "dominant_kernel": max(per_kernel, key=per_kernel.get), "launch_ms": ms,
                 "algorithmic_bytes": alg})
    form = "chunk-parallel (C = 64)" if chunked else "token-recurrent"
    line = {
        "metric": METRIC_BWD, "value": w.tokens / (ms * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: Falcon-1 backward, {form}", "variant": w.variant,
                   "batch": w.batch, "heads": w.heads, "seq_len": w.seqlen, "dk": w.dk, "dv": w.dv,
                   "io_dtype": w.dtype, "state_dtype": "f32", "parallelism": "none (1 GPU)",
                   "resident_sets": len(sets)},
        "roofline": roof,
        "kernels_ms": per_kernel, "wall_s_timed": wall,
    }
    if cpu is not None:
        line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)
    return 0

if __name__ == "__main__":
    sys.exit(main())
