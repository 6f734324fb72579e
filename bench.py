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
    args = ap.parse_args()
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
    traffic = None
    tpath = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                         f"traffic_{args.workload}.json")
    if os.path.exists(tpath):
        try:
            tj = json.load(open(tpath))
            from linear_recurrent_weight_amd.build import sources_digest
            if tj.get("sources_digest") == sources_digest():
                traffic = tj.get("bytes_per_call")
        except Exception:
            traffic = None

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
