"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
the fp64 oracle on the same seeded inputs, and compare."""
from __future__ import annotations

import numpy as np

import oracle
from linear_recurrent_weight_amd.inputs import Workload, make_inputs

TOL_BF16 = 2e-2   # max relative error, bf16 inputs with fp32 state
TOL_F32 = 1e-5    # max relative error, all-fp32 mode


def tol_for(w: Workload) -> float:
    return TOL_F32 if w.dtype == "f32" else TOL_BF16


def to_device(inp: dict, w: Workload):
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    out = {}
    for n in ("q", "k", "v"):
        out[n] = torch.from_numpy(inp[n]).to(dev).to(dt).contiguous()
    out["beta"] = torch.from_numpy(inp["beta"]).to(dev).contiguous()
    out["lam"] = torch.from_numpy(inp["lam"]).to(dev).contiguous()
    return out


def run_gpu(w: Workload, dev_inp: dict, chunk=None, state=None, want_state=True):
    from linear_recurrent_weight_amd import falcon as fb
    o, st = fb.fwd(dev_inp["q"], dev_inp["k"], dev_inp["v"], dev_inp["beta"], dev_inp["lam"],
                   variant=w.variant, chunk=w.chunk if chunk is None else chunk, window=w.window,
                   eps=w.eps, eps_gamma=w.eps_gamma, eps_rms=w.eps_rms, state=state,
                   want_state=want_state)
    return o, st


def gpu_state_to_oracle(st, heads=None) -> oracle.OracleState:
    S = st.S.double().cpu().numpy()
    B, H, dk, dv = S.shape
    sel = slice(None) if heads is None else heads
    S = S.reshape(B * H, dk, dv)[sel]
    xn = st.x_next.double().cpu().numpy().reshape(B * H, dk)[sel]
    n = st.n_tail
    tx = st.tail_x.double().cpu().numpy()
    ty = st.tail_y.double().cpu().numpy()
    h = tx.shape[2]
    tx = tx.reshape(B * H, h, dk)[sel][:, h - n:] if n else np.zeros((S.shape[0], 0, dk))
    ty = ty.reshape(B * H, h, dv)[sel][:, h - n:] if n else np.zeros((S.shape[0], 0, dv))
    return oracle.OracleState(S=S, fresh=bool(st.fresh), x_next=None if st.fresh else xn,
                              tail_x=tx, tail_y=ty)


def oracle_heads(w: Workload, inp: dict, heads, state_in=None, trace=False):
    """Run the oracle on a subset of flattened (b,h) heads."""
    B, H = w.batch, w.heads

    def pick(a):
        a = a.reshape(B * H, *a.shape[2:])[heads]
        return a[None]
    res = oracle.falcon_forward(w.variant, pick(inp["q"]), pick(inp["k"]), pick(inp["v"]),
                                pick(inp["beta"]), pick(inp["lam"]), window=w.window, eps=w.eps,
                                eps_gamma=w.eps_gamma, eps_rms=w.eps_rms, state_in=state_in,
                                trace=trace)
    return res


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over leading slices of max|got - ref| / max|ref| (last two axes
    are one slice: [T, dv] for outputs, [dk, dv] for states)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    g = got.reshape(-1, got.shape[-2] * got.shape[-1])
    r = ref.reshape(-1, ref.shape[-2] * ref.shape[-1])
    den = np.maximum(np.abs(r).max(axis=1), 1e-30)
    return float((np.abs(g - r).max(axis=1) / den).max())


def compare(w: Workload, heads, o_gpu, st_gpu, o_ref, st_ref):
    """Returns (err_o, err_S) on the sampled heads."""
    B, H = w.batch, w.heads
    og = o_gpu.double().cpu().numpy().reshape(B * H, w.seqlen, w.dv)[heads]
    err_o = max_rel_err(og, o_ref.reshape(-1, w.seqlen, w.dv)) if w.seqlen else 0.0
    err_s = 0.0
    if st_gpu is not None:
        sg = st_gpu.S.double().cpu().numpy().reshape(B * H, w.dk, w.dv)[heads]
        err_s = max_rel_err(sg, st_ref.S)
    return err_o, err_s


def sample_heads(w: Workload, n: int) -> np.ndarray:
    N = w.batch * w.heads
    if N <= n:
        return np.arange(N)
    return np.unique(np.linspace(0, N - 1, n).round().astype(int))


def small(variant, dtype="f32", B=2, H=3, T=150, dk=64, dv=64, chunk=0, window=1, seed=7, **kw):
    """A small synthetic workload of the given shape (same recipe as the
    named workloads)."""
    return Workload(f"small-{variant}", variant, B, H, T, dk, dv, chunk, window, dtype, "sigmoid",
                    0, 0, "uniform", kw.pop("lam_lo", 0.0), kw.pop("lam_hi", 0.3), seed=seed, **kw)


def make(w: Workload):
    return make_inputs(w)
