"""Single-token decode step (seqlen = 1, one kernel per call) against the
fp64 oracle: T consecutive one-token calls, each carrying the boundary state
(S, x_next, the last W - 1 pairs) into the next, must reproduce the oracle's
one-call run of the whole sequence, for every variant; and decode steps
after a chunk-parallel prefill must continue it exactly."""
from __future__ import annotations

import numpy as np
import pytest

from linear_recurrent_weight_amd.inputs import WORKLOADS
import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrent_weight_amd import falcon as fb
    fb.load_library()


def decode_chain(w, dev, start, stop, state):
    """Calls of one token each over tokens [start, stop)."""
    import torch
    outs = []
    for t in range(start, stop):
        part = {n: x[:, :, t:t + 1].contiguous() for n, x in dev.items()}
        o, state = gu.run_gpu(w.with_(seqlen=1), part, state=state)
        outs.append(o)
    return torch.cat(outs, 2), state


def check_against_oracle(w, inp, o, st, tol):
    heads = np.arange(w.batch * w.heads)
    o_ref, st_ref = gu.oracle_heads(w, inp, heads)
    eo, es = gu.compare(w, heads, o, st, o_ref, st_ref)
    print(f"    err_o={eo:.3e} err_S={es:.3e} tol={tol}", flush=True)
    assert eo <= tol and es <= tol, (eo, es)
    got = gu.gpu_state_to_oracle(st)
    assert np.allclose(got.x_next, st_ref.x_next, rtol=1e-5, atol=1e-5)
    if w.window > 1:
        assert st.n_tail == st_ref.n_tail
        assert np.allclose(got.tail_x, st_ref.tail_x, rtol=1e-5, atol=1e-5)
        assert np.allclose(got.tail_y, st_ref.tail_y, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("variant,window", [("F1", 1), ("F2", 1), ("F3", 3), ("F3", 8), ("F1A", 1),
                                            ("F2A", 1), ("F3A", 2), ("F3A", 8)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 64), (128, 32)])
def test_decode_chain_equals_one_call(variant, window, dtype, dk, dv):
    """A fresh sequence decoded token by token (the first call a strict
    no-op step), against the oracle over every head."""
    T = 12
    w = gu.small(variant, dtype, B=2, H=3, T=T, dk=dk, dv=dv, window=window, seed=dk + dv + window)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    print(f"[decode] {variant} W={window} {dtype} dk={dk} dv={dv} T={T}", flush=True)
    o, st = decode_chain(w, dev, 0, T, None)
    check_against_oracle(w, inp, o, st, gu.TOL_F32 if dtype == "f32" else gu.TOL_BF16)


@pytest.mark.parametrize("variant,window,chunk", [("F1", 1, 64), ("F2", 1, 64), ("F3", 4, 64),
                                                  ("F1A", 1, 64), ("F2A", 1, 64), ("F3A", 8, 64), ("F1", 1, 0)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_after_prefill(variant, window, chunk, dtype):
    """A chunk-parallel (or recurrent) prefill of 130 tokens, then 10
    single-token steps, equal the oracle's run of all 140 tokens."""
    import torch
    T, P = 140, 130
    w = gu.small(variant, dtype, B=2, H=2, T=T, dk=64, dv=64, chunk=chunk, window=window, seed=41)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    pre = {n: x[:, :, :P].contiguous() for n, x in dev.items()}
    print(f"[decode] prefill {variant} W={window} {dtype} chunk={chunk}", flush=True)
    o1, st = gu.run_gpu(w.with_(seqlen=P), pre)
    o2, st = decode_chain(w, dev, P, T, st)
    check_against_oracle(w, inp, torch.cat([o1, o2], 2), st,
                         gu.TOL_F32 if dtype == "f32" else gu.TOL_BF16)


def test_decode_c2_shape_all_heads():
    """The c2 shape (batch 8, 12 heads, d = 64, bf16): a chunk prefill of
    1000 tokens and 24 decode steps against the oracle over all 96 heads."""
    import torch
    w = WORKLOADS["c2"].with_(seqlen=1024)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    P = 1000
    pre = {n: x[:, :, :P].contiguous() for n, x in dev.items()}
    o1, st = gu.run_gpu(w.with_(seqlen=P), pre)
    o2, st = decode_chain(w, dev, P, w.seqlen, st)
    check_against_oracle(w, inp, torch.cat([o1, o2], 2), st, gu.TOL_BF16)


def test_decode_is_one_kernel():
    import ctypes
    from linear_recurrent_weight_amd import falcon as fb
    lib = fb.load_library()
    for var, W in (("F1", 1), ("F2", 1), ("F3", 5), ("F1A", 1), ("F2A", 1), ("F3A", 8)):
        for chunk in (0, 64):
            a = fb.make_args(variant=var, dtype="bf16", batch=2, heads=3, seqlen=1, dk=64, dv=64,
                             chunk=chunk, window=W)
            assert lib.falcon_kernel_name(ctypes.byref(a), 0) == b"decode"
            assert lib.falcon_kernel_name(ctypes.byref(a), 1) is None
            assert lib.falcon_fwd_workspace_size(ctypes.byref(a)) == 0
