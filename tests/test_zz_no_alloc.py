"""falcon_fwd_noalloc (workspace from the library's fixed per-GPU array)
against falcon_fwd (caller's workspace), called through the C ABI: two calls
in a row, the second on a smaller input, for a path whose kernels use
workspace, plus the rejection of a call that needs more than the array."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from linear_recurrent_weight_amd.inputs import WORKLOADS
import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrent_weight_amd import falcon as fb
    return fb.load_library()


def _call(lib, fn, w, dev, ws):
    """One call of `fn` (falcon_fwd or falcon_fwd_noalloc) on device inputs;
    returns (o, S, x_next, tail_x, tail_y, n_tail)."""
    import torch
    from linear_recurrent_weight_amd import falcon as fb
    dt = dev["q"].dtype
    o = torch.full((w.batch, w.heads, w.seqlen, w.dv), float("nan"), dtype=dt, device="cuda")
    st = fb.FalconState.empty(w.batch, w.heads, w.dk, w.dv, w.window, "cuda")
    for t in (st.S, st.x_next, st.tail_x, st.tail_y):
        t.fill_(float("nan"))
    st_c = st.to_c()
    a = fb.make_args(variant=w.variant, dtype=w.dtype, batch=w.batch, heads=w.heads, seqlen=w.seqlen,
                     dk=w.dk, dv=w.dv, chunk=w.chunk, window=w.window, eps=w.eps, eps_gamma=w.eps_gamma,
                     eps_rms=w.eps_rms, q=dev["q"], k=dev["k"], v=dev["v"], beta=dev["beta"],
                     lam=dev["lam"], o=o, state_out=st_c,
                     workspace=ws, workspace_bytes=0 if ws is None else ws.numel())
    rc = fn(ctypes.byref(a), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == fb.OK, rc
    torch.cuda.synchronize()
    return o, st.S, st.x_next, st.tail_x, st.tail_y, st_c.n_tail


@pytest.mark.parametrize("first,second", [
    (WORKLOADS["c2"], WORKLOADS["c2"].with_(batch=1, heads=3, seqlen=300)),
    (gu.small("F3A", "bf16", B=2, H=4, T=700, dk=64, dv=64, chunk=64, window=8, seed=3),
     gu.small("F3A", "bf16", B=1, H=2, T=130, dk=64, dv=64, chunk=64, window=8, seed=4)),
])
def test_noalloc_matches_falcon_fwd(lib, first, second):
    import torch
    from linear_recurrent_weight_amd import falcon as fb
    for w in (first, second):
        need = lib.falcon_fwd_workspace_size(ctypes.byref(fb.make_args(
            variant=w.variant, dtype=w.dtype, batch=w.batch, heads=w.heads, seqlen=w.seqlen, dk=w.dk,
            dv=w.dv, chunk=w.chunk, window=w.window)))
        assert 0 < need <= fb.NOALLOC_SCRATCH_BYTES
        inp = gu.make(w)
        dev = gu.to_device(inp, w)
        print(f"[noalloc] {w.name} {w.variant} ({w.batch},{w.heads},{w.seqlen}) workspace {need} B", flush=True)
        ref = _call(lib, lib.falcon_fwd, w, dev, torch.empty(need, dtype=torch.uint8, device="cuda"))
        got = _call(lib, lib.falcon_fwd_noalloc, w, dev, None)
        assert got[5] == ref[5]
        for g, r in zip(got[:5], ref[:5]):
            assert torch.equal(g, r)       # same kernels, deterministic: bitwise equal
        # and within the tolerance of the oracle (sampled heads)
        heads = gu.sample_heads(w, 3)
        o_ref, st_ref = gu.oracle_heads(w, inp, heads)
        og = got[0].double().cpu().numpy().reshape(w.batch * w.heads, w.seqlen, w.dv)[heads]
        assert gu.max_rel_err(og, o_ref.reshape(-1, w.seqlen, w.dv)) <= gu.tol_for(w)


def test_noalloc_rejects_more_than_its_array(lib):
    from linear_recurrent_weight_amd import falcon as fb
    fake = 1 << 20
    w = WORKLOADS["c2"].with_(batch=16)
    a = fb.make_args(variant=w.variant, dtype=w.dtype, batch=w.batch, heads=w.heads, seqlen=w.seqlen,
                     dk=w.dk, dv=w.dv, chunk=w.chunk, q=fake, k=2 * fake, v=3 * fake, beta=4 * fake,
                     lam=5 * fake, o=6 * fake)
    assert lib.falcon_fwd_workspace_size(ctypes.byref(a)) > fb.NOALLOC_SCRATCH_BYTES
    assert lib.falcon_fwd_noalloc(ctypes.byref(a), None) == fb.ERR_WORKSPACE
