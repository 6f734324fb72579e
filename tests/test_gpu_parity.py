"""GPU parity: the HIP path, called through the C ABI, against the fp64
oracle on the same seeded inputs.  Bound: max relative error (per head,
max|gpu - ref| / max|ref|) <= 2e-2 with bf16 inputs and fp32 state, and
<= 1e-5 in the all-fp32 mode."""
from __future__ import annotations

import numpy as np
import pytest

from linear_recurrent_weight_amd.inputs import WORKLOADS
import gpu_util as gu

pytestmark = pytest.mark.gpu

VARIANT_WINDOWS = [("F1", 1), ("F2", 1), ("F3", 3), ("F1A", 1), ("F2A", 1), ("F3A", 3), ("F3", 8), ("F3A", 8)]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrent_weight_amd import falcon as fb
    fb.load_library()          # raises when the HIP library is missing


def check(w, heads=None, chunk=None, tol=None, state=None, oracle_state=None):
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    heads = gu.sample_heads(w, 6) if heads is None else heads
    print(f"[parity] {w.name} {w.variant} chunk={w.chunk if chunk is None else chunk} "
          f"shape=({w.batch},{w.heads},{w.seqlen},{w.dk},{w.dv}) W={w.window} {w.dtype}", flush=True)
    o, st = gu.run_gpu(w, dev, chunk=chunk, state=state)
    o_ref, st_ref = gu.oracle_heads(w, inp, heads, state_in=oracle_state)
    eo, es = gu.compare(w, heads, o, st, o_ref, st_ref)
    tol = gu.tol_for(w) if tol is None else tol
    print(f"    err_o={eo:.3e} err_S={es:.3e} tol={tol}", flush=True)
    assert np.isfinite(eo) and np.isfinite(es)
    assert eo <= tol and es <= tol, (eo, es)
    return o, st, inp, dev


# -- the named workloads ----------------------------------------------------
# Every named workload is compared with the oracle over all of its heads; the
# oracle (vectorised over heads) runs once per workload and is shared by the
# chunk form, the recurrent form and the continuation tests.

_ORACLE = {}


def named_oracle(name):
    if name not in _ORACLE:
        w = WORKLOADS[name]
        inp = gu.make(w)
        print(f"[oracle] {name} all {w.batch * w.heads} heads", flush=True)
        o_ref, st_ref = gu.oracle_heads(w, inp, np.arange(w.batch * w.heads))
        _ORACLE[name] = (inp, o_ref, st_ref)
    return _ORACLE[name]


def check_named(name, chunk=None):
    w = WORKLOADS[name]
    inp, o_ref, st_ref = named_oracle(name)
    dev = gu.to_device(inp, w)
    print(f"[parity] {name} {w.variant} chunk={w.chunk if chunk is None else chunk} all heads", flush=True)
    o, st = gu.run_gpu(w, dev, chunk=chunk)
    heads = np.arange(w.batch * w.heads)
    eo, es = gu.compare(w, heads, o, st, o_ref, st_ref)
    tol = gu.tol_for(w)
    print(f"    err_o={eo:.3e} err_S={es:.3e} tol={tol}", flush=True)
    assert np.isfinite(eo) and np.isfinite(es)
    assert eo <= tol and es <= tol, (eo, es)
    got = gu.gpu_state_to_oracle(st)
    assert np.allclose(got.x_next, st_ref.x_next, rtol=1e-5, atol=1e-5)
    if w.window > 1:
        assert st.n_tail == w.window - 1
        assert np.allclose(got.tail_x, st_ref.tail_x, rtol=1e-5, atol=1e-5)
        assert np.allclose(got.tail_y, st_ref.tail_y, rtol=1e-6, atol=1e-6)
    return o, st, dev


def test_c1_recurrent_f32():
    check_named("c1")


def test_c2_chunk_f1_bf16():
    check_named("c2")


@pytest.mark.parametrize("name", ["c3", "c4", "c5", "c3clamp", "c5f3"])
def test_named_workloads_recurrent_form(name):
    """Every named workload through the token-recurrent HIP form."""
    check_named(name, chunk=0)


@pytest.mark.parametrize("name,splits", [("c5", [1024]), ("c2", [512]), ("c5", [300, 1100])])
def test_named_workload_continuation(name, splits):
    """The workload run as consecutive calls, each carrying (S, x_next and the
    last W - 1 pairs) into the next, against the oracle's one-call run over
    all heads and against the GPU's own one-call run."""
    import torch
    w = WORKLOADS[name]
    inp, o_ref, st_ref = named_oracle(name)
    dev = gu.to_device(inp, w)
    o_full, st_full = gu.run_gpu(w, dev)
    bounds = [0] + list(splits) + [w.seqlen]
    outs, st = [], None
    for a, b in zip(bounds[:-1], bounds[1:]):
        part = {n: t[:, :, a:b].contiguous() for n, t in dev.items()}
        print(f"[parity] {name} continuation tokens [{a}, {b})", flush=True)
        o, st = gu.run_gpu(w.with_(seqlen=b - a), part, state=st)
        outs.append(o)
    o_cat = torch.cat(outs, 2)
    heads = np.arange(w.batch * w.heads)
    eo, es = gu.compare(w, heads, o_cat, st, o_ref, st_ref)
    tol = gu.tol_for(w)
    print(f"    vs oracle: err_o={eo:.3e} err_S={es:.3e} tol={tol}", flush=True)
    assert eo <= tol and es <= tol, (eo, es)
    e1 = gu.max_rel_err(o_cat.double().cpu().numpy(), o_full.double().cpu().numpy())
    e2 = gu.max_rel_err(st.S.double().cpu().numpy(), st_full.S.double().cpu().numpy())
    print(f"    vs one call: err_o={e1:.3e} err_S={e2:.3e}", flush=True)
    assert e1 <= tol and e2 <= tol, (e1, e2)
    got = gu.gpu_state_to_oracle(st)
    assert np.allclose(got.x_next, st_ref.x_next, rtol=1e-5, atol=1e-5)
    if w.window > 1:
        assert st.n_tail == st_full.n_tail == w.window - 1
        assert np.allclose(got.tail_x, st_ref.tail_x, rtol=1e-5, atol=1e-5)
        assert np.allclose(got.tail_y, st_ref.tail_y, rtol=1e-6, atol=1e-6)
        assert torch.equal(st.tail_x, st_full.tail_x) and torch.equal(st.tail_y, st_full.tail_y)


# -- small cases of every variant ------------------------------------------

@pytest.mark.parametrize("variant,window", VARIANT_WINDOWS)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_recurrent_variants(variant, window, dtype):
    w = gu.small(variant, dtype, T=150, dk=64, dv=32, window=window)
    check(w)


@pytest.mark.parametrize("T", [1, 7, 8, 9, 15, 16, 17, 33])
@pytest.mark.parametrize("variant,window", [("F1", 1), ("F2", 1), ("F2A", 1), ("F3A", 3)])
def test_recurrent_lengths(variant, window, T):
    """Lengths around the token batches of the recurrent kernel (16 tokens, 8
    for Falcon-2), with reductions over 16 lanes (d_k = 16) and the whole wave."""
    check(gu.small(variant, "f32", B=1, H=2, T=T, dk=16, dv=16, window=window, seed=T))
    check(gu.small(variant, "f32", B=1, H=2, T=T, dk=64, dv=16, window=window, seed=T + 1))


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 16), (128, 128)])
def test_recurrent_head_dims(dk, dv):
    check(gu.small("F1", "f32", B=1, H=2, T=70, dk=dk, dv=dv))
    check(gu.small("F3A", "f32", B=1, H=2, T=70, dk=dk, dv=dv, window=4))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 256])
def test_chunk_f1_lengths(dtype, T):
    check(gu.small("F1", dtype, B=2, H=3, T=T, dk=64, dv=64, chunk=64))


@pytest.mark.parametrize("dk,dv", [(32, 16), (64, 16), (128, 32), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_f1_head_dims(dk, dv, dtype):
    check(gu.small("F1", dtype, B=1, H=3, T=130, dk=dk, dv=dv, chunk=64))


def test_chunk_f1_clamp_binds():
    """eta*lambda < beta, so beta in (1, 2) with a ridge well above ||x||^2 = 64
    puts alpha on the clamp 1 - eps_gamma for most tokens."""
    w = gu.small("F1", "f32", B=1, H=2, T=200, chunk=64, lam_lo=200.0, lam_hi=400.0, eps_gamma=0.3)
    inp = gu.make(w)
    inp["beta"] = (1.0 + inp["beta"]).astype(np.float32)
    dev = gu.to_device(inp, w)
    o, st = gu.run_gpu(w, dev)
    o_ref, st_ref, tr = gu.oracle_heads(w, inp, np.arange(2), trace=True)
    assert (tr.alpha >= 1 - 0.3 - 1e-9).mean() > 0.5
    eo, es = gu.compare(w, np.arange(2), o, st, o_ref, st_ref)
    assert eo <= 1e-5 and es <= 1e-5, (eo, es)


# -- continuation -------------------------------------------------------------

@pytest.mark.parametrize("variant,window,chunk", [("F1", 1, 0), ("F2", 1, 0), ("F3", 4, 0),
                                                  ("F1A", 1, 0), ("F3A", 8, 0), ("F1", 1, 64),
                                                  ("F1A", 1, 64), ("F3A", 3, 64), ("F3A", 8, 64)])
@pytest.mark.parametrize("split", [0, 3, 64, 100])
def test_continuation(variant, window, chunk, split):
    """Two calls carrying (S, x_next, tail) equal one call and the oracle."""
    import torch
    w = gu.small(variant, "f32", B=2, H=2, T=160, dk=32, dv=32, chunk=chunk, window=window, seed=11)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    o_full, st_full = gu.run_gpu(w, dev)
    a = {k: v[:, :, :split].contiguous() for k, v in dev.items()}
    b = {k: v[:, :, split:].contiguous() for k, v in dev.items()}
    o1, st1 = gu.run_gpu(w.with_(seqlen=split), a)
    o2, st2 = gu.run_gpu(w.with_(seqlen=160 - split), b, state=st1)
    o_cat = torch.cat([o1, o2], 2)
    heads = np.arange(4)
    o_ref, st_ref = gu.oracle_heads(w, inp, heads)
    eo, es = gu.compare(w, heads, o_cat, st2, o_ref, st_ref)
    assert eo <= 1e-5 and es <= 1e-5, (eo, es)
    # the split and unsplit GPU runs agree to fp32 rounding (chunk boundaries differ)
    assert gu.max_rel_err(o_cat.double().cpu().numpy(), o_full.double().cpu().numpy()) <= 1e-5
    assert st2.n_tail == st_full.n_tail == min(window - 1, 160)
    if window > 1:
        assert torch.allclose(st2.tail_x, st_full.tail_x) and torch.allclose(st2.tail_y, st_full.tail_y)
    assert torch.allclose(st2.x_next, st_full.x_next)


def test_continuation_with_state_from_oracle_layout():
    """A nonzero incoming state (S, x_next, partial tail) matches the oracle."""
    import torch
    from linear_recurrent_weight_amd import falcon as fb
    w = gu.small("F3A", "f32", B=1, H=2, T=40, dk=16, dv=16, window=5, seed=3)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((1, 2, 16, 16)).astype(np.float32)
    xn = rng.standard_normal((1, 2, 16)).astype(np.float32)
    tx = np.zeros((1, 2, 4, 16), np.float32)
    ty = np.zeros((1, 2, 4, 16), np.float32)
    tx[:, :, 2:] = rng.standard_normal((1, 2, 2, 16))
    ty[:, :, 2:] = rng.standard_normal((1, 2, 2, 16))
    cuda = lambda a: torch.from_numpy(a).cuda()
    st = fb.FalconState(cuda(S0), cuda(xn), cuda(tx), cuda(ty), n_tail=2, fresh=False)
    import oracle
    ost = oracle.OracleState(S=S0.reshape(2, 16, 16).astype(np.float64), fresh=False,
                             x_next=xn.reshape(2, 16).astype(np.float64),
                             tail_x=tx.reshape(2, 4, 16)[:, 2:].astype(np.float64),
                             tail_y=ty.reshape(2, 4, 16)[:, 2:].astype(np.float64))
    o, st_out = gu.run_gpu(w, dev, state=st)
    o_ref, st_ref = gu.oracle_heads(w, inp, np.arange(2), state_in=ost)
    eo, es = gu.compare(w, np.arange(2), o, st_out, o_ref, st_ref)
    assert eo <= 1e-5 and es <= 1e-5, (eo, es)
    assert st_out.n_tail == 4


# -- edge cases ---------------------------------------------------------------

def test_empty_sequence_passes_state_through():
    import torch
    from linear_recurrent_weight_amd import falcon as fb
    w = gu.small("F3A", "f32", B=1, H=2, T=0, dk=16, dv=16, window=3)
    S0 = torch.randn(1, 2, 16, 16, device="cuda")
    xn = torch.randn(1, 2, 16, device="cuda")
    tx = torch.randn(1, 2, 2, 16, device="cuda")
    ty = torch.randn(1, 2, 2, 16, device="cuda")
    st = fb.FalconState(S0, xn, tx, ty, n_tail=1, fresh=False)
    z = torch.zeros(1, 2, 0, 16, device="cuda")
    o, out = fb.fwd(z, z, z, torch.zeros(1, 2, 0, device="cuda"), torch.zeros(1, 2, 0, device="cuda"),
                    variant="F3A", chunk=0, window=3, state=st)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 16)
    assert torch.equal(out.S, S0) and torch.equal(out.x_next, xn)
    assert out.n_tail == 1 and not out.fresh
    assert torch.equal(out.tail_x[:, :, 1:], tx[:, :, 1:]) and torch.all(out.tail_x[:, :, :1] == 0)
    o, out = fb.fwd(z, z, z, torch.zeros(1, 2, 0, device="cuda"), torch.zeros(1, 2, 0, device="cuda"),
                    variant="F1", chunk=0)
    assert out.fresh and torch.all(out.S == 0)


def test_zero_keys_give_zero_step():
    """All-zero keys with lambda = eps = 0: the step denominator vanishes, eta
    = 0, the state stays zero and nothing is NaN."""
    import torch
    from linear_recurrent_weight_amd import falcon as fb
    for chunk in (0, 64):
        q = torch.randn(1, 1, 70, 64, device="cuda")
        k = torch.zeros(1, 1, 70, 64, device="cuda")
        v = torch.randn(1, 1, 70, 64, device="cuda")
        beta = torch.full((1, 1, 70), 0.5, device="cuda")
        lam = torch.zeros(1, 1, 70, device="cuda")
        o, st = fb.fwd(q, k, v, beta, lam, variant="F1", chunk=chunk, eps=0.0)
        assert torch.all(o == 0) and torch.all(st.S == 0)


def test_identity_feature_map():
    w = gu.small("F1", "f32", B=1, H=2, T=96, dk=32, dv=32, chunk=64)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    from linear_recurrent_weight_amd import falcon as fb
    import oracle
    for chunk in (0, 64):
        o, st = fb.fwd(dev["q"], dev["k"], dev["v"], dev["beta"], dev["lam"], variant="F1",
                       chunk=chunk, phi="identity")
        o_ref, st_ref = oracle.falcon_forward("F1", inp["q"], inp["k"], inp["v"], inp["beta"],
                                              inp["lam"], phi_kind=oracle.PHI_IDENTITY)
        assert gu.max_rel_err(o.double().cpu().numpy()[0], o_ref[0]) <= 1e-5


def test_deterministic():
    import torch
    w = WORKLOADS["c2"].with_(batch=2)
    dev = gu.to_device(gu.make(w), w)
    o1, s1 = gu.run_gpu(w, dev)
    o2, s2 = gu.run_gpu(w, dev)
    assert torch.equal(o1, o2) and torch.equal(s1.S, s2.S)


# -- bf16 Falcon-1 kernels for d_k = 64 ----------------------------------------

@pytest.mark.parametrize("dv", [32, 64, 128])
@pytest.mark.parametrize("T", [1, 64, 130, 300])
def test_chunk_f1_bf16_shapes(dv, T):
    check(gu.small("F1", "bf16", B=2, H=5, T=T, dk=64, dv=dv, chunk=64, seed=T + dv))


@pytest.mark.parametrize("B,H", [(1, 1), (1, 7), (3, 8), (5, 13)])
def test_chunk_f1_bf16_head_counts(B, H):
    """Head counts that do and do not divide by the 8-way workgroup
    interleave of the carry (every head compared)."""
    w = gu.small("F1", "bf16", B=B, H=H, T=200, dk=64, dv=64, chunk=64, seed=B * 100 + H)
    check(w, heads=np.arange(B * H))


@pytest.mark.parametrize("split", [64, 100])
def test_chunk_f1_bf16_continuation(split):
    """bf16 d_k = 64: two calls carrying the state match the oracle run of
    the whole sequence."""
    import torch
    w = gu.small("F1", "bf16", B=2, H=3, T=300, dk=64, dv=64, chunk=64, seed=13)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    a = {k: v[:, :, :split].contiguous() for k, v in dev.items()}
    b = {k: v[:, :, split:].contiguous() for k, v in dev.items()}
    o1, st1 = gu.run_gpu(w.with_(seqlen=split), a)
    o2, st2 = gu.run_gpu(w.with_(seqlen=300 - split), b, state=st1)
    heads = np.arange(6)
    o_ref, st_ref = gu.oracle_heads(w, inp, heads)
    eo, es = gu.compare(w, heads, torch.cat([o1, o2], 2), st2, o_ref, st_ref)
    assert eo <= gu.TOL_BF16 and es <= gu.TOL_BF16, (eo, es)
    assert torch.allclose(st2.x_next, torch.from_numpy(st_ref.x_next.reshape(2, 3, 64)).float().cuda(),
                          rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("eps_gamma", [1e-3, 1e-2])
def test_chunk_f1_bf16_strong_decay(eps_gamma):
    """Large ridge weights (eta lambda close to beta): a chunk decays by about
    2^-100, so some chunks take the separable decays and others form them
    pairwise."""
    w = gu.small("F1", "bf16", B=1, H=3, T=200, dk=64, dv=64, chunk=64, seed=29).with_(
        lam_lo=500.0, lam_hi=2000.0, eps_gamma=eps_gamma)
    check(w)


# Long walks over few heads split into segments: the segments' composed
# chunk maps are scanned, then every segment walks its chunks.  Shapes with
# whole and partial last segments and ragged last chunks, every d_v.
F1_SEGMENT_SHAPES = [(1, 3, 5000, 32), (1, 1, 3072, 128), (2, 6, 3100, 64), (1, 2, 7000, 64)]


@pytest.mark.parametrize("B,H,T,dv", F1_SEGMENT_SHAPES)
def test_chunk_f1_bf16_segments(B, H, T, dv):
    w = gu.small("F1", "bf16", B=B, H=H, T=T, dk=64, dv=dv, chunk=64, seed=T + dv)
    check(w, heads=np.arange(B * H))


def test_named_workload_c3f1_segments():
    """Falcon-1 over 16384 tokens and 24 heads: five segments of 52 chunks."""
    check_named("c3f1")


@pytest.mark.parametrize("split", [4000, 4160])
def test_chunk_f1_bf16_segments_continuation(split):
    """Two segmented calls carrying the state match one oracle run (the split
    falls inside a chunk, then on a chunk boundary)."""
    import torch
    B, H, T = 1, 3, 9000
    w = gu.small("F1", "bf16", B=B, H=H, T=T, dk=64, dv=64, chunk=64, seed=77)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    a = {k: v[:, :, :split].contiguous() for k, v in dev.items()}
    b = {k: v[:, :, split:].contiguous() for k, v in dev.items()}
    o1, st1 = gu.run_gpu(w.with_(seqlen=split), a)
    o2, st2 = gu.run_gpu(w.with_(seqlen=T - split), b, state=st1)
    heads = np.arange(B * H)
    o_ref, st_ref = gu.oracle_heads(w, inp, heads)
    eo, es = gu.compare(w, heads, torch.cat([o1, o2], 2), st2, o_ref, st_ref)
    print(f"    err_o={eo:.3e} err_S={es:.3e}", flush=True)
    assert eo <= gu.TOL_BF16 and es <= gu.TOL_BF16, (eo, es)
    got = gu.gpu_state_to_oracle(st2)
    assert np.allclose(got.x_next, st_ref.x_next, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("lam", [(0.0, 0.05), (500.0, 2000.0)])
def test_chunk_f1_bf16_segments_decay(lam):
    """Segment maps whose scalar part underflows (strong ridge: each chunk
    decays by about 2^-100) and ones that keep most of the state."""
    w = gu.small("F1", "bf16", B=1, H=2, T=4096, dk=64, dv=64, chunk=64, seed=91).with_(
        lam_lo=lam[0], lam_hi=lam[1])
    check(w, heads=np.arange(2))


# -- Falcon-1A / Falcon-3A chunk path -------------------------------------------

@pytest.mark.parametrize("name", ["c3", "c5", "c3clamp"])
def test_named_workloads_chunk_a(name):
    check_named(name)


@pytest.mark.parametrize("variant,window", [("F1A", 1), ("F3A", 2), ("F3A", 3), ("F3A", 8)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 5, 64, 130, 700])
def test_chunk_a_variants(variant, window, dtype, T):
    check(gu.small(variant, dtype, B=2, H=3, T=T, dk=64, dv=64, chunk=64, window=window, seed=T + window))


@pytest.mark.parametrize("B,H,T", [(1, 2, 1000), (4, 16, 1000), (8, 12, 1000), (8, 16, 2300)])
@pytest.mark.parametrize("variant,window", [("F1A", 1), ("F3A", 8)])
def test_chunk_a_segments(B, H, T, variant, window):
    """fp32 inner-product path: shapes whose segment lengths (chunks per
    workgroup, from the head and chunk counts) are 1, 2, 3 and 8."""
    check(gu.small(variant, "f32", B=B, H=H, T=T, dk=64, dv=64, chunk=64, window=window, seed=3),
          heads=gu.sample_heads(gu.small(variant, "f32", B=B, H=H, T=T), 8))


@pytest.mark.parametrize("dk,dv", [(32, 16), (32, 64), (64, 32), (64, 16)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_a_head_dims(dk, dv, dtype):
    check(gu.small("F3A", dtype, B=1, H=3, T=200, dk=dk, dv=dv, chunk=64, window=4))


def test_chunk_a_strong_ridge_clamp():
    """Clamp binding on most tokens (beta in (1, 2), ridge >> ||x||^2): the
    chunk-local carries stay exact through long products of small gammas."""
    w = gu.small("F1A", "f32", B=1, H=2, T=300, chunk=64, lam_lo=200.0, lam_hi=400.0, eps_gamma=0.05)
    inp = gu.make(w)
    inp["beta"] = (1.0 + inp["beta"]).astype(np.float32)
    dev = gu.to_device(inp, w)
    o, st = gu.run_gpu(w, dev)
    o_ref, st_ref, tr = gu.oracle_heads(w, inp, np.arange(2), trace=True)
    assert (tr.alpha >= 1 - 0.05 - 1e-9).mean() > 0.5
    eo, es = gu.compare(w, np.arange(2), o, st, o_ref, st_ref)
    assert eo <= 1e-5 and es <= 1e-5, (eo, es)


# -- bf16 Falcon-1A / 3A kernels for d_k = d_v = 64 (register operands) --------

@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 200, 1000])
def test_chunk_a1_bf16_lengths(T):
    check(gu.small("F1A", "bf16", B=2, H=3, T=T, dk=64, dv=64, chunk=64, seed=T + 7))


# (B, H, T) whose segment lengths (the fewest chunks per segment that keep
# every segment resident at once) are 1, 2, 5 and 16
A1_SEGMENT_SHAPES = [(1, 3, 1300), (2, 12, 2048), (4, 12, 3200), (8, 12, 5120)]


@pytest.mark.parametrize("B,H,T", A1_SEGMENT_SHAPES)
def test_chunk_a1_bf16_segments(B, H, T):
    """Chunks per segment do not change the result."""
    w = gu.small("F1A", "bf16", B=B, H=H, T=T, dk=64, dv=64, chunk=64, seed=17)
    check(w, heads=gu.sample_heads(w, 8))


@pytest.mark.parametrize("variant,window", [("F1A", 1), ("F3A", 2), ("F3A", 8)])
@pytest.mark.parametrize("split", [0, 3, 64, 100])
@pytest.mark.parametrize("B,H,T", [(2, 3, 300), (2, 12, 2048)])
def test_chunk_a1_bf16_continuation(variant, window, split, B, H, T):
    """Two calls carrying (S, x_next, the last W - 1 pairs) match the oracle
    run of the whole sequence; the carried pairs match the oracle's.  The
    second shape runs two chunks per segment."""
    import torch
    w = gu.small(variant, "bf16", B=B, H=H, T=T, dk=64, dv=64, chunk=64, window=window, seed=19)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    a = {k: v[:, :, :split].contiguous() for k, v in dev.items()}
    b = {k: v[:, :, split:].contiguous() for k, v in dev.items()}
    o1, st1 = gu.run_gpu(w.with_(seqlen=split), a)
    o2, st2 = gu.run_gpu(w.with_(seqlen=T - split), b, state=st1)
    heads = np.arange(B * H)
    o_ref, st_ref = gu.oracle_heads(w, inp, heads)
    eo, es = gu.compare(w, heads, torch.cat([o1, o2], 2), st2, o_ref, st_ref)
    assert eo <= gu.TOL_BF16 and es <= gu.TOL_BF16, (eo, es)
    assert torch.allclose(st2.x_next, torch.from_numpy(st_ref.x_next.reshape(B, H, 64)).float().cuda(),
                          rtol=1e-5, atol=1e-5)
    if window > 1:
        got = gu.gpu_state_to_oracle(st2)
        assert st2.n_tail == window - 1
        assert np.allclose(got.tail_x, st_ref.tail_x, rtol=1e-5, atol=1e-5)
        assert np.allclose(got.tail_y, st_ref.tail_y, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("B,H,T", A1_SEGMENT_SHAPES[:3])
@pytest.mark.parametrize("window", [3, 8])
def test_chunk_a3_bf16_segments(B, H, T, window):
    """Falcon-3A: chunks per segment (the halo carried in LDS or read from
    memory) do not change the result."""
    w = gu.small("F3A", "bf16", B=B, H=H, T=T, dk=64, dv=64, chunk=64, window=window, seed=29)
    check(w, heads=gu.sample_heads(w, 6))


@pytest.mark.parametrize("T", [1, 2, 7, 8, 9, 63, 64, 65, 200])
@pytest.mark.parametrize("window", [2, 8])
def test_chunk_a3_bf16_lengths(T, window):
    check(gu.small("F3A", "bf16", B=2, H=2, T=T, dk=64, dv=64, chunk=64, window=window, seed=T + 31))


@pytest.mark.parametrize("eps_gamma", [1e-3, 5e-2])
def test_chunk_a1_bf16_strong_decay(eps_gamma):
    """Large ridge weights: chunks decay far below 2^-100, so the scores take
    the pairwise decays instead of the separable ones."""
    w = gu.small("F1A", "bf16", B=1, H=3, T=300, dk=64, dv=64, chunk=64, seed=23).with_(
        lam_lo=500.0, lam_hi=2000.0, eps_gamma=eps_gamma)
    check(w)


def test_chunk_a1_bf16_identity_features():
    """phi = identity (no RMS scale): the unnormalised keys go straight into
    the step and the writes."""
    w = gu.small("F1A", "bf16", B=1, H=2, T=150, dk=64, dv=64, chunk=64, seed=5)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    from linear_recurrent_weight_amd import falcon as fb
    import oracle
    o, st = fb.fwd(dev["q"], dev["k"], dev["v"], dev["beta"], dev["lam"], variant="F1A",
                   chunk=64, phi="identity")
    o_ref, st_ref = oracle.falcon_forward("F1A", inp["q"], inp["k"], inp["v"], inp["beta"],
                                          inp["lam"], phi_kind=oracle.PHI_IDENTITY)
    assert gu.max_rel_err(o.double().cpu().numpy(), o_ref) <= gu.TOL_BF16


# -- Falcon-2 chunk path -------------------------------------------------------

def test_named_workload_c4_chunk_f2():
    check_named("c4")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 15, 16, 17, 63, 64, 65, 200])
def test_chunk_f2_lengths(dtype, T):
    """Ragged lengths across the 16-token solve blocks and the 64-token chunks."""
    check(gu.small("F2", dtype, B=2, H=3, T=T, dk=64, dv=64, chunk=64, seed=T))


@pytest.mark.parametrize("dk,dv,dtype", [(64, 16, "f32"), (64, 128, "f32"), (64, 32, "bf16"),
                                         (128, 16, "bf16"), (128, 128, "bf16")])
def test_chunk_f2_head_dims(dk, dv, dtype):
    check(gu.small("F2", dtype, B=1, H=3, T=300, dk=dk, dv=dv, chunk=64))


@pytest.mark.parametrize("T", [1, 17, 64, 65, 200])
@pytest.mark.parametrize("dv", [32, 128])
def test_chunk_f2_d128_lengths(dv, T):
    """bf16, d_k = 128, 32-column slices (the eight-wave workgroup): ragged
    lengths across the solve blocks and the chunks."""
    check(gu.small("F2", "bf16", B=1, H=3, T=T, dk=128, dv=dv, chunk=64, seed=T + dv))


@pytest.mark.parametrize("split", [3, 64, 100])
def test_chunk_f2_d128_continuation(split):
    """bf16, d_k = 128 (eight-wave workgroup): two calls carrying (S, x_next)
    match the oracle over the whole sequence."""
    import torch
    w = gu.small("F2", "bf16", B=1, H=2, T=200, dk=128, dv=64, chunk=64, seed=21)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    a = {k: v[:, :, :split].contiguous() for k, v in dev.items()}
    b = {k: v[:, :, split:].contiguous() for k, v in dev.items()}
    o1, st1 = gu.run_gpu(w.with_(seqlen=split), a)
    o2, st2 = gu.run_gpu(w.with_(seqlen=200 - split), b, state=st1)
    heads = np.arange(2)
    o_ref, st_ref = gu.oracle_heads(w, inp, heads)
    eo, es = gu.compare(w, heads, torch.cat([o1, o2], 2), st2, o_ref, st_ref)
    assert eo <= gu.tol_for(w) and es <= gu.tol_for(w), (eo, es)


def test_chunk_f2_equal_gains_is_falcon1():
    """With the same gain in every column, Falcon-2 is Falcon-1: the two
    chunk kernels agree to fp32 rounding."""
    w1 = gu.small("F1", "f32", B=2, H=2, T=333, dk=64, dv=64, chunk=64, seed=5)
    inp = gu.make(w1)
    dev1 = gu.to_device(inp, w1)
    o1, st1 = gu.run_gpu(w1, dev1)
    w2 = w1.with_(variant="F2")
    dev2 = dict(dev1)
    dev2["beta"] = dev1["beta"][..., None].expand(*dev1["beta"].shape, 64).contiguous()
    o2, st2 = gu.run_gpu(w2, dev2)
    assert gu.max_rel_err(o2.double().cpu().numpy(), o1.double().cpu().numpy()) <= 1e-5
    assert gu.max_rel_err(st2.S.double().cpu().numpy(), st1.S.double().cpu().numpy()) <= 1e-5


def test_chunk_f2_strong_ridge_clamp():
    """Clamp binding on most (token, column) pairs: long products of small
    per-column carries stay exact inside a chunk."""
    w = gu.small("F2", "f32", B=1, H=2, T=300, chunk=64, lam_lo=200.0, lam_hi=400.0, eps_gamma=0.05)
    inp = gu.make(w)
    inp["beta"] = (1.0 + inp["beta"]).astype(np.float32)
    dev = gu.to_device(inp, w)
    o, st = gu.run_gpu(w, dev)
    o_ref, st_ref, tr = gu.oracle_heads(w, inp, np.arange(2), trace=True)
    assert (tr.alpha >= 1 - 0.05 - 1e-9).mean() > 0.5
    eo, es = gu.compare(w, np.arange(2), o, st, o_ref, st_ref)
    assert eo <= 1e-5 and es <= 1e-5, (eo, es)


@pytest.mark.parametrize("split", [0, 3, 64, 100])
def test_chunk_f2_continuation(split):
    import torch
    w = gu.small("F2", "f32", B=2, H=2, T=160, dk=64, dv=32, chunk=64, seed=12)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    o_full, st_full = gu.run_gpu(w, dev)
    a = {k: v[:, :, :split].contiguous() for k, v in dev.items()}
    b = {k: v[:, :, split:].contiguous() for k, v in dev.items()}
    o1, st1 = gu.run_gpu(w.with_(seqlen=split), a)
    o2, st2 = gu.run_gpu(w.with_(seqlen=160 - split), b, state=st1)
    o_cat = torch.cat([o1, o2], 2)
    heads = np.arange(4)
    o_ref, st_ref = gu.oracle_heads(w, inp, heads)
    eo, es = gu.compare(w, heads, o_cat, st2, o_ref, st_ref)
    assert eo <= 1e-5 and es <= 1e-5, (eo, es)
    assert gu.max_rel_err(o_cat.double().cpu().numpy(), o_full.double().cpu().numpy()) <= 1e-5
    assert torch.allclose(st2.x_next, st_full.x_next)


# -- Falcon-3 chunk path (stacked window rows) ------------------------------------

def test_named_workload_c5f3_chunk():
    check_named("c5f3")


@pytest.mark.parametrize("window", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 7, 8, 9, 64, 130, 300])
def test_chunk_f3_windows(window, dtype, T):
    check(gu.small("F3", dtype, B=2, H=2, T=T, dk=64, dv=32, chunk=64, window=window, seed=T + 10 * window))


@pytest.mark.parametrize("dk,dv", [(32, 16), (128, 64), (64, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_f3_head_dims(dk, dv, dtype):
    check(gu.small("F3", dtype, B=1, H=3, T=200, dk=dk, dv=dv, chunk=64, window=4))


def test_chunk_f3_window1_is_falcon1():
    """At W = 1 the stacked form is the Falcon-1 chunk form."""
    w1 = gu.small("F1", "f32", B=2, H=2, T=200, dk=64, dv=32, chunk=64, seed=9)
    inp = gu.make(w1)
    dev = gu.to_device(inp, w1)
    o1, st1 = gu.run_gpu(w1, dev)
    o3, st3 = gu.run_gpu(w1.with_(variant="F3"), dev)
    assert gu.max_rel_err(o3.double().cpu().numpy(), o1.double().cpu().numpy()) <= 1e-5
    assert gu.max_rel_err(st3.S.double().cpu().numpy(), st1.S.double().cpu().numpy()) <= 1e-5


@pytest.mark.parametrize("window", [3, 8])
@pytest.mark.parametrize("split", [2, 100])
def test_chunk_f3_bf16_continuation(window, split):
    """bf16, d_k = 64: the second call's first chunk stacks the incoming tail
    pairs (fp32, rounded to bf16 as they are staged) with its own rows."""
    import torch
    w = gu.small("F3", "bf16", B=1, H=2, T=160, dk=64, dv=32, chunk=64, window=window, seed=17)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    a = {k: v[:, :, :split].contiguous() for k, v in dev.items()}
    b = {k: v[:, :, split:].contiguous() for k, v in dev.items()}
    o1, st1 = gu.run_gpu(w.with_(seqlen=split), a)
    o2, st2 = gu.run_gpu(w.with_(seqlen=160 - split), b, state=st1)
    heads = np.arange(2)
    o_ref, st_ref = gu.oracle_heads(w, inp, heads)
    eo, es = gu.compare(w, heads, torch.cat([o1, o2], 2), st2, o_ref, st_ref)
    assert eo <= gu.tol_for(w) and es <= gu.tol_for(w), (eo, es)


@pytest.mark.parametrize("window", [3, 8])
@pytest.mark.parametrize("split", [0, 2, 8, 100])
def test_chunk_f3_continuation(window, split):
    """Carrying (S, x_next, the last W-1 pairs) across calls equals one call."""
    import torch
    w = gu.small("F3", "f32", B=2, H=2, T=160, dk=32, dv=32, chunk=64, window=window, seed=13)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    o_full, st_full = gu.run_gpu(w, dev)
    a = {k: v[:, :, :split].contiguous() for k, v in dev.items()}
    b = {k: v[:, :, split:].contiguous() for k, v in dev.items()}
    o1, st1 = gu.run_gpu(w.with_(seqlen=split), a)
    o2, st2 = gu.run_gpu(w.with_(seqlen=160 - split), b, state=st1)
    o_cat = torch.cat([o1, o2], 2)
    heads = np.arange(4)
    o_ref, st_ref = gu.oracle_heads(w, inp, heads)
    eo, es = gu.compare(w, heads, o_cat, st2, o_ref, st_ref)
    assert eo <= 1e-5 and es <= 1e-5, (eo, es)
    assert gu.max_rel_err(o_cat.double().cpu().numpy(), o_full.double().cpu().numpy()) <= 1e-5
    assert st2.n_tail == st_full.n_tail == window - 1
    assert torch.allclose(st2.tail_x, st_full.tail_x) and torch.allclose(st2.tail_y, st_full.tail_y)


# -- Falcon-3 through 64-token transfer operators (bf16, d_k = d_v = 64, W in
#    {2, 4, 8}): W sub-chunks of 64 stacked rows, then the Falcon-1 carry ----

def _f3x(**kw):
    base = dict(B=2, H=3, dk=64, dv=64, chunk=64)
    base.update(kw)
    return gu.small("F3", "bf16", **base)


def test_chunk_f3_xfer_takes_the_transfer_path():
    import ctypes
    from linear_recurrent_weight_amd import falcon as fb
    lib = fb.load_library()
    a = fb.make_args(variant="F3", dtype="bf16", batch=2, heads=3, seqlen=300, dk=64, dv=64, chunk=64, window=8)
    names = []
    while (nm := lib.falcon_kernel_name(ctypes.byref(a), len(names))) is not None:
        names.append(nm.decode())
    assert names == ["a3_window", "f3_xfer", "f1_carry"]


@pytest.mark.parametrize("window", [2, 4, 8])
@pytest.mark.parametrize("T", [7, 8, 9, 64, 65, 130, 300])
def test_chunk_f3_xfer_lengths(window, T):
    """Chunks of 64 tokens in W sub-chunks, ragged last chunk, sub-chunks
    past the end of the sequence.  (Below 7 tokens a head's whole output is
    one or two rows whose size can rest on a single dot product: the
    per-head relative error then measures that dot product's bf16 rounding,
    about 1e-3 absolute as everywhere else, against a reference of a few
    1e-3; the shortest lengths are the same as the other Falcon-3 tests'.)"""
    check(_f3x(T=T, window=window, seed=T + 7 * window), heads=np.arange(6))


@pytest.mark.parametrize("window", [4, 8])
@pytest.mark.parametrize("split", [1, 5, 64, 100])
def test_chunk_f3_xfer_continuation(window, split):
    """The second call's first sub-chunk stacks the incoming tail pairs
    (fp32, rounded to bf16 as staged) with its own rows; the carried state
    enters through the Falcon-1 walk."""
    import torch
    w = _f3x(B=1, H=2, T=200, window=window, seed=23)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    a = {k: v[:, :, :split].contiguous() for k, v in dev.items()}
    b = {k: v[:, :, split:].contiguous() for k, v in dev.items()}
    o1, st1 = gu.run_gpu(w.with_(seqlen=split), a)
    o2, st2 = gu.run_gpu(w.with_(seqlen=200 - split), b, state=st1)
    heads = np.arange(2)
    o_ref, st_ref = gu.oracle_heads(w, inp, heads)
    eo, es = gu.compare(w, heads, torch.cat([o1, o2], 2), st2, o_ref, st_ref)
    print(f"    split={split} W={window} err_o={eo:.3e} err_S={es:.3e}", flush=True)
    assert eo <= gu.tol_for(w) and es <= gu.tol_for(w), (eo, es)


@pytest.mark.parametrize("window", [4, 8])
def test_chunk_f3_xfer_strong_decay(window):
    """Steps near the clamp with a tiny eps_gamma: sub-chunks decay below
    2^-100, which takes the pairwise (non-separable) decay form."""
    w = _f3x(B=1, H=2, T=300, window=window, seed=29, lam_lo=5e3, lam_hi=1e4, eps_gamma=1e-6)
    inp = gu.make(w)
    inp["beta"] = (1.0 + inp["beta"]).astype(np.float32)
    dev = gu.to_device(inp, w)
    o, st = gu.run_gpu(w, dev)
    o_ref, st_ref, tr = gu.oracle_heads(w, inp, np.arange(2), trace=True)
    lg = np.log2(1.0 - tr.alpha)
    assert (lg < -12.5).mean() > 0.5   # sub-chunks of 8 or 16 such tokens span more than 2^-100
    eo, es = gu.compare(w, np.arange(2), o, st, o_ref, st_ref)
    assert eo <= gu.tol_for(w) and es <= gu.tol_for(w), (eo, es)


def test_chunk_f3_strong_ridge_clamp():
    w = gu.small("F3", "f32", B=1, H=2, T=300, chunk=64, window=4, lam_lo=200.0, lam_hi=400.0,
                 eps_gamma=0.05)
    inp = gu.make(w)
    inp["beta"] = (1.0 + inp["beta"]).astype(np.float32)
    dev = gu.to_device(inp, w)
    o, st = gu.run_gpu(w, dev)
    o_ref, st_ref, tr = gu.oracle_heads(w, inp, np.arange(2), trace=True)
    assert (tr.alpha >= 1 - 0.05 - 1e-9).mean() > 0.5
    eo, es = gu.compare(w, np.arange(2), o, st, o_ref, st_ref)
    assert eo <= 1e-5 and es <= 1e-5, (eo, es)


@pytest.mark.parametrize("eps_gamma,lam_hi,dtype", [(1e-4, 400.0, "f32"), (1e-3, 30.0, "f32"),
                                                    (1e-4, 400.0, "bf16")])
def test_chunk_f2_steep_decay_blocks(eps_gamma, lam_hi, dtype):
    """Blocks whose carry falls below 2^-100 take the exact in-block form;
    with the clamp binding everywhere (first case) every block does, with a
    ridge spread (second case) the two forms alternate."""
    w = gu.small("F2", dtype, B=1, H=2, T=200, dk=64, dv=32, chunk=64, lam_lo=0.0, lam_hi=lam_hi,
                 eps_gamma=eps_gamma, seed=21)
    inp = gu.make(w)
    inp["beta"] = (1.0 + inp["beta"]).astype(np.float32)
    dev = gu.to_device(inp, w)
    o, st = gu.run_gpu(w, dev)
    o_ref, st_ref = gu.oracle_heads(w, inp, np.arange(2))
    eo, es = gu.compare(w, np.arange(2), o, st, o_ref, st_ref)
    tol = gu.tol_for(w)
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("dk,dv,lam_lo,lam_hi", [(128, 64, 100.0, 200.0), (64, 32, 40.0, 80.0)])
def test_chunk_f2_block_frames(dk, dv, lam_lo, lam_hi):
    """Chunks that decay below 2^-100 while their 16-token blocks stay above
    it: the solve keeps a frame per block and rescales the earlier writes (the
    chunk-start frame needs e^{b_C} >= 2^-100 in every column of a slice).
    d_k = 128 is the c4 kernel's shape."""
    w = gu.small("F2", "bf16", B=1, H=2, T=200, dk=dk, dv=dv, chunk=64, lam_lo=lam_lo, lam_hi=lam_hi,
                 eps_gamma=1e-3, seed=77)
    inp = gu.make(w)
    inp["beta"] = (1.0 + inp["beta"]).astype(np.float32)
    dev = gu.to_device(inp, w)
    o, st = gu.run_gpu(w, dev)
    o_ref, st_ref, tr = gu.oracle_heads(w, inp, np.arange(2), trace=True)
    # per (chunk, column) log2 decay of whole chunks and of 16-token blocks
    lg = np.log2(np.maximum(1.0 - np.asarray(tr.alpha, np.float64), 1e-300))   # [head, t, column]
    lg = lg[:, :192].reshape(lg.shape[0], 3, 4, 16, lg.shape[2])   # three whole chunks
    chunk_decay = lg.sum(axis=(2, 3))
    block_decay = lg.sum(axis=3)
    assert (chunk_decay < -100).mean() > 0.5, "most chunks leave the chunk frame"
    assert (block_decay >= -100).mean() > 0.9, "the blocks stay separable"
    eo, es = gu.compare(w, np.arange(2), o, st, o_ref, st_ref)
    tol = gu.tol_for(w)
    assert eo <= tol and es <= tol, (eo, es)


# -- Falcon-2A chunk path -------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 200, 700])
def test_chunk_f2a_lengths(dtype, T):
    check(gu.small("F2A", dtype, B=2, H=3, T=T, dk=64, dv=64, chunk=64, seed=T + 3))


@pytest.mark.parametrize("dk,dv", [(32, 16), (32, 64), (64, 32), (64, 128), (64, 16)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_f2a_head_dims(dk, dv, dtype):
    """Slices of 16, 32 and 64 value columns (d_v = 128: two workgroups per
    head), d_k of 32 and 64."""
    w = gu.small("F2A", dtype, B=1, H=3, T=200, dk=dk, dv=dv, chunk=64, seed=dk + dv)
    check(w, heads=np.arange(3))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_f2a_strong_decay_runs_token_by_token(dtype):
    """beta in (1, 2) and a ridge far above ||x||^2 put the clamp on most
    (token, column) pairs: chunks whose decay falls below 2^-64 take the
    token-by-token form; others the renormalised one."""
    w = gu.small("F2A", dtype, B=1, H=2, T=300, dk=64, dv=32, chunk=64, lam_lo=0.0, lam_hi=400.0,
                 eps_gamma=0.01, seed=77)
    inp = gu.make(w)
    inp["beta"] = (1.0 + inp["beta"]).astype(np.float32)
    dev = gu.to_device(inp, w)
    o, st = gu.run_gpu(w, dev)
    o_ref, st_ref, tr = gu.oracle_heads(w, inp, np.arange(2), trace=True)
    assert (tr.alpha >= 1 - 0.01 - 1e-9).mean() > 0.3
    eo, es = gu.compare(w, np.arange(2), o, st, o_ref, st_ref)
    tol = gu.tol_for(w)
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("split", [0, 3, 64, 100])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_f2a_continuation(split, dtype):
    import torch
    w = gu.small("F2A", dtype, B=2, H=2, T=160, dk=64, dv=32, chunk=64, seed=12)
    inp = gu.make(w)
    dev = gu.to_device(inp, w)
    a = {k: v[:, :, :split].contiguous() for k, v in dev.items()}
    b = {k: v[:, :, split:].contiguous() for k, v in dev.items()}
    o1, st1 = gu.run_gpu(w.with_(seqlen=split), a)
    o2, st2 = gu.run_gpu(w.with_(seqlen=160 - split), b, state=st1)
    heads = np.arange(4)
    o_ref, st_ref = gu.oracle_heads(w, inp, heads)
    eo, es = gu.compare(w, heads, torch.cat([o1, o2], 2), st2, o_ref, st_ref)
    tol = gu.tol_for(w)
    assert eo <= tol and es <= tol, (eo, es)


def test_named_workload_c2f2a_chunk():
    """Falcon-2A at the c2 shape over all 96 heads."""
    check_named("c2f2a")


def test_chunk_f2a_equal_gains_is_falcon1a():
    """The same gain in every column: the Falcon-2A chunk kernel and the
    Falcon-1A chunk kernels agree to fp32 rounding."""
    w1 = gu.small("F1A", "f32", B=2, H=2, T=333, dk=64, dv=64, chunk=64, seed=5)
    inp = gu.make(w1)
    dev1 = gu.to_device(inp, w1)
    o1, st1 = gu.run_gpu(w1, dev1)
    dev2 = dict(dev1)
    dev2["beta"] = dev1["beta"][..., None].expand(*dev1["beta"].shape, 64).contiguous()
    o2, st2 = gu.run_gpu(w1.with_(variant="F2A"), dev2)
    assert gu.max_rel_err(o2.double().cpu().numpy(), o1.double().cpu().numpy()) <= 1e-5
    assert gu.max_rel_err(st2.S.double().cpu().numpy(), st1.S.double().cpu().numpy()) <= 1e-5
