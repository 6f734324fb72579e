"""GPU parity of the Falcon-1 backward pass (falcon_bwd through the C ABI)
against the fp64 backward oracle on the same seeded inputs.

Bound, per gradient tensor, max|gpu - ref| / max|ref| (over all heads):
  * all-fp32 calls: 1e-4 (fp32 sums over up to a few hundred steps of the
    reverse recursion, against fp64);
  * bf16 inputs: the oracle takes the same bf16-rounded inputs; d_q, d_k,
    d_v are written in bf16 (2^-9 relative rounding) and get 1e-2, the fp32
    gradients (d_beta, d_lambda, d_S_in, d_x_next_in) 1e-4."""
from __future__ import annotations

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16_IO = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from linear_recurrent_weight_amd import falcon as fb
    fb.load_library()


def make(seed, B, H, T, dk, dv, dtype, lam=(0.0, 0.05), continued=False, with_out_grads=True):
    """Inputs of the c2 recipe (q, k, v standard normal, beta a sigmoid of a
    normal, lambda uniform), the incoming gradients standard normal; bf16
    calls round q, k, v and d_o to bf16 first, so both sides see the same
    numbers."""
    from linear_recurrent_weight_amd.inputs import round_to_bf16
    rng = np.random.default_rng(seed)
    f = (lambda a: round_to_bf16(a.astype(np.float32)).astype(np.float64)) if dtype == "bf16" else (lambda a: a)
    inp = dict(q=f(rng.standard_normal((B, H, T, dk))), k=f(rng.standard_normal((B, H, T, dk))),
               v=f(rng.standard_normal((B, H, T, dv))),
               beta=(1 / (1 + np.exp(-rng.standard_normal((B, H, T))))).astype(np.float32).astype(np.float64),
               lam=rng.uniform(*lam, (B, H, T)).astype(np.float32).astype(np.float64))
    up = dict(d_o=f(rng.standard_normal((B, H, T, dv))))
    if with_out_grads:
        up["d_S_out"] = rng.standard_normal((B, H, dk, dv)).astype(np.float32).astype(np.float64)
        up["d_x_next_out"] = rng.standard_normal((B, H, dk)).astype(np.float32).astype(np.float64)
    st = None
    if continued:
        import oracle
        st = oracle.OracleState(S=(0.3 * rng.standard_normal((B * H, dk, dv))).astype(np.float32).astype(np.float64),
                                fresh=False,
                                x_next=rng.standard_normal((B * H, dk)).astype(np.float32).astype(np.float64),
                                tail_x=np.zeros((B * H, 0, dk)), tail_y=np.zeros((B * H, 0, dv)))
    return inp, up, st


def run_gpu(inp, up, st, dtype, **kw):
    import torch
    from linear_recurrent_weight_amd import falcon as fb
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    t = {n: torch.from_numpy(inp[n]).to(dev).to(dt).contiguous() for n in ("q", "k", "v")}
    for n in ("beta", "lam"):
        t[n] = torch.from_numpy(inp[n]).to(dev).float().contiguous()
    d_o = torch.from_numpy(up["d_o"]).to(dev).to(dt).contiguous()
    extra = {}
    for n in ("d_S_out", "d_x_next_out"):
        if n in up:
            extra[n] = torch.from_numpy(up[n]).to(dev).float().contiguous()
    state = None
    if st is not None:
        B, H = inp["q"].shape[:2]
        dk, dv = inp["q"].shape[-1], inp["v"].shape[-1]
        state = fb.FalconState(torch.from_numpy(st.S.reshape(B, H, dk, dv)).to(dev).float().contiguous(),
                               torch.from_numpy(st.x_next.reshape(B, H, dk)).to(dev).float().contiguous(),
                               torch.zeros(B, H, 0, dk, device=dev), torch.zeros(B, H, 0, dv, device=dev),
                               n_tail=0, fresh=st.fresh)
    g = fb.bwd(t["q"], t["k"], t["v"], t["beta"], t["lam"], d_o, state=state, **extra, **kw)
    torch.cuda.synchronize()
    return {n: v.double().cpu().numpy() for n, v in g.items()}


def run_oracle(inp, up, st, **kw):
    from oracle.falcon_backward import falcon1_backward
    return falcon1_backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["lam"], up["d_o"],
                            d_S_out=up.get("d_S_out"), d_x_next_out=up.get("d_x_next_out"),
                            state_in=st, **kw)


def compare(got, ref, dtype, what=""):
    errs = {}
    for n in ("dq", "dk", "dv", "dbeta", "dlam", "dS_in", "dx_next_in"):
        a, b = got[n], ref[n].reshape(got[n].shape)
        assert np.all(np.isfinite(a)), (what, n)
        scale = np.max(np.abs(b)) if b.size else 0.0
        err = float(np.max(np.abs(a - b)) / scale) if scale > 0 else float(np.max(np.abs(a), initial=0.0))
        errs[n] = err
        tol = TOL_BF16_IO if (dtype == "bf16" and n in ("dq", "dk", "dv")) else TOL_F32
        assert err <= tol, (what, n, err, tol)
    print(f"    {what} " + " ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    return errs


def check(seed, B, H, T, dk, dv, dtype, continued=False, with_out_grads=True, lam=(0.0, 0.05), **kw):
    print(f"[bwd] seed={seed} shape=({B},{H},{T},{dk},{dv}) {dtype} continued={continued} {kw}", flush=True)
    inp, up, st = make(seed, B, H, T, dk, dv, dtype, lam=lam, continued=continued, with_out_grads=with_out_grads)
    got = run_gpu(inp, up, st, dtype, **kw)
    ref = run_oracle(inp, up, st, **{k: v for k, v in kw.items() if k != "phi"},
                     phi_kind=1 if kw.get("phi") == "identity" else 0)
    return compare(got, ref, dtype, f"T={T} dk={dk} dv={dv}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 2, 37, 200])
def test_bwd_lengths(dtype, T):
    check(T, 2, 3, T, 64, 64, dtype)


@pytest.mark.parametrize("T", [63, 64, 65, 128, 129, 300, 640])
def test_bwd_chunk_boundaries(T):
    """Lengths at and around the 64-token chunks of the chunk-parallel form
    (one chunk, a full last chunk, a one-token tail, ten chunks)."""
    check(100 + T, 1, 3, T, 64, 64, "f32", continued=True)


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (64, 32), (128, 16), (16, 128), (128, 128)])
def test_bwd_head_dims(dk, dv):
    check(dk + dv, 1, 3, 40, dk, dv, "f32", continued=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_continued_state(dtype):
    check(5, 2, 2, 120, 64, 64, dtype, continued=True)


def test_bwd_without_output_gradients():
    check(6, 1, 4, 60, 64, 32, "f32", continued=True, with_out_grads=False)


def test_bwd_identity_features():
    check(7, 2, 2, 50, 32, 32, "f32", continued=True, phi="identity")


def test_bwd_clamp_binds():
    """Large ridge (lambda >> ||x||^2 ~ d_k) with eps_gamma = 0.3 and beta
    either 0.3 or 0.99: eta lambda is about 0.26-0.29 or 0.85-0.97, so the
    clamp at 0.7 binds on about half the steps and the decay gradient stops
    there."""
    inp, up, st = make(8, 1, 3, 80, 64, 64, "f32", lam=(400.0, 2000.0), continued=True)
    rng = np.random.default_rng(80)
    inp["beta"] = np.where(rng.uniform(size=inp["beta"].shape) < 0.5, 0.3, 0.99).astype(np.float32).astype(np.float64)
    import oracle
    _, _, tr = oracle.falcon_forward("F1", inp["q"], inp["k"], inp["v"], inp["beta"], inp["lam"],
                                     state_in=st, trace=True, eps_gamma=0.3)
    a_un = tr.eta * inp["lam"].reshape(tr.eta.shape)
    assert (a_un >= 0.7).any() and (a_un < 0.7).any()
    assert np.min(np.abs(a_un - 0.7)) > 1e-4   # no decision within rounding of the kink
    got = run_gpu(inp, up, st, "f32", eps_gamma=0.3)
    ref = run_oracle(inp, up, st, eps_gamma=0.3)
    compare(got, ref, "f32", "clamp")


def test_bwd_zero_denominator_is_masked():
    """eps = 0, lambda_t = 0 and a zero key k_{t-1}: that step's denominator is
    0; its gradients are 0 on both sides and nothing is NaN."""
    inp, up, st = make(9, 1, 2, 30, 32, 32, "f32", continued=True)
    inp["k"][0, 1, 10] = 0.0
    inp["lam"][0, 1, 11] = 0.0
    got = run_gpu(inp, up, st, "f32", eps=0.0)
    ref = run_oracle(inp, up, st, eps=0.0)
    assert got["dbeta"][0, 1, 11] == 0 and got["dlam"][0, 1, 11] == 0
    compare(got, ref, "f32", "masked")


def test_bwd_fresh_first_step_is_a_constant():
    inp, up, st = make(10, 2, 2, 20, 64, 64, "f32")
    got = run_gpu(inp, up, st, "f32")
    assert np.all(got["dbeta"][:, :, 0] == 0) and np.all(got["dlam"][:, :, 0] == 0)
    assert np.all(got["dv"][:, :, 0] == 0) and np.all(got["dx_next_in"] == 0)
    compare(got, run_oracle(inp, up, st), "f32", "fresh")


def test_bwd_empty_segment_passes_gradients_through():
    inp, up, st = make(11, 2, 2, 0, 64, 32, "f32", continued=True)
    got = run_gpu(inp, up, st, "f32")
    assert np.array_equal(got["dS_in"], up["d_S_out"].astype(np.float32))
    assert np.array_equal(got["dx_next_in"], up["d_x_next_out"].astype(np.float32))


@pytest.mark.parametrize("split", [1, 64, 150])
def test_bwd_chained_segments_equal_one_call(split):
    """GPU backward of two segments, the later call's d_S_in and d_x_next_in
    fed to the earlier call, against the oracle's one-call backward."""
    import torch
    import oracle
    from linear_recurrent_weight_amd import falcon as fb
    B, H, T, dk, dv = 1, 4, 240, 64, 64
    inp, up, st = make(12, B, H, T, dk, dv, "f32", continued=True)
    ref = run_oracle(inp, up, st)
    a = {n: v[:, :, :split] for n, v in inp.items()}
    b = {n: v[:, :, split:] for n, v in inp.items()}
    _, mid = oracle.falcon_forward("F1", a["q"], a["k"], a["v"], a["beta"], a["lam"], state_in=st)
    mid.S = mid.S.astype(np.float32).astype(np.float64)
    gb = run_gpu(b, dict(d_o=up["d_o"][:, :, split:], d_S_out=up["d_S_out"], d_x_next_out=up["d_x_next_out"]),
                 mid, "f32")
    ga = run_gpu(a, dict(d_o=up["d_o"][:, :, :split], d_S_out=gb["dS_in"], d_x_next_out=gb["dx_next_in"]),
                 st, "f32")
    got = {n: np.concatenate([ga[n], gb[n]], axis=2) for n in ("dq", "dk", "dv", "dbeta", "dlam")}
    got["dS_in"], got["dx_next_in"] = ga["dS_in"], ga["dx_next_in"]
    compare(got, ref, "f32", f"split={split}")
    del torch, fb


def test_bwd_deterministic():
    import torch
    inp, up, st = make(13, 2, 3, 90, 64, 64, "bf16", continued=True)
    g1 = run_gpu(inp, up, st, "bf16")
    g2 = run_gpu(inp, up, st, "bf16")
    for n in g1:
        assert np.array_equal(g1[n], g2[n]), n
    del torch


def test_bwd_c2_full_shape_sampled_heads():
    """The c2 workload shape (8 x 12 heads, T = 1024, d_k = d_v = 64, bf16) in
    the launch configuration the bench times: all 96 heads in one call, fresh
    state, no outgoing x_next gradient.  Eight heads spread over the batch are
    compared with the fp64 oracle (heads are independent), to the bf16 bounds
    above."""
    from linear_recurrent_weight_amd.inputs import WORKLOADS, make_inputs, round_to_bf16
    w = WORKLOADS["c2"]
    B, H, T, dk, dv = w.batch, w.heads, w.seqlen, w.dk, w.dv
    raw = make_inputs(w)
    f = lambda a: round_to_bf16(np.asarray(a, np.float32)).astype(np.float64)
    inp = dict(q=f(raw["q"]), k=f(raw["k"]), v=f(raw["v"]),
               beta=np.asarray(raw["beta"], np.float64), lam=np.asarray(raw["lam"], np.float64))
    rng = np.random.default_rng(2024)
    up = dict(d_o=f(rng.standard_normal((B, H, T, dv))),
              d_S_out=rng.standard_normal((B, H, dk, dv)).astype(np.float32).astype(np.float64))
    print(f"[bwd] c2 full shape ({B},{H},{T},{dk},{dv}) bf16", flush=True)
    got = run_gpu(inp, up, None, "bf16")
    heads = np.unique(np.linspace(0, B * H - 1, 8).round().astype(int))
    sel = lambda a: np.asarray(a).reshape(B * H, *np.asarray(a).shape[2:])[heads][None]
    ref = run_oracle({n: sel(v) for n, v in inp.items()}, {n: sel(v) for n, v in up.items()}, None,
                     eps=w.eps, eps_gamma=w.eps_gamma, eps_rms=w.eps_rms)
    compare({n: sel(v) for n, v in got.items()}, ref, "bf16", "c2 sampled heads")
