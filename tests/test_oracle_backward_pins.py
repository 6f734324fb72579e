"""Pins of the Falcon-1 backward oracle against things other than itself:

  * central finite differences of the forward oracle, for every element of
    every input (q, k, v, beta, lambda, the initial state S and the carried
    feature x_next) on tiny shapes: fresh and continued segments, the clamp
    binding on some steps and not on others, the identity feature map, and
    gradients arriving at the final state and at the carried feature;
  * the zero-step convention: where the step's denominator is 0 the step is
    0 and its gradients are 0 (no 0/0), while every other gradient still
    matches finite differences;
  * linearity in the incoming gradients;
  * chaining: the backward of two segments, the later one's input-state
    gradients fed to the earlier one, equals the one-call backward;
  * an empty segment passes the state gradients through.
CPU only."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import OracleState, falcon_forward, PHI_IDENTITY, PHI_RMSNORM
from oracle.falcon_backward import falcon1_backward

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def make_case(seed, B=1, H=2, T=5, dk=4, dv=3, lam=(0.0, 0.5), beta=(0.2, 0.9), continued=False,
              k_scale=1.0):
    rng = np.random.default_rng(seed)
    inp = dict(
        q=rng.standard_normal((B, H, T, dk)),
        k=rng.standard_normal((B, H, T, dk)) * k_scale,
        v=rng.standard_normal((B, H, T, dv)),
        beta=rng.uniform(*beta, (B, H, T)),
        lam=rng.uniform(*lam, (B, H, T)),
    )
    st = None
    if continued:
        st = OracleState(S=rng.standard_normal((B * H, dk, dv)) * 0.5, fresh=False,
                         x_next=rng.standard_normal((B * H, dk)), tail_x=np.zeros((B * H, 0, dk)),
                         tail_y=np.zeros((B * H, 0, dv)))
    up = dict(d_o=rng.standard_normal((B, H, T, dv)),
              d_S_out=rng.standard_normal((B, H, dk, dv)),
              d_x_next_out=rng.standard_normal((B, H, dk)))
    return inp, st, up


def loss(inp, st, up, kw):
    """L = <d_o, o> + <d_S_out, S_T> + <d_x_next_out, x_next_out>, by the forward oracle."""
    o, so = falcon_forward("F1", inp["q"], inp["k"], inp["v"], inp["beta"], inp["lam"],
                           state_in=st, **kw)
    B, H = o.shape[:2]
    L = np.sum(up["d_o"] * o) + np.sum(up["d_S_out"].reshape(so.S.shape) * so.S)
    if so.x_next is not None:
        L += np.sum(up["d_x_next_out"].reshape(so.x_next.shape) * so.x_next)
    return L


def fd_grads(inp, st, up, kw, h=1e-5):
    """Central differences of the loss for every input element."""
    out = {}
    for name in ("q", "k", "v", "beta", "lam"):
        g = np.zeros_like(inp[name])
        for idx in np.ndindex(*inp[name].shape):
            for sgn in (1, -1):
                p = {kk: vv.copy() for kk, vv in inp.items()}
                p[name][idx] += sgn * h
                g[idx] += sgn * loss(p, st, up, kw) / (2 * h)
        out[name] = g
    if st is not None:
        for name in ("S", "x_next"):
            base = getattr(st, name)
            g = np.zeros_like(base)
            for idx in np.ndindex(*base.shape):
                for sgn in (1, -1):
                    arr = base.copy()
                    arr[idx] += sgn * h
                    s2 = OracleState(S=arr if name == "S" else st.S, fresh=st.fresh,
                                     x_next=arr if name == "x_next" else st.x_next,
                                     tail_x=st.tail_x, tail_y=st.tail_y)
                    g[idx] += sgn * loss(inp, s2, up, kw) / (2 * h)
            out[name] = g
    return out


def backward(inp, st, up, kw):
    return falcon1_backward(inp["q"], inp["k"], inp["v"], inp["beta"], inp["lam"], up["d_o"],
                            d_S_out=up["d_S_out"], d_x_next_out=up["d_x_next_out"], state_in=st, **kw)


def assert_close(got, want, what, rtol=1e-6):
    scale = max(np.max(np.abs(want)), 1e-12)
    err = np.max(np.abs(got - want)) / scale
    assert err <= rtol, (what, err)


CASES = {
    "fresh": dict(seed=1),
    "continued": dict(seed=2, continued=True),
    "identity_phi": dict(seed=3, continued=True, phi_kind=PHI_IDENTITY),
    "longer": dict(seed=4, T=9, dk=5, dv=2, continued=True),
}


def clamp_mixed_case():
    """Large ridge with eps_gamma = 0.3: eta lambda is about 0.29 or 0.92
    against the clamp at 0.7, so some steps clamp and others do not, each
    far from the kink."""
    inp, st, up = make_case(5, T=7, lam=(80.0, 120.0), continued=True)
    rng = np.random.default_rng(50)
    inp["beta"] = np.where(rng.uniform(size=inp["beta"].shape) < 0.5, 0.3, 0.95)
    return inp, st, up, dict(eps_gamma=0.3)


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_matches_finite_differences(name):
    c = dict(CASES[name])
    phi_kind = c.pop("phi_kind", PHI_RMSNORM)
    inp, st, up = make_case(**c)
    kw = dict(phi_kind=phi_kind)
    g = backward(inp, st, up, kw)
    fd = fd_grads(inp, st, up, kw)
    for ours, theirs in [("dq", "q"), ("dk", "k"), ("dv", "v"), ("dbeta", "beta"), ("dlam", "lam")]:
        assert_close(g[ours], fd[theirs], (name, ours))
    if st is not None:
        assert_close(g["dS_in"].reshape(st.S.shape), fd["S"], (name, "dS_in"))
        assert_close(g["dx_next_in"].reshape(st.x_next.shape), fd["x_next"], (name, "dx_next_in"))


def test_backward_with_clamp_binding_matches_finite_differences():
    inp, st, up, kw = clamp_mixed_case()
    o, so, tr = falcon_forward("F1", inp["q"], inp["k"], inp["v"], inp["beta"], inp["lam"],
                               state_in=st, trace=True, **kw)
    a_un = tr.eta * inp["lam"].reshape(tr.eta.shape)
    clamped = a_un >= 1 - 0.3
    assert clamped.any() and (~clamped).any()
    assert np.min(np.abs(a_un - 0.7)) > 0.05
    g = backward(inp, st, up, kw)
    fd = fd_grads(inp, st, up, kw)
    for ours, theirs in [("dq", "q"), ("dk", "k"), ("dv", "v"), ("dbeta", "beta"), ("dlam", "lam")]:
        assert_close(g[ours], fd[theirs], ("clamp", ours))
    assert_close(g["dS_in"].reshape(st.S.shape), fd["S"], ("clamp", "dS_in"))


def test_fresh_first_step_gets_no_step_gradient():
    """The strict no-op first step is a boundary constant: beta_1 and
    lambda_1 get exactly 0, and so does v_1 (its pair never writes)."""
    inp, st, up = make_case(6)
    g = backward(inp, st, up, {})
    assert np.all(g["dbeta"][..., 0] == 0) and np.all(g["dlam"][..., 0] == 0)
    assert np.all(g["dv"][..., 0, :] == 0)
    assert np.all(g["dx_next_in"] == 0)


def test_zero_denominator_steps_are_masked():
    """eps = 0, lambda = 0 and a zero key make one step's denominator 0: that
    step is 0 and its beta / lambda gradients are 0, not NaN; the gradients
    of every other input still match finite differences (that token's lambda
    and the zero key excluded: a nonzero perturbation of either makes the
    denominator nonzero and the step jumps from 0 to beta / denominator)."""
    inp, st, up = make_case(7, T=6, continued=True)
    inp["k"][0, 1, 2] = 0.0            # x_4 of head 1 is phi(0) = 0
    inp["lam"][0, 1, 3] = 0.0
    kw = dict(eps=0.0)
    g = backward(inp, st, up, kw)
    for v in g.values():
        assert np.all(np.isfinite(v))
    assert g["dbeta"][0, 1, 3] == 0 and g["dlam"][0, 1, 3] == 0
    fd = fd_grads(inp, st, up, kw)
    for ours, theirs in [("dq", "q"), ("dv", "v"), ("dbeta", "beta")]:
        assert_close(g[ours], fd[theirs], ("masked", ours))
    keep = np.ones(inp["lam"].shape, bool)
    keep[0, 1, 3] = False
    assert_close(g["dlam"][keep], fd["lam"][keep], ("masked", "dlam"))
    keep_k = np.ones(inp["k"].shape, bool)
    keep_k[0, 1, 2, :] = False
    assert_close(g["dk"][keep_k], fd["k"][keep_k], ("masked", "dk"))


def test_backward_is_linear_in_the_incoming_gradients():
    inp, st, up = make_case(8, continued=True)
    up2 = make_case(9, continued=True)[2]
    a, b = 0.7, -1.3
    mix = {k: a * up[k] + b * up2[k] for k in up}
    g1, g2, gm = backward(inp, st, up, {}), backward(inp, st, up2, {}), backward(inp, st, mix, {})
    for k in g1:
        assert_close(gm[k], a * g1[k] + b * g2[k], ("linear", k), rtol=1e-12)


@pytest.mark.parametrize("split", [1, 3, 4])
def test_chained_segments_equal_one_call(split):
    """Run the forward in two calls; the backward of the second call gives
    dL/dS and dL/dx_next at the split, which the first call's backward takes
    as its d_S_out and d_x_next_out."""
    inp, st, up = make_case(10, T=6, continued=True)
    kw = {}
    whole = backward(inp, st, up, kw)
    a = {k: v[:, :, :split] for k, v in inp.items()}
    b = {k: v[:, :, split:] for k, v in inp.items()}
    _, mid = falcon_forward("F1", a["q"], a["k"], a["v"], a["beta"], a["lam"], state_in=st)
    up_b = dict(d_o=up["d_o"][:, :, split:], d_S_out=up["d_S_out"], d_x_next_out=up["d_x_next_out"])
    gb = backward(b, mid, up_b, kw)
    up_a = dict(d_o=up["d_o"][:, :, :split], d_S_out=gb["dS_in"], d_x_next_out=gb["dx_next_in"])
    ga = backward(a, st, up_a, kw)
    for name in ("dq", "dk", "dv", "dbeta", "dlam"):
        assert_close(np.concatenate([ga[name], gb[name]], axis=2), whole[name], ("chain", name), 1e-12)
    assert_close(ga["dS_in"], whole["dS_in"], ("chain", "dS_in"), 1e-12)
    assert_close(ga["dx_next_in"], whole["dx_next_in"], ("chain", "dx_next_in"), 1e-12)


def test_empty_segment_passes_the_gradients_through():
    inp, st, up = make_case(11, T=0, continued=True)
    g = backward(inp, st, up, {})
    assert np.array_equal(g["dS_in"], up["d_S_out"])
    assert np.array_equal(g["dx_next_in"], up["d_x_next_out"])
