"""Plain fp64 CPU oracle for the Falcon-1 backward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite may import this module.  The
HIP library never calls it and shares no code with it.

What is computed (per head, state S with d_k rows and d_v columns): the
gradients of a scalar loss L through the Falcon-1 forward pass of
``falcon_oracle.falcon_forward`` (same readings R1-R7), given
  d_o       dL/do_t for every output,
  d_S_out   dL/dS_T (optional; 0 when absent),
  d_x_next_out  dL/d(phi(k_T)), the carried feature of the next segment
            (optional; 0 when absent),
as the reverse of the token recurrence:
  * o_t = S_t^T qh_t gives  G_t += qh_t do_t^T  and  dqh_t = S_t do_t, where
    G_t = dL/dS_t;
  * S_t = gamma_t S_{t-1} + eta_t x_t r_t^T with r_t = y_t - S_{t-1}^T x_t,
    that is S_t = (gamma_t I - eta_t x_t x_t^T) S_{t-1} + eta_t x_t y_t^T,
    gives, with w_t = G_t^T x_t,
      G_{t-1} = gamma_t G_t - eta_t x_t w_t^T,
      dgamma_t = <G_t, S_{t-1}>,  deta_t = w_t . r_t,  dy_t = eta_t w_t,
      dx_t = eta_t (G_t r_t - S_{t-1} w_t);
  * alpha_t = min(eta_t lambda_t, 1 - eps_gamma), gamma_t = 1 - alpha_t: the
    decay adjoint reaches eta_t and lambda_t only where the clamp does not
    bind (eta_t lambda_t < 1 - eps_gamma) ([summary §D.2 "Backward Pass",
    §G.3 "Forward and Backward Algorithms"]);
  * eta_t = beta_t / d_t, d_t = ||x_t||^2 + lambda_t + eps: dbeta_t =
    deta_t / d_t, dd_t = -deta_t eta_t / d_t, which reaches lambda_t and
    x_t (2 dd_t x_t) ([summary §G.3]);
  * where d_t = 0 the step is 0 by definition and its gradients are masked to
    0 instead of forming 0/0 ([summary §E.3 "Chunk-Parallel Backward Pass"]);
  * the strict no-op first step of a fresh sequence (eta = alpha = 0, the
    sentinel x_1 = 0) is a boundary constant: it passes G through and its
    beta_1, lambda_1 get no gradient ([summary §D.2, §G.3]);
  * the features: qh_t = phi(q_t), x_t = phi(k_{t-1}); phi's vector-Jacobian
    product for QK-RMSNorm, phi(z) = z s, s = (mean(z^2) + eps_rms)^(-1/2):
    dz = s g - (s^3 / d_k) (z . g) z (0 where mean(z^2) + eps_rms = 0); the
    identity map passes g;
  * returned: dq, dk, dv, dbeta, dlambda, dS_in = G_0 (the gradient of the
    initial state, [summary §G.3]) and dx_next_in = dx_1 for a continued
    segment (the gradient of the carried feature; 0 for a fresh one).
    k_T feeds only the next segment's first pair, so dk_T comes from
    d_x_next_out alone.

Reading B1 (the pages give the backward's structure, not this level of
detail): at the clamp boundary eta_t lambda_t == 1 - eps_gamma exactly, the
step counts as clamped (the indicator is the strict eta lambda < 1 - eps_gamma).
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .falcon_oracle import PHI_IDENTITY, PHI_RMSNORM, OracleState, phi


def phi_vjp(z: np.ndarray, g: np.ndarray, eps_rms: float, kind: int = PHI_RMSNORM) -> np.ndarray:
    """dL/dz given g = dL/dphi(z), over the last axis."""
    z = np.asarray(z, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    if kind == PHI_IDENTITY:
        return g.copy()
    d = z.shape[-1]
    ms = np.mean(z * z, axis=-1, keepdims=True) + eps_rms
    ok = ms > 0
    s = np.where(ok, 1.0 / np.sqrt(np.where(ok, ms, 1.0)), 0.0)
    zg = np.sum(z * g, axis=-1, keepdims=True)
    return np.where(ok, s * g - (s ** 3 / d) * zg * z, 0.0)


def falcon1_backward(q, k, v, beta, lam, d_o, *, d_S_out=None, d_x_next_out=None,
                     eps: float = 1e-6, eps_gamma: float = 1e-3, eps_rms: float = 1e-6,
                     phi_kind: int = PHI_RMSNORM, state_in: Optional[OracleState] = None):
    """Gradients of the Falcon-1 forward pass.  Shapes as falcon_forward:
    q, k [B,H,T,dk]; v, d_o [B,H,T,dv]; beta, lam [B,H,T]; d_S_out
    [B,H,dk,dv]; d_x_next_out [B,H,dk].  Returns a dict with dq, dk, dv (input
    shapes), dbeta, dlam [B,H,T], dS_in [B,H,dk,dv], dx_next_in [B,H,dk]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    N = B * H
    qf = q.reshape(N, T, dk)
    kf = k.reshape(N, T, dk)
    vf = v.reshape(N, T, dv)
    betaf = np.asarray(beta, np.float64).reshape(N, T)
    lamf = np.asarray(lam, np.float64).reshape(N, T)
    dof = np.asarray(d_o, np.float64).reshape(N, T, dv)

    qh = phi(qf, eps_rms, phi_kind)
    kh = phi(kf, eps_rms, phi_kind)
    if state_in is None:
        S = np.zeros((N, dk, dv))
        fresh = True
        x_first = np.zeros((N, dk))
    else:
        S = np.array(state_in.S, np.float64).reshape(N, dk, dv).copy()
        fresh = bool(state_in.fresh)
        x_first = np.zeros((N, dk)) if fresh else np.asarray(state_in.x_next, np.float64).reshape(N, dk)

    # forward replay, keeping what the reverse sweep needs
    S_prev = np.zeros((T, N, dk, dv))
    S_post = np.zeros((T, N, dk, dv))
    xs = np.zeros((T, N, dk))
    rs = np.zeros((T, N, dv))
    etas = np.zeros((T, N))
    gammas = np.ones((T, N))
    dens = np.zeros((T, N))
    unclamped = np.zeros((T, N), dtype=bool)
    for t in range(T):
        x_t = x_first if t == 0 else kh[:, t - 1]
        xs[t] = x_t
        S_prev[t] = S
        if fresh and t == 0:
            S_post[t] = S
            continue
        den = np.sum(x_t * x_t, axis=-1) + lamf[:, t] + eps
        eta = np.zeros(N)
        np.divide(betaf[:, t], den, out=eta, where=den != 0)
        a_un = eta * lamf[:, t]
        unclamped[t] = a_un < 1.0 - eps_gamma
        gamma = 1.0 - np.where(unclamped[t], a_un, 1.0 - eps_gamma)
        r = vf[:, t] - np.einsum("nkv,nk->nv", S, x_t)
        S = gamma[:, None, None] * S + eta[:, None, None] * np.einsum("nk,nv->nkv", x_t, r)
        S_post[t] = S
        rs[t], etas[t], gammas[t], dens[t] = r, eta, gamma, den

    # reverse sweep
    G = np.zeros((N, dk, dv)) if d_S_out is None else np.asarray(d_S_out, np.float64).reshape(N, dk, dv).copy()
    dqh = np.zeros((N, T, dk))
    dx = np.zeros((T, N, dk))
    dvf = np.zeros((N, T, dv))
    dbeta = np.zeros((N, T))
    dlam = np.zeros((N, T))
    for t in reversed(range(T)):
        # read after write: o_t = S_t^T qh_t
        G = G + np.einsum("nk,nv->nkv", qh[:, t], dof[:, t])
        dqh[:, t] = np.einsum("nkv,nv->nk", S_post[t], dof[:, t])
        if fresh and t == 0:
            continue                      # boundary step: G passes through
        x_t, r, eta, gamma = xs[t], rs[t], etas[t], gammas[t]
        Sp = S_prev[t]
        w = np.einsum("nkv,nk->nv", G, x_t)
        dgamma = np.einsum("nkv,nkv->n", G, Sp)
        deta = np.sum(w * r, axis=-1)
        dvf[:, t] = eta[:, None] * w
        dx[t] += eta[:, None] * (np.einsum("nkv,nv->nk", G, r) - np.einsum("nkv,nv->nk", Sp, w))
        G = gamma[:, None, None] * G - eta[:, None, None] * np.einsum("nk,nv->nkv", x_t, w)
        # gamma = 1 - alpha, alpha = eta lambda where the clamp does not bind
        dalpha = -dgamma
        deta = deta + np.where(unclamped[t], dalpha * lamf[:, t], 0.0)
        dl = np.where(unclamped[t], dalpha * eta, 0.0)
        # eta = beta / den, den = ||x||^2 + lambda + eps (masked where den = 0)
        den = dens[t]
        nz = den != 0
        safe = np.where(nz, den, 1.0)
        dbeta[:, t] = np.where(nz, deta / safe, 0.0)
        dden = np.where(nz, -deta * eta / safe, 0.0)
        dlam[:, t] = dl + dden
        dx[t] += 2.0 * dden[:, None] * x_t

    dq = phi_vjp(qf, dqh, eps_rms, phi_kind)
    dkf = np.zeros((N, T, dk))
    for t in range(1, T):
        dkf[:, t - 1] = phi_vjp(kf[:, t - 1], dx[t], eps_rms, phi_kind)
    if d_x_next_out is not None and T > 0:
        dkf[:, T - 1] += phi_vjp(kf[:, T - 1], np.asarray(d_x_next_out, np.float64).reshape(N, dk),
                                 eps_rms, phi_kind)
    if fresh:
        dxn = np.zeros((N, dk))
    elif T == 0:   # the state passes through: x_next_out is x_next_in
        dxn = np.zeros((N, dk)) if d_x_next_out is None else np.asarray(d_x_next_out, np.float64).reshape(N, dk)
    else:
        dxn = dx[0]
    return {
        "dq": dq.reshape(B, H, T, dk),
        "dk": dkf.reshape(B, H, T, dk),
        "dv": dvf.reshape(B, H, T, dv),
        "dbeta": dbeta.reshape(B, H, T),
        "dlam": dlam.reshape(B, H, T),
        "dS_in": G.reshape(B, H, dk, dv),
        "dx_next_in": dxn.reshape(B, H, dk),
    }
