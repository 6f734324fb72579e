"""Plain fp64 CPU oracle for the Falcon fast-weight forward pass.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import
this module.  The HIP library never calls it and shares no code with it.

The oracle is the token-by-token recurrence, exactly as the pages define it,
in float64, vectorised only over the independent (batch, head) pairs.  It is
slow on purpose: every line is one step of the definition.

Sources (cited by page title and section; no code exists on any page):
  [summary]   paperlayer.ai source-linked summary of "Fast Weight Attention
              for Continual Learning" (arXiv 2608.27763v1); sections as the
              summary labels them.
  [explainer] agihunt.info, "Falcon realigns fast-weight writes: learn v_t
              from the previous key, not the current one", section "Method".
  [blog]      sungsoo.github.io post on the same paper (Korean), the
              paragraphs on the pre-update prediction, the window step size
              and the decay clamp.

What is computed, per head (state S has d_k rows and d_v columns):
  * features: qh_t = phi(q_t), kh_t = phi(k_t); phi is QK-RMSNorm over d_k
    with no gain, or the identity ("unkernelized" case)
    ([summary §5, §H.3 "The Falcon-3 Recurrence"], [explainer, Method]);
  * write pair: x_t = kh_{t-1}, y_t = v_t; a fresh sequence starts with the
    sentinel x_1 = 0 and its first step is a strict no-op
    ([summary §3, Appendix, §4.6, §H.3 "Identification of Drivers"]);
  * step: eta_t = beta_t / (mu_t + lambda_t + eps), 0 if the denominator is
    0; mu_t = ||x_t||^2 (Falcon-1, -2, -1A) or the top eigenvalue of the
    window covariance (Falcon-3, -3A)
    ([summary §3.1, Appendix, §C.6], [explainer, Method], [blog]);
  * carry: alpha_t = min(eta_t*lambda_t, 1-eps_gamma), gamma_t = 1-alpha_t
    ([summary §C.3, §4.6], [blog]);
  * writes (residual at the pre-update state S_{t-1}):
      F1 : S_t = gamma S + eta x (y - S^T x)^T
      F2 : per value column j with its own eta_{t,j}, gamma_{t,j}
      F3 : S_t = gamma S + (eta/B_t) sum_{j in I_t} x_j (y_j - S^T x_j)^T
      F1A: S_t = gamma S + eta x y^T
      F2A: per value column j, S_t[:, j] = gamma_{t,j} S[:, j] + eta_{t,j} x y_{t,j}
      F3A: S_t = gamma S + (eta/B_t) sum_{j in I_t} x_j y_j^T
    ([summary §1, §4, §4.3, §4.4, §4.5, App. F, "B. Falcon-2A: per-channel
    inner-product write", Figures 6-8], [explainer, Method]);
  * read-after-write: o_t = S_t^T qh_t ([summary §C.2], [explainer, Method]);
  * boundary state for exact continuation: S_T, the next pair's feature
    phi(k_T) and the last W-1 pairs ([summary §C.7, §4.4], [blog]).

Readings where the pages are silent or ambiguous (each also listed with the
design notes of the repository):
  R1  the residual uses S_{t-1} (pre-update), not S_t;
  R2  a fresh t = 1 is a strict no-op (eta = alpha = 0, gamma = 1), and the
      sentinel pair (0, y_1) still enters the window list and counts in B_t;
  R3  phi(z) = z / sqrt(mean(z^2) + eps_rms), per head over d_k, no gain;
      when mean(z^2) + eps_rms == 0 the feature is 0;
  R4  lambda_t is shared by all columns in Falcon-2; only beta is per column;
  R5  when the clamp binds, eta keeps its unclamped value and only gamma
      changes;
  R6  Falcon-3A normalises by the same lambda_max of the window covariance as
      Falcon-3;
  R7  the continuation state also carries x_next = phi(k_T), because the
      next segment's first pair uses the previous key;
  R8  Falcon-2A is the inner-product write of Falcon-1A with the per-column
      gains of Falcon-2: beta_{t,j} per value column, the same energy
      ||x_t||^2 and ridge lambda_t for every column (reading R4), so
      eta_{t,j} = beta_{t,j} / (||x_t||^2 + lambda_t + eps), alpha_{t,j} =
      min(eta_{t,j} lambda_t, 1 - eps_gamma), and each column decays and is
      written on its own ([summary §4.3, §4.5 and the bullets on the A family
      under "C. Falcon-3" and Figures 6-8]: per-column analogue, per-column
      decay-weighted masks, alpha derived as eta lambda).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

F1, F2, F3, F1A, F2A, F3A = 1, 2, 3, 11, 12, 13
VARIANTS = {"F1": F1, "F2": F2, "F3": F3, "F1A": F1A, "F2A": F2A, "F3A": F3A}
PER_COLUMN = (F2, F2A)
WINDOW_VARIANTS = (F3, F3A)
PHI_RMSNORM, PHI_IDENTITY = 0, 1


@dataclass
class OracleState:
    """Boundary state of a segment (fp64 arrays over the flattened heads).

    S       [N, dk, dv] fast-weight state after the last token.
    fresh   True when no pair has been consumed yet (next step is t = 1).
    x_next  [N, dk] the write feature of the next segment's first pair.
    tail_x  [N, n_tail, dk], tail_y [N, n_tail, dv]: the last pairs, oldest first.
    """
    S: np.ndarray
    fresh: bool
    x_next: Optional[np.ndarray]
    tail_x: np.ndarray
    tail_y: np.ndarray

    @property
    def n_tail(self) -> int:
        return int(self.tail_x.shape[1])


@dataclass
class OracleTrace:
    """Per-token scalars the recurrence used (for unit checks of features)."""
    mu: np.ndarray       # [N, T]
    eta: np.ndarray      # [N, T] (F2: [N, T, dv])
    alpha: np.ndarray    # same shape as eta
    gamma: np.ndarray    # same shape as eta
    window: np.ndarray   # [T] realised window size B_t (1 for non-window variants)
    x: np.ndarray        # [N, T, dk] write features actually used
    extra: dict = field(default_factory=dict)


def phi(z: np.ndarray, eps_rms: float, kind: int = PHI_RMSNORM) -> np.ndarray:
    """QK-RMSNorm over the last axis (reading R3), or the identity map.

    [summary §5] says the fast-weight blocks use QK-RMSNorm; [explainer,
    Method] says Q/K default to RMSNorm; [summary §H.3] names the identity
    ("unkernelized") case.
    """
    z = np.asarray(z, dtype=np.float64)
    if kind == PHI_IDENTITY:
        return z.copy()
    ms = np.mean(z * z, axis=-1, keepdims=True) + eps_rms
    safe = np.where(ms > 0, ms, 1.0)
    return np.where(ms > 0, z / np.sqrt(safe), 0.0)


def window_lambda_max(xw: np.ndarray) -> np.ndarray:
    """Top eigenvalue of the window covariance (1/B) sum_j x_j x_j^T.

    xw: [N, B, dk].  The non-zero spectrum of X^T X / B equals that of the
    B x B Gram X X^T / B, so the small Gram is diagonalised exactly with a
    library eigen-solver ([summary §C.6]: the exact top eigenvalue of the
    active-window Gram is allowed; [blog]: mu = lambda_max of the window
    covariance).
    """
    b = xw.shape[1]
    gram = np.einsum("nik,njk->nij", xw, xw) / b
    return np.linalg.eigvalsh(gram)[:, -1]


def falcon_forward(variant, q, k, v, beta, lam, *, window: int = 1,
                   eps: float = 1e-6, eps_gamma: float = 1e-3,
                   eps_rms: float = 1e-6, phi_kind: int = PHI_RMSNORM,
                   state_in: Optional[OracleState] = None,
                   trace: bool = False):
    """Run the recurrence.  Shapes: q, k [B,H,T,dk]; v [B,H,T,dv];
    beta [B,H,T] ([B,H,T,dv] for F2 and F2A); lam [B,H,T].

    Returns (o [B,H,T,dv], OracleState) or, with trace=True,
    (o, OracleState, OracleTrace).  All arithmetic is float64.
    """
    if isinstance(variant, str):
        variant = VARIANTS[variant]
    if variant not in (F1, F2, F3, F1A, F2A, F3A):
        raise ValueError(f"unknown variant {variant}")
    if window < 1:
        raise ValueError("window must be >= 1")
    if variant not in WINDOW_VARIANTS and window != 1:
        raise ValueError("window > 1 only applies to Falcon-3 / Falcon-3A")

    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    N = B * H
    qf = q.reshape(N, T, dk)
    kf = k.reshape(N, T, dk)
    vf = v.reshape(N, T, dv)
    lamf = lam.reshape(N, T)
    betaf = beta.reshape(N, T, dv) if variant in PER_COLUMN else beta.reshape(N, T)

    qh = phi(qf, eps_rms, phi_kind)
    kh = phi(kf, eps_rms, phi_kind)

    if state_in is None:
        S = np.zeros((N, dk, dv))
        fresh = True
        x_next = None
        pairs_x: List[np.ndarray] = []
        pairs_y: List[np.ndarray] = []
    else:
        S = np.array(state_in.S, dtype=np.float64).reshape(N, dk, dv).copy()
        fresh = bool(state_in.fresh)
        x_next = None if fresh else np.asarray(state_in.x_next, np.float64).reshape(N, dk)
        pairs_x = [np.asarray(state_in.tail_x[:, i], np.float64) for i in range(state_in.n_tail)]
        pairs_y = [np.asarray(state_in.tail_y[:, i], np.float64) for i in range(state_in.n_tail)]

    o = np.zeros((N, T, dv))
    col_shape = (N, T, dv) if variant in PER_COLUMN else (N, T)
    tr_mu = np.zeros((N, T))
    tr_eta = np.zeros(col_shape)
    tr_alpha = np.zeros(col_shape)
    tr_gamma = np.ones(col_shape)
    tr_win = np.zeros(T, dtype=np.int64)
    tr_x = np.zeros((N, T, dk))

    for t in range(T):
        # write pair (x_t, y_t) = (phi(k_{t-1}), v_t); sentinel x = 0 when fresh
        if t == 0:
            x_t = np.zeros((N, dk)) if fresh else x_next
        else:
            x_t = kh[:, t - 1]
        y_t = vf[:, t]
        pairs_x.append(x_t)
        pairs_y.append(y_t)
        tr_x[:, t] = x_t
        noop = fresh and t == 0

        # active window I_t: the last min(W, #pairs) pairs (reading R2)
        bt = min(window, len(pairs_x))
        tr_win[t] = bt
        if noop:
            o[:, t] = np.einsum("nkv,nk->nv", S, qh[:, t])
            continue
        xw = np.stack(pairs_x[-bt:], axis=1)        # [N, bt, dk]
        yw = np.stack(pairs_y[-bt:], axis=1)        # [N, bt, dv]

        # smoothness / energy scale mu_t
        if variant in WINDOW_VARIANTS:
            mu = window_lambda_max(xw)
        else:
            mu = np.sum(x_t * x_t, axis=-1)
        tr_mu[:, t] = mu

        # normalised step eta_t and clamped ridge carry gamma_t
        den = mu + lamf[:, t] + eps
        if variant in PER_COLUMN:
            num = betaf[:, t, :]
            den_b = np.broadcast_to(den[:, None], num.shape)
            lam_b = lamf[:, t][:, None]
        else:
            num = betaf[:, t]
            den_b = den
            lam_b = lamf[:, t]
        eta = np.zeros_like(num)
        np.divide(num, den_b, out=eta, where=den_b != 0)
        alpha = np.minimum(eta * lam_b, 1.0 - eps_gamma)
        gamma = 1.0 - alpha
        tr_eta[:, t] = eta
        tr_alpha[:, t] = alpha
        tr_gamma[:, t] = gamma

        # state write
        if variant == F1:
            r = y_t - np.einsum("nkv,nk->nv", S, x_t)
            S = gamma[:, None, None] * S + eta[:, None, None] * np.einsum("nk,nv->nkv", x_t, r)
        elif variant == F2:
            r = y_t - np.einsum("nkv,nk->nv", S, x_t)
            S = gamma[:, None, :] * S + np.einsum("nk,nv->nkv", x_t, eta * r)
        elif variant == F3:
            rw = yw - np.einsum("nkv,nbk->nbv", S, xw)      # residuals at S_{t-1}
            g = np.einsum("nbk,nbv->nkv", xw, rw)
            S = gamma[:, None, None] * S + (eta / bt)[:, None, None] * g
        elif variant == F1A:
            S = gamma[:, None, None] * S + eta[:, None, None] * np.einsum("nk,nv->nkv", x_t, y_t)
        elif variant == F2A:
            S = gamma[:, None, :] * S + np.einsum("nk,nv->nkv", x_t, eta * y_t)
        else:  # F3A
            g = np.einsum("nbk,nbv->nkv", xw, yw)
            S = gamma[:, None, None] * S + (eta / bt)[:, None, None] * g

        # read-after-write
        o[:, t] = np.einsum("nkv,nk->nv", S, qh[:, t])

    # boundary state for exact continuation (reading R7)
    keep = window - 1
    if T == 0:
        out_fresh = fresh
        out_xnext = x_next
    else:
        out_fresh = False
        out_xnext = kh[:, T - 1].copy()
    tail = list(zip(pairs_x, pairs_y))[-keep:] if keep > 0 else []
    tail_x = np.stack([p[0] for p in tail], axis=1) if tail else np.zeros((N, 0, dk))
    tail_y = np.stack([p[1] for p in tail], axis=1) if tail else np.zeros((N, 0, dv))
    st = OracleState(S=S, fresh=out_fresh,
                     x_next=out_xnext, tail_x=tail_x, tail_y=tail_y)
    o = o.reshape(B, H, T, dv)
    if trace:
        return o, st, OracleTrace(mu=tr_mu, eta=tr_eta, alpha=tr_alpha, gamma=tr_gamma,
                                  window=tr_win, x=tr_x)
    return o, st
