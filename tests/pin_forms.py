"""Second and third computations of the Falcon forward pass, used only to pin
the recurrent oracle.  They share no code with ``oracle/``: scalars, windows
and features are recomputed here from the inputs.

* Masked-parallel forms (the O(T^2) unrolled form; "Fast Weight Attention for
  Continual Learning" summary, Figure 2 and Figure 4; §4.6 and §D.1 for the
  Falcon-3A mask; §H "Falcon-3 ParallelFlow Implementation" for the
  block-strict-causal Falcon-3 system).  The triangular systems are solved
  with ``scipy.linalg.solve_triangular``.
* Positive-decay renormalised recurrence (summary §C.6, §E, §G.1): divide the
  state by the running decay, the step by gamma_t and the target by the
  decay up to t-1, and the ridge disappears.
* fp64 chunk form: the masked form applied chunk by chunk, with the
  log-prefix restarted at 0 in each chunk and the previous pairs carried as a
  halo (summary §D.1 "Chunk-Local Evaluation", §C.7).

Derivation of the masked F1 form.  With u_t = eta_t (y_t - S_{t-1}^T x_t) the
write is S_t = gamma_t S_{t-1} + x_t u_t^T, so with b_t = sum_{s<=t} log gamma_s
(b_0 = 0):  S_t = e^{b_t} S_0 + sum_{j<=t} e^{b_t - b_j} x_j u_j^T.  Putting
S_{t-1} into the residual gives a unit-lower system for U:
    u_t + eta_t sum_{j<t} e^{b_{t-1}-b_j} (x_t . x_j) u_j
        = eta_t (y_t - e^{b_{t-1}} S_0^T x_t),
and the read-after-write output is
    o_t = e^{b_t} S_0^T qh_t + sum_{j<=t} e^{b_t-b_j} (qh_t . x_j) u_j.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular

F1, F2, F3, F1A, F2A, F3A = 1, 2, 3, 11, 12, 13
NAMES = {"F1": F1, "F2": F2, "F3": F3, "F1A": F1A, "F2A": F2A, "F3A": F3A}


def rms_feature(z, eps_rms, identity=False):
    z = np.asarray(z, np.float64)
    if identity:
        return z.copy()
    ms = (z ** 2).sum(-1, keepdims=True) / z.shape[-1] + eps_rms
    with np.errstate(divide="ignore", invalid="ignore"):
        out = z / np.sqrt(ms)
    return np.where(ms > 0, out, 0.0)


def cov_top_eig(xw):
    """Top eigenvalue of the d x d window covariance (1/B) X^T X, computed on
    the d x d matrix (the oracle uses the B x B Gram instead)."""
    xw = np.asarray(xw, np.float64)
    c = xw.T @ xw / xw.shape[0]
    return float(np.linalg.eigvalsh(c)[-1])


class Segment:
    """One head's inputs for a segment, with the carried boundary."""

    def __init__(self, q, k, v, beta, lam, S0=None, x_first=None, tail_x=None,
                 tail_y=None, eps_rms=1e-6, identity=False):
        self.qh = rms_feature(q, eps_rms, identity)
        kh = rms_feature(k, eps_rms, identity)
        T, dk = self.qh.shape
        dv = v.shape[1]
        self.fresh = x_first is None
        x = np.zeros((T, dk))
        if T:
            x[0] = 0.0 if self.fresh else x_first
            x[1:] = kh[:-1]
        self.x = x
        self.k_last = kh[-1] if T else x_first
        self.y = np.asarray(v, np.float64)
        self.beta = np.asarray(beta, np.float64)
        self.lam = np.asarray(lam, np.float64)
        self.S0 = np.zeros((dk, dv)) if S0 is None else np.asarray(S0, np.float64)
        self.tail_x = np.zeros((0, dk)) if tail_x is None else np.asarray(tail_x, np.float64)
        self.tail_y = np.zeros((0, dv)) if tail_y is None else np.asarray(tail_y, np.float64)


def step_scalars(variant, seg: Segment, window, eps, eps_gamma):
    """eta, log gamma and the window sets for every token of the segment.

    Returns (eta [T] or [T,dv], logg same shape, windows: list of pair-index
    lists into the concatenated pair list (tail pairs first), bsize [T])."""
    T = seg.x.shape[0]
    px = np.concatenate([seg.tail_x, seg.x], 0)
    nt = seg.tail_x.shape[0]
    per_col = variant in (F2, F2A)
    shape = seg.beta.shape if per_col else (T,)
    eta = np.zeros(shape)
    logg = np.zeros(shape)
    windows, bsize = [], np.zeros(T)
    for t in range(T):
        p = nt + t
        lo = max(0, p - window + 1)
        win = list(range(lo, p + 1))
        windows.append(win)
        bsize[t] = len(win)
        if seg.fresh and t == 0:
            continue
        if variant in (F3, F3A):
            mu = cov_top_eig(px[win])
        else:
            mu = float(seg.x[t] @ seg.x[t])
        den = mu + seg.lam[t] + eps
        e = seg.beta[t] / den if den != 0 else np.zeros_like(seg.beta[t])
        eta[t] = e
        a = np.minimum(e * seg.lam[t], 1.0 - eps_gamma)
        logg[t] = np.log1p(-a)
    return eta, logg, windows, bsize


def masked_segment(variant, seg: Segment, window=1, eps=1e-6, eps_gamma=1e-3):
    """Masked-parallel evaluation of one head over one segment.

    Returns (O [T,dv], S_T [dk,dv])."""
    T = seg.x.shape[0]
    dk, dv = seg.S0.shape
    if T == 0:
        return np.zeros((0, dv)), seg.S0.copy()
    eta, logg, windows, bsize = step_scalars(variant, seg, window, eps, eps_gamma)
    X, Y, Q, S0 = seg.x, seg.y, seg.qh, seg.S0
    if variant == F2:
        O = np.zeros((T, dv))
        ST = np.zeros((dk, dv))
        for j in range(dv):
            o_j, s_j = _masked_delta(X, Y[:, j:j + 1], Q, S0[:, j:j + 1], eta[:, j], logg[:, j])
            O[:, j] = o_j[:, 0]
            ST[:, j] = s_j[:, 0]
        return O, ST
    if variant == F1:
        return _masked_delta(X, Y, Q, S0, eta, logg)
    if variant == F2A:
        # per value column j: decay-weighted mask e^{b_tj - b_sj} eta_sj on
        # the shared scores q_t . x_s (summary Figures 6-8: per-column masks)
        O = np.zeros((T, dv))
        ST = np.zeros((dk, dv))
        QX = Q @ X.T
        for j in range(dv):
            b = np.cumsum(logg[:, j])
            P = np.tril(np.exp(b[:, None] - b[None, :]) * QX)
            u = eta[:, j] * Y[:, j]
            O[:, j] = np.exp(b) * (Q @ S0[:, j]) + P @ u
            ST[:, j] = np.exp(b[-1]) * S0[:, j] + (np.exp(b[-1] - b)[:, None] * X).T @ u
        return O, ST
    if variant == F1A:
        b = np.cumsum(logg)
        U = eta[:, None] * Y
        P = np.tril(np.exp(b[:, None] - b[None, :]) * (Q @ X.T))
        O = np.exp(b)[:, None] * (Q @ S0) + P @ U
        ST = np.exp(b[-1]) * S0 + (np.exp(b[-1] - b)[:, None] * X).T @ U
        return O, ST
    # window variants: pairs are the carried tail followed by this segment's pairs
    PX = np.concatenate([seg.tail_x, X], 0)
    PY = np.concatenate([seg.tail_y, Y], 0)
    b = np.cumsum(logg)
    bprev = np.concatenate([[0.0], b[:-1]])
    if variant == F3A:
        npairs = PX.shape[0]
        M = np.zeros((T, npairs))
        c = np.zeros(npairs)
        for t in range(T):
            for s in range(t + 1):
                w = eta[s] / bsize[s]
                for p in windows[s]:
                    M[t, p] += np.exp(b[t] - b[s]) * w
        for s in range(T):
            for p in windows[s]:
                c[p] += np.exp(b[-1] - b[s]) * eta[s] / bsize[s]
        O = np.exp(b)[:, None] * (Q @ S0) + (M * (Q @ PX.T)) @ PY
        ST = np.exp(b[-1]) * S0 + (c[:, None] * PX).T @ PY
        return O, ST
    # F3: stacked rows (s, p) for p in I_s, ordered by s; block-strict-causal
    rows = [(s, p) for s in range(T) for p in windows[s]]
    R = len(rows)
    A = np.zeros((R, R))
    Dg = np.zeros(R)
    rhs = np.zeros((R, dv))
    for r, (s, p) in enumerate(rows):
        Dg[r] = eta[s] / bsize[s]
        rhs[r] = Dg[r] * (PY[p] - np.exp(bprev[s]) * (S0.T @ PX[p]))
        for r2, (s2, p2) in enumerate(rows):
            if s2 < s:
                A[r, r2] = np.exp(bprev[s] - b[s2]) * (PX[p] @ PX[p2])
    L = np.eye(R) + Dg[:, None] * A
    U = solve_triangular(L, rhs, lower=True, unit_diagonal=True)
    O = np.exp(b)[:, None] * (Q @ S0)
    ST = np.exp(b[-1]) * S0
    for r, (s, p) in enumerate(rows):
        for t in range(s, T):
            O[t] += np.exp(b[t] - b[s]) * (Q[t] @ PX[p]) * U[r]
        ST += np.exp(b[-1] - b[s]) * np.outer(PX[p], U[r])
    return O, ST


def _masked_delta(X, Y, Q, S0, eta, logg):
    """Masked F1 form for one head (eta, logg: [T])."""
    b = np.cumsum(logg)
    bprev = np.concatenate([[0.0], b[:-1]])
    T = X.shape[0]
    A = np.tril(np.exp(bprev[:, None] - b[None, :]) * (X @ X.T), -1)
    L = np.eye(T) + eta[:, None] * A
    rhs = eta[:, None] * (Y - np.exp(bprev)[:, None] * (X @ S0))
    U = solve_triangular(L, rhs, lower=True, unit_diagonal=True)
    P = np.tril(np.exp(b[:, None] - b[None, :]) * (Q @ X.T))
    O = np.exp(b)[:, None] * (Q @ S0) + P @ U
    ST = np.exp(b[-1]) * S0 + (np.exp(b[-1] - b)[:, None] * X).T @ U
    return O, ST


def renormalized_f1(seg: Segment, eps=1e-6, eps_gamma=1e-3):
    """No-ridge recurrence on rescaled quantities (F1 only):
    St_t = St_{t-1} + et_t x_t (yt_t - St_{t-1}^T x_t)^T, with St = S/G_t,
    et_t = eta_t/gamma_t, yt_t = y_t/G_{t-1}; o_t = G_t St_t^T qh_t."""
    eta, logg, _, _ = step_scalars(F1, seg, 1, eps, eps_gamma)
    T = seg.x.shape[0]
    St = seg.S0.copy()
    G = 1.0
    O = np.zeros((T, seg.S0.shape[1]))
    for t in range(T):
        g = np.exp(logg[t])
        Gprev, G = G, G * g
        et = eta[t] / g
        yt = seg.y[t] / Gprev
        St = St + et * np.outer(seg.x[t], yt - St.T @ seg.x[t])
        O[t] = G * (St.T @ seg.qh[t])
    return O, G * St


def chunked(variant, q, k, v, beta, lam, C, window=1, eps=1e-6, eps_gamma=1e-3,
            eps_rms=1e-6, identity=False, S0=None):
    """fp64 chunk form: masked evaluation per chunk of C tokens, with the
    log-prefix restarted in every chunk and (S, x_next, last W-1 pairs)
    carried across the boundary.  One head: q,k [T,dk], v [T,dv]."""
    T = q.shape[0]
    dk, dv = q.shape[1], v.shape[1]
    S = np.zeros((dk, dv)) if S0 is None else S0
    x_first = None
    tail_x = np.zeros((0, dk))
    tail_y = np.zeros((0, dv))
    kh = rms_feature(k, eps_rms, identity)
    outs = []
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        seg = Segment(q[sl], k[sl], v[sl], beta[sl], lam[sl], S0=S, x_first=x_first,
                      tail_x=tail_x, tail_y=tail_y, eps_rms=eps_rms, identity=identity)
        O, S = masked_segment(variant, seg, window, eps, eps_gamma)
        outs.append(O)
        px = np.concatenate([tail_x, seg.x], 0)
        py = np.concatenate([tail_y, seg.y], 0)
        keep = window - 1
        tail_x, tail_y = (px[px.shape[0] - keep:], py[py.shape[0] - keep:]) if keep else (px[:0], py[:0])
        x_first = kh[sl.stop - 1]
    return np.concatenate(outs, 0), S
