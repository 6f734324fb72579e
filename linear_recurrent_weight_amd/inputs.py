"""Seeded synthetic inputs for the Falcon forward pass.

This module only draws random numbers and rounds them to the storage type;
it holds none of the method's arithmetic, so both the HIP path and the fp64
oracle can be fed from it.

Recipe (per workload): ``numpy.random.default_rng(seed)``; draw q, k, v as
float32 ``standard_normal`` of shape [B, H, T, d], then the beta source, then
lambda.  For bf16 workloads q, k, v are rounded once to bfloat16
(round-to-nearest-even) on the host, so the GPU and the oracle read the same
values.  beta and lambda stay float32.

The workloads stand in for the mixer activations of the ~130M-parameter,
length-1024 language models the paper trains; no dataset is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    variant: str          # F1, F2, F3, F1A, F2A, F3A
    batch: int
    heads: int
    seqlen: int
    dk: int
    dv: int
    chunk: int            # 0 = recurrent form
    window: int
    dtype: str            # "bf16" or "f32"
    beta_kind: str        # "uniform(a,b)" or "sigmoid"
    beta_lo: float
    beta_hi: float
    lam_kind: str         # "const" or "uniform"
    lam_lo: float
    lam_hi: float
    seed: int
    eps: float = 1e-6
    eps_gamma: float = 1e-3
    eps_rms: float = 1e-6

    @property
    def tokens(self) -> int:
        return self.batch * self.heads * self.seqlen

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Falcon-1 recurrent, fp32, 1 x 1 x 64 x 16
    "c1": Workload("c1", "F1", 1, 1, 64, 16, 16, 0, 1, "f32", "uniform", 0.1, 0.9,
                   "const", 0.01, 0.01, seed=1),
    # Falcon-1 chunk-parallel, bf16, 8 x 12 x 1024 x 64, C = 64
    "c2": Workload("c2", "F1", 8, 12, 1024, 64, 64, 64, 1, "bf16", "sigmoid", 0, 0,
                   "uniform", 0.0, 0.05, seed=2),
    # Falcon-1A, bf16, 2 x 12 x 16384 x 64, C = 64, strong ridge
    "c3": Workload("c3", "F1A", 2, 12, 16384, 64, 64, 64, 1, "bf16", "sigmoid", 0, 0,
                   "uniform", 0.5, 1.0, seed=3),
    # Falcon-2 per-column, bf16, 4 x 16 x 4096 x 128, C = 64
    "c4": Workload("c4", "F2", 4, 16, 4096, 128, 128, 64, 1, "bf16", "sigmoid", 0, 0,
                   "uniform", 0.0, 0.05, seed=4),
    # Falcon-3A window 8, bf16, 8 x 12 x 2048 x 64, C = 64
    "c5": Workload("c5", "F3A", 8, 12, 2048, 64, 64, 64, 8, "bf16", "sigmoid", 0, 0,
                   "uniform", 0.0, 0.05, seed=5),
    # single-token decode step at the c2 shape, continuing from a carried
    # state (the state is part of the inputs: see decode_state)
    "c2dec": Workload("c2dec", "F1", 8, 12, 1, 64, 64, 64, 1, "bf16", "sigmoid", 0, 0,
                      "uniform", 0.0, 0.05, seed=21),
    # parity-only extras
    "c3clamp": Workload("c3clamp", "F1A", 2, 12, 2048, 64, 64, 64, 1, "bf16", "sigmoid",
                        0, 0, "uniform", 0.5, 1.0, seed=31, eps_gamma=0.994),
    # Falcon-1 over the long sequences of c3 (2 x 12 x 16384 x 64, C = 64) with
    # c2's step distributions: few heads, a 256-chunk walk per head
    "c3f1": Workload("c3f1", "F1", 2, 12, 16384, 64, 64, 64, 1, "bf16", "sigmoid", 0, 0,
                     "uniform", 0.0, 0.05, seed=33),
    # Falcon-2A (per-column gains, inner-product write) at the c2 shape; its
    # chunk kernel takes d_k <= 64, so c4's d = 128 shape runs it token by token
    "c2f2a": Workload("c2f2a", "F2A", 8, 12, 1024, 64, 64, 64, 1, "bf16", "sigmoid", 0, 0,
                      "uniform", 0.0, 0.05, seed=22),
    "c5f3": Workload("c5f3", "F3", 8, 12, 512, 64, 64, 64, 8, "bf16", "sigmoid", 0, 0,
                     "uniform", 0.0, 0.05, seed=51),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned
    as float32 holding exactly representable bf16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def make_inputs(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw the workload's inputs.  Returns float32 numpy arrays
    q, k [B,H,T,dk]; v [B,H,T,dv]; beta [B,H,T] (F2: [B,H,T,dv]); lam [B,H,T]."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    shp_k = (w.batch, w.heads, w.seqlen, w.dk)
    shp_v = (w.batch, w.heads, w.seqlen, w.dv)
    q = rng.standard_normal(shp_k, dtype=np.float32)
    k = rng.standard_normal(shp_k, dtype=np.float32)
    v = rng.standard_normal(shp_v, dtype=np.float32)
    bshape = shp_v if w.variant in ("F2", "F2A") else shp_k[:3]
    if w.beta_kind == "sigmoid":
        z = rng.standard_normal(bshape)
        beta = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    else:
        beta = rng.uniform(w.beta_lo, w.beta_hi, bshape).astype(np.float32)
    if w.lam_kind == "const":
        lam = np.full(shp_k[:3], w.lam_lo, dtype=np.float32)
    else:
        lam = rng.uniform(w.lam_lo, w.lam_hi, shp_k[:3]).astype(np.float32)
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    return {"q": q, "k": k, "v": v, "beta": beta, "lam": lam}


def decode_state(w: Workload, seed: Optional[int] = None) -> dict:
    """A carried boundary state for a workload that continues a sequence:
    S [B,H,dk,dv] ~ N(0, 1/dk), x_next [B,H,dk] an RMS-normalised N(0,1)
    vector (a feature, as the previous call leaves it), and W-1 tail pairs
    (features and values) when the window is wider than 1.  float32."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 1000)
    B, H = w.batch, w.heads
    S = (rng.standard_normal((B, H, w.dk, w.dv)) / np.sqrt(w.dk)).astype(np.float32)
    xn = rng.standard_normal((B, H, w.dk))
    xn = (xn / np.sqrt(np.mean(xn * xn, axis=-1, keepdims=True))).astype(np.float32)
    h = max(w.window - 1, 0)
    tx = rng.standard_normal((B, H, h, w.dk))
    if h:
        tx = tx / np.sqrt(np.mean(tx * tx, axis=-1, keepdims=True))
    ty = rng.standard_normal((B, H, h, w.dv))
    return {"S": S, "x_next": xn, "tail_x": tx.astype(np.float32), "tail_y": ty.astype(np.float32),
            "n_tail": h}
