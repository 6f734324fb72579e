"""Host build of the kernels' window statistic (lambda_max of the small
window Gram, linear_recurrent_weight_amd/csrc/lambda_max.h) checked against
numpy's symmetric eigen-solver: rank-one, repeated and clustered spectra
(where an iteration from above can step onto or just past the largest root),
zero rows and duplicates.  CPU only (compiled with g++)."""
from __future__ import annotations

import ctypes
import pathlib
import shutil
import subprocess

import numpy as np
import pytest

CSRC = pathlib.Path(__file__).resolve().parent.parent / "linear_recurrent_weight_amd" / "csrc"

SHIM = r'''
#include "lambda_max.h"
extern "C" float lmax(const float *g, int n) {
    float G[8][8];
    for (int i = 0; i < 8; ++i)
        for (int j = 0; j < 8; ++j) G[i][j] = g[i * 8 + j];
    return falcon::psd_lambda_max(G, n);
}
'''


@pytest.fixture(scope="module")
def lmax(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("lmax")
    (d / "shim.cpp").write_text(SHIM)
    so = d / "liblmax.so"
    subprocess.run([gxx, "-O2", "-shared", "-fPIC", f"-I{CSRC}", str(d / "shim.cpp"), "-o", str(so)],
                   check=True)
    lib = ctypes.CDLL(str(so))
    lib.lmax.restype = ctypes.c_float
    lib.lmax.argtypes = [np.ctypeslib.ndpointer(np.float32, flags="C"), ctypes.c_int]
    return lib


@pytest.mark.parametrize("kind", ["random", "x_and_minus_x", "duplicates", "zero_rows", "collinear",
                                  "rms_normalised", "clustered", "repeated_top"])
def test_window_lambda_max_matches_eigvalsh(lmax, kind):
    rng = np.random.default_rng(hash(kind) % 2**32)
    for _ in range(400):
        n = int(rng.integers(1, 9))
        X = rng.standard_normal((n, 64))
        if kind == "x_and_minus_x" and n >= 2:
            X[1] = -X[0]
        elif kind == "duplicates" and n >= 3:
            X[2] = X[0]
            X[1] = 0
        elif kind == "zero_rows":
            X[: n // 2] = 0
        elif kind == "collinear":
            X[:] = X[0] * rng.choice([-1.0, 1.0, 0.5], size=(n, 1))
        elif kind == "rms_normalised":
            X *= 8.0 / np.linalg.norm(X, axis=1, keepdims=True)
        elif kind == "clustered":   # near-orthogonal rows of almost equal norm: all eigenvalues close
            Q, _ = np.linalg.qr(rng.standard_normal((64, n)))
            X = (Q.T * 8.0) * (1.0 + 1e-4 * rng.standard_normal((n, 1)))
        elif kind == "repeated_top" and n >= 2:   # the largest eigenvalue twice
            Q, _ = np.linalg.qr(rng.standard_normal((64, n)))
            s = rng.uniform(0.1, 1.0, n)
            s[:2] = 2.0
            X = (Q * s).T
        G = np.zeros((8, 8), np.float32)
        G[:n, :n] = X @ X.T
        ref = np.linalg.eigvalsh(X @ X.T)[-1]
        got = lmax.lmax(G.ravel().copy(), n)
        assert abs(got - ref) <= 2e-6 * max(ref, 1e-30) + 1e-30, (n, ref, got)


def test_zero_window(lmax):
    assert lmax.lmax(np.zeros(64, np.float32), 8) == 0.0
