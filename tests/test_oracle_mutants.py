"""The oracle's pins must catch plausible mistakes.  Each case plants one
mistake in a temporary copy of the oracle (never in the real file), runs the
pin suite against the copy, and expects it to fail.  CPU only."""
from __future__ import annotations

import pathlib
import shutil
import subprocess
import sys

import pytest

ROOT = pathlib.Path(__file__).resolve().parent.parent

MUTANTS = {
    "key_not_shifted": ("x_t = kh[:, t - 1]", "x_t = kh[:, t]"),
    "residual_sign": ('r = y_t - np.einsum("nkv,nk->nv", S, x_t)\n            S = gamma[:, None, None]',
                      'r = np.einsum("nkv,nk->nv", S, x_t) - y_t\n            S = gamma[:, None, None]'),
    "transposed_read": ('o[:, t] = np.einsum("nkv,nk->nv", S, qh[:, t])\n\n    # boundary',
                        'o[:, t] = np.einsum("nvk,nk->nv", S, qh[:, t])\n\n    # boundary'),
    "read_before_write": ('        # read-after-write\n        o[:, t] = np.einsum("nkv,nk->nv", S, qh[:, t])',
                          "        pass"),
    "ridge_dropped_from_step": ("den = mu + lamf[:, t] + eps", "den = mu + eps"),
    "no_decay": ("gamma = 1.0 - alpha", "gamma = 1.0 - 0*alpha"),
    "no_clamp": ("alpha = np.minimum(eta * lam_b, 1.0 - eps_gamma)", "alpha = eta * lam_b"),
    "f3_residual_not_at_state": ('rw = yw - np.einsum("nkv,nbk->nbv", S, xw)', "rw = yw"),
    "f3_window_not_averaged": ("S = gamma[:, None, None] * S + (eta / bt)[:, None, None] * g\n        elif",
                               "S = gamma[:, None, None] * S + (eta)[:, None, None] * g\n        elif"),
    "window_off_by_one": ("bt = min(window, len(pairs_x))", "bt = min(window + 1, len(pairs_x))"),
    "first_step_not_noop": ("noop = fresh and t == 0", "noop = False"),
    "trace_instead_of_lambda_max": ("mu = window_lambda_max(xw)", 'mu = np.einsum("nbk,nbk->n", xw, xw) / bt'),
    "f2_shared_carry": ('S = gamma[:, None, :] * S + np.einsum("nk,nv->nkv", x_t, eta * r)',
                        'S = gamma.mean(-1)[:, None, None] * S + np.einsum("nk,nv->nkv", x_t, eta * r)'),
    "l2_instead_of_rms": ("ms = np.mean(z * z, axis=-1, keepdims=True) + eps_rms",
                          "ms = np.sum(z * z, axis=-1, keepdims=True) + eps_rms"),
    "tail_too_long": ("keep = window - 1", "keep = window"),
    "f2a_first_columns_gain": ('S = gamma[:, None, :] * S + np.einsum("nk,nv->nkv", x_t, eta * y_t)',
                               'S = gamma[:, None, :] * S + np.einsum("nk,nv->nkv", x_t, eta[:, :1] * y_t)'),
    "f2a_shared_decay": ('S = gamma[:, None, :] * S + np.einsum("nk,nv->nkv", x_t, eta * y_t)',
                         'S = gamma[:, None, :1] * S + np.einsum("nk,nv->nkv", x_t, eta * y_t)'),
    "wrong_x_next": ("out_xnext = kh[:, T - 1].copy()", "out_xnext = kh[:, T - 2].copy()"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = (ROOT / "oracle" / "falcon_oracle.py").read_text()
    old, new = MUTANTS[name]
    assert old in src, f"mutation site for {name} no longer exists"
    shutil.copytree(ROOT / "oracle", tmp_path / "oracle")
    shutil.copytree(ROOT / "tests", tmp_path / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutants.py", "test_gpu*"))
    pkg = tmp_path / "linear_recurrent_weight_amd"
    pkg.mkdir()
    shutil.copy(ROOT / "linear_recurrent_weight_amd" / "inputs.py", pkg / "inputs.py")
    (pkg / "__init__.py").write_text("")
    (tmp_path / "oracle" / "falcon_oracle.py").write_text(src.replace(old, new, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0, f"planted mistake {name} went unnoticed:\n{r.stdout[-2000:]}"
