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


# planted mistakes in the backward oracle, caught by its own pins
MUTANTS_BWD = {
    "bwd_dx_state_term_dropped": (
        'dx[t] += eta[:, None] * (np.einsum("nkv,nv->nk", G, r) - np.einsum("nkv,nv->nk", Sp, w))',
        'dx[t] += eta[:, None] * np.einsum("nkv,nv->nk", G, r)'),
    "bwd_clamp_not_gated": ("deta = deta + np.where(unclamped[t], dalpha * lamf[:, t], 0.0)",
                            "deta = deta + dalpha * lamf[:, t]"),
    "bwd_decay_adjoint_at_post_state": ('dgamma = np.einsum("nkv,nkv->n", G, Sp)',
                                        'dgamma = np.einsum("nkv,nkv->n", G, S_post[t])'),
    "bwd_rank_one_adjoint_dropped": (
        'G = gamma[:, None, None] * G - eta[:, None, None] * np.einsum("nk,nv->nkv", x_t, w)',
        "G = gamma[:, None, None] * G"),
    "bwd_energy_term_dropped": ("dx[t] += 2.0 * dden[:, None] * x_t", "dx[t] += 0.0 * x_t"),
    "bwd_rms_vjp_sign": ("s * g - (s ** 3 / d) * zg * z", "s * g + (s ** 3 / d) * zg * z"),
    "bwd_read_at_pre_state": ('dqh[:, t] = np.einsum("nkv,nv->nk", S_post[t], dof[:, t])',
                              'dqh[:, t] = np.einsum("nkv,nv->nk", S_prev[t], dof[:, t])'),
    "bwd_key_gradient_shifted": ("dkf[:, t - 1] = phi_vjp(kf[:, t - 1], dx[t], eps_rms, phi_kind)",
                                 "dkf[:, t - 1] = phi_vjp(kf[:, t - 1], dx[t - 1], eps_rms, phi_kind)"),
}


def _run_pins_on_mutant(tmp_path, target, old, new, pins):
    src = (ROOT / "oracle" / target).read_text()
    assert old in src, "mutation site no longer exists"
    shutil.copytree(ROOT / "oracle", tmp_path / "oracle")
    shutil.copytree(ROOT / "tests", tmp_path / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutants.py", "test_gpu*"))
    pkg = tmp_path / "linear_recurrent_weight_amd"
    pkg.mkdir()
    shutil.copy(ROOT / "linear_recurrent_weight_amd" / "inputs.py", pkg / "inputs.py")
    (pkg / "__init__.py").write_text("")
    (tmp_path / "oracle" / target).write_text(src.replace(old, new, 1))
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           f"tests/{pins}"], cwd=tmp_path, capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    r = _run_pins_on_mutant(tmp_path, "falcon_oracle.py", old, new, "test_oracle_pins.py")
    assert r.returncode != 0, f"planted mistake {name} went unnoticed:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTANTS_BWD))
def test_backward_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS_BWD[name]
    r = _run_pins_on_mutant(tmp_path, "falcon_backward.py", old, new, "test_oracle_backward_pins.py")
    assert r.returncode != 0, f"planted mistake {name} went unnoticed:\n{r.stdout[-2000:]}"
