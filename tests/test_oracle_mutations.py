"""The pins in test_oracle.py and test_oracle_tail.py must fail for plausible mistakes in
the oracle.

Each case plants one mistake (an update order swapped, a dropped modifier term, a
flipped sign, a wrong dual in a factor, a transposed contraction, a missing scale,
a mirrored band offset, the wrong plan on V) in a temporary copy of the oracle and
runs the pin tests against that copy; every copy must fail.  CPU only.
"""

import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sinkhorn_band.py")

MUTATIONS = {
    "update_order_column_first": (
        "        u = row_update(S, v, h)\n        v = col_update(S, u, h)\n    if R == 0:",
        "        v = col_update(S, u, h)\n        u = row_update(S, v, h)\n    if R == 0:"),
    "drop_modifier_C_term": ("- C[None, :] * _row_vec(G, h))", ")"),
    "sign_of_dv1": ("dv1 = -ev1 * _col_sum", "dv1 = ev1 * _col_sum"),
    "wrong_dual_in_G": ("ev0 = np.exp(v0 - v2)", "ev0 = np.exp(v1 - v2)"),
    "transposed_dK": ("dK = s * _band_matvec_cols(dS, Q, h)", "dK = s * _band_matvec_rows(dS, Q, h)"),
    "missing_epsilon": ("s = 1.0 / (np.sqrt(d) * eps)", "s = 1.0 / np.sqrt(d)"),
    "du1_missing_column_factor": (
        "du1 = -eu1 * _row_sum(P22 * _row_vec(ev1 * dv1, h))",
        "du1 = -eu1 * _row_sum(P22 * _row_vec(dv1, h))"),
    "direct_four_wrong_P11": ("P11 = staircase_plan(S, u1, v1, h)", "P11 = staircase_plan(S, u2, v1, h)"),
    "mirrored_band_offset": ("j = i + _offsets(h)[:, None]", "j = i - _offsets(h)[:, None]"),
    "output_uses_P21": ("    uR, vR = duals[-2], duals[-1]", "    uR, vR = duals[-2], duals[-3]"),
}

# mistakes in the general-R adjoint forms, caught by the pins in test_oracle_tail.py
TAIL_MUTATIONS = {
    "tail_drop_column_modifier_term": (
        "        M = M - eu[a][None, :] * _row_vec(ev[a] * dv[a], h)\n", ""),
    "tail_wrong_level_in_dv": (
        "dv[a] = -ev[a] * _col_sum(P * (eu[a + 1] * du[a + 1])[None, :], h)",
        "dv[a] = -ev[a] * _col_sum(P * (eu[a] * du[a + 1])[None, :], h)"),
    "tail_wrong_column_factor_in_row_term": (
        "(eu[a] * du[a])[None, :] * _row_vec(ev[a - 1], h)",
        "(eu[a] * du[a])[None, :] * _row_vec(ev[a], h)"),
    "tail_sign_of_du": ("du[a] = -eu[a] * _row_sum(", "du[a] = eu[a] * _row_sum("),
    "tail_step_form_wrong_row_plan": (
        "Pab = staircase_plan(S, us[a], vs[a - 1], h)", "Pab = staircase_plan(S, us[a], vs[a], h)"),
    "tail_step_form_skips_column_term": (
        "        dS = dS - Paa * _row_vec(dv[a], h)\n", ""),
    "r0_base_duals_swapped": (
        "        return [u.copy(), v.copy()]\n", "        return [v.copy(), u.copy()]\n"),
    "full_backprop_one_step_short": (
        "pf = BandProblem(W=prob.W, T=0, R=prob.T + prob.R, eps=prob.eps)",
        "pf = BandProblem(W=prob.W, T=0, R=prob.T + prob.R - 1, eps=prob.eps)"),
}


# mistakes in the projective contraction certificate, caught by test_oracle_contraction.py
CONTRACTION_MUTATIONS = {
    "diameter_with_unpaired_columns": (
        "delta[rb, o + m] = float(np.max(diff.max(axis=2) - diff.min(axis=2)))",
        "delta[rb, o + m] = float(np.max(S.max(axis=1)[:, None] - S.min(axis=1)[None, :]))"),
    "block_active_one_token_too_far": (
        "if max(r1 - 1 - c0, c1 - 1 - r0) > h:", "if max(r1 - 1 - c0, c1 - 1 - r0) > h + 1:"),
    "coefficient_tanh_of_half": ("np.tanh(np.maximum(delta, 0.0) / 4.0)",
                                 "np.tanh(np.maximum(delta, 0.0) / 2.0)"),
    "diameter_misses_temperature": ("scale = 1.0 / (np.sqrt(d) * prob.eps)",
                                    "scale = 1.0 / np.sqrt(d)"),
}

CONTRACTION_SRC = os.path.join(ROOT, "oracle", "contraction.py")

# mistakes in the training step, caught by test_oracle_training.py
TRAINING_MUTATIONS = {
    "training_input_not_masked": ("    Xin = X * (1.0 - mask)[..., None]\n    Q, K, V = Xin @ Wq",
                                  "    Xin = X\n    Q, K, V = Xin @ Wq"),
    "training_dWo_transposed": ("dWo = O.reshape(-1, D).T @ dY.reshape(-1, D)",
                                "dWo = (O.reshape(-1, D).T @ dY.reshape(-1, D)).T"),
    "training_loss_gradient_not_halved": ("dY = 2.0 * diff / n", "dY = diff / n"),
    "training_heads_merged_wrong": (
        "    return Xh.transpose(0, 2, 1, 3).reshape(B, L, H * d)",
        "    return Xh.transpose(0, 2, 3, 1).reshape(B, L, H * d)"),
}

TRAINING_SRC = os.path.join(ROOT, "oracle", "training.py")

CASES = [(n, "tests/test_oracle.py") for n in sorted(MUTATIONS)] + \
        [(n, "tests/test_oracle_tail.py") for n in sorted(TAIL_MUTATIONS)] + \
        [(n, "tests/test_oracle_contraction.py") for n in sorted(CONTRACTION_MUTATIONS)] + \
        [(n, "tests/test_oracle_training.py") for n in sorted(TRAINING_MUTATIONS)]


@pytest.mark.parametrize("name,pins", CASES, ids=[c[0] for c in CASES])
def test_pins_catch_planted_mistake(name, pins):
    if name in CONTRACTION_MUTATIONS:
        before, after = CONTRACTION_MUTATIONS[name]
        path = CONTRACTION_SRC
    elif name in TRAINING_MUTATIONS:
        before, after = TRAINING_MUTATIONS[name]
        path = TRAINING_SRC
    else:
        before, after = {**MUTATIONS, **TAIL_MUTATIONS}[name]
        path = SRC
    src = open(path).read()
    assert before in src, f"mutation anchor for {name} no longer present"
    with tempfile.TemporaryDirectory() as d:
        shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                        ignore=shutil.ignore_patterns("__pycache__"))
        shutil.copytree(os.path.join(ROOT, "tests"), os.path.join(d, "tests"),
                        ignore=shutil.ignore_patterns("__pycache__", "golden"))
        with open(os.path.join(d, "oracle", os.path.basename(path)), "w") as f:
            f.write(src.replace(before, after))
        r = subprocess.run([sys.executable, "-m", "pytest", pins, "-q", "-x",
                            "-p", "no:cacheprovider"], cwd=d, capture_output=True, text=True,
                           timeout=300)
    assert r.returncode != 0, f"planted mistake {name} passed every pin:\n{r.stdout[-2000:]}"
