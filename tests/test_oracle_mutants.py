"""The oracle pins must catch plausible mistakes (CPU only).

Each case plants one mistake in a temporary copy of the oracle's C source
(never in the oracle itself), builds it, and runs tests/test_oracle_pins.py
against that copy in a subprocess.  The pins pass on the real oracle, so every
planted mistake must make at least one of them fail.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name -> (text in dp_oracle.c, replacement)
MUTANTS = {
    "reverse_substep_order": (
        "for (int j = 0; j < n_h; ++j) {\n            const size_t sub = tok * n_h + j;",
        "for (int jj = 0; jj < n_h; ++jj) {\n            const int j = n_h - 1 - jj;\n"
        "            const size_t sub = tok * n_h + j;"),
    "residual_sign": ("e[c] = vv[c] - acc;", "e[c] = vv[c] + acc;"),
    "transposed_state_read": ("acc += S[(size_t)r * dv + c] * kh[r];",
                              "acc += S[(size_t)c * dv + r] * kh[r];"),
    "beta_not_clamped": ("const double bt = clampd(beta[sub], 0.0, 2.0);",
                         "const double bt = beta[sub];"),
    "write_key_ignored": ("const double* w = kt ? kt + sub * dk : kh;", "const double* w = kh;"),
    "key_not_normalised": ("for (int r = 0; r < dk; ++r) kh[r] = kr[r] / den;",
                           "for (int r = 0; r < dk; ++r) kh[r] = kr[r];"),
    "gate_after_substeps": (
        "        if (g) {\n            /* H_{i,0} = g_i H_{i-1}: once per token, before its sub-steps */\n"
        "            const double gt = g[tok];\n"
        "            for (size_t x = 0; x < (size_t)dk * dv; ++x) S[x] *= gt;\n        }\n"
        "        for (int j = 0; j < n_h; ++j) {",
        "        for (int j = 0; j < n_h; ++j) {\n"
        "            if (g && j == 1) {\n                const double gt = g[tok];\n"
        "                for (size_t x = 0; x < (size_t)dk * dv; ++x) S[x] *= gt;\n            }"),
    "readout_before_last_substep": ("        /* o = H^T q after the token's last sub-step */",
                                    "        if (0) /* moved */"),
    "phase1_missing_beta_in_a": ("const double a = bu * ds;", "const double a = ds;"),
    "phase1_emit_after_update": (
        "            for (int r = 0; r < dk; ++r) ko[r] = d[r] * kh[r];\n",
        "            double* ko_late = ko;\n"),
    "phase1_no_projection": ("d[r] = clampd(rt * d[r] + coef * (kh[r] * kh[r]), dmin, dmax);",
                             "d[r] = rt * d[r] + coef * (kh[r] * kh[r]);"),
    "phase1_retention_ignored": ("const double rt = ret ? ret[tok] : 1.0;", "const double rt = 1.0;"),
    "phase1_retention_on_the_step": (
        "d[r] = clampd(rt * d[r] + coef * (kh[r] * kh[r]), dmin, dmax);",
        "d[r] = clampd(rt * (d[r] + coef * (kh[r] * kh[r])), dmin, dmax);"),
    "phase1_beta_free_keeps_beta": ("const double bu = beta_aware ? bt : 1.0;",
                                    "const double bu = bt;"),
    "channel_gate_on_columns": ("for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] *= al[r];",
                                "for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] *= al[c % dk];"),
    "channel_gate_ignored": ("for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] *= al[r];",
                             "for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] *= 1.0;"),
}

# mistakes in the gradient, caught by tests/test_oracle_bwd_pins.py
BWD_MUTANTS = {
    "bwd_drop_state_term_in_dk": ("dr -= Sj[(size_t)r * dv + c] * de[c];", "dr -= 0.0 * de[c];"),
    "bwd_state_grad_sign": ("dH[(size_t)r * dv + c] -= khj[r] * de[c];",
                            "dH[(size_t)r * dv + c] += khj[r] * de[c];"),
    "bwd_gate_grad_on_gated_state": ("for (size_t x = 0; x < DS; ++x) acc += dH[x] * Hp[x];",
                                     "for (size_t x = 0; x < DS; ++x) acc += dH[x] * Hs[x];"),
    "bwd_dq_from_earlier_state": ("const double* Hl = Hs + (size_t)n_h * DS;",
                                  "const double* Hl = Hs + (size_t)(n_h - 1) * DS;"),
    "bwd_norm_projection_dropped": ("dkj[r] = (dkh[r] - khj[r] * p) / nrm;", "dkj[r] = dkh[r] / nrm;"),
    "bwd_dbeta_ignores_clamp": ("(braw >= 0.0 && braw <= 2.0) ? dbt : 0.0", "dbt"),
    "bwd_write_grad_missing_beta": ("dr += bt * acc;", "dr += acc;"),
    "bwd_gate_not_applied_to_state_grad": ("for (size_t x = 0; x < DS; ++x) dH[x] *= g[tok];",
                                           "for (size_t x = 0; x < DS; ++x) dH[x] *= 1.0;"),
    # the phase-1 gradient
    "p1bwd_drop_step_term_in_dd": ("gd[r] = rt * gx[r] - eta * bu * bu / nb * gxs * (kh[r] * kh[r]) + kh[r] * gk[r];",
                                   "gd[r] = rt * gx[r] + kh[r] * gk[r];"),
    "p1bwd_write_key_not_into_d": ("gd[r] = rt * gx[r] - eta * bu * bu / nb * gxs * (kh[r] * kh[r]) + kh[r] * gk[r];",
                                   "gd[r] = rt * gx[r] - eta * bu * bu / nb * gxs * (kh[r] * kh[r]);"),
    "p1bwd_write_key_not_into_k": ("gkh[r] = 2.0 * kh[r] * gs + dt[r] * gk[r];", "gkh[r] = 2.0 * kh[r] * gs;"),
    "p1bwd_projection_mask_ignored": ("gx[r] = (x >= dmin && x <= dmax) ? gd[r] : 0.0;", "gx[r] = gd[r];"),
    "p1bwd_retention_not_applied": ("gd[r] = rt * gx[r] - eta", "gd[r] = gx[r] - eta"),
    "p1bwd_beta_term": ("const double gbu = gxs * eta * (1.0 - 2.0 * a) / nb;",
                        "const double gbu = gxs * eta * (1.0 - a) / nb;"),
    "p1bwd_norm_term_dropped": ("const double cn = n > eps ? coef / nb : 0.0;", "const double cn = 0.0;"),
    "p1bwd_emitted_key_uses_next_d": ("gkh[r] = 2.0 * kh[r] * gs + dt[r] * gk[r];",
                                      "gkh[r] = 2.0 * kh[r] * gs + (dt[r] + coef * kh[r] * kh[r]) * gk[r];"),
}

_EMIT_LATE = (
    "            for (int r = 0; r < dk; ++r) d[r] = clampd(rt * d[r] + coef * (kh[r] * kh[r]), dmin, dmax);\n",
    "            for (int r = 0; r < dk; ++r) d[r] = clampd(rt * d[r] + coef * (kh[r] * kh[r]), dmin, dmax);\n"
    "            for (int r = 0; r < dk; ++r) ko_late[r] = d[r] * kh[r];\n")

_READOUT_FIX = (
    "        if (0) /* moved */\n        const double* qq = q + tok * dk;",
    "        const double* qq = q + tok * dk;")


def _mutate(src, name):
    if name in BWD_MUTANTS:
        a, b = BWD_MUTANTS[name]
        assert src.count(a) == 1, name
        return src.replace(a, b)
    a, b = MUTANTS[name]
    assert src.count(a) >= 1, name
    s = src.replace(a, b)
    if name == "phase1_emit_after_update":
        # the first update of d is phase 1's own (the gradient's forward pass repeats the line)
        s = s.replace(*_EMIT_LATE, 1)
    if name == "readout_before_last_substep":
        # read out after the first sub-step instead of the last
        s = s.replace(_READOUT_FIX[0], _READOUT_FIX[1])
        s = s.replace(
            "                for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] += bw * e[c];\n            }\n        }",
            "                for (int c = 0; c < dv; ++c) S[(size_t)r * dv + c] += bw * e[c];\n            }\n"
            "            if (j == 0) {\n                const double* q0 = q + tok * dk;\n"
            "                double* o0 = out_h + (size_t)t * out_stride;\n"
            "                for (int c = 0; c < dv; ++c) {\n                    double acc = 0.0;\n"
            "                    for (int r = 0; r < dk; ++r) acc += S[(size_t)r * dv + c] * q0[r];\n"
            "                    o0[c] = acc;\n                }\n            }\n        }\n        if (0) {")
        s = s.replace("            oo[c] = acc;\n        }\n    }\n    if (fs_h)",
                      "            oo[c] = acc;\n        }\n        }\n    }\n    if (fs_h)")
    return s


@pytest.mark.parametrize("name", sorted(MUTANTS) + sorted(BWD_MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    pins = "test_oracle_bwd_pins.py" if name in BWD_MUTANTS else "test_oracle_pins.py"
    src = open(os.path.join(ROOT, "oracle", "dp_oracle.c")).read()
    mut = _mutate(src, name)
    assert mut != src
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    shutil.copytree(os.path.join(ROOT, "tests"), tmp_path / "tests",
                    ignore=shutil.ignore_patterns("__pycache__", "test_oracle_mutants.py",
                                                  "test_*gpu*.py", "test_api*.py"))
    (tmp_path / "oracle" / "dp_oracle.c").write_text(mut)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC",
                    str(tmp_path / "oracle" / "dp_oracle.c"), "-o",
                    str(tmp_path / "oracle" / "liboracle.so"), "-lm"], check=True)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "--rootdir", str(tmp_path), str(tmp_path / "tests" / pins)],
                       capture_output=True, text=True, cwd=str(tmp_path), timeout=600)
    assert "passed" in r.stdout or "failed" in r.stdout, r.stdout + r.stderr
    assert r.returncode != 0, f"mutant {name} survived every pin:\n{r.stdout[-2000:]}"
