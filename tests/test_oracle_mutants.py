"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant is a one-line edit of oracle/fa_oracle.c of the kind a plausible
bug would make (a dropped term, a wrong sign, index or unit, a transposed
operand, a missing guard). The copy is built on the CPU in a temporary
directory and run through tests/pins.py; the real oracle passes all pins
(test_oracle.py), so a mutant that passes them all would mean a blind spot.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "fa_oracle.c")

MUTANTS = {
    "mask_in_natural_units": ("s[j] += ORACLE_LOG2E * mr[j];", "s[j] += mr[j];"),
    "mask_dropped": ("\n    if (p->mask) {", "\n    if (0) {"),
    "exp_sign_flipped": ("s[j] = exp2f(s[j] - m);", "s[j] = exp2f(m - s[j]);"),
    "causal_off_by_one": ("\n        for (int64_t j = q_abs + 1; j < kl; ++j)",
                          "\n        for (int64_t j = q_abs; j < kl; ++j)"),
    "causal_offset_dropped": ("\n    const int64_t q_abs = (kl > ql ? kl - ql : 0) + i;",
                              "\n    const int64_t q_abs = i;"),
    "causal_offset_unclamped": [("\n    const int64_t q_abs = (kl > ql ? kl - ql : 0) + i;",
                                 "\n    const int64_t q_abs = (kl - ql) + i;"),
                                ("\n        for (int64_t j = q_abs + 1; j < kl; ++j)",
                                 "\n        for (int64_t j = (q_abs + 1 > 0 ? q_abs + 1 : 0); j < kl; ++j)")],
    "gqa_modulo_map": ("const int64_t kvh = h / (p->H / p->Hkv);",
                       "const int64_t kvh = h % p->Hkv;"),
    "k_transposed": ("\n            dot += qr[d] * kh[j * D + d];",
                     "\n            dot += qr[d] * kh[d * kl + j];"),
    "scale_dropped": ("s[j] = dot * q_scale;", "s[j] = dot * ORACLE_LOG2E;"),
    "log2e_dropped": ("const float q_scale = p->scale * ORACLE_LOG2E;",
                      "const float q_scale = p->scale;"),
    "lse_without_max": ("*l_out = m * ORACLE_LN2 + logf(sum);", "*l_out = logf(sum);"),
    "lse_base2_max": ("*l_out = m * ORACLE_LN2 + logf(sum);", "*l_out = m + logf(sum);"),
    "no_normalisation": ("const float w = s[j] / safe;", "const float w = s[j];"),
    "infinite_sentinel": ("float m = -FLT_MAX / 2.0f;", "float m = -INFINITY;"),
    "no_empty_row_guard": ("const float safe = (sum == 0.0f) ? 1.0f : sum;",
                           "const float safe = sum;"),
    "v_from_head_zero": ("\n    const float *vh = p->v + (b * p->Hkv + kvh) * kl * D;\n\n",
                         "\n    const float *vh = p->v + (b * p->Hkv) * kl * D;\n\n"),
    "k_batch_dropped": ("const float *qr = p->q + row * D;\n    const float *kh = p->k + (b * p->Hkv + kvh) * kl * D;",
                        "const float *qr = p->q + row * D;\n    const float *kh = p->k + kvh * kl * D;"),
    "v_row_off_by_one": ("const float *vr = vh + j * D;",
                         "const float *vr = vh + (j + 1 < kl ? j + 1 : j) * D;"),
    "window_off_by_one": ("for (int64_t j = 0; j < q_abs - p->window && j < kl; ++j)\n            s[j]",
                          "for (int64_t j = 0; j <= q_abs - p->window && j < kl; ++j)\n            s[j]"),
    "window_too_wide": ("for (int64_t j = 0; j < q_abs - p->window && j < kl; ++j)\n            s[j]",
                        "for (int64_t j = 0; j < q_abs - p->window - 1 && j < kl; ++j)\n            s[j]"),
    "window_offset_dropped": ("for (int64_t j = 0; j < q_abs - p->window && j < kl; ++j)\n            s[j]",
                              "for (int64_t j = 0; j < i - p->window && j < kl; ++j)\n            s[j]"),
    "window_ignored": ("\n    if (p->window >= 0) {", "\n    if (0) {"),
    "window_without_causal": ("oracle_problem p = {q, k, v, mask, H, Hkv, ql, kl, D, scale, 1, window};",
                              "oracle_problem p = {q, k, v, mask, H, Hkv, ql, kl, D, scale, 0, window};"),
    "max_skips_last_key": ("for (int64_t j = 0; j < kl; ++j)\n        if (s[j] > m)",
                           "for (int64_t j = 0; j + 1 < kl; ++j)\n        if (s[j] > m)"),
}


def _build_mutant(tmp, name, edits):
    src = open(SRC).read()
    if isinstance(edits, tuple):
        edits = [edits]
    for old, new in edits:
        assert src.count(old) == 1, f"mutation site for {name} not unique"
        src = src.replace(old, new)
    path_c = os.path.join(tmp, f"{name}.c")
    path_so = os.path.join(tmp, f"lib{name}.so")
    with open(path_c, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-pthread", "-o", path_so, path_c, "-lm"], check=True)
    return path_so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    with tempfile.TemporaryDirectory() as tmp:
        fwd = oracle.bind(_build_mutant(tmp, name, MUTANTS[name]))
        caught = []
        for pin_name, pin in pins.ALL_PINS:
            try:
                pin(fwd)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin_name)
        assert caught, f"no pin catches mutant {name}"


# Planted mistakes in the backward part of the oracle, caught by tests/pins_bwd.py.
BWD_MUTANTS = {
    "bwd_dq_scale_dropped": ("dqr[d] += p->scale * ds * kh[j * D + d];",
                             "dqr[d] += ds * kh[j * D + d];"),
    "bwd_ds_sign_flipped": ("const float ds = pr[j] * (s[j] - d_i);",
                            "const float ds = pr[j] * (d_i - s[j]);"),
    "bwd_D_dropped": ("d_i += pr[j] * dp;", "d_i += 0.0f * dp;"),
    "bwd_p_base2": ("expf(s[j] - l_i)", "exp2f(s[j] - l_i)"),
    "bwd_causal_off_by_one": ("for (int64_t j = q_abs + 1; j < kl; ++j)\n                    s[j] = -INFINITY;",
                              "for (int64_t j = q_abs + 2; j < kl; ++j)\n                    s[j] = -INFINITY;"),
    "bwd_dk_uses_k": ("dkh[j * D + d] += p->scale * ds * qr[d];",
                      "dkh[j * D + d] += p->scale * ds * kh[j * D + d];"),
    "bwd_dv_uses_q": ("dvh[j * D + d] += pr[j] * dor[d];", "dvh[j * D + d] += pr[j] * qr[d];"),
    "bwd_group_first_head_only": ("for (int64_t h = kvh * G; h < (kvh + 1) * G; ++h) {",
                                  "for (int64_t h = kvh * G; h < kvh * G + 1; ++h) {"),
    "bwd_mask_ignored": ("if (p->mask) {\n                    const float m = p->mask[row * kl + j];",
                         "if (0) {\n                    const float m = p->mask[row * kl + j];"),
    "bwd_dp_uses_q": ("dp += dor[d] * vh[j * D + d];", "dp += qr[d] * vh[j * D + d];"),
    "bwd_mask_base2": ("s[j] += m;", "s[j] += 1.44269504f * m;"),
    "bwd_lse_ignored": ("expf(s[j] - l_i)", "expf(s[j])"),
    "bwd_window_off_by_one": ("for (int64_t j = 0; j < q_abs - p->window && j < kl; ++j)\n                    s[j] = -INFINITY;",
                              "for (int64_t j = 0; j <= q_abs - p->window && j < kl; ++j)\n                    s[j] = -INFINITY;"),
    "bwd_window_ignored": ("if (p->window >= 0) {\n                for", "if (0) {\n                for"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_backward_pins_catch_planted_mistake(name):
    from tests import pins_bwd
    with tempfile.TemporaryDirectory() as tmp:
        bwd = oracle.bind_bwd(_build_mutant(tmp, name, BWD_MUTANTS[name]))
        caught = []
        for pin_name, pin in pins_bwd.ALL_PINS:
            try:
                pin(bwd)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin_name)
        assert caught, f"no backward pin catches mutant {name}"
