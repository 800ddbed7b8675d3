"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant is a small edit of oracle/fa_oracle.c of the kind a plausible
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
    "mask_dropped": ("    if (p->mask)\n        s += p->mask[row * p->kl + j];", ""),
    "mask_in_base2_units": ("s += p->mask[row * p->kl + j];",
                            "s += 1.44269504f * p->mask[row * p->kl + j];"),
    "mask_of_first_head": ("s += p->mask[row * p->kl + j];",
                           "s += p->mask[(row % p->ql) * p->kl + j];"),
    "exp_sign_flipped": ("e[j] = expf(e[j] - m);", "e[j] = expf(m - e[j]);"),
    "exp_base2": ("e[j] = expf(e[j] - m);", "e[j] = exp2f(e[j] - m);"),
    "causal_off_by_one": ("if ((p->causal || p->window >= 0) && j > pos)",
                          "if ((p->causal || p->window >= 0) && j >= pos)"),
    "causal_offset_dropped": ("return (p->kl > p->ql ? p->kl - p->ql : 0) + i;", "return i;"),
    "causal_offset_unclamped": ("return (p->kl > p->ql ? p->kl - p->ql : 0) + i;",
                                "return (p->kl - p->ql) + i;"),
    "gqa_modulo_map": ("*kvhead = b * p->Hkv + h / (p->H / p->Hkv);",
                       "*kvhead = b * p->Hkv + h % p->Hkv;"),
    "k_transposed": ("dot += qr[d] * kh[j * p->D + d];", "dot += qr[d] * kh[d * p->kl + j];"),
    "dot_drops_last_dim": ("for (int64_t d = 0; d < p->D; ++d)\n        dot +=",
                           "for (int64_t d = 0; d + 1 < p->D; ++d)\n        dot +="),
    "scale_dropped": ("float s = p->scale * dot;", "float s = dot;"),
    "scale_squared": ("float s = p->scale * dot;", "float s = p->scale * p->scale * dot;"),
    "lse_without_max": ("*l = m + logf(z);", "*l = logf(z);"),
    "lse_base2_sum": ("*l = m + logf(z);", "*l = m + log2f(z);"),
    "no_normalisation": ("const float w = e[j] / z;", "const float w = e[j];"),
    "no_empty_row_guard": ("    if (m == -INFINITY) { /* no visible key */\n        *l = -INFINITY;"
                           "\n        return;\n    }\n", ""),
    "v_from_head_zero": ("const float *vh = p->v + kvh * p->kl * p->Dv;\n    float m",
                         "const float *vh = p->v + (kvh - kvh % p->Hkv) * p->kl * p->Dv;\n    float m"),
    "k_batch_dropped": ("const float *kh = p->k + kvh * p->kl * p->D;\n    const float *vh",
                        "const float *kh = p->k + (kvh % p->Hkv) * p->kl * p->D;\n    const float *vh"),
    "v_row_off_by_one": ("o[d] += w * vh[j * p->Dv + d];",
                         "o[d] += w * vh[(j + 1 < p->kl ? j + 1 : j) * p->Dv + d];"),
    "max_skips_last_key": ("if (e[j] > m)\n            m = e[j];",
                           "if (e[j] > m && j + 1 < p->kl)\n            m = e[j];"),
    "window_off_by_one": ("if (p->window >= 0 && j < pos - p->window)",
                          "if (p->window >= 0 && j <= pos - p->window)"),
    "window_too_wide": ("if (p->window >= 0 && j < pos - p->window)",
                        "if (p->window >= 0 && j < pos - p->window - 1)"),
    "window_offset_dropped": ("if (p->window >= 0 && j < pos - p->window)",
                              "if (p->window >= 0 && j < pos - (p->kl > p->ql ? p->kl - p->ql : 0)"
                              " - p->window)"),
    "window_ignored": ("if (p->window >= 0 && j < pos - p->window)",
                       "if (0 && j < pos - p->window)"),
    "window_without_causal": [("if ((p->causal || p->window >= 0) && j > pos)",
                               "if (p->causal && j > pos)"),
                              ("D, D, scale, 1, window, rows,", "D, D, scale, 0, window, rows,")],
    # value width: V or O addressed with the key width where it differs (the
    # smaller of the two widths, so that every access stays inside the buffers)
    "v_head_stride_uses_D": ("const float *vh = p->v + kvh * p->kl * p->Dv;\n    float m",
                             "const float *vh = p->v + kvh * p->kl * (p->D < p->Dv ? p->D : p->Dv);"
                             "\n    float m"),
    "v_row_stride_uses_D": ("o[d] += w * vh[j * p->Dv + d];",
                            "o[d] += w * vh[j * (p->D < p->Dv ? p->D : p->Dv) + d];"),
    "output_width_uses_D": ("forward_row(c->p, c->rows ? c->rows[t] : t, c->O + t * c->p->Dv,",
                            "forward_row(c->p, c->rows ? c->rows[t] : t, "
                            "c->O + t * (c->p->D < c->p->Dv ? c->p->D : c->p->Dv),"),
    # sinks: left out of the max, out of the sum, read for the wrong head, or
    # taken in base-2 units
    "sink_not_in_max": ("    if (sink > m)\n        m = sink;\n", ""),
    "sink_not_in_sum": ("    z += expf(sink - m);", "    z += 0.0f * expf(sink - m);"),
    "sink_of_kv_head": ("p->sinks[(row / p->ql) % p->H]", "p->sinks[(row / p->ql) % p->Hkv]"),
    "sink_base2": ("    z += expf(sink - m);", "    z += exp2f(sink - m);"),
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
        path = _build_mutant(tmp, name, MUTANTS[name])
        fwd, fwd_dv = oracle.bind(path), oracle.bind_dv(path)
        caught = []
        for pin_name, pin, f in ([(n, p, fwd) for n, p in pins.ALL_PINS]
                                 + [(n, p, fwd_dv) for n, p in pins.DV_PINS]
                                 + [(n, p, fwd_dv) for n, p in pins.SINK_PINS]):
            try:
                pin(f)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin_name)
        assert caught, f"no pin catches mutant {name}"


# Planted mistakes in the backward part of the oracle, caught by tests/pins_bwd.py.
BWD_MUTANTS = {
    "bwd_dq_scale_dropped": ("const float coef = p->scale * (P[j] * (dP[j] - d_i));",
                             "const float coef = (P[j] * (dP[j] - d_i));"),
    "bwd_ds_sign_flipped": ("const float coef = p->scale * (P[j] * (dP[j] - d_i));",
                            "const float coef = p->scale * (P[j] * (d_i - dP[j]));"),
    "bwd_D_dropped": ("d_i += P[j] * dp;", "d_i += 0.0f * dp;"),
    "bwd_p_base2": [("P[j] = (s == -INFINITY) ? 0.0f : expf(s - l_i);",
                     "P[j] = (s == -INFINITY) ? 0.0f : exp2f(s - l_i);"),
                    ("const float P = (s == -INFINITY) ? 0.0f : expf(s - c->L[row]);",
                     "const float P = (s == -INFINITY) ? 0.0f : exp2f(s - c->L[row]);")],
    "bwd_lse_ignored": [("P[j] = (s == -INFINITY) ? 0.0f : expf(s - l_i);",
                         "P[j] = (s == -INFINITY) ? 0.0f : expf(s);"),
                        ("const float P = (s == -INFINITY) ? 0.0f : expf(s - c->L[row]);",
                         "const float P = (s == -INFINITY) ? 0.0f : expf(s);")],
    "bwd_keys_position_off_by_one": ("if (!key_allowed(p, pos, j))\n                continue;\n"
                                     "            const float *qr",
                                     "if (!key_allowed(p, pos + 1, j))\n                continue;\n"
                                     "            const float *qr"),
    "bwd_dk_uses_k": ("dk[d] += coef * qr[d];", "dk[d] += coef * kh[j * p->D + d];"),
    "bwd_dk_scale_dropped": ("const float coef = p->scale * (P * (dp - c->Di[t]));",
                             "const float coef = (P * (dp - c->Di[t]));"),
    "bwd_dv_uses_q": ("dv[d] += P * gr[d];", "dv[d] += P * qr[d];"),
    "bwd_dv_missing_p": ("dv[d] += P * gr[d];", "dv[d] += gr[d];"),
    "bwd_group_first_head_only": ("for (int64_t r = 0; r < c->G * p->ql; ++r) {",
                                  "for (int64_t r = 0; r < p->ql; ++r) {"),
    "bwd_D_of_group_zero": ("(dp - c->Di[t])", "(dp - c->Di[r])"),
    "bwd_dp_uses_q": ("dp += gr[d] * vh[j * p->Dv + d];\n            dP[j] = dp;",
                      "dp += qr[d] * vh[j * p->Dv + d];\n            dP[j] = dp;"),
    "bwd_keys_dp_uses_q": ("dp += gr[d] * vh[j * p->Dv + d];\n            const float coef",
                           "dp += qr[d] * vh[j * p->Dv + d];\n            const float coef"),
    "bwd_dq_uses_q": ("dq[d] += coef * kh[j * p->D + d];", "dq[d] += coef * qr[d];"),
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


# Planted mistakes in the sink-gradient part of the oracle, caught by the sink
# pins of tests/pins_bwd.py.
SINK_BWD_MUTANTS = {
    "sink_grad_sign_flipped": ("dsinks[h] = (float)(-acc);", "dsinks[h] = (float)(acc);"),
    "sink_grad_weight_inverted": ("const float p_i = expf(sinks[h] - L[row]);",
                                  "const float p_i = expf(L[row] - sinks[h]);"),
    "sink_grad_weight_dropped": ("acc += (double)(p_i * Di[row]);", "acc += (double)(Di[row]);"),
    "sink_grad_first_batch_only": ("for (int64_t b = 0; b < B; ++b)\n                    for",
                                   "for (int64_t b = 0; b < 1; ++b)\n                    for"),
    "sink_grad_rows_of_head_zero": ("const int64_t row = (b * H + h) * ql + i;",
                                    "const int64_t row = (b * H) * ql + i;"),
    "sink_grad_D_unweighted": ("            d_i += P * dp;\n        }\n        c->Di[row] = d_i;",
                               "            d_i += dp;\n        }\n        c->Di[row] = d_i;"),
}


@pytest.mark.parametrize("name", sorted(SINK_BWD_MUTANTS))
def test_sink_pins_catch_planted_mistake(name):
    from tests import pins_bwd
    with tempfile.TemporaryDirectory() as tmp:
        path = _build_mutant(tmp, name, SINK_BWD_MUTANTS[name])
        bwd, bwd_sinks = oracle.bind_bwd(path), oracle.bind_bwd_sinks(path)
        caught = []
        for pin_name, pin in pins_bwd.SINK_PINS:
            try:
                pin(bwd, bwd_sinks)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin_name)
        assert caught, f"no sink pin catches mutant {name}"


# Planted mistakes in the given-O reading of D (D_i = rowsum(O_i * dO_i)),
# caught by the given-O pins of tests/pins_bwd.py.
GIVEN_O_MUTANTS = {
    "given_o_ignored": ("if (c->O) {", "if (0) {"),
    "given_o_row_of_head_zero": ("c->O + row * p->Dv", "c->O + (row % p->ql) * p->Dv"),
    "given_o_sign_flipped": ("d_i += orow[d] * gr[d];", "d_i -= orow[d] * gr[d];"),
    "given_o_not_reset": ("            d_i = 0.0f;\n            for (int64_t d = 0; d < p->Dv",
                          "            for (int64_t d = 0; d < p->Dv"),
    "given_o_squares_o": ("d_i += orow[d] * gr[d];", "d_i += orow[d] * orow[d];"),
}


@pytest.mark.parametrize("name", sorted(GIVEN_O_MUTANTS))
def test_given_o_pins_catch_planted_mistake(name):
    from tests import pins_bwd
    with tempfile.TemporaryDirectory() as tmp:
        bwd = oracle.bind_bwd(_build_mutant(tmp, name, GIVEN_O_MUTANTS[name]))
        caught = []
        for pin_name, pin in pins_bwd.GIVEN_O_PINS:
            try:
                pin(bwd)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin_name)
        assert caught, f"no given-O pin catches mutant {name}"
