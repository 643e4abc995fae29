"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one of them: a dropped term, a wrong sign, a wrong index,
a transposed or shifted operand, a wrong threshold, a wrong packing code."""
import os

import pytest

import oracle
import pins

ORACLE_SRC = open(oracle.SRC).read()

# (name, original text, planted text)
MUTANTS = [
    ("strict_threshold", "if (v >= theta) t = 1;", "if (v > theta) t = 1;"),
    ("dropped_sign", "else if (v <= -theta) t = -1;", "else if (v <= -theta) t = 1;"),
    ("scale_row_index", "weff[r * out + c] = (double)scale[c] * (double)tern[r * out + c];",
     "weff[r * out + c] = (double)scale[r % out] * (double)tern[r * out + c];"),
    ("fwd_dropped_last_term",
     "for (int64_t r = 0; r < in; r++) {\n            double x = widen_one(X, dtype, t * in + r);",
     "for (int64_t r = 0; r < in - 1; r++) {\n            double x = widen_one(X, dtype, t * in + r);"),
    ("fwd_reversed_operand",
     "double x = widen_one(X, dtype, t * in + r);\n            const double *w = weff + r * out;",
     "double x = widen_one(X, dtype, t * in + (in - 1 - r));\n            const double *w = weff + r * out;"),
    ("dx_wrong_sign", "for (int64_t c = 0; c < out; c++) s += g[c] * w[c];",
     "for (int64_t c = 0; c < out; c++) s -= g[c] * w[c];"),
    ("dx_first_column_dropped", "for (int64_t c = 0; c < out; c++) s += g[c] * w[c];",
     "for (int64_t c = 1; c < out; c++) s += g[c] * w[c];"),
    ("gq_wrong_scale_index", "gq[r * nc + j] = acc[r * nc + j] * (double)scale[c];",
     "gq[r * nc + j] = acc[r * nc + j] * (double)scale[r % out];"),
    ("sgrad_uses_gq", "s += acc[r * nc + j] * (double)tern[r * out + c];",
     "s += acc[r * nc + j] * (double)scale[c] * (double)tern[r * out + c];"),
    ("wgrad_shifted_dY", "dys[t * nc + j] = widen_one(dY, dtype, t * out + c);",
     "dys[t * nc + j] = widen_one(dY, dtype, t * out + (c + 1) % out);"),
    ("pack_minus_one_code", "else if (t == -1) code = 3;  /* 11 */",
     "else if (t == -1) code = 2;  /* 11 */"),
    ("unpack_sign", "else if (code == 3) tern[r * out + c] = -1;",
     "else if (code == 3) tern[r * out + c] = 1;"),
    ("bf16_widen_shift", "uint32_t u = (uint32_t)((const uint16_t *)src)[i] << 16;",
     "uint32_t u = (uint32_t)((const uint16_t *)src)[i] << 15;"),
    ("pack_bit_order", "word |= code << (2 * j);", "word |= code << (30 - 2 * j);"),
    ("adamw_bias_correction_step", "bc1 = 1.0 - pow(b1, (double)t)", "bc1 = 1.0 - pow(b1, (double)t + 1.0)"),
    ("adamw_eps_inside_sqrt", "(sqrt(vhat) + eps)", "sqrt(vhat + eps)"),
    ("adamw_no_one_minus_b1", "m[c] = b1 * m[c] + (1.0 - b1) * g;", "m[c] = b1 * m[c] + g;"),
    ("adamw_coupled_decay", "const double g = sgrad[c] * scale_lr / lr;",
     "const double g = sgrad[c] * scale_lr / lr + wd * scale[c];"),
    ("adamw_dropped_lr_ratio", "const double g = sgrad[c] * scale_lr / lr;", "const double g = sgrad[c];"),
    ("panel_dead_inclusive", "if (mag < theta) counts[5] += h;", "if (mag <= theta) counts[5] += h;"),
    ("panel_rail_uses_theta", "if (mag == q_clamp) counts[4] += h;", "if (mag == theta) counts[4] += h;"),
    ("panel_churn_ignores_sign", "counts[6] += prev_tern[k] != now;", "counts[6] += (prev_tern[k] != 0) != (now != 0);"),
    ("panel_zero_counted_as_pos", "if (v >= theta) counts[3] += h;", "if (v >= 0) counts[3] += h;"),
    ("panel_scale_min_skips_first", "for (int64_t c = 0; c < out; c++) {\n        const double sv",
     "for (int64_t c = 1; c < out; c++) {\n        const double sv"),
    ("panel_histogram_off_by_one", "bins[(int)q[k] + 128]++;", "bins[(int)q[k] + 127 + (q[k] == -128)]++;"),
]


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, orig, planted):
    assert ORACLE_SRC.count(orig) == 1, f"mutation site for {name} is not unique"
    src = tmp_path / "tern_oracle.c"
    src.write_text(ORACLE_SRC.replace(orig, planted))
    lib = str(tmp_path / "libmut.so")
    oracle.build(src=str(src), out=lib, extra=["-I", os.path.dirname(oracle.SRC)])
    mut = oracle.Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(mut)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught the planted mistake {name}"
