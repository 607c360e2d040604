"""Planted mistakes in a copy of the CPU oracle must each fail at least one pin.

Each mutant is the oracle's C source with one plausible error (a dropped term, a wrong
sign, index or operand, a changed constant), compiled on the CPU into a temporary
library and loaded by the pin tests through BEAM_ORACLE_LIB.  The real oracle is never
modified.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "beam_oracle.c")

MUTANTS = {
    "sigmoid_scale": ("return 1.0 / (1.0 + exp(-a));", "return 1.0 / (1.0 + exp(-2.0 * a));"),
    "group_score_max_only": ("gs32[g] = (gsize >= 2) ? a1 + a2 : a1;", "gs32[g] = a1;"),
    "no_group_limit": ("if (kept[e / gsize]) cand[nc++] = e;", "cand[nc++] = e;"),
    "interleaved_groups": ("if (kept[e / gsize]) cand[nc++] = e;", "if (kept[e % n_group]) cand[nc++] = e;"),
    "bias_in_weights": ("ssum += s64[best];", "ssum += sb64[best];"),
    "no_rho": ("wts[t * K + j] = rho * s64", "wts[t * K + j] = s64"),
    "ties_to_higher_index": ("return va > vb || (va == vb && a < b); }\nstatic int before_d",
                             "return va > vb || (va == vb && a > b); }\nstatic int before_d"),
    "silu_on_up": ("hh[i] = a * sigmoid(a) * c;", "hh[i] = c * sigmoid(c) * a;"),
    "gelu_like_gate": ("hh[i] = a * sigmoid(a) * c;", "hh[i] = a * sigmoid(1.702 * a) * c;"),
    "down_transposed": ("z += wval(w_down, s_down, base + i, w_fmt, &tabs) * hh[i];",
                        "z += wval(w_down, s_down, e * H * I + i * H + o, w_fmt, &tabs) * hh[i];"),
    "e4m3_exponent_bias_8": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 8.0, e - 8)"),
    "e4m3_subnormal_as_normal": ("e == 0 ? ldexp((double)m, -9)", "e == 0 ? ldexp(1.0 + m / 8.0, -7)"),
    "e4m3_mantissa_4_bits": ("ldexp(1.0 + m / 8.0, e - 7)", "ldexp(1.0 + m / 16.0, e - 7)"),
    "e8m0_scale_bias": ("ldexp(1.0, (int)s - 127); }", "ldexp(1.0, (int)s - 128); }"),
    "e8m0_no_nan": ("return s == 0xFF ? NAN : ldexp", "return s == 0x100 ? NAN : ldexp"),
    "e8m0_zero_byte_is_zero": ("return s == 0xFF ? NAN : ldexp", "return s == 0 ? 0.0 : s == 0xFF ? NAN : ldexp"),
    "scale_block_of_16": ("t->code[((const uint8_t*)p)[i]] * t->scale[sc[i >> 5]]",
                          "t->code[((const uint8_t*)p)[i]] * t->scale[sc[i >> 4]]"),
    "e2m1_exponent_bias_2": ("ldexp(1.0 + m / 2.0, e - 1)", "ldexp(1.0 + m / 2.0, e - 2)"),
    "e2m1_subnormal_as_normal": ("e == 0 ? 0.5 * m", "e == 0 ? ldexp(1.0 + m / 2.0, -1)"),
    "e2m1_sign_bit_2": ("const int sgn = (code >> 3) & 1", "const int sgn = (code >> 2) & 1"),
    "e2m1_nibbles_swapped": ("(i & 1) ? b >> 4 : b & 15", "(i & 1) ? b & 15 : b >> 4"),
    "e2m1_scale_block_of_16": ("t->fp4[(i & 1) ? b >> 4 : b & 15] * t->scale[sc[i >> 5]]",
                               "t->fp4[(i & 1) ? b >> 4 : b & 15] * t->scale[sc[i >> 4]]"),
    "weights_reversed": ("double wj = wts[t * K + j];", "double wj = wts[t * K + (K - 1 - j)];"),
    "rms_sum_not_mean": ("float r = (float)(1.0 / sqrt(ss / (double)H + (double)eps));",
                         "float r = (float)(1.0 / sqrt(ss + (double)eps));"),
    "rms_eps_outside_sqrt": ("float r = (float)(1.0 / sqrt(ss / (double)H + (double)eps));",
                             "float r = (float)(1.0 / (sqrt(ss / (double)H) + (double)eps));"),
    "rms_no_gain": ("float b = a * gain[h];", "float b = a;"),
    "residual_keep_weight_one": ("double a = sqrt((k - 1.0) / k), b = 1.0 / sqrt(k);",
                                 "double a = 1.0, b = 1.0 / sqrt(k);"),
    "residual_add_weight_1_over_k": ("double a = sqrt((k - 1.0) / k), b = 1.0 / sqrt(k);",
                                     "double a = sqrt((k - 1.0) / k), b = 1.0 / k;"),
    "post_norm_no_gain": ("b * ((double)gain[h] * yr[h] * r)", "b * (yr[h] * r)"),
    "post_norm_no_rsqrt": ("double r = 1.0 / sqrt(ss / (double)H + (double)eps);", "double r = 1.0;"),
}


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "pattern for %s must occur once" % name
    path = os.path.join(tmp, name + ".c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(tmp, name + ".so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-o", lib, path, "-lm"])
    env = dict(os.environ, BEAM_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, p.returncode, p.stdout[-400:]


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda n: _run_mutant(n, tmp), sorted(MUTANTS)))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, "mutants not caught by any pin: %s" % [n for n, _ in survivors]
