"""Mutation check of the oracle's pins.

Each case plants one plausible mistake in a private copy of
oracle/gemm_oracle.c (a dropped term, a sign, a misplaced bias, a wrong
exponent or rounding rule), compiles it, and runs every pin of
test_oracle_pins.py that takes the oracle as an argument. At least one pin must
fail for every mutant; a mutant that survives means the pins have a blind spot.
Mutants are compiled on the CPU only and never touch a GPU.
"""
import inspect
import os

import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gemm_oracle.c")

MUTANTS = {
    "drop_last_k": ("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = 0; k < K - 1; ++k)"),
    "bias_by_row": ("if (j->bias) z += dec(j->dtype, j->bias[c]);",
                    "if (j->bias) z += dec(j->dtype, j->bias[i % N]);"),
    "bias_after_act": ("o[c] = act_apply(j->act, z);",
                       "o[c] = act_apply(j->act, acc[c]) + (z - acc[c]);"),
    "gelu_sign": ("erfc(-z / sqrt(2.0))", "erfc(z / sqrt(2.0))"),
    "gelu_no_half": ("return 0.5 * z * erfc", "return z * erfc"),
    "gelu_scale": ("erfc(-z / sqrt(2.0))", "erfc(-z / 2.0)"),
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(z));"),
    "sigmoid_neg_branch": ("return e / (1.0 + e);", "return 1.0 / (1.0 + e);"),
    "softplus_drops_z": ("return z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z));",
                         "return z > 0.0 ? log1p(exp(-z)) : log1p(exp(z));"),
    "softplus_log_not_log1p": ("return z > 0.0 ? z + log1p(exp(-z)) : log1p(exp(z));",
                               "return z > 0.0 ? z + log(exp(-z)) : log1p(exp(z));"),
    "gelu_tanh_cubic_coeff": ("0.044715 * z * z * z", "0.04715 * z * z * z"),
    "gelu_tanh_neg_branch": ("return z * e / (1.0 + e);", "return z / (1.0 + e);"),
    "e4m3_exponent_bias": ("ldexp((double)(fr | 0x8), ex - 10)", "ldexp((double)(fr | 0x8), ex - 11)"),
    "e4m3_nan_rule": ("else if (ex == 15 && fr == 7)", "else if (ex == 15)"),
    "e5m2_hidden_bit": ("ldexp((double)(fr | 0x4), ex - 17)", "ldexp((double)(fr | 0x8), ex - 17)"),
    "fp8_scale_dropped": ("double z = j->scale * acc[c];", "double z = acc[c];"),
    "fp8_scale_on_bias": ("if (j->bias) z += dec(j->dtype, j->bias[c]);",
                          "if (j->bias) z += j->scale * dec(j->dtype, j->bias[c]);"),
    "leaky_relu": ("return z > 0.0 ? z : 0.0;", "return z > 0.0 ? z : 0.01 * z;"),
    "f16_exp_off_by_one": ("ldexp((double)(fr | 0x400), ex - 25)", "ldexp((double)(fr | 0x400), ex - 24)"),
    "f16_subnormal_scale": ("ldexp((double)fr, -24)", "ldexp((double)fr, -25)"),
    "bf16_hidden_bit": ("ldexp((double)(fr | 0x80), ex - 134)", "ldexp((double)(fr | 0x100), ex - 134)"),
    "round_truncates": ("double r = rint(a / q);", "double r = floor(a / q);"),
    "round_half_up": ("double r = rint(a / q);", "double r = floor(a / q + 0.5);"),
    "abs_sum_signed": ("aacc[c] += aa * fabs(brow[c]);", "aacc[c] += aa * brow[c];"),
    "transpose_b_reads_kn": ("d->b_nk ? j * d->K + k : t", "d->b_nk ? k * d->N + j : t"),
    "transpose_a_reads_mk": ("j->a_km ? k * j->M + i : i * K + k",
                             "j->a_km ? i * K + k : i * K + k"),
    "second_operand_row": ("const double *brow = j->Bd + k * N;",
                           "const double *brow = j->Bd + (K - 1 - k) * N;"),
}


def _pins():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        params = inspect.signature(fn).parameters
        if "orc" not in params:
            continue
        marks = getattr(fn, "pytestmark", [])
        grid = [dict()]
        for m in marks:
            if m.name == "parametrize":
                argnames = [a.strip() for a in m.args[0].split(",")]
                new = []
                for g in grid:
                    for v in m.args[1]:
                        vals = v if len(argnames) > 1 else (v,)
                        new.append({**g, **dict(zip(argnames, vals))})
                grid = new
        out.extend((name, fn, g) for g in grid)
    return out


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(mutant, tmp_path):
    before, after = MUTANTS[mutant]
    src = open(SRC).read()
    assert src.count(before) == 1, "mutation site not found: %r" % before
    path = tmp_path / ("mutant_%s.c" % mutant)
    path.write_text(src.replace(before, after))
    so = oracle.build(force=True, src=str(path), out=str(tmp_path / ("lib%s.so" % mutant)))
    orc = oracle.Oracle(so)
    failed = []
    for name, fn, kw in _pins():
        try:
            fn(orc=orc, **kw)
        except Exception:   # an assertion or a rejected argument both count as caught
            failed.append(name)
    assert failed, "mutant %s survived every pin" % mutant
