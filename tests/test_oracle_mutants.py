"""The oracle's pins must catch plausible mistakes.

Each case compiles a copy of ``oracle/prox_oracle.c`` with one planted
mistake (on the CPU, into a temporary directory), points the oracle shim
at it, runs every pin in ``test_oracle_pins.py`` and requires at least one
to fail.  The real oracle is restored afterwards.
"""
import inspect
import os
import subprocess

import pytest

import oracle as oracle_mod
from tests import test_oracle_pins as pins

MUTANTS = [
    ("silu with exp(+z)", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("k rounded down", "floor((1.0 - sparsity) * (double)F + 0.5)", "floor((1.0 - sparsity) * (double)F)"),
    ("quantizer truncates", "float t = rintf(w[i] / s);", "float t = truncf(w[i] / s);"),
    ("scale absmax/(qmax+1)", "float s = a / (float)qmax;", "float s = a / (float)(qmax + 1);"),
    ("int4 group index i%128", "scale[j * (d / 128) + i / 128]", "scale[j * (d / 128) + i % (d / 128)]"),
    ("tie goes to higher index", "return (a->idx < b->idx) ? -1 : (a->idx > b->idx) ? 1 : 0;",
     "return (a->idx < b->idx) ? 1 : (a->idx > b->idx) ? -1 : 0;"),
    ("up proxy reads gate codes", "u += xb[i] * dequant(qu, scu,", "u += xb[i] * dequant(qg, scg,"),
    ("salience from gate only", "return fabs(h * u);", "return fabs(h);"),
    ("batch salience not summed", "sc += salience_term(signal, act, g, u);", "sc = salience_term(signal, act, g, u);"),
    ("gate signal reads up", "if (signal == 1) return fabs(h);", "if (signal == 1) return fabs(u);"),
    ("up signal reads gate", "if (signal == 2) return fabs(u);", "if (signal == 2) return fabs(h);"),
    ("gelu without the cubic term", "(z + 0.044715 * z * z * z)", "(z + 0.044715 * z * z)"),
    ("activation choice ignored", "return act == 1 ? oracle_gelu_tanh(z) : oracle_silu(z);", "return oracle_silu(z);"),
    ("exact gate uses up weights", "g += (double)wg[j * d + i] * xb[i];", "g += (double)wu[j * d + i] * xb[i];"),
    ("down weight transposed", "(double)wd[m * F + sel[t]]", "(double)wd[(sel[t] * d + m) % (d * F)]"),
    ("one input too few kept", "for (int64_t t = 0; t < k_in; ++t)", "for (int64_t t = 0; t + 1 < k_in; ++t)"),
    ("rmsnorm without eps", "sqrt(ss / (double)d + eps)", "sqrt(ss / (double)d)"),
    ("rmsnorm sum not reset per token", "for (int64_t b = 0; b < B; ++b) {\n        double ss = 0.0;",
     "double ss = 0.0;\n    for (int64_t b = 0; b < B; ++b) {"),
    ("rmsnorm squares of token 0 for all", "ss += h[b * d + i] * h[b * d + i];", "ss += h[i] * h[i];"),
    ("silu missing z", "return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    ("e4m3 exponent bias 8", "v = ldexp(1.0 + (double)m / 8.0, e - 7);", "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("e4m3 subnormals 2^-10", "v = ldexp((double)m, -9);", "v = ldexp((double)m, -10);"),
    ("e4m3 ties away from zero", "(above == below && ((c + 1) & 1) == 0)", "(above == below)"),
    ("e4m3 no saturation", "if (a >= 448.0) return sign | 0x7E;", "if (a >= 464.0) return sign | 0x7F;"),
    ("fp8 scale for max 240", "float sc = a / 448.0f;", "float sc = a / 240.0f;"),
    ("fp8 up uses gate scale", "u += (double)su[j] *", "u += (double)sg[j] *"),
    ("fp8 down scale per column", "acc += (double)sd[m] * oracle_e4m3_decode(qd[m * F + sel[t]])",
     "acc += (double)sd[sel[t] % d] * oracle_e4m3_decode(qd[m * F + sel[t]])"),
]


def _pin_tests():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if params:
            argnames = [a.strip() for a in params[0].args[0].split(",")]
            for vals in params[0].args[1]:
                vals = vals if isinstance(vals, tuple) else (vals,)
                out.append((name, fn, dict(zip(argnames, vals))))
        else:
            out.append((name, fn, {}))
    return out


@pytest.mark.parametrize("label,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, label, old, new):
    src = open(os.path.join(os.path.dirname(oracle_mod.__file__), "prox_oracle.c")).read()
    assert src.count(old) == 1, "mutation site not found: " + old
    c = tmp_path / "mutant.c"
    c.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
                           "-shared", "-fPIC", "-o", str(so), str(c), "-lm"])
    caught = []
    oracle_mod.use_library(str(so))
    try:
        for name, fn, kw in _pin_tests():
            try:
                fn(oracle_mod, **kw)
            except (AssertionError, ValueError, IndexError):
                caught.append(name)
    finally:
        oracle_mod.use_library(None)
    assert caught, "no pin caught the planted mistake: " + label
