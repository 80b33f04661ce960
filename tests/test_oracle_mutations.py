"""Planted mistakes in the oracle are caught by its pins (CPU only).

Each case copies ``oracle/oracle.c``, plants one plausible mistake (a
transposed operand, a dropped term, an ignored leading dimension, a wrong
rounding, exponent bias, block size or tolerance), compiles the copy with
the oracle's own flags into a temporary library, and runs the oracle's pin
tests (``tests/test_oracle.py``) against it through ``ORACLE_LIB``: they
must fail.  The unmodified copy, built the same way, must pass.  The
in-tree oracle is never touched.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (what, text in oracle.c, replacement, which occurrence)
MUTATIONS = [
    ("A.B^T reads B transposed",
     "bt64[j * K + k] = (layout == ORACLE_NT) ? oracle_decode(fmt, B[j * ldb + k])",
     "bt64[j * K + k] = (layout == ORACLE_NT) ? oracle_decode(fmt, B[k * ldb + j])", 1),
    ("A.B reads B as N-strided", ": oracle_decode(fmt, B[k * ldb + j]);\n#pragma",
     ": oracle_decode(fmt, B[k * N + j]);\n#pragma", 1),
    ("lda ignored", "a64[i * K + k] = oracle_decode(fmt, A[i * lda + k])",
     "a64[i * K + k] = oracle_decode(fmt, A[i * K + k])", 1),
    ("last K term dropped", "for (int64_t k = 0; k < K; ++k) {\n        double prod",
     "for (int64_t k = 0; k < K - 1; ++k) {\n        double prod", 1),
    ("single entries of A.B read B transposed",
     "                                     : oracle_decode(fmt, B[k * ldb + j]);\n    double prod",
     "                                     : oracle_decode(fmt, B[j * ldb + k]);\n    double prod", 1),
    ("single entries of A.B^T read B transposed",
     "double b = (layout == ORACLE_NT) ? oracle_decode(fmt, B[j * ldb + k])",
     "double b = (layout == ORACLE_NT) ? oracle_decode(fmt, B[k * ldb + j])", 1),
    ("single entries of A.B^T stride B by K instead of ldb",
     "double b = (layout == ORACLE_NT) ? oracle_decode(fmt, B[j * ldb + k])",
     "double b = (layout == ORACLE_NT) ? oracle_decode(fmt, B[j * K + k])", 1),
    ("single entries ignore lda", "double a = oracle_decode(fmt, A[i * lda + k]);",
     "double a = oracle_decode(fmt, A[i * K + k]);", 1),
    ("single entries of A.B stride B by K instead of ldb",
     "                                     : oracle_decode(fmt, B[k * ldb + j]);\n    double prod",
     "                                     : oracle_decode(fmt, B[k * K + j]);\n    double prod", 1),
    ("sum of |a b| signed", "s += fabs(prod);\n      }", "s += prod;\n      }", 1),
    ("rounding truncates", "double r = nearbyint(a / q) * q;", "double r = trunc(a / q) * q;", 1),
    ("rounding half away from zero", "double r = nearbyint(a / q) * q;",
     "double r = floor(a / q + 0.5) * q;", 1),
    ("FP16 minimum exponent off by one",
     "static int fmt_emin(int fmt) { return fmt == ORACLE_FMT_F16 ? -14 : -126; }",
     "static int fmt_emin(int fmt) { return fmt == ORACLE_FMT_F16 ? -15 : -126; }", 1),
    ("ulp one binade off", "return ldexp(1.0, E - fmt_p(fmt) + 1);",
     "return ldexp(1.0, E - fmt_p(fmt));", 1),
    ("tolerance doubled", "double tol = oracle_ulp(fmt, d[t]) + ldexp(s[t], -11);",
     "double tol = oracle_ulp(fmt, d[t]) + ldexp(s[t], -10);", 1),
    # (">=" -> ">" here would be an equivalent mutant: a value rounded to
    # exactly 2^(emax+1) encodes as the infinity pattern either way)
    ("overflow one binade early", "if (r >= ldexp(1.0, emax + 1)) return sign | inf;",
     "if (r >= ldexp(1.0, emax)) return sign | inf;", 1),
    ("FP8: E4M3 exponent bias off by one", "ldexp((double)(8 + m), e - 10)",
     "ldexp((double)(8 + m), e - 9)", 1),
    ("FP8: E4M3 subnormal scale", "ldexp((double)m, -9)", "ldexp((double)m, -8)", 1),
    ("FP8: E4M3 NaN code decoded as a number", "if (e == 15 && m == 7) return NAN;",
     "if (e == 16) return NAN;", 1),
    ("FP8: E8M0 bias off by one", "ldexp(1.0, (int)e - 127)", "ldexp(1.0, (int)e - 126)", 1),
    ("FP8: scale blocks of 16", "SX[r * ldsx + k / 32]", "SX[r * ldsx + k / 16]", 1),
    ("FP8: last K term dropped", "for (int64_t k = 0; k < K; ++k) {\n        double prod",
     "for (int64_t k = 0; k < K - 1; ++k) {\n        double prod", 2),
]


def _build(text: str, out_dir: str) -> str:
    src = os.path.join(out_dir, "oracle.c")
    lib = os.path.join(out_dir, "liboracle.so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-w", "-o", lib, src,
                    "-lm"], check=True)
    return lib


def _pins_pass(lib: str) -> bool:
    env = dict(os.environ, ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle.py"), "-x",
                        "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                       text=True)
    return r.returncode == 0


def _plant(text: str, old: str, new: str, nth: int) -> str:
    pos = -1
    for _ in range(nth):
        pos = text.find(old, pos + 1)
        assert pos >= 0, "the oracle no longer contains %r" % old
    return text[:pos] + new + text[pos + len(old):]


def test_unmodified_copy_passes(tmp_path):
    assert _pins_pass(_build(open(SRC).read(), str(tmp_path)))


@pytest.mark.parametrize("what,old,new,nth", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(what, old, new, nth, tmp_path):
    text = _plant(open(SRC).read(), old, new, nth)
    assert not _pins_pass(_build(text, str(tmp_path))), "pins missed: " + what
