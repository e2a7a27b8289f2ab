"""The pins have teeth: each plausible mistake, planted in a copy of the
oracle's C source on the CPU, makes at least one pin test fail.

The planted copies live in a temporary directory; the oracle itself is never
modified.  Each mutant is built with the same gcc flags and the pin suite is
run against it in a subprocess (stopping at the first failure)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, original text, replacement) -- each must match exactly once
MUTANTS = [
    ("h-not-rounded", "h[j] = oracle_round(s, J->c_dt);", "h[j] = s;"),
    ("h-rounded-to-output-dtype", "h[j] = oracle_round(s, J->c_dt);", "h[j] = oracle_round(s, J->o_dt);"),
    ("bias-fused-in-affine", "v = oracle_round(acc, J->o_dt) + bias;", "v = acc + bias;"),
    ("ties-away-from-zero", "(d > 0.5 || (d == 0.5 && fmod(fl, 2.0) == 1.0))", "(d >= 0.5)"),
    ("round-via-fp32", "    if (isnan(v)) return v;\n    if (v == 0.0", "    v = (double)(float)v;\n    if (isnan(v)) return v;\n    if (v == 0.0"),
    ("flush-subnormals", "if (e < emin) e = emin;", "if (e < emin) return copysign(0.0, v);"),
    ("operands-not-cast", "xc[k] = oracle_round(widen(J->x, J->x_dt, m * K + k), J->c_dt);", "xc[k] = widen(J->x, J->x_dt, m * K + k);"),
    ("output-is-compute", "*output = h32 ? OR_F32 : c;", "*output = c;"),
    ("mixed-half-accepted", "if (h16 && hbf) return OR_MIXED_HALF;", ""),
    ("bypass-sign", "v = acc + J->scale * f + bias;", "v = acc - J->scale * f + bias;"),
    ("up-transposed", "f += h[j] * J->uc[n * r + j];", "f += h[j] * J->uc[j * N + n];"),
    ("lora-bias-dropped", "v = acc + J->scale * f + bias;", "v = acc + J->scale * f;"),
    ("overflow-threshold", "if (a >= maxv + ldexp(1.0, emax - p))", "if (a > maxv + ldexp(1.0, emax - p))"),
    ("scale-ignored", "v = acc + J->scale * f + bias;", "v = acc + f + bias;"),
    ("down-index", "s += xc[k] * J->dc[j * K + k];", "s += xc[k] * J->dc[k];"),
    ("fp16-exponent-bias", "else v = ldexp((double)(1024 + m), e - 25);", "else v = ldexp((double)(1024 + m), e - 24);"),
    ("merge-delta-rounded-first", "const double v = widen(J->w, J->w_dt, n * K + k) + J->scale * d;",
     "const double v = widen(J->w, J->w_dt, n * K + k) + J->scale * oracle_round(d, J->o_dt);"),
    ("merge-weight-cast", "const double v = widen(J->w, J->w_dt, n * K + k) + J->scale * d;",
     "const double v = oracle_round(widen(J->w, J->w_dt, n * K + k), J->o_dt == OR_F32 ? OR_F16 : J->o_dt) + J->scale * d;"),
    ("merge-scale-ignored", "const double v = widen(J->w, J->w_dt, n * K + k) + J->scale * d;",
     "const double v = widen(J->w, J->w_dt, n * K + k) + d;"),
    ("merge-down-transposed", "d += J->uc[n * r + j] * J->dc[j * K + k];", "d += J->uc[n * r + j] * J->dc[k * r + j];"),
    ("bwd-gh-not-rounded", "return oracle_round(B->scale * s, B->c_dt);", "return B->scale * s;"),
    ("bwd-gh-scale-missing", "return oracle_round(B->scale * s, B->c_dt);", "return oracle_round(s, B->c_dt);"),
    ("bwd-gh-up-transposed", "s += B->gc[m * B->N + n] * B->uc[n * B->r + j];",
     "s += B->gc[m * B->N + n] * B->uc[(j * B->N + n) % (B->N * B->r)];"),
    ("bwd-dx-fold-dropped", "const double v = s + f;", "const double v = s;"),
    ("bwd-dup-scale-missing", "const double v = B->scale * s;", "const double v = s;"),
    ("bwd-ddown-uses-x-not-cast", "double* xc = cast_all(x, x_dt, c_dt, M * K);\n    double* wc = cast_all(w, w_dt, c_dt, N * K);\n    double* dc = cast_all(down, down_dt, c_dt, r * K);\n    double* uc = cast_all(up, up_dt, c_dt, N * r);\n    double* gc",
     "double* xc = cast_all(x, x_dt, x_dt, M * K);\n    double* wc = cast_all(w, w_dt, c_dt, N * K);\n    double* dc = cast_all(down, down_dt, c_dt, r * K);\n    double* uc = cast_all(up, up_dt, c_dt, N * r);\n    double* gc"),
    ("dora-norm-without-delta", "const double v = widen(D->w, D->w_dt, n * K + k) + D->scale * d;",
     "const double v = widen(D->w, D->w_dt, n * K + k);"),
    ("dora-norm-not-rooted", "const double s = sqrt(q);", "const double s = q;"),
    ("dora-gain-inverted", "const double g = widen(D->m, D->m_dt, n) / (double)D->norms[n];",
     "const double g = (double)D->norms[n] / widen(D->m, D->m_dt, n);"),
    ("dora-bias-scaled", "const double v = g * (acc + D->scale * f) + bias;", "const double v = g * (acc + D->scale * f + bias);"),
    ("dora-gain-on-base-only", "const double v = g * (acc + D->scale * f) + bias;", "const double v = g * acc + D->scale * f + bias;"),
    ("bwd-dx-rounded-to-compute", "if (B->dx) store(B->dx, B->x_dt, i * K + k, oracle_round(v, B->x_dt));",
     "if (B->dx) store(B->dx, B->x_dt, i * K + k, oracle_round(oracle_round(v, B->c_dt), B->x_dt));"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name}: pattern not unique in oracle.c"
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o", str(lib),
                           str(mutant), "-lm", "-lpthread"])
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
