"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of rr_oracle.c (on the CPU, in a
temporary directory), builds it, and runs the oracle pin tests against the
copy in a subprocess; at least one pin must fail.
"""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rr_oracle.c")
PINS = ["tests/test_oracle_estimate.py", "tests/test_oracle_select.py",
        "tests/test_oracle_attention.py", "tests/test_oracle_xattn.py",
        "tests/test_oracle_rescue.py"]

MUTANTS = [
    ("E1 sum instead of mean", "Kbar[((size_t)g * ns + j) * d + k] = sum / (double)S;",
     "Kbar[((size_t)g * ns + j) * d + k] = sum;"),
    ("E1 first token only", "sum += bf16_value(K[((size_t)(j * S + t) * Hkv + g) * d + k]);",
     "sum += bf16_value(K[((size_t)(j * S) * Hkv + g) * d + k]);"),
    ("E2 no rotation", "int t = i * S + (h % S);", "int t = i * S;"),
    ("E2 rotation by kv-head", "int t = i * S + (h % S);", "int t = i * S + ((h / (Hq / 2 > 0 ? 2 : 1)) % S);"),
    ("E2 missing scale", "    for (int j = 0; j <= i; ++j) s[j] *= sigma;\n", "\n"),
    ("E2 wrong kv-head", "stride_scores(Q, KbarT + (size_t)(h / G) * d * ns, ns, Hq, d, S, h, i, p);",
     "stride_scores(Q, KbarT + (size_t)(h % Hkv) * d * ns, ns, Hq, d, S, h, i, p);"),
    ("E3 strict causality", "for (int j = 0; j <= i; ++j) Arow[j / c] += p[j];",
     "for (int j = 0; j < i; ++j) Arow[j / c] += p[j];"),
    ("E3 no max shift sign", "        s[j] = exp(s[j] - m);", "        s[j] = exp(m - s[j]);"),
    ("E4 wrong block of stride", "Arow[j / c] += p[j];", "Arow[(j + 1) / c < nb ? (j + 1) / c : nb - 1] += p[j];"),
    ("E5 strict threshold", "if (kstar < 0 && C >= tau * W) kstar = k;", "if (kstar < 0 && C > tau * W) kstar = k;"),
    ("E5 ties by larger index", "return (u->j > v->j) - (u->j < v->j);", "return (u->j < v->j) - (u->j > v->j);"),
    ("E5 ascending order", "if (u->a > v->a) return -1;\n    if (u->a < v->a) return 1;",
     "if (u->a > v->a) return 1;\n    if (u->a < v->a) return -1;"),
    ("E5 off by one", "for (int k = 0; k <= kstar; ++k) kp[ord[k].j] = 1;",
     "for (int k = 0; k < kstar; ++k) kp[ord[k].j] = 1;"),
    ("E6 wrong kv-head", "int h = toks[2 * r], t = toks[2 * r + 1], g = h / G, I = t / B;",
     "int h = toks[2 * r], t = toks[2 * r + 1], g = h % Hkv, I = t / B;"),
    ("E6 strict causality", "for (int nn = 0; nn <= t; ++nn) {\n                if (!mrow[nn / B]) continue;\n                const uint16_t *kr",
     "for (int nn = 0; nn < t; ++nn) {\n                if (!mrow[nn / B]) continue;\n                const uint16_t *kr"),
    ("E6 missing scale", "l[nn] = sigma * dot;", "l[nn] = dot;"),
    ("X1 main diagonal", "const double *kk = Kd + ((size_t)(j * S + S - 1 - t) * Hkv + g) * d;",
     "const double *kk = Kd + ((size_t)(j * S + t) * Hkv + g) * d;"),
    ("X1 missing scale", "x[j] = sc * acc;", "x[j] = acc;"),
    ("X1 average ignored", "    if (average) sc /= (double)S;\n", "\n"),
    ("X1 wrong kv-head", "int g = h / (Hq / Hkv);", "int g = h % Hkv;"),
    ("X1 one query per stride", "bf16_value(Q[((size_t)(i * S + t) * Hq + h) * d + k]);",
     "bf16_value(Q[((size_t)(i * S) * Hq + h) * d + k]);"),
    ("R1 radius ignored", "Arow[J] = sigma * (dot + qn * rad[(size_t)g * nb + J]);",
     "Arow[J] = sigma * dot;"),
    ("R1 short block divided by B", "for (int k = 0; k < d; ++k) c[k] /= (double)(n1 - n0);",
     "for (int k = 0; k < d; ++k) c[k] /= (double)B;"),
    ("R1 radius as mean distance", "if (sqrt(s2) > r) r = sqrt(s2);", "r += sqrt(s2) / (double)(n1 - n0);"),
    ("R1 wrong kv-head", "int h = r / nb, I = r % nb, g = h / G;", "int h = r / nb, I = r % nb, g = h % Hkv;"),
    ("E6 mask ignored", "            for (int nn = 0; nn <= t; ++nn) {\n                if (!mrow[nn / B]) continue;\n                double p",
     "            for (int nn = 0; nn <= t; ++nn) {\n                if (!mrow[t / B]) continue;\n                double p"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mutated = src.replace(old, new)
    with tempfile.TemporaryDirectory() as tmp:
        c = os.path.join(tmp, "m.c")
        so = os.path.join(tmp, "libm.so")
        open(c, "w").write(mutated)
        subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC",
                        "-shared", "-o", so, c, "-lm"], check=True)
        env = dict(os.environ, RR_ORACLE_LIB=so, OMP_NUM_THREADS="4")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"]
                           + PINS, cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
        assert r.returncode != 0, "planted mistake '%s' passed every pin" % name
