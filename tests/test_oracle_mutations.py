"""The oracle's pins catch plausible mistakes: each case plants one mistake in a copy of the
oracle's C source, builds it, and runs the pin suite against it; at least one pin must fail.

The mistakes are the kinds the pins are meant to rule out: a dropped factor, a wrong sign, a
wrong rounding or clipping rule, the tie rule reversed, max and sum confused, a missing mean,
a wrong decoding of binary16 scales, a transposed index.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "cq_oracle.c")

MUTATIONS = [
    ("diagonal dropped", "F = F + (double)d[i] * t2;", "F = F + t2;"),
    ("residual sign", "double t = (double)w[i] - s * (double)q[i];", "double t = (double)w[i] + s * (double)q[i];"),
    ("round half up", "float r = rintf(x);", "float r = floorf(x + 0.5f);"),
    ("clip at -7", "if (r < -8.0f) r = -8.0f;", "if (r < -7.0f) r = -7.0f;"),
    ("tie keeps the higher pattern", "if (F < best) { second = best; best = F; best_b = b; }",
     "if (F <= best) { second = best; best = F; best_b = b; }"),
    ("sum instead of max", "if (Fe[e] > F) F = Fe[e];", "F = F + Fe[e];"),
    ("pooled without the mean", "            P = P / (double)E;\n            /* ascending b",
     "            /* ascending b"),
    ("subnormal scale decoded one binade low", "return ldexp((double)man, -24);", "return ldexp((double)man, -25);"),
    ("normal scale exponent off by one", "return ldexp((double)(1024u + man), (int)ex - 25);",
     "return ldexp((double)(1024u + man), (int)ex - 24);"),
    ("environment stride", "out[e] = env_error(w, d + (size_t)e * GROUP, s, q);",
     "out[e] = env_error(w, d + (size_t)e, s, q);"),
    ("quotient transposed", "float x = w / s;", "float x = s / w;"),
]


@pytest.fixture(scope="module")
def source():
    text = open(SRC).read()
    for _, old, _ in MUTATIONS:
        assert text.count(old) == 1, old  # every mutation applies to exactly one place
    return text


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_reject_mutant(name, old, new, source, tmp_path):
    src = tmp_path / "cq_oracle_mutant.c"
    src.write_text(source.replace(old, new, 1))
    lib = tmp_path / "libcq_oracle_mutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                           "-shared", "-fPIC", str(src), "-o", str(lib), "-lm"])
    env = dict(os.environ, CQ_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"), "-x", "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"the pins did not notice: {name}\n{r.stdout[-2000:]}"
    failed = [l for l in r.stdout.splitlines() if l.startswith("FAILED")]
    print(f"{name}: {failed[0] if failed else r.stdout.splitlines()[-1]}")
