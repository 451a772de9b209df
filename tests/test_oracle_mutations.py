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
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "cq_oracle.c")

MUTATIONS = [
    ("diagonal dropped", "F = F + (double)d[i] * t2;", "F = F + t2;"),
    ("residual sign", "double t = (double)w[i] - s * (double)q[i];", "double t = (double)w[i] + s * (double)q[i];"),
    ("round half up", "float r = rintf(x);", "float r = floorf(x + 0.5f);"),
    ("clip one above qmin", "if (r < (float)qmin) r = (float)qmin;",
     "if (r < (float)(qmin + 1)) r = (float)(qmin + 1);"),
    ("clip one below qmax", "if (r > (float)qmax) r = (float)qmax;",
     "if (r > (float)(qmax - 1)) r = (float)(qmax - 1);"),
    ("tie keeps the higher pattern", "if (F < best) { second = best; best = F; best_b = b; }",
     "if (F <= best) { second = best; best = F; best_b = b; }"),
    ("sum instead of max", "if (Fe[e] > F) F = Fe[e];", "F = F + Fe[e];"),
    ("pooled without the mean", "            P = P / (double)E;\n            /* ascending b",
     "            /* ascending b"),
    ("pooled drops environments", "                P = P + Fe[e];\n", ""),
    ("pooled tie keeps the higher pattern", "if (P < bestp) { secondp = bestp; bestp = P; bestp_b = b; }",
     "if (P <= bestp) { secondp = bestp; bestp = P; bestp_b = b; }"),
    ("subnormal scale decoded one binade low", "return ldexp((double)man, -24);", "return ldexp((double)man, -25);"),
    ("normal scale exponent off by one", "return ldexp((double)(1024u + man), (int)ex - 25);",
     "return ldexp((double)(1024u + man), (int)ex - 24);"),
    ("environment stride", "out[e] = env_error(w, d + (size_t)e * G, G, s, q);",
     "out[e] = env_error(w, d + (size_t)e, G, s, q);"),
    ("environment stride fixed at 128", "out[e] = env_error(w, d + (size_t)e * G, G, s, q);",
     "out[e] = env_error(w, d + (size_t)e * 128, G, s, q);"),
    ("group stride fixed at 128", "const float *wg = w + (size_t)g * G;", "const float *wg = w + (size_t)g * 128;"),
    ("quotient transposed", "float x = w / s;", "float x = s / w;"),
    ("AbsMax divides by 7 whatever the range", "oracle_fp16_round(m / (float)qmax);", "oracle_fp16_round(m / 7.0f);"),
]


def _run_mutant(name, old, new, text, tmp):
    """Build the oracle with one planted mistake and run the pin suite against it; returns
    (return code, first failed pin or the last line of the run)."""
    src = os.path.join(tmp, "cq_oracle_mutant.c")
    with open(src, "w") as f:
        f.write(text.replace(old, new, 1))
    lib = os.path.join(tmp, "libcq_oracle_mutant.so")
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                           "-shared", "-fPIC", src, "-o", lib, "-lm"])
    env = dict(os.environ, CQ_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"), "-x", "-q",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    failed = [l for l in r.stdout.splitlines() if l.startswith("FAILED")]
    return r.returncode, (failed[0] if failed else (r.stdout.splitlines() or [""])[-1])


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    """Every mutant's pin run, several at once (each run is mostly single-threaded Python)."""
    text = open(SRC).read()
    for _, old, _ in MUTATIONS:
        assert text.count(old) == 1, old  # every mutation applies to exactly one place
    with ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
        futs = {name: ex.submit(_run_mutant, name, old, new, text, str(tmp_path_factory.mktemp("m")))
                for name, old, new in MUTATIONS}
        return {name: f.result() for name, f in futs.items()}


@pytest.mark.parametrize("name", [m[0] for m in MUTATIONS])
def test_pins_reject_mutant(name, outcomes):
    rc, first = outcomes[name]
    assert rc != 0, f"the pins did not notice: {name}\n{first}"
    print(f"{name}: {first}")
