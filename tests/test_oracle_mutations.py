"""Planted mistakes in the oracle must be caught by its pins.

Each case copies ``oracle/ssm_oracle.c`` with one plausible mistake (a dropped
term, a wrong sign, a transposed operand, a wrong index, a skipped reset, an
off-by-one rollback), builds it on the CPU, and runs the pin suite against it
in a child process: the suite has to fail.  Nothing here touches a GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ssm_oracle.c")

MUTATIONS = {
    "output_before_update": (
        "    for (int n = 0; n < N; ++n) row[n] = decay * row[n] + u * Bg[n];\n"
        "    double acc = 0.0;\n"
        "    for (int n = 0; n < N; ++n) acc += row[n] * Cg[n];\n",
        "    double acc = 0.0;\n"
        "    for (int n = 0; n < N; ++n) acc += row[n] * Cg[n];\n"
        "    for (int n = 0; n < N; ++n) row[n] = decay * row[n] + u * Bg[n];\n"),
    "dropped_skip_term": ("y[p] = acc + Dh * x[p];", "y[p] = acc;"),
    "decay_sign": ("exp(dt * c->A[h])", "exp(-dt * c->A[h])"),
    "B_C_swapped": ("row[n] = decay * row[n] + u * Bg[n];", "row[n] = decay * row[n] + u * Cg[n];"),
    "dt_not_applied": ("double u = dt * x[p];", "double u = x[p];"),
    "group_index": ("const int g = (int)(h / (H / G));\n  const int64_t PN = (int64_t)P * N;\n  double *s = c->state + h * PN;",
                    "const int g = (int)(h % G);\n  const int64_t PN = (int64_t)P * N;\n  double *s = c->state + h * PN;"),
    "reset_ignored": ("if (c->reset && c->reset[t]) memset(s, 0, sizeof(double) * PN);", ""),
    "rollback_off_by_one": ("if (k == a - 1) memcpy(kept", "if (k == (a < n_in ? a : a - 1)) memcpy(kept"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, name
    mutated = tmp_path / "mut.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-o", str(lib),
                    str(mutated), "-lm", "-lpthread"], check=True)
    env = dict(os.environ, SSM_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutation {name} survived the pins:\n{r.stdout[-2000:]}"
