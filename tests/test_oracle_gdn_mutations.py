"""Planted mistakes in the Gated DeltaNet oracle must be caught by its pins.

Each case copies ``oracle/gdn_oracle.c`` with one plausible mistake, builds it
on the CPU and runs ``tests/test_oracle_gdn.py`` against it in a child
process: the suite has to fail.  Nothing here touches a GPU.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

MUTATIONS = {
    # the recurrence
    "erase_sign": ("alpha * (row[n] - beta * d * k[n])", "alpha * (row[n] + beta * d * k[n])"),
    "erase_not_gated": ("alpha * (row[n] - beta * d * k[n])", "alpha * row[n] - beta * d * k[n]"),
    "write_without_beta": ("+ beta * v[p] * k[n];", "+ v[p] * k[n];"),
    "read_with_query": ("for (int n = 0; n < N; ++n) d += row[n] * k[n];",
                        "for (int n = 0; n < N; ++n) d += row[n] * q[n];"),
    "output_with_key": ("for (int n = 0; n < N; ++n) acc += row[n] * q[n];",
                        "for (int n = 0; n < N; ++n) acc += row[n] * k[n];"),
    "output_before_update": (
        "    for (int n = 0; n < N; ++n) row[n] = alpha * (row[n] - beta * d * k[n]) + beta * v[p] * k[n];\n"
        "    double acc = 0.0;\n"
        "    for (int n = 0; n < N; ++n) acc += row[n] * q[n];\n",
        "    double acc = 0.0;\n"
        "    for (int n = 0; n < N; ++n) acc += row[n] * q[n];\n"
        "    for (int n = 0; n < N; ++n) row[n] = alpha * (row[n] - beta * d * k[n]) + beta * v[p] * k[n];\n"),
    "gate_sign": ("const double alpha = exp(c->dt[t * H + h] * c->A[h]);",
                  "const double alpha = exp(-c->dt[t * H + h] * c->A[h]);"),
    "group_index": ("const int g = (int)(h / (H / G));\n  const int64_t PN = (int64_t)P * N;\n  double *s = c->state + h * PN;",
                    "const int g = (int)(h % G);\n  const int64_t PN = (int64_t)P * N;\n  double *s = c->state + h * PN;"),
    "rollback_off_by_one": ("if (i == a - 1) memcpy(kept", "if (i == (a < n_in ? a : a - 1)) memcpy(kept"),
    # the replay form
    "replay_query_not_gated": ("w[n] = alpha * (w[n] - c[j] * kj[n]);", "w[n] = w[n] - c[j] * kj[n];"),
    "replay_fold_factor_order": (
        "T2[a * N + b] = alpha * (T[a * N + b] - beta * kj[a] * r[b]);",
        "T2[a * N + b] = alpha * (T[a * N + b] - beta * r[a] * kj[b]);"),
    "replay_entry_term_skips_self": ("for (int j = 0; j <= m; ++j) acc += c[j]",
                                     "for (int j = 0; j < m; ++j) acc += c[j]"),
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
    env = dict(os.environ, SSM_GDN_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_gdn.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutation {name} survived the pins:\n{r.stdout[-2000:]}"
