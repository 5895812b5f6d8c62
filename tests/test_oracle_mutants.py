"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the pin
suite rejects every one of them.  This shows the pins constrain each term of the
recurrence, not only the oracle's agreement with itself."""

import os
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
SRC = ROOT / "oracle" / "oracle.c"

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("additive_writes_query", "for (int j = 0; j < dk; ++j) s[j] += vt * kt[j];",
     "for (int j = 0; j < dk; ++j) s[j] += vt * qt[j];"),
    ("gated_gates_the_write", "s[j] = a * s[j] + b * vt * kt[j];", "s[j] = a * (s[j] + b * vt * kt[j]);"),
    ("gated_drops_beta", "const double b = beta ? beta[t] : 1.0;\n      for (int j = 0; j < dk; ++j) s[j] = a * s[j]",
     "const double b = 1.0;\n      for (int j = 0; j < dk; ++j) s[j] = a * s[j]"),
    ("delta_sign", "s[j] = a * (s[j] - b * r * kt[j]) + b * vt * kt[j];",
     "s[j] = a * (s[j] + b * r * kt[j]) + b * vt * kt[j];"),
    ("delta_reads_with_query", "for (int j = 0; j < dk; ++j) r += s[j] * kt[j];",
     "for (int j = 0; j < dk; ++j) r += s[j] * qt[j];"),
    ("delta_ungated_erase", "s[j] = a * (s[j] - b * r * kt[j]) + b * vt * kt[j];",
     "s[j] = a * s[j] - b * r * kt[j] + b * vt * kt[j];"),
    ("read_previous_query", "const double *qt = q + (size_t)t * dk;\n    const double vt",
     "const double *qt = q + (size_t)(t > 0 ? t - 1 : 0) * dk;\n    const double vt"),
    ("value_row_index", "const double vt = v[(size_t)t * dv + row];", "const double vt = v[(size_t)t * dv + (dv - 1 - row)];"),
    ("based_feature_scale", "const double inv_sqrt2 = 1.0 / sqrt(2.0);\n  f[0] = 1.0;",
     "const double inv_sqrt2 = 0.5;\n  f[0] = 1.0;"),
    ("based_no_constant_feature", "f[0] = 1.0;", "f[0] = 0.0;"),
    ("based_square_only", "f[1 + dp + i * dp + j] = x[i] * x[j] * inv_sqrt2;", "f[1 + dp + i * dp + j] = x[i] * x[i] * inv_sqrt2;"),
    ("based_den_uses_key", "for (int f = 0; f < D; ++f) den += z[f] * fq[f];", "for (int f = 0; f < D; ++f) den += z[f] * fk[f];"),
    ("based_read_before_write_z", "z[f] += fk[f];\n    }", "z[f] += 0.0 * fk[f];\n    }"),
    ("compact_square_unscaled", "f[n++] = (a == b) ? x[a] * x[a] * inv_sqrt2 : x[a] * x[b];",
     "f[n++] = (a == b) ? x[a] * x[a] : x[a] * x[b];"),
    ("compact_cross_scaled", "f[n++] = (a == b) ? x[a] * x[a] * inv_sqrt2 : x[a] * x[b];",
     "f[n++] = (a == b) ? x[a] * x[a] * inv_sqrt2 : x[a] * x[b] * inv_sqrt2;"),
    ("compact_lower_triangle", "for (int b = a; b < dp; ++b) f[n++]", "for (int b = 0; b <= a; ++b) f[n++]"),
    ("write_mean_not_renormalised", "dot += (kb[t * dk + j] / n) * (mu[j] / mn);", "dot += (kb[t * dk + j] / n) * mu[j];"),
    ("write_keys_not_normalised", "if (n > 0.0)\n            for (int j = 0; j < dk; ++j) mu[j] += kb[t * dk + j] / n;",
     "if (n > 0.0)\n            for (int j = 0; j < dk; ++j) mu[j] += kb[t * dk + j];"),
    ("window_ignores_tail", "const long lo = c * C - tail > 0 ? c * C - tail : 0, hi = (c + 1) * C;",
     "const long lo = c * C, hi = (c + 1) * C;"),
    ("window_ties_to_latest", "if (v > bv) {", "if (v >= bv) {"),
    ("address_ties_to_latest", "if (d[t] > d[ts]) ts = t;", "if (d[t] >= d[ts]) ts = t;"),
    ("vote_uses_last_question_token", "if (c > m) m = c;", "m = c;"),
    ("vote_ranking_prefers_later_note", "if (pick < 0 || votes[i] > votes[pick]) pick = i;",
     "if (pick < 0 || votes[i] >= votes[pick]) pick = i;"),
    ("selection_not_in_document_order", "if (positions[y] < positions[x] || (positions[y] == positions[x] && y < x)) {",
     "if (0) {"),
    ("start_state_ignored", "memcpy(s, S0 + (bh * dv + row) * dk, sizeof(double) * dk);",
     "memset(s, 0, sizeof(double) * dk);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_planted_mistake(tmp_path, name, old, new):
    text = SRC.read_text()
    assert text.count(old) == 1, f"mutation site for {name} is not unique"
    (tmp_path / "oracle.c").write_text(text.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    str(tmp_path / "oracle.c"), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        str(ROOT / "tests" / "test_oracle_pins.py"),
                        str(ROOT / "tests" / "test_oracle_notebank_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pin suite:\n{r.stdout[-2000:]}"
