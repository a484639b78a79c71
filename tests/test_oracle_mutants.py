"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch each one.  The oracle source itself is never modified."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mla_oracle.c")

# (name, text in the source, replacement)
MUTANTS = [
    ("matvec_transposed_operand", "acc += A[(size_t)i * n + j] * x[j];", "acc += A[(size_t)j * m + i % m] * x[j % m];"),
    ("rope_term_dropped", "double rope = d_r > 0 ? mla_oracle_dot(d_r, q_r, KR + (size_t)t * d_r) : 0.0;",
     "double rope = 0.0;"),
    ("explicit_rope_key_dropped", "if (d_r > 0) memcpy(K + (size_t)t * dq + d_h, rope_row(P, b, t), sizeof(double) * d_r);",
     "if (d_r > 0) memset(K + (size_t)t * dq + d_h, 0, sizeof(double) * d_r);"),
    ("causal_offset_off_by_one", "const int vis = L - n_q + m + 1; /* tokens 0 .. L - n_q + m */",
     "const int vis = L - n_q + m; /* tokens 0 .. L - n_q + m */"),
    ("softmax_max_not_subtracted_wrong_sign", "p[t] = exp(s[t] - mx);", "p[t] = exp(mx - s[t]);"),
    ("page_row_index", "(size_t)(t % P->page_size)) * P->d_c", "(size_t)(t / P->page_size)) * P->d_c"),
    ("scale_ignored", "s[t] = scale * (content + rope);", "s[t] = (content + rope);"),
    ("output_projection_heads_reversed", "const double ox = o[(size_t)r * k + x];",
     "const double ox = o[(size_t)r * k + (k - 1 - x)];"),
    ("output_projection_rows_shifted", "const double* wx = w_o + (size_t)x * d;",
     "const double* wx = w_o + (size_t)((x + 1) % k) * d;"),
    ("rope_sine_sign", "y[2 * j] = x0 * c - x1 * s;", "y[2 * j] = x0 * c + x1 * s;"),
    ("rope_pairs_are_halves", "const double x0 = x[2 * j], x1 = x[2 * j + 1];",
     "const double x0 = x[j], x1 = x[j + d / 2];"),
    ("rope_frequency_exponent", "theta[j] = pow(base, -2.0 * j / d);", "theta[j] = pow(base, -1.0 * j / d);"),
    ("cache_append_page_row", "const size_t row = (size_t)page * page_size + (size_t)(pos[r] % page_size);",
     "const size_t row = (size_t)page * page_size + (size_t)(pos[r] / page_size % page_size);"),
    ("query_side_head_stride", "mla_oracle_matvec(d_h, d_qc, w_uq + (size_t)i * d_h * d_qc, cq,",
     "mla_oracle_matvec(d_h, d_qc, w_uq + (size_t)(i % 1) * d_h * d_qc, cq,"),
]


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor missing: " + name
    mutated = src.replace(old, new)
    c_file = tmp_path / "mutant.c"
    c_file.write_text(mutated)
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-o", str(so), str(c_file), "-lm"],
                   check=True)
    env = dict(os.environ, MLA_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pages.py"),
                        os.path.join(ROOT, "tests", "test_oracle_identities.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "planted mistake %s passed every pin:\n%s" % (name, r.stdout[-2000:])
