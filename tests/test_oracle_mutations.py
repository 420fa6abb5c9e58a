"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/pda_oracle.c (on the CPU),
builds it, and runs the pin suites against it in a child pytest; the suites
must fail.  The unmodified oracle passes the same suites (the other test files).
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pda_oracle.c")
PIN_FILES = ["tests/test_oracle_pins.py", "tests/test_oracle_mla.py",
             "tests/test_oracle_multitoken.py", "tests/test_oracle_append.py"]

MUTATIONS = [
    ("interleaved head grouping", "int kvh = h / G;", "int kvh = h % Hkv;"),
    ("softmax scale dropped", "s[j] = scale * acc;", "s[j] = acc;"),
    ("log base 2 in the LSE", "*lse = m + log(z);", "*lse = m + log2(z);"),
    ("output not normalized", "out[e] /= z;", "out[e] /= 1.0;"),
    ("page slot off by one", "int64_t slot = j % P;", "int64_t slot = (j + 1) % P;"),
    ("wrong logical page", "int32_t page = table_row[j / P];",
     "int32_t page = table_row[j / (P + 1)];"),
    ("dequant scale dropped", "dec_elem(dtype, cache, base + i) * mult;",
     "dec_elem(dtype, cache, base + i);"),
    ("fp8 exponent bias", "ldexp(1.0 + (double)m / 8.0, e - 7)",
     "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    ("fp16 mantissa width", "ldexp(1.0 + (double)m / 1024.0, e - 15)",
     "ldexp(1.0 + (double)m / 512.0, e - 15)"),
    ("bf16 exponent bias", "ldexp(1.0 + (double)m / 128.0, e - 127)",
     "ldexp(1.0 + (double)m / 128.0, e - 126)"),
    ("V read from the K cache", "int rv = gather_rows(v_cache,", "int rv = gather_rows(k_cache,"),
    ("MLA value taken from the record's tail",
     "P, (int64_t)P * rec, rec, 0,\n                           d_latent, kv_scale,",
     "P, (int64_t)P * rec, rec, d_rope,\n                           d_latent, kv_scale,"),
    ("MLA value missing the latent scale",
     "d_latent, kv_scale, t0, t1, V);", "d_latent, 1.0, t0, t1, V);"),
    ("MLA rope block dropped from the score",
     "attend_rows(qd, K, V, n, rec, d_latent,", "attend_rows(qd, K, V, n, d_latent, d_latent,"),
    ("combine: plain average of splits", "double w = exp(l - mx);", "double w = 1.0;"),
    ("combine: LSE missing the denominator", "lse[r] = mx + log(denom);", "lse[r] = mx;"),
    ("running max never updated", "if (s[j] > m) m = s[j];", "if (s[j] > m) m = s[0];"),
    ("causal window off by one", "causal ? n - (int64_t)(q_len - 1 - i) : n;",
     "causal ? n - (int64_t)(q_len - i) : n;"),
    ("causal window aligned top-left", "causal ? n - (int64_t)(q_len - 1 - i) : n;",
     "causal ? (int64_t)(i + 1) : n;"),
    ("causal flag ignored", "causal ? n - (int64_t)(q_len - 1 - i) : n;",
     "n - (int64_t)(q_len - 1 - i);"),
    # sites below occur in both the GQA and the MLA routine: both are mutated
    ("lse stored query-major", "int64_t lse_row = ((int64_t)b * Hq + h) * q_len + i;",
     "int64_t lse_row = ((int64_t)b * q_len + i) * Hq + h;"),
    ("query index from the wrong axis", "int i = (int)((r / Hq) % q_len);",
     "int i = (int)(r % q_len);"),
    ("append slot off by one", "int64_t dst0 = ((int64_t)page * P + p % P) * row;",
     "int64_t dst0 = ((int64_t)page * P + (p + 1) % P) * row;"),
    ("append source token ignored", "int64_t src0 = ((int64_t)b * s_new + t) * row;",
     "int64_t src0 = ((int64_t)b * s_new) * row;"),
    ("append quantizes x * scale", "float q = x / scale;", "float q = x * scale;"),
    ("append rounds ties toward zero",
     "d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)", "d < best_d"),
    ("append page from the next table entry",
     "block_tables[(int64_t)b * max_pages + p / P];",
     "block_tables[(int64_t)b * max_pages + (p + P) / P];"),
]


def _run_mutant(args):
    desc, old, new, tmp = args
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site missing: %r" % old
    path = os.path.join(tmp, "m%d.c" % abs(hash(desc)))
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = path[:-2] + ".so"
    sys.path.insert(0, ROOT)
    from oracle import build as ob
    ob.build(src=path, lib=lib)
    env = dict(os.environ, PDA_ORACLE_MUTANT=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_FILES], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    return desc, r.returncode


def test_pins_catch_planted_mistakes():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(_run_mutant, [(d, o, n, tmp) for d, o, n in MUTATIONS]))
    survived = [d for d, rc in results if rc == 0]
    assert not survived, "pins did not catch: %s" % survived
