"""The oracle's pin suites run against a build of the oracle instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer (gcc, CPU only): no
out-of-bounds access, use after free or undefined arithmetic anywhere the pins
reach.  A control build with a planted one-past-the-end read must be caught,
which shows the sanitizers are active in the child process."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pda_oracle.c")
PINS = ["tests/test_oracle_pins.py", "tests/test_oracle_mla.py",
        "tests/test_oracle_multitoken.py", "tests/test_oracle_append.py",
        "tests/test_oracle_layout.py"]


def _runtime(name):
    path = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                          text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


ASAN, UBSAN = _runtime("libasan.so"), _runtime("libubsan.so")
pytestmark = pytest.mark.skipif(not (ASAN and UBSAN), reason="gcc sanitizer runtimes missing")


def _build(src, lib):
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-fopenmp",
                    "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-fno-sanitize-recover=undefined", "-o", lib, src, "-lm"], check=True)


def _run_pins(lib, files):
    env = dict(os.environ, PDA_ORACLE_MUTANT=lib, LD_PRELOAD=ASAN + ":" + UBSAN,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-s", "-p",
                           "no:cacheprovider", *files], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=900)


def test_pin_suites_clean_under_asan_and_ubsan(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    _build(SRC, lib)
    r = _run_pins(lib, PINS)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]


def test_planted_overflow_is_caught(tmp_path):
    src = open(SRC).read()
    old = "for (int64_t j = 0; j < n; ++j) {\n    double acc = 0.0;"
    assert src.count(old) == 1
    bad = tmp_path / "bad.c"
    bad.write_text(src.replace(old, "for (int64_t j = 0; j <= n; ++j) {\n    double acc = 0.0;"))
    lib = str(tmp_path / "liboracle_bad.so")
    _build(str(bad), lib)
    r = _run_pins(lib, ["tests/test_oracle_pins.py"])
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stdout + r.stderr
