"""The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

oracle/ssm_oracle.c and tests/oracle_sanitize_driver.c are compiled together
with gcc's -fsanitize=address,undefined (OpenMP left out, so the channel
loop runs serially) and the driver calls every oracle entry point on small
shapes and edge cases with arrays of exactly the size their layout needs.
A second build from a copy of the oracle with one index moved past the end
of x must be stopped by the sanitizer, so the check is not vacuous.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE_SRC = os.path.join(HERE, "..", "oracle", "ssm_oracle.c")
DRIVER_SRC = os.path.join(HERE, "oracle_sanitize_driver.c")
FLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-std=c11"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _build(tmp_path, oracle_src, name):
    exe = str(tmp_path / name)
    res = subprocess.run(["gcc", *FLAGS, oracle_src, DRIVER_SRC, "-o", exe, "-lm"],
                         capture_output=True, text=True)
    if res.returncode != 0 and "sanitize" in res.stderr:
        pytest.skip(f"gcc cannot build with sanitizers here: {res.stderr[-300:]}")
    assert res.returncode == 0, res.stderr
    return exe


@pytest.fixture(scope="module")
def _gcc():
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")


def test_oracle_clean_under_sanitizers(_gcc, tmp_path):
    exe = _build(tmp_path, ORACLE_SRC, "oracle_san")
    res = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), \
        res.stdout[-2000:] + res.stderr[-4000:]


def test_sanitizers_catch_a_planted_overflow(_gcc, tmp_path):
    with open(ORACLE_SRC) as f:
        src = f.read()
    needle = "const double u = x[i_tok];"
    assert needle in src
    bad = tmp_path / "ssm_oracle_overflow.c"
    bad.write_text(src.replace(needle, "const double u = x[i_tok + 1];", 1))
    exe = _build(tmp_path, str(bad), "oracle_bad")
    res = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=300)
    assert res.returncode != 0
    assert "heap-buffer-overflow" in res.stderr
