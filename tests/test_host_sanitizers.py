"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (no GPU).

The CPU oracle (oracle/oracle.c, with OpenMP) and the C ABI's argument checks
(top_search_resident_amd/csrc/validate.cpp, the same source the library links)
are compiled by the host compilers with -fsanitize=address,undefined and
-fno-sanitize-recover=all, together with a driver that exercises them
(tests/sanitize/), and run: any out-of-bounds access, leak, overflow or other
undefined behaviour aborts with a nonzero status."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def _run(cmd, env=None):
    res = subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, " ".join(cmd) + "\n" + res.stdout + res.stderr
    return res.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no host C compiler")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", *FLAGS, "-fopenmp", "-o", exe, os.path.join(HERE, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "oracle.c"), "-lm"])
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    assert _run([exe], env=env).strip() == "ok"


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_abi_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "validate_driver")
    _run(["g++", "-std=c++17", *FLAGS, "-I" + os.path.join(ROOT, "include"), "-o", exe,
          os.path.join(HERE, "validate_driver.cpp"),
          os.path.join(ROOT, "top_search_resident_amd", "csrc", "validate.cpp")])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    assert _run([exe], env=env).strip() == "ok"
