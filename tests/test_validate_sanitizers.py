"""The C-ABI argument checks under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/native/validate_cases.cpp includes the library's own checks
(head_attention_mha_amd/csrc/mha_validate.hpp, plain host C++) and runs them
on a table of calls: valid ones, every kind of invalid argument, and sizes
at and past each limit up to INT_MAX. It is compiled here with g++ and both
sanitizers in non-recovering mode, so an out-of-range access or a signed
integer overflow inside the checks fails the test, as does any status that
differs from the one include/mha.h states. Host only: no GPU, no HIP call."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "validate_cases.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_argument_checks_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "validate_cases")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", SRC, "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert " of " in r.stdout and "cases as the contract states" in r.stdout
    ran, total = r.stdout.split(" cases")[0].split(" of ")
    assert ran == total and int(total) >= 70
