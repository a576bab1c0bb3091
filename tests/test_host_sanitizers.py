"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Two check programs under tests/host/ are built with gcc/g++ and
-fsanitize=address,undefined (no GPU code involved) and run in a child
process:

* sched_check: the schedule builders of the library's host side
  (csrc/tra_sched.cpp: Jaccard pairing, merged block lists, chunk orders,
  CSR transpose) on seeded random and banded block masks, against set
  computations and a replay of the pairing rule;
* oracle_check: every entry point of the C oracle on small inputs, against
  element-by-element agreement of its mask functions and closed forms of
  its attention, gradient, linear-branch and SALAD results.

Any out-of-bounds access, use after free, leak or undefined operation ends
the check program with an error, as does a failed check.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
CSRC = os.path.join(ROOT, "static_sparse_spatiotemporal_amd", "csrc")
ORACLE = os.path.join(ROOT, "oracle")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-Wall", "-Werror"]


def _build_and_run(tmp_path, compiler, args, name):
    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not found")
    exe = str(tmp_path / name)
    r = subprocess.run([compiler, *SAN, *args, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "checks passed" in r.stdout


def test_schedule_builders_under_sanitizers(tmp_path):
    _build_and_run(tmp_path, "g++", ["-std=c++17", "-I", CSRC, os.path.join(HOST, "sched_check.cpp"),
                                     os.path.join(CSRC, "tra_sched.cpp")], "sched_check")


def test_oracle_under_sanitizers(tmp_path):
    _build_and_run(tmp_path, "gcc", ["-std=c11", "-I", ORACLE, os.path.join(HOST, "oracle_check.c"),
                                     os.path.join(ORACLE, "oracle.c"), "-lm", "-lpthread"], "oracle_check")
