"""The host planner and the oracle built with AddressSanitizer and UBSan
(host compilers only) run a host program over small grids and error paths; any
sanitizer report or wrong result fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                    reason="needs the host compilers")
def test_planner_and_oracle_under_sanitizers(tmp_path):
    oc = str(tmp_path / "oracle.o")
    exe = str(tmp_path / "sanitize_host")
    subprocess.check_call(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN, "-c",
                           os.path.join(ROOT, "oracle", "oracle.c"), "-o", oc])
    subprocess.check_call(["g++", "-std=c++17", *SAN,
                           "-I", os.path.join(ROOT, "include"),
                           "-I", os.path.join(ROOT, "zero_sharded_mixed_grads_amd", "csrc"),
                           os.path.join(ROOT, "tests", "sanitize_host.cpp"),
                           os.path.join(ROOT, "zero_sharded_mixed_grads_amd", "csrc",
                                        "zero_host.cpp"),
                           oc, "-fopenmp", "-lm", "-o", exe])
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "sanitized host checks passed" in r.stdout
