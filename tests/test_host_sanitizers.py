"""The host code built with AddressSanitizer and UndefinedBehaviorSanitizer (CPU only, gcc/g++):
the trie builder, minimum-call planner, plan descriptor validator and tree-attention tables
(tests/host/plan_check.cpp, which also corrupts valid plans field by field and expects the
validator's error codes), and the float64 oracle's recurrent forward and reverse pass
(tests/host/oracle_check.c).  Any sanitizer report fails the test."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")


def _run(cmd, tmp):
    exe = os.path.join(tmp, "a.out")
    r = subprocess.run(cmd + ["-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    p = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=600)
    out = p.stdout + p.stderr
    assert p.returncode == 0 and "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
    return out


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_planner_and_validator_under_sanitizers(tmp_path):
    host = os.path.join(ROOT, "chunkwise_linear_attention_gated_amd", "csrc", "host")
    out = _run(["g++", "-std=c++17"] + SAN + [os.path.join(ROOT, "tests", "host", "plan_check.cpp"),
                                               os.path.join(host, "plan.cpp"), os.path.join(host, "attn_tables.cpp")],
               str(tmp_path))
    assert "0 failures" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_recurrence_under_sanitizers(tmp_path):
    out = _run(["gcc", "-std=c99", "-fopenmp"] + SAN + [os.path.join(ROOT, "tests", "host", "oracle_check.c"), "-lm"],
               str(tmp_path))
    assert "finite" in out and "NON-FINITE" not in out
