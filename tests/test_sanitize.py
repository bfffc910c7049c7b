"""The fp64 oracle and the LeanTile planner under host sanitizers.

Builds ``oracle/attn_oracle.c`` (gcc) and ``tests/harness/sanitize_driver.cpp`` (g++,
which includes the plan harness and through it the kernels' plan header) with
AddressSanitizer and UndefinedBehaviorSanitizer, every report fatal, and runs the
driver over seeded small cases: ragged, empty and one-key contexts, FP8, multi-token,
split-and-merge, causal prefill, and 300 random plans.  No GPU is involved.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="needs gcc and g++")
def test_oracle_and_planner_under_asan_ubsan(tmp_path):
    obj = tmp_path / "attn_oracle.o"
    exe = tmp_path / "sanitize_driver"
    subprocess.run(["gcc", "-std=c99", "-ffp-contract=off", *SAN, "-c", os.path.join(ROOT, "oracle", "attn_oracle.c"),
                    "-o", str(obj)], check=True)
    subprocess.run(["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "tests", "harness"),
                    os.path.join(ROOT, "tests", "harness", "sanitize_driver.cpp"), str(obj), "-lm", "-o", str(exe)],
                   check=True)
    # the environment may preload a library ahead of the ASan runtime: allow that link order
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "clean" in r.stdout
