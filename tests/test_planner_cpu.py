"""The prefill launch planner (host code, dequant_gemm_q4_amd/csrc/plan.cpp)
checked on the CPU: tests/planner_check.cpp is built against it with hipcc
(host code only) and run over 370 groups of problems, from one decoder
layer at M = 2 .. 8192 to ragged single projections, SwiGLU pairs, a mixed
group of eight and the LM head.  For every plan: each problem's n-tiles are
covered exactly once, every split-K piece is non-empty and the pieces cover
K exactly, Q6_K pieces start on even blocks, SwiGLU problems are never split,
partial sums stay within the workspace bound, the heights are valid, the
plan is deterministic and the cache returns it, and its simulated time is no
worse than running every problem unsplit at 32 rows."""
import os
import subprocess

import pytest

from dequant_gemm_q4_amd import build as dmq_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "dequant_gemm_q4_amd", "csrc")


def test_planner_invariants(tmp_path):
    exe = str(tmp_path / "planner_check")
    cmd = [dmq_build.hipcc(), "-O2", "-std=c++17", "-x", "hip", "--cuda-host-only",
           os.path.join(ROOT, "tests", "planner_check.cpp"), os.path.join(CSRC, "plan.cpp"),
           "-I", CSRC, "-o", exe]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    except FileNotFoundError:
        pytest.skip("hipcc not available")
    assert r.returncode == 0, r.stderr[-2000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(run.stdout[-2000:])
    assert run.returncode == 0 and " 0 failures" in run.stdout, run.stdout[-4000:]
