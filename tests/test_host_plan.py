"""The library's work planning and argument checks (ltree_plan.cpp, plain C++)
built for the host with g++ under the address and undefined-behaviour
sanitizers, driven over extreme and random sizes by tests/c_abi/plan_driver.cpp
(CPU only, no device code)."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tree_attention_amd", "csrc")


def _rocm_include():
    for cand in ("/opt/rocm/include", os.path.join(os.environ.get("ROCM_PATH", ""), "include")):
        if os.path.exists(os.path.join(cand, "hip", "hip_runtime_api.h")):
            return cand
    return None


@pytest.mark.skipif(shutil.which("g++") is None or _rocm_include() is None,
                    reason="needs g++ and the HIP headers")
def test_plan_under_sanitizers(tmp_path):
    exe = tmp_path / "plan_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", _rocm_include(), "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "ltree_plan.cpp"),
           os.path.join(ROOT, "tests", "c_abi", "plan_driver.cpp"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "plans checked:" in run.stdout
    assert "runtime error" not in run.stderr, run.stderr[-4000:]
