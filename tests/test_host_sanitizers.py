"""The C-ABI layer's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

gqa_kv_cache_qwen3_amd/csrc/mtd_api.cpp (every argument check and size query) is built with g++ for
the host only, with stand-in launchers that abort if reached, together with
tests/host_sanitize/abi_errors.cpp, which drives every entry point through its refusal paths and
the size queries through their extremes.  Any sanitizer report, wrong status or missing error
detail fails the run.  No GPU and no GPU code are involved."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "gqa_kv_cache_qwen3_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_abi_host_code_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "abi_errors"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", f"-I{ROCM}/include", f"-I{ROOT}/include", f"-I{CSRC}",
           os.path.join(CSRC, "mtd_api.cpp"), os.path.join(ROOT, "tests", "host_sanitize", "abi_errors.cpp"),
           f"-L{ROCM}/lib", "-lamdhip64", f"-Wl,-rpath,{ROCM}/lib", "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert run.returncode == 0, (run.stdout + run.stderr)[-3000:]
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-3000:]
    assert "all passed" in run.stdout
