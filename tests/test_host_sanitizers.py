"""The library's host code built with AddressSanitizer and
UndefinedBehaviorSanitizer (g++, no device code: the kernel launchers are
test doubles that record their argument blocks) and driven through every
entry point, valid and invalid, on the CPU."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_asan")
CSRC = os.path.join(ROOT, "gqa_attention_rope_02_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

needs_toolchain = pytest.mark.skipif(
    shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "lib", "libamdhip64.so")),
    reason="g++ or the HIP runtime library is not available")


@needs_toolchain
def test_host_code_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "driver"
    cmd = ["g++", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", HERE,
           os.path.join(CSRC, "llama_attn.cpp"), os.path.join(HERE, "stub_launchers.cpp"),
           os.path.join(HERE, "driver.cpp"), "-o", str(exe),
           "-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    env.pop("LLAMA_ATTN_DEBUG", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "all host checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
