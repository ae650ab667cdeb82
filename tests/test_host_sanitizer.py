"""The host library (hl_host.cpp) under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

tests/host_abi_sanitize.cpp drives every host path of the C ABI (plan
validation and variant choice for every element type, mode and a range of
vocabulary sizes; workspace layout; the per-call checks; the enqueue sequence
on a stand-in workspace, with the kernel launchers replaced by stubs). It is
built with g++ (host code only, no device code) with -fsanitize=address,
undefined and run; any sanitizer report or failed check fails the test.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_library_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "host_abi_sanitize"
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]
    cmd = ["g++", "-std=c++17", "-O1", "-g", *san, "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "lm_head_vocab_amd", "csrc"),
           "-I", os.path.join(ROCM, "include"),
           os.path.join(ROOT, "tests", "host_abi_sanitize.cpp"),
           os.path.join(ROOT, "lm_head_vocab_amd", "csrc", "hl_host.cpp"),
           "-L", os.path.join(ROCM, "lib"), "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64",
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", HIP_VISIBLE_DEVICES="")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "host ABI checks passed" in out
