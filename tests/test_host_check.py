"""The C-ABI layer built for the host alone with AddressSanitizer and
UndefinedBehaviorSanitizer (g++, no GPU code): tests/host_check/abi_host.cpp
links csrc/api.cpp against launchers that only record what they were asked
to launch, and checks every entry point's argument validation, the planner's
tile and split choices where they change with M, the workspace layout of
the split products, the LoRA layer and the no-allocation entry point, and
size arithmetic at very large dimensions.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_abi_layer_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_host")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "invariant_reduction_amd", "csrc"), "-I", "/opt/rocm/include",
           os.path.join(ROOT, "invariant_reduction_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "host_check", "abi_host.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "host ABI checks passed" in r.stdout
