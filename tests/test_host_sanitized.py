"""Host planning and cache index helpers under AddressSanitizer and
UndefinedBehaviorSanitizer (no GPU).

tests/cpu/host_check.cpp is compiled with plan.cpp by the host compiler, with
the kernel launchers replaced by recorders, and run: it checks that decode
splits cover every visible key exactly once, that the K / V element offsets
are bijections onto a segment, that page ids clamp into range, and that
every decode / prefill launch plan the C ABI makes keeps its grid, merge
class and workspace indices within bounds (see the file's header).
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_host_check_under_sanitizers(tmp_path):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "host_check")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I" + os.path.join(ROCM, "include"), "-D__HIP_PLATFORM_AMD__",
           os.path.join(ROOT, "decode_attention_gemma_amd", "csrc", "plan.cpp"),
           os.path.join(ROOT, "tests", "cpu", "host_check.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert r.returncode == 0 and "host_check OK" in r.stdout, r.stdout[-4000:] + r.stderr[-4000:]
