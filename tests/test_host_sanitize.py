"""The host half of libvcoll (validation, schedules, ledgers, the alpha-beta
model, MoE plans) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer, kernel launchers replaced by recording stubs,
driven through the C ABI by tests/c/host_sanitize.cpp. No GPU involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "collective_communication_algorithms_vcoll_amd", "csrc")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE), reason="no g++ or HIP headers")
def test_host_library_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "host_sanitize")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INCLUDE}", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(ROOT, "tests", "c", "host_sanitize.cpp"), os.path.join(CSRC, "vcoll_api.cpp"),
           os.path.join(CSRC, "schedule.cpp"), os.path.join(CSRC, "model.cpp"), "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0 and res.stdout.startswith("OK"), (res.stdout + res.stderr)[-4000:]
