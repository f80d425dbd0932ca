"""The C ABI from C and C++, without Python or torch.

CPU: include/vcoll.h and include/vcoll_bench.h compile as strict C99 and as
C++17, and tests/c/abi_smoke.c (a C consumer of the library) compiles and
links against libvcoll.so. GPU: that program runs the 4-device worked
example ([NCC] section 4.1) through the ring all-reduce, reduce-scatter and
all-gather and checks the ring ledger, printing OK.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
PKG = os.path.join(ROOT, "collective_communication_algorithms_vcoll_amd")
LIB = os.path.join(PKG, "libvcoll.so")
ROCM = "/opt/rocm"
SMOKE = os.path.join(ROOT, "tests", "c", "abi_smoke.c")

needs_cc = pytest.mark.skipif(shutil.which("gcc") is None or shutil.which("g++") is None, reason="no gcc / g++")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, f"{' '.join(cmd)}\n{res.stdout}\n{res.stderr}"
    return res.stdout


@needs_cc
@pytest.mark.parametrize("lang", ["c99", "c++17"])
def test_headers_compile_strictly(tmp_path, lang):
    src = tmp_path / ("h.c" if lang == "c99" else "h.cpp")
    src.write_text('#include "vcoll.h"\n#include "vcoll_bench.h"\nint main(void) { return vcoll_abi_version() > 0 ? 0 : 1; }\n')
    cc = "gcc" if lang == "c99" else "g++"
    _run([cc, f"-std={lang}", "-Wall", "-Wextra", "-Werror", "-pedantic", "-fsyntax-only", f"-I{INCLUDE}", str(src)])


def _build_smoke(tmp_path) -> str:
    if not os.path.exists(LIB):
        pytest.skip("libvcoll.so is not built")
    exe = str(tmp_path / "abi_smoke")
    _run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", f"-I{INCLUDE}",
          f"-I{ROCM}/include", SMOKE, "-o", exe, LIB, f"-L{ROCM}/lib", "-lamdhip64",
          f"-Wl,-rpath,{PKG}", f"-Wl,-rpath,{ROCM}/lib"])
    return exe


@needs_cc
def test_c_program_links_against_the_library(tmp_path):
    assert os.path.exists(_build_smoke(tmp_path))


@needs_cc
@pytest.mark.gpu
def test_c_program_runs_the_worked_example(tmp_path):
    exe = _build_smoke(tmp_path)
    assert _run([exe]).strip() == "OK"
