"""The benchmark's command-line contract on a machine without a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "8"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_the_contract_flags():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for flag in ("--gpus", "--steps", "--warmup"):
        assert flag in r.stdout


def test_headline_kernel_code_is_found_in_the_library():
    """The counter traffic is keyed to the headline kernel's machine code,
    read back from the built library's gfx950 code object."""
    sys.path.insert(0, ROOT)
    import bench
    h = bench.kernel_code_hash()
    assert h is not None and len(h) == 16
    assert bench.kernel_code_hash("copy_kernel") not in (None, h)
