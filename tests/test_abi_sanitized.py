"""The C ABI's argument validation under host ASan and UBSan (CPU only): a
sanitized copy of the library runs the argument-check tests in a child
process (tests/sanitize_abi.py)."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SCRIPT = os.path.join(ROOT, "tests", "sanitize_abi.py")


def test_abi_validation_clean_under_asan_ubsan():
    if not glob.glob(os.path.join(ROOT, "fp4_quantized_prep_amd", "_build", "*.o")):
        pytest.skip("the library's objects are not built here (run the build first)")
    if not glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"):
        pytest.skip("no host ASan runtime in this image")
    res = subprocess.run([sys.executable, SCRIPT], capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stdout + res.stderr[-3000:]
    assert "argument-check tests passed under ASan/UBSan" in res.stdout
