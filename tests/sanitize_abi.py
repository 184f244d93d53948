"""Host AddressSanitizer / UndefinedBehaviorSanitizer check of the C ABI's
argument validation.

Builds a copy of libiqprep.so whose host code in abi.hip carries ASan and
UBSan (device code is untouched: each -fsanitize= applies to the host pass
only), linked with the regular build's other objects, then runs the CPU
argument-check tests (tests/test_abi_cpu.py, the ones that take only the
library) against it in a child process with the ASan runtime preloaded. No
GPU is used: every call returns from validation before touching a device.

    python tests/sanitize_abi.py      # exit status 0 = clean
"""
import glob
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG_DIR = os.path.join(ROOT, "fp4_quantized_prep_amd")
sys.path.insert(0, PKG_DIR)
import build as B  # noqa: E402

SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

CHILD = r"""
import inspect, sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import fp4_quantized_prep_amd as iqp
iqp.LIB_PATH = {lib!r}
iqp._lib = iqp._load()
import test_abi_cpu as T
n = 0
for name in sorted(dir(T)):
    f = getattr(T, name)
    if name.startswith("test_") and list(inspect.signature(f).parameters) == ["iqp"]:
        f(iqp)
        n += 1
print(f"{{n}} argument-check tests passed under ASan/UBSan")
"""


def asan_runtime() -> str:
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("no host ASan runtime under /opt/rocm/lib/llvm")
    return hits[-1]


def main() -> int:
    objs = sorted(o for o in glob.glob(os.path.join(PKG_DIR, "_build", "*.o")) if not o.endswith("abi.hip.o"))
    if not objs:
        raise FileNotFoundError("build the library first (its objects are linked in)")
    with tempfile.TemporaryDirectory() as tmp:
        abi_o = os.path.join(tmp, "abi.o")
        lib = os.path.join(tmp, "libiqprep.so")
        subprocess.run([B.hipcc()] + B.compile_flags() + SAN + ["-c", os.path.join(PKG_DIR, "csrc", "abi.hip"),
                       "-o", abi_o], check=True, capture_output=True)
        # the host object must carry the instrumentation (ASan report hooks)
        nm = subprocess.run(["nm", "-u", abi_o], check=True, capture_output=True,
                            text=True).stdout
        if "__asan_report" not in nm or "__ubsan_handle" not in nm:
            raise RuntimeError("abi.hip's host object is not instrumented")
        subprocess.run([B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-Xarch_host",
                        "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", lib, abi_o] + objs,
                       check=True, capture_output=True)
        env = dict(os.environ, LD_PRELOAD=asan_runtime(), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
                   UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
        code = CHILD.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
        res = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=600)
        sys.stdout.write(res.stdout)
        sys.stderr.write(res.stderr[-4000:])
        return res.returncode


if __name__ == "__main__":
    sys.exit(main())
