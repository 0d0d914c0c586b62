"""Host AddressSanitizer build of the C ABI layer (CPU only): every csrc/*.hip is compiled with the
sanitizer on its host side alone (argument validation, workspace planning, the bit allocation,
the rotation's Jacobi solver, the codebook fit's host loop; device code is built as usual) and
linked into liboscar_asan.so. With --test, the CPU tests of the C ABI run against it:

    python -m bit_rotated_kv_amd.build_asan --test

The tests load the library named by OSCAR_LIB; the sanitizer runtime is preloaded into that
pytest process (leak detection off: the interpreter keeps its allocations at exit). Nothing here
touches a GPU."""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

from . import build as B

ASAN_DIR = os.path.join(B.OBJDIR, "asan")
ASAN_LIB = os.path.join(B.HERE, "liboscar_asan.so")
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
TESTS = ["tests/test_abi.py", "tests/test_allocate.py", "tests/test_rotation_abi.py", "tests/test_ops_checks.py"]


def runtime() -> str:
    """The sanitizer's shared runtime of the ROCm LLVM toolchain."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found under /opt/rocm/llvm")
    return hits[-1]


def _compile(src: str) -> str:
    obj = os.path.join(ASAN_DIR, os.path.basename(src) + ".o")
    cmd = [B.hipcc(), *B.HIPFLAGS, *HOST_ASAN, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(ASAN_DIR, exist_ok=True)
    srcs = sorted(os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = ASAN_LIB + ".tmp"
    cmd = [B.hipcc(), f"--offload-arch={B.ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-shared-libsan", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


def _env() -> dict:
    env = dict(os.environ)
    pre = env.get("LD_PRELOAD")
    env["LD_PRELOAD"] = runtime() + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["OSCAR_LIB"] = ASAN_LIB
    return env


# A host read past a caller's buffer: two 8x8 covariances requested from a buffer holding one.
_OVERFLOW = """
import numpy as np
from bit_rotated_kv_amd import _lib
c = np.eye(8)
r = np.zeros((2, 8, 8), np.float32)
_lib.lib().oscar_rotation_from_covariance(2, 8, c.ctypes.data, r.ctypes.data, None, None)
"""


def self_check() -> bool:
    """The sanitizer is live in this setup: an out-of-bounds host read through the library is
    reported (the process aborts with a heap-buffer-overflow report)."""
    r = subprocess.run([sys.executable, "-c", _OVERFLOW], cwd=B.ROOT, env=_env(), capture_output=True, text=True)
    return r.returncode != 0 and "heap-buffer-overflow" in r.stderr


def run_tests(extra=()) -> int:
    cmd = [sys.executable, "-m", "pytest", "-q", "-m", "not gpu", *TESTS, *extra]
    return subprocess.run(cmd, cwd=B.ROOT, env=_env()).returncode


if __name__ == "__main__":
    print(f"built {build()}")
    if "--test" in sys.argv[1:]:
        if not self_check():
            print("the sanitizer did not report a planted host overflow: the setup is not live")
            sys.exit(1)
        print("sanitizer live: a planted host overflow is reported")
        sys.exit(run_tests())
