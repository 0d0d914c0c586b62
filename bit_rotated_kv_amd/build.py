"""Build liboscar.so (the gfx950 HIP library behind include/oscar.h) in-tree with hipcc, and
liboscar_timeline.so, the same library with per-workgroup timestamps in the decode kernels (a
diagnostic build: decode.hip compiled with OSCAR_TIMELINE; every other object shared).

    python -m bit_rotated_kv_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "liboscar.so")
TIMELINE_LIB = os.path.join(HERE, "liboscar_timeline.so")
TIMELINE_SOURCES = ("decode.hip",)
ARCH = "gfx950"

# Packed-FP32 instructions are disabled for every HIP object (-packed-fp32-ops).
HIPFLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-ffp-contract=fast-honor-pragmas",
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", INCLUDE]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, timeline: bool = False) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + (".tl.o" if timeline else ".o"))
    cmd = [hipcc(), *HIPFLAGS, *(["-DOSCAR_TIMELINE=1"] if timeline else []), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, lib: str):
    tmp = lib + ".tmp"
    # -z defs: a symbol left undefined (such as a kernel whose host stub the compiler dropped)
    # fails the link instead of the first load
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every csrc/*.hip for gfx950, link liboscar.so and liboscar_timeline.so; returns the
    path of liboscar.so."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    jobs = [(s, False) for s in srcs] + [(s, True) for s in srcs if os.path.basename(s) in TIMELINE_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(lambda j: _compile(*j), jobs))
    plain = objs[:len(srcs)]
    tl = {os.path.basename(s): o for (s, t), o in zip(jobs, objs) if t}
    _link(plain, LIB)
    _link([tl.get(os.path.basename(s), o) for s, o in zip(srcs, plain)], TIMELINE_LIB)
    if verbose:
        print(f"built {LIB} and {TIMELINE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
