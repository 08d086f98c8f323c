"""Compile the HIP sources under csrc/ into lib/libscaledfp8.so for gfx950, and the
measurement kernels under calib/ into lib/libfp8calib.so.

Each .hip file is compiled to an object in parallel, then linked into its shared
library.  Run as ``python -m scaled_quantize_gemm_amd.build`` or call ``build()``.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
CALIB = os.path.join(HERE, "calib")
CALIB_LIBNAME = "libfp8calib.so"
LIBDIR = os.path.join(HERE, "lib")
LIBNAME = "libscaledfp8.so"
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # packed fp32 VALU ops stay off (they are not needed by these kernels)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the FP8 library)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every csrc/*.hip and calib/*.hip and link lib/libscaledfp8.so and
    lib/libfp8calib.so; returns the FP8 library's path."""
    cc = hipcc()
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    libs = {LIBNAME: [], CALIB_LIBNAME: []}
    jobs_ = []
    for libname, srcdir in ((LIBNAME, CSRC), (CALIB_LIBNAME, CALIB)):
        for src in sorted(f for f in os.listdir(srcdir) if f.endswith(".hip")):
            obj = os.path.join(objdir, src[:-4] + ".o")
            libs[libname].append(obj)
            jobs_.append((obj, [cc, *HIPCC_FLAGS, "-c", os.path.join(srcdir, src), "-o", obj]))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(jobs_)))) as ex:
        for (obj, cmd), out in zip(jobs_, ex.map(lambda j: _run(j[1]), jobs_)):
            if verbose and out.strip():
                print(out)
    for libname, objs in libs.items():
        lib = os.path.join(LIBDIR, libname)
        tmp = lib + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
        os.replace(tmp, lib)
        if verbose:
            print(f"built {lib}")
    return os.path.join(LIBDIR, LIBNAME)


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
