"""Compile the HIP sources into the in-tree shared library ``libpa.so`` (gfx950 only).

Usage: python -m pagedattention_block_table_amd.build [--jobs N] [--verbose]

Every ``csrc/*.hip`` file is one translation unit, compiled in parallel with hipcc,
then linked into ``pagedattention_block_table_amd/libpa.so``. Packed-FP32 instruction
selection is disabled for all device code.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libpa.so")
ARCH = "gfx950"

# Packed-FP32 selection off; MFMA accumulators in ordinary VGPRs: the kernels rescale them
# with vector ops, and AGPR accumulators would cost copies both ways at every rescale (and
# one more occupancy step for the 8-head decode engine)
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                "-mllvm", "-amdgpu-mfma-vgpr-form"]
FILE_FLAGS = {}  # per translation unit extras


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def _compile(src: str, verbose: bool, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src).replace(".hip", ".o"))
    cmd = [hipcc(), "-c", "-fPIC", "-O3", "-std=c++17", f"--offload-arch={ARCH}", *DEVICE_FLAGS,
           *FILE_FLAGS.get(os.path.basename(src), []),
           *[f"-D{d}" for d in defines],
           "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC, "-o", obj, src]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(jobs: int = 0, verbose: bool = False, out: str = LIB, defines=()) -> str:
    """Compile and link; `defines` (NAME=VALUE) select compile-time tuning knobs and
    `out` names the library file (the package loads LIB unless told otherwise)."""
    build_dir = BUILD if out == LIB else os.path.join(BUILD, "v_" + os.path.basename(out).replace(".so", ""))
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources found")
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    t0 = time.time()
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, defines), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources in {time.time() - t0:.1f}s", flush=True)
    return out


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=0)
    ap.add_argument("--verbose", action="store_true")
    ap.add_argument("--out", default=LIB)
    ap.add_argument("-D", dest="defines", action="append", default=[])
    a = ap.parse_args()
    print(build(a.jobs, a.verbose, os.path.abspath(a.out), a.defines))


if __name__ == "__main__":
    main()
