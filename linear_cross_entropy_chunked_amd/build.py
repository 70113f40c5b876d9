"""Build the gfx950 HIP libraries in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with packed-fp32 instructions
disabled (``-Xclang -target-feature -Xclang -packed-fp32-ops``).  The path's
sources are linked into ``libflce.so`` (the C ABI of ``include/flce.h``); the
benchmark's measurement probes (``include/flce_probe.h``) into a library of
their own, ``libflce_probe.so``, both next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libflce.so")
SOURCES = ["flce_api.hip", "flce_gemm.hip", "flce_rowops.hip"]
PROBE_LIB = os.path.join(PKG, "libflce_probe.so")
PROBE_SOURCES = ["flce_probe.hip"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags(debug: bool = False) -> list[str]:
    f = ["--offload-arch=gfx950", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    f += ["-O0", "-g"] if debug else ["-O3"]
    return f


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()

    def compile_one(src: str) -> str:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmd = [cc, *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        errs = [l for l in (r.stderr or "").splitlines()
                if "packed-fp32-ops' is not a recognized feature" not in l]
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(errs))
        if verbose and errs:
            print("\n".join(errs), file=sys.stderr)
        return obj

    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(compile_one, srcs)))
    for lib, group in ((LIB, SOURCES), (PROBE_LIB, PROBE_SOURCES)):
        tmp = lib + ".tmp"
        subprocess.run([cc, "--offload-arch=gfx950", "-shared", "-o", tmp,
                        *(objs[s] for s in group)], check=True)
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
