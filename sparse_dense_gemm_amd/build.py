"""Build the HIP library ``libspense.so`` in-tree for gfx950.

Run ``python -m sparse_dense_gemm_amd.build``; ``__graft_entry__.build()``
calls :func:`build`.  The library is written next to this file so it travels
with the source tree.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libspense.so")
SOURCES = [os.path.join(HERE, "csrc", f) for f in ("spense_kernels.hip", "spense_tile.hip", "spense_score.hip",
                                                   "spense_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
# The linear kernels rely on fully unrolled epilogue loops over register-
# blocked accumulator tiles (up to 64 16x16 tiles per wave); above the default
# size limit of a forced unroll the tile array would live in scratch memory.
EXTRA = {f: ["-mllvm", "-pragma-unroll-threshold=200000"] for f in ("spense_kernels.hip", "spense_tile.hip")}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("command failed: " + " ".join(cmd))
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if msg.strip():
        sys.stderr.write(msg + "\n")


def build(verbose: bool = False) -> str:
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs, procs = [], []
    for src in SOURCES:  # the translation units compile in parallel
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    for cmd, pr in procs:
        out, err = pr.communicate()
        if pr.returncode != 0:
            sys.stderr.write(out + err)
            raise RuntimeError("command failed: " + " ".join(cmd))
        noise = "is not a recognized feature for this target"
        msg = "\n".join(l for l in (out + err).splitlines() if noise not in l)
        if msg.strip():
            sys.stderr.write(msg + "\n")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    _run(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
