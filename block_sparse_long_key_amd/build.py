"""Build the gfx950 MoBA library (``libmoba_amd.so``) in-tree with hipcc.

Every ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in
parallel) and linked into ``block_sparse_long_key_amd/libmoba_amd.so``.
Flags: gfx950 only, -O3, packed-fp32 instructions disabled (hipcc's host
pass warns that it does not know that feature; the warning is harmless), and
MFMA accumulators kept in VGPRs.

The same sources with -DMOBA_DEBUG_BOUNDS give ``libmoba_amd_debug.so``
(objects in ``_build/debug/``): the kernels check every index they take
from data against the region it addresses and record violations, which
``moba_debug_violations`` reports.  Tests load it; the package binding
loads the release library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmoba_amd.so")
DEBUG_LIB = os.path.join(PKG, "libmoba_amd_debug.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs (no AGPR round trips)
    "-Xarch_device", "-mllvm=-amdgpu-mfma-vgpr-form=true",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, debug: bool = True) -> str:
    """Compile and link the release library and (with debug) the
    bounds-checking one; returns the release library's path."""
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    variants = [(BUILD, LIB, [])]
    if debug:
        variants.append((os.path.join(BUILD, "debug"), DEBUG_LIB, ["-DMOBA_DEBUG_BOUNDS"]))
    objs = {}
    procs = []
    for bdir, lib, extra in variants:
        os.makedirs(bdir, exist_ok=True)
        objs[lib] = []
        for src in srcs:
            obj = os.path.join(bdir, os.path.basename(src)[:-4] + ".o")
            objs[lib].append(obj)
            cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT)))
    failed = False
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        lines = [l for l in out.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"hipcc failed on {src}:\n" + "\n".join(lines) + "\n")
        elif verbose and lines:
            print("\n".join(lines))
    if failed:
        raise RuntimeError("HIP compilation failed")
    for _, lib, _ in variants:
        tmp = lib + ".tmp"
        subprocess.check_call([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC",
                               *objs[lib], "-o", tmp])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
