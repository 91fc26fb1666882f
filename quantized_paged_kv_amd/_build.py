"""Build libtq.so in-tree with hipcc for gfx950.

Usage: python quantized_paged_kv_amd/_build.py [-v] [--trace]   (or __graft_entry__.build());
the script is run by path, since importing the package needs the library.

Every HIP source is compiled with the packed-FP32 target feature off, the
quantise-on-write source additionally with -ffp-contract=off so that no
multiply-add is fused on the bit-exact fp64 path, and the decode source
without the atomic optimizer (its block counter is read one block late).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtq.so")
ARCH = "gfx950"

COMMON = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
          "-Wno-unused-variable", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]

SOURCES = {
    "tq_host.cpp": ["-x", "hip"],
    "write_kv.hip": ["-ffp-contract=off"],
    # one lane takes the next block index with an LDS atomic whose result is
    # read a block later; the atomic optimizer would turn it into a wave-wide
    # reduction that waits for the result immediately
    "decode.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"],
    "window.hip": [],
    "qjl.hip": ["-ffp-contract=off"],
}


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", shutil.which("hipcc") or ""):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


TRACE_LIB = os.path.join(HERE, "libtq_trace.so")


def build(verbose: bool = False, trace: bool = False) -> str:
    """Compile every source and link libtq.so; trace=True builds the
    phase-timestamp variant (TQ_PHASE_TRACE, see tq_debug_phase_trace) as
    libtq_trace.so instead, for performance analysis only."""
    bdir = BUILD + ("_trace" if trace else "")
    lib = TRACE_LIB if trace else LIB
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()
    procs = []
    objs = []
    t0 = time.time()
    for src, extra in SOURCES.items():
        obj = os.path.join(bdir, src + ".o")
        objs.append(obj)
        cmd = [cc, *COMMON, *extra, *(["-DTQ_PHASE_TRACE"] if trace else []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, pr in procs:
        out, _ = pr.communicate()
        text = out.decode(errors="replace")
        text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
        if pr.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        msg = "\n".join(f"--- {s}\n{t}" for s, t in failed)
        raise RuntimeError(f"HIP build failed:\n{msg}")
    tmp = lib + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout.decode(errors="replace"))
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib} in {time.time() - t0:.1f}s", flush=True)
    return lib


if __name__ == "__main__":
    build(verbose="-v" in sys.argv, trace="--trace" in sys.argv)
