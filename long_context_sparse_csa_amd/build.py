"""Build the CSA HIP library (libcsa.so) in-tree for gfx950 with hipcc.

Usage: ``python -m long_context_sparse_csa_amd.build`` (or ``build()`` from Python).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcsa.so")
SOURCES = ["indexer.hip", "topk.hip", "attention.hip", "compressor.hip", "noalloc.hip", "api.cpp"]
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
    # keep the compiler from emitting packed-fp32 VALU ops (see the design notes)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the accumulation-register form made the compiler copy
    # the 128 attention accumulators between register files on every tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-result",
]
# sources whose matrix-core accumulators may live in the accumulation registers (none at present)
NO_VGPR_FORM: set = set()


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel: one hipcc per file), then link the library.
    Each translation unit carries its own gfx950 code object; no device symbol crosses files."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    jobs = []
    for src in SOURCES:
        obj = os.path.join(objdir, src + ".o")
        flags = compile_flags
        if src in NO_VGPR_FORM:
            flags = [f for k, f in enumerate(compile_flags)
                     if not (f == "-mllvm" and compile_flags[k + 1] == "-amdgpu-mfma-vgpr-form")
                     and f != "-amdgpu-mfma-vgpr-form"]
        jobs.append((obj, [hipcc(), *flags, "-I", os.path.join(ROOT, "include"), "-c",
                           os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(min(len(jobs), max(1, os.cpu_count() or 1))) as ex:
        list(ex.map(lambda j: _run(j[1], verbose), jobs))
    tmp = LIB + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
