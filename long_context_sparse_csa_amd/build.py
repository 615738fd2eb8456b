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
SOURCES = ["indexer.hip", "topk.hip", "attention.hip", "compressor.hip", "noalloc.hip", "plan.cpp", "api.cpp"]
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


DEBUG_LIB = os.path.join(HERE, "libcsa_debug.so")


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every source to an object (in parallel: one hipcc per file), then link the library.
    Each translation unit carries its own gfx950 code object; no device symbol crosses files.
    debug=True builds libcsa_debug.so with CSA_DEBUG_CHECKS (the kernels count the values they mask
    as invalid; csa_debug_violations reads the count)."""
    from concurrent.futures import ThreadPoolExecutor

    objdir = os.path.join(HERE, "_build_debug" if debug else "_build")
    os.makedirs(objdir, exist_ok=True)
    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"] + (["-DCSA_DEBUG_CHECKS"] if debug else [])
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
    out = DEBUG_LIB if debug else LIB
    tmp = out + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *[o for o, _ in jobs], "-o", tmp], verbose)
    os.replace(tmp, out)
    return out


HOST_ASAN_LIB = os.path.join(HERE, "libcsa_host_asan.so")
HOST_SOURCES = ["api.cpp", "plan.cpp", "launch_stubs.cpp"]


def build_host_sanitized(verbose: bool = False) -> str:
    """The C ABI layer built by the host compiler with address and undefined-behaviour sanitizers,
    kernel launchers replaced by stubs that fail (launch_stubs.cpp): the CPU ABI tests run against
    it.  Not a GPU build; loading it in place of libcsa.so launches nothing."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = f"{HOST_ASAN_LIB}.tmp{os.getpid():x}"   # concurrent builders (test workers) each rename their own
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-D__HIP_PLATFORM_AMD__",
           "-Wno-attributes", "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           *[os.path.join(CSRC, f) for f in HOST_SOURCES], "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed ({r.returncode}):\n{r.stdout}{r.stderr}")
    os.replace(tmp, HOST_ASAN_LIB)
    return HOST_ASAN_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build(verbose="-v" in sys.argv, debug=True))
    print(build_host_sanitized(verbose="-v" in sys.argv))
