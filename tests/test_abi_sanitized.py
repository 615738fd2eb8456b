"""The C ABI layer under address and undefined-behaviour sanitizers, and the host fault-injection
flag (CPU only).  Both run against the host-only build of api.cpp + plan.cpp whose kernel launchers
are stubs that fail (launch_stubs.cpp), in child processes so that the sanitizer runtime can be
preloaded: nothing here can reach a GPU."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _asan_runtime():
    if shutil.which("g++") is None:
        return None
    r = subprocess.run(["g++", "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.fixture(scope="module")
def host_lib():
    if _asan_runtime() is None:
        pytest.skip("no g++ / libasan to build the sanitizer host library")
    from long_context_sparse_csa_amd import build
    return build.build_host_sanitized()


def _env(lib, **extra):
    env = dict(os.environ)
    env.update(CSA_LIB=lib, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONPATH=ROOT)
    env.update(extra)
    return env


def test_abi_tests_pass_under_sanitizers(host_lib):
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_abi.py"), "-q", "-x",
                        "-p", "no:cacheprovider"], cwd=ROOT, env=_env(host_lib), capture_output=True, text=True,
                       timeout=600)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail


_PROBE = r"""
import ctypes
import long_context_sparse_csa_amd as csa
L = csa.lib()
FAKE = 1 << 20
st = L.csa_topk(FAKE, 1024, FAKE, 2, 1000, 512, FAKE, 512, FAKE, 1 << 30, None)
print(st, L.csa_last_hip_error())
"""


@pytest.mark.parametrize("inject,expect", [("launch", "-7 719"), ("", "-7 801")])
def test_fault_injection_fails_before_any_launch(host_lib, inject, expect):
    """CSA_FAULT_INJECT=launch: a call that passes validation returns CSA_ERR_HIP with
    hipErrorLaunchFailure (719) before enqueuing anything; without the flag the same call reaches
    the stub launcher of this build (hipErrorNotSupported, 801)."""
    r = subprocess.run([sys.executable, "-c", _PROBE], cwd=ROOT, env=_env(host_lib, CSA_FAULT_INJECT=inject),
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip().splitlines()[-1] == expect
