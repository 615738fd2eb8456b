"""The CSA_DEBUG_CHECKS build (libcsa_debug.so): the kernels count the device-resident values they
mask as invalid.  Run in a child process that loads that build: explicit index lists with only
valid and -1 slots count nothing; out-of-range window and compressed indices and a slot on an
unmapped page are counted; a decode whose page table leaves a visible page unmapped is counted by
the indexer and the selection."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "long_context_sparse_csa_amd", "libcsa_debug.so")

_CHILD = r"""
import json, sys
import numpy as np, torch
import long_context_sparse_csa_amd as csa
from workloads import configs, run, torch_io
print("[gpu] child: debug-checks build", flush=True)
res = {}
wl = configs.make_decode("dbg", [3000, 5000], H=16, HI=16, seed=3)
d = torch_io.to_device(wl, "cuda")
n_win, n_comp = 128, 64
idx = np.empty((wl.Q, n_win + n_comp), np.int32)
idx[:, :n_win] = np.arange(n_win)
idx[:, n_win:] = np.arange(n_comp)
idx[0, 5] = -1
idx[1, n_win + 3] = -1
t = lambda x: torch.from_numpy(x).to("cuda")
csa.csa_debug_violations()
run.sparse_attn(wl, d, t(idx), n_win, n_comp); torch.cuda.synchronize()
res["valid"] = csa.csa_debug_violations()
bad = idx.copy()
bad[0, 7] = wl.win_rows.shape[1] + 3                   # window index past the ring
bad[1, n_win + 9] = wl.max_pages * 64 + 100            # compressed index past the table
run.sparse_attn(wl, d, t(bad), n_win, n_comp); torch.cuda.synchronize()
res["out_of_range"] = csa.csa_debug_violations()
pt = wl.page_table.copy()
pt[1, 2] = -1                                          # a visible page of request 1 unmapped
import dataclasses
wl2 = dataclasses.replace(wl, page_table=pt)
d2 = torch_io.to_device(wl2, "cuda")
run.decode(wl2, d2); torch.cuda.synchronize()
res["unmapped_decode"] = csa.csa_debug_violations()
print(json.dumps(res), flush=True)
"""


def test_debug_build_counts_masked_values():
    if not os.path.exists(DEBUG_LIB):
        pytest.skip("libcsa_debug.so is not built")
    env = dict(os.environ, CSA_LIB=DEBUG_LIB, PYTHONPATH=ROOT)
    print("[gpu] debug-checks child process", flush=True)
    r = subprocess.run([sys.executable, "-c", _CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=240)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    res = json.loads(r.stdout.strip().splitlines()[-1])
    print(f"[gpu] {res}", flush=True)
    assert res["valid"] == 0
    assert res["out_of_range"] > 0
    assert res["unmapped_decode"] > 0
