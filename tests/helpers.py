"""Acceptance checks shared by the GPU parity tests (they compare library output with the oracle)."""
from __future__ import annotations

import numpy as np

from oracle import csa_oracle as O

BF16_TOL = 2e-2     # max-abs on attention output in bf16 mode
F32_TOL = 1e-5      # max-abs on attention output in fp32 mode
TOPK_BAND = 1e-3    # relative near-tie band at the k-th / (k+1)-th oracle score


def check_topk_row(gpu_row: np.ndarray, scores: np.ndarray, n_vis: int, k: int, where: str = ""):
    """GPU top-k row vs the oracle's scores of the same query.

    n_vis <= k: the row must be exactly 0..n_vis-1 then -1.  Otherwise the row is k distinct visible
    indices in ascending order; when the oracle's k-th and (k+1)-th scores differ by at least 1e-3
    relative the set must equal the oracle's, else every element of the symmetric difference must
    lie within that band around the k-th score.
    """
    gpu_row = np.asarray(gpu_row, np.int64)
    if n_vis <= k:
        expect = list(range(n_vis)) + [-1] * (k - n_vis)
        assert gpu_row.tolist() == expect, f"{where}: short-context selection differs"
        return
    assert np.all(gpu_row >= 0) and np.all(gpu_row < n_vis), f"{where}: invalid index"
    assert np.all(np.diff(gpu_row) > 0), f"{where}: not strictly ascending / duplicates"
    ref = O.topk_select(scores, n_vis, k)
    s_k = scores[ref[k - 1]]
    s_k1 = scores[np.lexsort((np.arange(n_vis), -scores[:n_vis]))[k]]
    band = TOPK_BAND * max(abs(s_k), abs(s_k1))
    got, exp = set(gpu_row.tolist()), set(ref.tolist())
    if abs(s_k - s_k1) >= band:
        assert got == exp, f"{where}: top-k set differs ({len(got ^ exp)} elements) outside a near tie"
    else:
        for c in got ^ exp:
            assert abs(scores[c] - s_k) <= band, f"{where}: index {c} outside the tie band"


def check_attention(gpu: np.ndarray, ref: np.ndarray, tol: float, where: str = ""):
    err = float(np.max(np.abs(gpu - ref))) if gpu.size else 0.0
    assert np.all(np.isfinite(gpu)), f"{where}: non-finite output"
    assert err <= tol, f"{where}: max-abs error {err:.3e} > {tol:.1e}"
    return err
