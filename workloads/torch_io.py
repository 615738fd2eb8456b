"""Upload a workload's byte arrays to device memory as PyTorch tensors (plumbing only)."""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np
import torch

import long_context_sparse_csa_amd as csa

from .configs import DT_F32, Workload


def _t(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def to_device(wl: Workload, device="cuda") -> SimpleNamespace:
    d = SimpleNamespace()
    d.q = _t(wl.q, device)
    d.sink = _t(wl.sink, device)
    d.qI = _t(wl.qI, device)
    d.qI_scale = None if wl.qI_scale is None else _t(wl.qI_scale, device)
    d.w = _t(wl.w, device)
    # FP8 / FP4 key pages go to the device in the library's operand order
    d.ik_keys = _t(wl.ik_keys if wl.idx_dt == DT_F32 else csa.pack_index_keys(wl.ik_keys), device)
    d.ik_scales = None if wl.ik_scales is None else _t(wl.ik_scales, device)
    d.kv_pool = _t(wl.kv_pool, device)
    d.win_rows = _t(wl.win_rows, device)
    d.page_table = _t(wl.page_table, device)
    d.q_req = _t(wl.q_req, device)
    d.n_vis = _t(wl.n_vis, device)
    d.ctx_len = None if wl.ctx_len is None else _t(wl.ctx_len, device)
    return d


def empty_out(wl: Workload, device="cuda") -> torch.Tensor:
    dt = torch.float32 if wl.out_dt == DT_F32 else torch.bfloat16
    return torch.empty((wl.Q, wl.H, 512), dtype=dt, device=device)


def out_to_numpy(out: torch.Tensor) -> np.ndarray:
    return out.float().cpu().numpy().astype(np.float64)
