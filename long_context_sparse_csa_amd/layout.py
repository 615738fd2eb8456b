"""Byte order of the index-key pages the library reads and writes (host-side marshalling only).

FP8 and FP4 index-key pages are kept in matrix-core operand order rather than row-major: slot
s = 4n + kg of a page holds its bytes [64h + 16g, +16) in kilobyte kg·halves + h, at lane
n + 16g's 16-byte chunk, where halves = 2 for FP8 (128-byte slots) and 1 for FP4 (64-byte
slots).  These helpers convert row-major ``[P][64][R]`` uint8 pages to and from that order.
"""
from __future__ import annotations

import numpy as np


def _split(R: int) -> int:
    if R not in (64, 128):
        raise ValueError(f"index-key rows are 128 (FP8) or 64 (FP4) bytes, not {R}")
    return R // 64


def pack_index_keys(rows: np.ndarray) -> np.ndarray:
    """Row-major ``[P][64][R]`` key bytes -> operand-order pages (returned with the same shape)."""
    rows = np.asarray(rows)
    P, S, R = rows.shape
    if S != 64 or rows.dtype != np.uint8:
        raise ValueError("expected uint8 pages of 64 slots")
    h = _split(R)
    # axes: page, n (slot // 4), kg (slot % 4), half, g, byte -> page, kg, half, g, n, byte
    t = rows.reshape(P, 16, 4, h, 4, 16).transpose(0, 2, 3, 4, 1, 5)
    return np.ascontiguousarray(t).reshape(P, 64, R)


def unpack_index_keys(pages: np.ndarray) -> np.ndarray:
    """Operand-order pages ``[P][64][R]`` (or ``[P][64·R]``) -> row-major ``[P][64][R]`` bytes."""
    pages = np.asarray(pages)
    P = pages.shape[0]
    R = pages.size // (P * 64)
    h = _split(R)
    t = pages.reshape(P, 4, h, 4, 16, 16).transpose(0, 4, 1, 2, 3, 5)
    return np.ascontiguousarray(t).reshape(P, 64, R)
