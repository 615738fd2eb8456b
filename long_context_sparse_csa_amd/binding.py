"""ctypes binding of libcsa.so (include/csa.h).  Argument marshalling only: every step of the path
runs in the library's HIP kernels.  Tensors are PyTorch device tensors; their data pointers and the
current HIP stream are handed to the C entry points of the same names."""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
# CSA_LIB names another build of the library to load instead (the host-only sanitizer build the
# CPU ABI tests run against); by default the in-tree gfx950 build
LIB_PATH = os.environ.get("CSA_LIB") or os.path.join(HERE, "libcsa.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "csa.h")

CSA_F32, CSA_BF16, CSA_FP8_E4M3FN, CSA_FP4_E2M1 = 0, 1, 2, 3
CSA_KV_F32, CSA_KV_BF16, CSA_KV_FP8NOPE_BF16ROPE = 0, 1, 2
STATUS = {0: "CSA_OK", -1: "CSA_ERR_NULL", -2: "CSA_ERR_SHAPE", -3: "CSA_ERR_DTYPE", -4: "CSA_ERR_ALIGN",
          -5: "CSA_ERR_WORKSPACE", -6: "CSA_ERR_UNSUPPORTED", -7: "CSA_ERR_HIP", -8: "CSA_ERR_SCRATCH"}
NOALLOC_SCRATCH_BYTES = 32 << 20   # CSA_NOALLOC_SCRATCH_BYTES of include/csa.h


class CsaError(RuntimeError):
    def __init__(self, fn: str, status: int, hip: int = 0):
        self.status = status
        self.hip = hip
        super().__init__(f"{fn} -> {STATUS.get(status, status)}" + (f" (hipError {hip})" if hip else ""))


class PagedKV(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_void_p), ("fmt", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class PagedIdx(ctypes.Structure):
    _fields_ = [("keys", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("dt", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_P, _I32, _I64, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGS = {
    "csa_indexer_logits": (_I32, [_P, _P, _I32, _P, ctypes.POINTER(PagedIdx), _P, _I32, _P, _I32, _I32, _I64, _P, _I64, _P]),
    "csa_topk_workspace_bytes": (_SZ, [_I32, _I64, _I32]),
    "csa_topk": (_I32, [_P, _I64, _P, _I32, _I64, _I32, _P, _I64, _P, _SZ, _P]),
    "csa_sparse_attn_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "csa_sparse_attn": (_I32, [_P, _I32, _I32, _I32, _P, _P, _I32, _I64, ctypes.POINTER(PagedKV), _P, _I32, _P,
                               _I64, _I32, _I32, _F32, _P, _I32, _P, _SZ, _P]),
    "csa_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I64, _I32]),
    "csa_decode": (_I32, [_I32, _I32, _I32, _I32, _P, _I32, _P, _P, _P, _I32, _P, ctypes.POINTER(PagedIdx),
                          ctypes.POINTER(PagedKV), _P, _I32, _P, _I64, _F32, _P, _I32, _P, _P, _SZ, _P]),
    "csa_decode_noalloc": (_I32, [_I32, _I32, _I32, _I32, _P, _I32, _P, _P, _P, _I32, _P, ctypes.POINTER(PagedIdx),
                                  ctypes.POINTER(PagedKV), _P, _I32, _P, _I64, _F32, _P, _I32, _P, _P]),
    "csa_decode_multi_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I64, _I32]),
    "csa_decode_multi": (_I32, [_I32, _I32, _I32, _I32, _I32, _P, _I32, _P, _P, _P, _I32, _P,
                                ctypes.POINTER(PagedIdx), ctypes.POINTER(PagedKV), _P, _I32, _I32, _P, _I64, _F32,
                                _P, _I32, _P, _P, _SZ, _P]),
    "csa_prefill_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I64, _I32]),
    "csa_prefill": (_I32, [_I32, _I32, _I32, _I32, _P, _I32, _P, _P, _P, _I32, _P, ctypes.POINTER(PagedIdx),
                           ctypes.POINTER(PagedKV), _P, _I32, _I64, _I64, _F32, _P, _I32, _P, _P, _SZ, _P]),
    "csa_hca_decode_workspace_bytes": (_SZ, [_I32, _I32, _I64, _I32]),
    "csa_hca_decode": (_I32, [_I32, _I32, _P, _I32, _P, ctypes.POINTER(PagedKV), _P, _I32, _P, _I64, _I32, _F32,
                              _P, _I32, _P, _SZ, _P]),
    "csa_hca_prefill_workspace_bytes": (_SZ, [_I32, _I32, _I64, _I32]),
    "csa_hca_prefill": (_I32, [_I32, _I32, _P, _I32, _P, ctypes.POINTER(PagedKV), _P, _I32, _I64, _I64, _I32,
                               _F32, _P, _I32, _P, _SZ, _P]),
    "csa_compress_kv": (_I32, [_P, _P, _I32, _I64, _I64, _I64, _I32, _P, _P, _F32, _P, _P, _I64, _I32, _P, _I32, _I32,
                               _P, _I32, _P]),
    "csa_compress_index_keys": (_I32, [_P, _P, _I32, _I64, _I64, _I64, _I32, _P, _P, _F32, _P, _P, _I64, _I32, _P, _P,
                                       _I32, _I32, _P, _I32, _P]),
    "csa_status_string": (ctypes.c_char_p, [_I32]),
    "csa_last_hip_error": (_I32, []),
    "csa_debug_violations": (_I32, [ctypes.POINTER(ctypes.c_uint64)]),
    "csa_profile_enable": (_I32, [_I32]),
    "csa_profile_collect": (_I32, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
    "csa_profile_reset": (_I32, []),
}

_lib = None


def lib():
    """Load libcsa.so (fails loudly if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m long_context_sparse_csa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/csa.h declares."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_[a-z0-9_]+)\s*\(", txt)))


def _check(fn: str, status: int):
    if status != 0:
        raise CsaError(fn, status, lib().csa_last_hip_error() if status == -7 else 0)


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def paged_kv(rows, fmt: int, page_table, num_pages: int | None = None) -> PagedKV:
    return PagedKV(_ptr(rows), fmt, int(rows.shape[0] if num_pages is None else num_pages), _ptr(page_table),
                   int(page_table.shape[-1]), 0)


def paged_idx(keys, scales, dt: int, page_table, num_pages: int | None = None) -> PagedIdx:
    return PagedIdx(_ptr(keys), _ptr(scales), dt, int(keys.shape[0] if num_pages is None else num_pages),
                    _ptr(page_table), int(page_table.shape[-1]), 0)


# ------------------------------------------------------------------------------------------------
def csa_indexer_logits(qI, qI_scale, qI_dt, w, keys: PagedIdx, q_req, n_req, n_vis, Q, HI, max_n_vis,
                       logits, ld, stream=None):
    _check("csa_indexer_logits", lib().csa_indexer_logits(
        _ptr(qI), _ptr(qI_scale), qI_dt, _ptr(w), ctypes.byref(keys), _ptr(q_req), n_req, _ptr(n_vis), Q, HI,
        max_n_vis, _ptr(logits), ld, _stream(stream)))


def csa_topk_workspace_bytes(Q, max_n_vis, k) -> int:
    return int(lib().csa_topk_workspace_bytes(Q, max_n_vis, k))


def csa_topk(logits, ld, n_vis, Q, max_n_vis, k, idx, ld_idx, ws, ws_bytes, stream=None):
    _check("csa_topk", lib().csa_topk(_ptr(logits), ld, _ptr(n_vis), Q, max_n_vis, k, _ptr(idx), ld_idx,
                                      _ptr(ws), ws_bytes, _stream(stream)))


def csa_sparse_attn_workspace_bytes(Q, H, n_idx) -> int:
    return int(lib().csa_sparse_attn_workspace_bytes(Q, H, n_idx))


def csa_sparse_attn(q, q_dt, Q, H, sink, win_rows, win_fmt, win_rows_per_req, comp: PagedKV | None, q_req,
                    n_req, idx, ld_idx, n_win, n_comp, softmax_scale, out, out_dt, ws, ws_bytes, stream=None):
    _check("csa_sparse_attn", lib().csa_sparse_attn(
        _ptr(q), q_dt, Q, H, _ptr(sink), _ptr(win_rows), win_fmt, win_rows_per_req,
        ctypes.byref(comp) if comp is not None else None, _ptr(q_req), n_req, _ptr(idx), ld_idx, n_win,
        n_comp, softmax_scale, _ptr(out), out_dt, _ptr(ws), ws_bytes, _stream(stream)))


def csa_decode_workspace_bytes(B, H, HI, max_ctx, k) -> int:
    return int(lib().csa_decode_workspace_bytes(B, H, HI, max_ctx, k))


def csa_decode(B, H, HI, k, q, q_dt, sink, qI, qI_scale, qI_dt, w, keys: PagedIdx, comp: PagedKV, win_ring,
               win_fmt, ctx_len, max_ctx, softmax_scale, out, out_dt, idx_out, ws, ws_bytes, stream=None):
    _check("csa_decode", lib().csa_decode(
        B, H, HI, k, _ptr(q), q_dt, _ptr(sink), _ptr(qI), _ptr(qI_scale), qI_dt, _ptr(w), ctypes.byref(keys),
        ctypes.byref(comp), _ptr(win_ring), win_fmt, _ptr(ctx_len), max_ctx, softmax_scale, _ptr(out), out_dt,
        _ptr(idx_out), _ptr(ws), ws_bytes, _stream(stream)))


def csa_decode_noalloc(B, H, HI, k, q, q_dt, sink, qI, qI_scale, qI_dt, w, keys: PagedIdx, comp: PagedKV, win_ring,
                       win_fmt, ctx_len, max_ctx, softmax_scale, out, out_dt, idx_out, stream=None):
    _check("csa_decode_noalloc", lib().csa_decode_noalloc(
        B, H, HI, k, _ptr(q), q_dt, _ptr(sink), _ptr(qI), _ptr(qI_scale), qI_dt, _ptr(w), ctypes.byref(keys),
        ctypes.byref(comp), _ptr(win_ring), win_fmt, _ptr(ctx_len), max_ctx, softmax_scale, _ptr(out), out_dt,
        _ptr(idx_out), _stream(stream)))


def csa_decode_multi_workspace_bytes(B, S, H, HI, max_ctx, k) -> int:
    return int(lib().csa_decode_multi_workspace_bytes(B, S, H, HI, max_ctx, k))


def csa_decode_multi(B, S, H, HI, k, q, q_dt, sink, qI, qI_scale, qI_dt, w, keys: PagedIdx, comp: PagedKV, win_ring,
                     win_fmt, ring_slots, ctx_len, max_ctx, softmax_scale, out, out_dt, idx_out, ws, ws_bytes,
                     stream=None):
    _check("csa_decode_multi", lib().csa_decode_multi(
        B, S, H, HI, k, _ptr(q), q_dt, _ptr(sink), _ptr(qI), _ptr(qI_scale), qI_dt, _ptr(w), ctypes.byref(keys),
        ctypes.byref(comp), _ptr(win_ring), win_fmt, ring_slots, _ptr(ctx_len), max_ctx, softmax_scale, _ptr(out),
        out_dt, _ptr(idx_out), _ptr(ws), ws_bytes, _stream(stream)))


def csa_prefill_workspace_bytes(Q, H, HI, T, k) -> int:
    return int(lib().csa_prefill_workspace_bytes(Q, H, HI, T, k))


def csa_prefill(Q, H, HI, k, q, q_dt, sink, qI, qI_scale, qI_dt, w, keys: PagedIdx, comp: PagedKV, raw_rows,
                raw_fmt, T, pos0, softmax_scale, out, out_dt, idx_out, ws, ws_bytes, stream=None):
    _check("csa_prefill", lib().csa_prefill(
        Q, H, HI, k, _ptr(q), q_dt, _ptr(sink), _ptr(qI), _ptr(qI_scale), qI_dt, _ptr(w), ctypes.byref(keys),
        ctypes.byref(comp), _ptr(raw_rows), raw_fmt, T, pos0, softmax_scale, _ptr(out), out_dt, _ptr(idx_out),
        _ptr(ws), ws_bytes, _stream(stream)))


def csa_hca_decode_workspace_bytes(B, H, max_ctx, ratio) -> int:
    return int(lib().csa_hca_decode_workspace_bytes(B, H, max_ctx, ratio))


def csa_hca_decode(B, H, q, q_dt, sink, comp: PagedKV, win_ring, win_fmt, ctx_len, max_ctx, ratio, softmax_scale,
                   out, out_dt, ws, ws_bytes, stream=None):
    _check("csa_hca_decode", lib().csa_hca_decode(
        B, H, _ptr(q), q_dt, _ptr(sink), ctypes.byref(comp), _ptr(win_ring), win_fmt, _ptr(ctx_len), max_ctx, ratio,
        softmax_scale, _ptr(out), out_dt, _ptr(ws), ws_bytes, _stream(stream)))


def csa_hca_prefill_workspace_bytes(Q, H, T, ratio) -> int:
    return int(lib().csa_hca_prefill_workspace_bytes(Q, H, T, ratio))


def csa_hca_prefill(Q, H, q, q_dt, sink, comp: PagedKV, raw_rows, raw_fmt, T, pos0, ratio, softmax_scale, out, out_dt,
                    ws, ws_bytes, stream=None):
    _check("csa_hca_prefill", lib().csa_hca_prefill(
        Q, H, _ptr(q), q_dt, _ptr(sink), ctypes.byref(comp), _ptr(raw_rows), raw_fmt, T, pos0, ratio, softmax_scale,
        _ptr(out), out_dt, _ptr(ws), ws_bytes, _stream(stream)))


def csa_compress_kv(kv_proj, score_proj, proj_dt, ld_proj, tok0, n_tok, ratio, ape, norm_w, eps, rope_cos, rope_sin,
                    c_begin, c_count, pool_rows, pool_fmt, num_pages, page_table_row, max_pages, stream=None):
    _check("csa_compress_kv", lib().csa_compress_kv(
        _ptr(kv_proj), _ptr(score_proj), proj_dt, ld_proj, tok0, n_tok, ratio, _ptr(ape), _ptr(norm_w), eps,
        _ptr(rope_cos), _ptr(rope_sin), c_begin, c_count, _ptr(pool_rows), pool_fmt, num_pages, _ptr(page_table_row),
        max_pages, _stream(stream)))


def csa_compress_index_keys(kv_proj, score_proj, proj_dt, ld_proj, tok0, n_tok, ratio, ape, norm_w, eps, rope_cos,
                            rope_sin, c_begin, c_count, keys, scales, key_dt, num_pages, page_table_row, max_pages,
                            stream=None):
    _check("csa_compress_index_keys", lib().csa_compress_index_keys(
        _ptr(kv_proj), _ptr(score_proj), proj_dt, ld_proj, tok0, n_tok, ratio, _ptr(ape), _ptr(norm_w), eps,
        _ptr(rope_cos), _ptr(rope_sin), c_begin, c_count, _ptr(keys), _ptr(scales), key_dt, num_pages,
        _ptr(page_table_row), max_pages, _stream(stream)))


def csa_status_string(status: int) -> str:
    return lib().csa_status_string(status).decode()


def csa_last_hip_error() -> int:
    return int(lib().csa_last_hip_error())


def csa_debug_violations() -> int:
    """Masked-value count of a debug build since the last call (raises on release builds)."""
    n = ctypes.c_uint64(0)
    _check("csa_debug_violations", lib().csa_debug_violations(ctypes.byref(n)))
    return int(n.value)


def csa_profile_enable(on: bool):
    _check("csa_profile_enable", lib().csa_profile_enable(1 if on else 0))


def csa_profile_collect(kernel: str):
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check("csa_profile_collect", lib().csa_profile_collect(kernel.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def csa_profile_reset():
    _check("csa_profile_reset", lib().csa_profile_reset())
