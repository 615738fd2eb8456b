"""CPU oracle for the compressed-sparse-attention (CSA) hot path: indexer -> top-k -> sparse_attn.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or call this module.  The product path (the HIP library and its binding)
never does, and this module imports nothing from it.

Plain, slow and float64 throughout.  It has its own decoders for the stored byte formats and
evaluates the method's definitions directly, with no blocking, fusion or reordering beyond what the
definitions state.  Sources (the pages as titled; sections named on each function):

* [P1] "DeepSeek-V4 全面解读：架构设计与 inference/encoding 源码深度解析" (wangjunjian.com)
* [P2] "DeepSeek-V4 in SGLang 深度理解分析" (kenforever1.github.io)
* [P3] "tilelang量化内核拆解DeepSeek-V4.1-Flash-NVFP4的fp4_gemm与sparse_attn实现" (wzjinhao.cn)

Readings taken where the pages are silent or disagree (each also listed in the design notes):
  * the visibility mask is applied before selection (a query never selects an entry it cannot see);
  * equal scores are ordered by ascending entry index;
  * the running max starts at the finite -1e30 of [P3], which the plain definition below reaches
    without special cases: an empty index set gives an all-zero output;
  * the sink enters the softmax denominator only, unscaled, as in [P1] section 3.7;
  * window and compressed entries are both attended even when they cover the same tokens.
"""
from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 512
NOPE_DIM = 448
DI = 128
PAGE = 64
WINDOW = 128
COMPRESS = 4

KV_F32, KV_BF16, KV_FP8 = 0, 1, 2
DT_F32, DT_BF16, DT_FP8, DT_FP4 = 0, 1, 2, 3


# ------------------------------------------------------------------------------------------------
# Decoders of the stored formats.  [P1] section 3.2 lists the element types (float8_e4m3, E8M0
# scales, bfloat16); [P2] concept 5 describes the nope-FP8 / rope-BF16 KV row.
# ------------------------------------------------------------------------------------------------

def fp8_e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3FN byte: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent 0 is
    subnormal; S.1111.111 is NaN and there are no infinities."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:
        return sign * m * 2.0 ** -9          # m/8 * 2^(1-7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_FP8_TABLE = np.array([fp8_e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def fp8_decode(codes: np.ndarray) -> np.ndarray:
    return _FP8_TABLE[np.asarray(codes, dtype=np.uint8)]


def fp4_e2m1_value(code: int) -> float:
    """Value of one FP4 E2M1 nibble ([P1] section 3.5, fp4_quant_kernel: the FP4 indexer format,
    largest value 6.0): 1 sign, 2 exponent (bias 1), 1 mantissa bit; exponent 0 is subnormal
    (m * 0.5); no infinities or NaN."""
    code = int(code) & 0xF
    sign = -1.0 if code & 0x8 else 1.0
    e = (code >> 1) & 0x3
    m = code & 0x1
    if e == 0:
        return sign * m * 0.5
    return sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)


_FP4_TABLE = np.array([fp4_e2m1_value(c) for c in range(16)], dtype=np.float64)


def fp4_decode_packed(packed: np.ndarray) -> np.ndarray:
    """Two E2M1 values per byte ([P1] section 3.5: float4_e2m1fn_x2), element 2i in the low nibble
    and 2i+1 in the high nibble: [..., n] bytes -> [..., 2n] values."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty((*b.shape[:-1], 2 * b.shape[-1]), dtype=np.float64)
    out[..., 0::2] = _FP4_TABLE[b & np.uint8(0xF)]
    out[..., 1::2] = _FP4_TABLE[b >> np.uint8(4)]
    return out


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale byte e -> 2**(e-127); 0xFF is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    v = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, v)


def bf16_decode(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32_decode(raw: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(raw).view(np.float32).astype(np.float64)


def kv_row_values(row_bytes: np.ndarray, fmt: int) -> np.ndarray:
    """Dequantised 512-dim KV rows from stored byte rows [..., row_bytes].

    FP8 rows: nope[i] = fp8(byte i) * scale[i // 64] for i < 448 (scale = fp32 at byte 576 + 4*(i//64)),
    then 64 bf16 rope dims from byte 448 ([P2] concept 5; rope is the last 64 dims of the head,
    [P1] section 2.11 step 8).
    """
    rb = np.ascontiguousarray(row_bytes, dtype=np.uint8)
    lead = rb.shape[:-1]
    if fmt == KV_F32:
        return f32_decode(rb.reshape(*lead, 2048)).reshape(*lead, 512)
    if fmt == KV_BF16:
        return bf16_decode(rb.reshape(*lead, 1024).view(np.uint16)).reshape(*lead, 512)
    assert fmt == KV_FP8 and rb.shape[-1] == 608
    nope = fp8_decode(rb[..., :448]).reshape(*lead, 7, 64)
    scale = f32_decode(np.ascontiguousarray(rb[..., 576:604])).reshape(*lead, 7)
    out = np.empty((*lead, 512), dtype=np.float64)
    out[..., :448] = (nope * scale[..., None]).reshape(*lead, 448)
    out[..., 448:] = bf16_decode(np.ascontiguousarray(rb[..., 448:576]).view(np.uint16))
    return out


def q_values(q: np.ndarray, dt: int) -> np.ndarray:
    return np.asarray(q, dtype=np.float64) if dt == DT_F32 else bf16_decode(q)


def indexer_q_values(qI: np.ndarray, qI_scale, dt: int) -> np.ndarray:
    """Indexer query [..., HI, 128]: fp8 (or fp4, two per byte) value times the E8M0 scale of its
    32-element block."""
    if dt == DT_F32:
        return np.asarray(qI, dtype=np.float64)
    v = fp4_decode_packed(qI) if dt == DT_FP4 else fp8_decode(qI)
    s = e8m0_decode(qI_scale)                                  # [..., HI, 4]
    return (v.reshape(*v.shape[:-1], 4, 32) * s[..., None]).reshape(v.shape)


def indexer_key_values(ik_keys: np.ndarray, ik_scales, dt: int, page: int, slots=None) -> np.ndarray:
    """Indexer keys of one page [64, 128] (or the given slots); scales are stored [4 blocks][64 slots]."""
    slots = np.arange(PAGE) if slots is None else np.asarray(slots)
    if dt == DT_F32:
        return np.asarray(ik_keys[page][slots], dtype=np.float64)
    raw = ik_keys[page][slots]
    v = fp4_decode_packed(raw) if dt == DT_FP4 else fp8_decode(raw)   # [n,128]
    s = e8m0_decode(ik_scales[page][:, slots]).T              # [n,4]
    return (v.reshape(-1, 4, 32) * s[:, :, None]).reshape(-1, DI)


# ------------------------------------------------------------------------------------------------
# Method.
# ------------------------------------------------------------------------------------------------

def indexer_scores(q_hat: np.ndarray, k_hat: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Indexer score of every key: s[c] = sum_h w[h] * max(0, q_hat[h] . k_hat[c]).

    [P1] section 2.10 (forward steps 5-8: head logits by einsum, ReLU, times the per-head weight,
    summed over heads); [P2] concept 3 and algorithm 2 (the FP8 logits pass of the indexer).
    q_hat [HI, d], k_hat [N, d], w [HI] -> s [N].
    """
    logits = np.asarray(k_hat, np.float64) @ np.asarray(q_hat, np.float64).T     # [N, HI]
    return np.maximum(logits, 0.0) @ np.asarray(w, np.float64)


def topk_select(s: np.ndarray, n_vis: int, k: int) -> np.ndarray:
    """Indices of the k largest visible scores, -1 padded.

    Only entries c < n_vis are candidates (mask before selection).  When n_vis <= k every visible
    entry is taken ([P2] algorithm 2 notes that short contexts need no selection).  Ties are broken
    by ascending index.  [P1] section 2.10 steps 9-10; [P2] concept 3 (top-512).
    """
    n_vis = int(n_vis)
    if n_vis <= k:
        return np.concatenate([np.arange(n_vis), np.full(k - n_vis, -1)]).astype(np.int64)
    vis = np.asarray(s[:n_vis], dtype=np.float64)
    order = np.lexsort((np.arange(n_vis), -vis))
    return order[:k].astype(np.int64)


def window_decode(ctx_len: int, window: int = WINDOW, ring: int = WINDOW) -> np.ndarray:
    """Ring-slot indices of the sliding window at decode ([P1] section 2.8, get_window_topk_idxs:
    a ring buffer at decode, -1 for absent positions).

    With ``ctx_len`` raw tokens (the current one included), slot j of the list holds position
    ``p = ctx_len - window + j``; it is valid when p >= 0 and lives in ring slot ``p % ring`` (a
    ring of ``window`` slots for one query per request; multi-query decode keeps ``ring`` >=
    window + queries - 1 slots so the earliest query's window is still held).
    """
    p = ctx_len - window + np.arange(window)
    return np.where(p >= 0, p % ring, -1).astype(np.int64)


def decode_tokens_seen(ctx_len: int, queries: int, j: int) -> int:
    """Raw tokens at or before query j of a request decoding ``queries`` tokens at once (the last
    ``queries`` of its ``ctx_len`` tokens, as in multi-token prediction / speculative decoding,
    [P1] sections 2.17 and [P2]'s NextN variant): query j sits at position ctx_len - queries + j
    and causally sees the tokens up to it."""
    return max(int(ctx_len) - (int(queries) - 1 - int(j)), 0)


def window_prefill(t: int, window: int = WINDOW) -> np.ndarray:
    """Raw positions [t-window+1, t] of a causal prefill query, -1 before position 0 ([P1] 2.8)."""
    p = t - window + 1 + np.arange(window)
    return np.where(p >= 0, p, -1).astype(np.int64)


def sparse_attention(q: np.ndarray, rows: np.ndarray, valid: np.ndarray, sink: np.ndarray,
                     scale: float) -> np.ndarray:
    """Index-gathered MQA with an attention sink, for one query.

    q [H, D], rows [J, D] (the gathered KV; K and V are the same rows), valid [J] bool, sink [H].
        S[h, j] = scale * q[h] . rows[j]                for valid j
        out[h]  = sum_j e^{S[h,j]} rows[j] / (sum_j e^{S[h,j]} + e^{sink[h]})
    computed with the common factor e^{-m}, m = max(sink[h], max_j S[h, j]).  This is what the
    online-softmax kernel of [P1] section 3.7 accumulates block by block; the sink term is the one
    added to the denominator after the loop, and an empty valid set gives exactly zero ([P3],
    sparse_attn section).  Duplicate rows count once per occurrence (gather semantics).
    """
    q = np.asarray(q, np.float64)
    H, D = q.shape
    sink = np.asarray(sink, np.float64).reshape(H)
    kv = np.asarray(rows, np.float64)[np.asarray(valid, bool)]
    if kv.shape[0] == 0:
        return np.zeros((H, D))
    S = scale * (q @ kv.T)                                       # [H, J]
    m = np.maximum(S.max(axis=1), sink)                          # [H]
    e = np.exp(S - m[:, None])
    denom = e.sum(axis=1) + np.exp(sink - m)
    return (e @ kv) / denom[:, None]


# ------------------------------------------------------------------------------------------------
# Whole-path drivers on a workload (the ABI byte layouts).
# ------------------------------------------------------------------------------------------------

def _entry_rows(page_table_row: np.ndarray, entries: np.ndarray):
    entries = np.asarray(entries, np.int64)
    pages = page_table_row[entries // PAGE].astype(np.int64)
    return pages, entries % PAGE


def query_scores(wl, qi: int) -> np.ndarray:
    """Indexer scores of every visible compressed entry of query ``qi`` of a workload."""
    r = int(wl.q_req[qi])
    n = int(wl.n_vis[qi])
    if n == 0:
        return np.zeros(0)
    qh = indexer_q_values(wl.qI[qi], None if wl.qI_scale is None else wl.qI_scale[qi], wl.idx_dt)
    ent = np.arange(n)
    pages, slots = _entry_rows(wl.page_table[r], ent)
    k_hat = np.empty((n, DI))
    for p in np.unique(pages):
        sel = pages == p
        k_hat[sel] = indexer_key_values(wl.ik_keys, wl.ik_scales, wl.idx_dt, int(p), slots[sel])
    return indexer_scores(qh, k_hat, wl.w[qi])


def query_window(wl, qi: int) -> np.ndarray:
    if wl.kind == "decode":
        S = wl.q_per_req
        seen = decode_tokens_seen(int(wl.ctx_len[wl.q_req[qi]]), S, qi % S)
        return window_decode(seen, wl.window, wl.ring)
    return window_prefill(int(wl.positions[qi]), wl.window)


def gather_rows(wl, qi: int, win_idx: np.ndarray, comp_idx: np.ndarray):
    """Dequantised rows for [window ++ compressed] index lists of query ``qi`` and their validity.

    An index is valid when it is >= 0 and inside its source (window source: the request's
    ``win_rows``; compressed source: entries mapped by the page table).  Invalid slots give a zero
    row and are masked out of the softmax, as the -1 slots are in [P1] section 3.7.
    """
    r = int(wl.q_req[qi])
    idx = np.concatenate([np.asarray(win_idx, np.int64), np.asarray(comp_idx, np.int64)])
    nw = len(win_idx)
    rows = np.zeros((idx.size, HEAD_DIM))
    valid = np.zeros(idx.size, dtype=bool)
    wr = wl.win_rows.shape[1]
    for j, c in enumerate(idx):
        if j < nw:
            if 0 <= c < wr:
                rows[j] = kv_row_values(wl.win_rows[r, c], wl.win_fmt)
                valid[j] = True
        else:
            if 0 <= c < wl.page_table.shape[1] * PAGE:
                p = int(wl.page_table[r, c // PAGE])
                if 0 <= p < wl.kv_pool.shape[0]:
                    rows[j] = kv_row_values(wl.kv_pool[p, c % PAGE], wl.kv_fmt)
                    valid[j] = True
    return rows, valid


def attend(wl, qi: int, win_idx, comp_idx) -> np.ndarray:
    rows, valid = gather_rows(wl, qi, win_idx, comp_idx)
    qv = q_values(wl.q[qi], wl.q_dt)
    return sparse_attention(qv, rows, valid, wl.sink, wl.softmax_scale)


def compressed_visible(n_tokens: int, ratio: int) -> int:
    """Compressed entries a query can see when ``n_tokens`` raw tokens (positions 0..n_tokens-1) are
    at or before it: entry c summarises raw tokens [c*ratio, (c+1)*ratio) and is visible once all of
    them are ([P1] section 2.8, get_compress_topk_idxs: causal by compression ratio at prefill, the
    entries up to the current position at decode; section 2.10 for the C4 case)."""
    return max(int(n_tokens), 0) // int(ratio)


def dense_compressed_indices(n_vis: int) -> np.ndarray:
    """Index list of a layer without an indexer: every visible compressed entry, in order ([P1]
    section 2.8 get_compress_topk_idxs; section 2.11, the attention forward's branch without an
    indexer)."""
    return np.arange(int(n_vis), dtype=np.int64)


def run_query_dense(wl, qi: int) -> np.ndarray:
    """Attention of a layer without an indexer for query ``qi``: [window ++ all visible compressed
    entries] through the same sparse attention."""
    return attend(wl, qi, query_window(wl, qi), dense_compressed_indices(int(wl.n_vis[qi])))


def run_query(wl, qi: int):
    """Whole path for one query: scores -> top-k -> [window ++ top-k] -> sparse attention.

    Returns (out [H, 512] float64, top-k indices [k], scores [n_vis]).
    """
    s = query_scores(wl, qi)
    top = topk_select(s, int(wl.n_vis[qi]), wl.topk)
    out = attend(wl, qi, query_window(wl, qi), top)
    return out, top, s


# ------------------------------------------------------------------------------------------------
# Compressor: the step that writes the compressed cache the path reads ([P1] section 2.9; [P2]
# concept 2).  Token projections (the kv and gate linear maps of the hidden state) are inputs: they
# are plain matrix products outside the step.  Readings (also in the design notes): with overlap
# (ratio 4) each token's 2D-wide projection splits into an overlapping half [0, D), lent to the
# next window, and a normal half [D, 2D); the learned position embedding `ape` [ratio, coff*D] is
# added to the gate scores per position inside the window before the halves are placed; the first
# window has no previous window, so its borrowed positions are absent.
# ------------------------------------------------------------------------------------------------

def compressor_window(kv_tok: np.ndarray, score_tok: np.ndarray, ape: np.ndarray, entry: int, ratio: int,
                      overlap: bool, D: int):
    """Positions of compressed entry ``entry``: (kv [P, D], score [P, D]) for its window of ``ratio``
    tokens ([P1] section 2.9, overlap_transform: the current window's normal half in place, the
    previous window's overlapping half shifted in front).  ``kv_tok`` / ``score_tok`` are indexed
    by raw token position ([T, coff*D])."""
    r = ratio
    cur = np.arange(entry * r, (entry + 1) * r)
    s_cur = np.asarray(score_tok[cur], np.float64) + np.asarray(ape, np.float64)
    if not overlap:
        return np.asarray(kv_tok[cur], np.float64)[:, :D], s_cur[:, :D]
    kv = [np.asarray(kv_tok[cur], np.float64)[:, D:2 * D]]
    sc = [s_cur[:, D:2 * D]]
    if entry > 0:
        prev = cur - r
        kv.insert(0, np.asarray(kv_tok[prev], np.float64)[:, :D])
        sc.insert(0, (np.asarray(score_tok[prev], np.float64) + np.asarray(ape, np.float64))[:, :D])
    return np.concatenate(kv), np.concatenate(sc)


def gated_pool(kv: np.ndarray, score: np.ndarray) -> np.ndarray:
    """Softmax of the gate scores over the window positions, per feature, then the weighted sum of
    the kv rows ([P1] section 2.9 forward step 5)."""
    s = np.asarray(score, np.float64)
    e = np.exp(s - s.max(axis=0, keepdims=True))
    return (e * np.asarray(kv, np.float64)).sum(axis=0) / e.sum(axis=0)


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * weight ([P1] section 2.9 step 6: RMSNorm)."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(weight, np.float64)


def rope_pairs(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotary embedding on consecutive pairs (x[2i], x[2i+1]) read as complex numbers and multiplied
    by cos + i sin ([P1] section 2.6 apply_rotary_emb: the last dimension split into (-1, 2) pairs,
    complex multiplication by freqs_cis)."""
    x = np.asarray(x, np.float64)
    a, b = x[..., 0::2], x[..., 1::2]
    c, s = np.asarray(cos, np.float64), np.asarray(sin, np.float64)
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def hadamard_rotate(x: np.ndarray) -> np.ndarray:
    """Walsh-Hadamard transform of the last dimension scaled by n^-1/2 ([P1] section 2.7
    rotate_activation), by the butterfly definition H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        y = y.reshape(*y.shape[:-1], n // (2 * h), 2, h)
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :], y[..., 1, :] = a + b, a - b
        y = y.reshape(*y.shape[:-3], n)
        h *= 2
    return y / math.sqrt(n)


def compress_entries(kv_tok, score_tok, ape, norm_w, eps, rope_cos, rope_sin, c_begin: int, c_count: int,
                     ratio: int, rope_dims: int = 64, rotate: bool = False) -> np.ndarray:
    """Compressed rows of entries c_begin .. c_begin+c_count-1 before quantisation ([P1] section 2.9
    forward steps 4-7): overlap placement (ratio 4), gated softmax pooling, RMSNorm, RoPE on the
    last ``rope_dims`` dims with the angles of each entry (rope_cos/rope_sin [c_count, rope_dims/2]),
    then for ``rotate`` the Hadamard rotation of the whole row (the indexer's key compressor)."""
    D = int(np.asarray(norm_w).shape[0])
    overlap = ratio == 4
    out = np.empty((c_count, D))
    for i in range(c_count):
        kv, sc = compressor_window(kv_tok, score_tok, ape, c_begin + i, ratio, overlap, D)
        y = rms_norm(gated_pool(kv, sc), norm_w, eps)
        y[D - rope_dims:] = rope_pairs(y[D - rope_dims:], rope_cos[i], rope_sin[i])
        out[i] = hadamard_rotate(y) if rotate else y
    return out


def compressor_reference(ci, c_begin: int, c_count: int, rotate: bool = False) -> np.ndarray:
    """compress_entries on a workload's stored projections (bf16 or fp32 rows)."""
    kv = q_values(ci.kv_tok, ci.proj_dt)
    sc = q_values(ci.score_tok, ci.proj_dt)
    return compress_entries(kv, sc, ci.ape, ci.norm_w, ci.eps, ci.rope_cos[c_begin:c_begin + c_count],
                            ci.rope_sin[c_begin:c_begin + c_count], c_begin, c_count, ci.ratio, rotate=rotate)
