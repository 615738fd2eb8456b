"""Seeded synthetic workloads for the CSA hot path, in the byte layouts the C ABI consumes.

Every array is drawn from ``numpy.random.Generator(PCG64)`` seeded through ``SeedSequence``; large
arrays are drawn in fixed-size chunks, each with its own spawned child seed, so the bytes do not
depend on how many threads fill them.  Nothing here computes scores, selections or attention: the
one piece of linear algebra (the planted direction of the long-context workload) builds an input,
it does not evaluate the method.

Layouts (little-endian, C order), shared with ``include/csa.h``:

* ``q``            [Q][H][512]   bf16 bits (uint16) or float32
* ``sink``         [H]           float32
* ``qI``           [Q][HI][128]  fp8 e4m3fn codes (uint8) or float32;  ``qI_scale`` [Q][HI][4] E8M0
* ``w``            [Q][HI]       float32 (already carries softmax_scale * HI**-0.5)
* ``ik_keys``      [P][64][128]  fp8 codes or float32, row-major (uploads pack fp8 / fp4 pages into the library's operand order);  ``ik_scales`` [P][4][64] E8M0 (block-major)
* ``kv_pool``      [P][64][row_bytes]  KV rows (see workloads.codec)
* ``win_rows``     [B][Wr][row_bytes]  window source (a 128-slot ring at decode, raw rows at prefill)
* ``page_table``   [B][max_pages] int32, -1 for unused entries; entry c of request b lives in page
                   ``page_table[b][c >> 6]``, slot ``c & 63``
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from . import codec

PAGE = 64
DI = 128
WINDOW = 128
TOPK = 512
COMPRESS = 4

DT_F32, DT_BF16, DT_FP8, DT_FP4 = 0, 1, 2, 3
KV_F32, KV_BF16, KV_FP8 = codec.KV_F32, codec.KV_BF16, codec.KV_FP8

_CHUNK = 1 << 20  # values per independently seeded chunk


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _normal_rows(ss: np.random.SeedSequence, n_rows: int, dim: int, transform, out: np.ndarray):
    """Fill ``out[i] = transform(N(0,1) rows)`` chunk by chunk with spawned seeds (thread-parallel)."""
    rows_per_chunk = max(1, _CHUNK // dim)
    n_chunks = (n_rows + rows_per_chunk - 1) // rows_per_chunk
    if n_chunks == 0:
        return out
    kids = ss.spawn(n_chunks)

    def work(i):
        lo = i * rows_per_chunk
        hi = min(n_rows, lo + rows_per_chunk)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        x = g.standard_normal((hi - lo, dim), dtype=np.float32)
        out[lo:hi] = transform(x, lo, hi)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(work, range(n_chunks)))
    return out


@dataclass
class Workload:
    name: str
    kind: str                 # "decode" or "prefill"
    B: int
    Q: int
    H: int
    HI: int
    q_dt: int
    out_dt: int
    idx_dt: int
    kv_fmt: int
    win_fmt: int
    q: np.ndarray
    sink: np.ndarray
    qI: np.ndarray
    qI_scale: np.ndarray | None
    w: np.ndarray
    ik_keys: np.ndarray
    ik_scales: np.ndarray | None
    kv_pool: np.ndarray
    win_rows: np.ndarray
    page_table: np.ndarray
    q_req: np.ndarray
    n_vis: np.ndarray
    ctx_len: np.ndarray | None = None      # decode: raw context length per request (incl. current)
    positions: np.ndarray | None = None    # prefill: raw position of each query
    topk: int = TOPK
    window: int = WINDOW
    softmax_scale: float = 1.0 / math.sqrt(512.0)
    planted: list = field(default_factory=list)   # long-context workload: planted entries per request
    ratio: int = COMPRESS                          # raw tokens per compressed entry
    q_per_req: int = 1                             # decode: queries per request (the last tokens)
    ring: int = WINDOW                             # decode: window ring slots per request
    notes: str = ""

    @property
    def num_pages(self) -> int:
        return int(self.kv_pool.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def win_rows_per_req(self) -> int:
        return int(self.win_rows.shape[1])

    @property
    def max_n_vis(self) -> int:
        return int(self.n_vis.max()) if self.n_vis.size else 0

    @property
    def row_bytes(self) -> int:
        return codec.ROW_BYTES[self.kv_fmt]


def _encode_q(x: np.ndarray, dt: int) -> np.ndarray:
    return x.astype(np.float32) if dt == DT_F32 else codec.bf16_encode(x)


def _page_table(rng: np.random.Generator, n_entries: list[int]):
    pages = [max(1, -(-n // PAGE)) for n in n_entries]
    total = int(sum(pages))
    perm = rng.permutation(total).astype(np.int32)
    maxp = max(pages) if pages else 1
    pt = np.full((len(n_entries), maxp), -1, dtype=np.int32)
    off = 0
    for b, p in enumerate(pages):
        pt[b, :p] = perm[off:off + p]
        off += p
    return pt, total


def _indexer_pool(ss, total_pages: int, idx_dt: int, override=None):
    """Indexer keys [P][64][128] (fp8; fp4: [P][64][64], two values per byte) and E8M0 scales
    [P][4][64] (block-major within a page)."""
    n = total_pages * PAGE
    if idx_dt == DT_F32:
        keys = np.empty((n, DI), dtype=np.float32)
        _normal_rows(ss, n, DI, lambda x, lo, hi: x, keys)
        if override is not None:
            override(keys, None)
        return keys.reshape(total_pages, PAGE, DI), None
    width = DI // 2 if idx_dt == DT_FP4 else DI
    quant = codec.quantize_fp4_e8m0_blocks if idx_dt == DT_FP4 else codec.quantize_fp8_e8m0_blocks
    codes = np.empty((n, width), dtype=np.uint8)
    scales = np.empty((n, DI // 32), dtype=np.uint8)

    def tf(x, lo, hi):
        c, e = quant(x, 32)
        scales[lo:hi] = e
        return c

    _normal_rows(ss, n, DI, tf, codes)
    if override is not None:
        override(codes, scales)
    sc = scales.reshape(total_pages, PAGE, 4).transpose(0, 2, 1).copy()   # [P][4][64]
    return codes.reshape(total_pages, PAGE, width), sc


def _kv_rows(ss, n_rows: int, fmt: int) -> np.ndarray:
    out = np.empty((n_rows, codec.ROW_BYTES[fmt]), dtype=np.uint8)
    _normal_rows(ss, n_rows, 512, lambda x, lo, hi: codec.pack_kv_rows(x, fmt), out)
    return out


def _indexer_queries(g: np.random.Generator, Q: int, HI: int, idx_dt: int):
    x = g.standard_normal((Q, HI, DI), dtype=np.float32)
    if idx_dt == DT_F32:
        return x, x, None
    if idx_dt == DT_FP4:
        codes, e = codec.quantize_fp4_e8m0_blocks(x, 32)
    else:
        codes, e = codec.quantize_fp8_e8m0_blocks(x, 32)
    return x, codes, e


def make_decode(name: str, ctx_len, H: int, HI: int, *, q_dt=DT_BF16, out_dt=DT_BF16,
                idx_dt=DT_FP8, kv_fmt=KV_FP8, win_fmt=None, seed: int = 0,
                planted_frac: float = 0.0, topk: int = TOPK, ratio: int = COMPRESS,
                q_per_req: int = 1, planted_contiguous: bool = False) -> Workload:
    """``q_per_req`` queries per request: the last tokens of a context of ``ctx_len[b]`` raw tokens
    (query b*q_per_req + j sits at position ctx_len[b] - q_per_req + j).  The window ring holds
    128 + q_per_req - 1 slots, so the earliest query's window is still in it.

    Sub-streams, spawned in this order: page permutation, q, sink, indexer q, w, indexer key pool,
    KV pool, window ring, planted entries.  ``planted_contiguous`` puts each request's planted
    entries in one run of consecutive entries at a seeded offset instead of spreading them.
    """
    win_fmt = kv_fmt if win_fmt is None else win_fmt
    ctx_len = np.asarray(ctx_len, dtype=np.int32)
    B = int(ctx_len.shape[0])
    S = int(q_per_req)
    Q = B * S
    ring = WINDOW + S - 1
    n_c = [int(t) // ratio for t in ctx_len]
    # visible entries of each query: every entry whose tokens are all at or before its position
    n_vis = [max(int(ctx_len[q // S]) - (S - 1 - q % S), 0) // ratio for q in range(Q)]
    ss = np.random.SeedSequence(seed).spawn(9)
    g = [np.random.Generator(np.random.PCG64(s)) for s in ss]

    page_table, total_pages = _page_table(g[0], n_c)
    q_f = g[1].standard_normal((Q, H, 512), dtype=np.float32)
    sink = g[2].standard_normal(H, dtype=np.float32)
    qI_f, qI, qI_s = _indexer_queries(g[3], Q, HI, idx_dt)
    w = (g[4].standard_normal((Q, HI), dtype=np.float32) * np.float32(DI ** -0.5 * HI ** -0.5)).astype(np.float32)

    planted = []
    key_override = None
    if planted_frac > 0:
        pg = g[8]
        for b in range(B):
            n_plant = int(round(planted_frac * n_c[b]))
            if planted_contiguous:
                start = int(pg.integers(0, n_c[b] - n_plant + 1))
                planted.append(np.arange(start, start + n_plant, dtype=np.int64))
            else:
                planted.append(np.sort(pg.choice(n_c[b], size=n_plant, replace=False)).astype(np.int64))

        def key_override(codes, scales):
            # planted indexer key = alpha * u_b + 0.25 * N(0, I), where u_b is the unit vector whose
            # dot product with each head's indexer query has the sign of that head's weight.
            for b in range(B):
                qb = b * S + S - 1                                   # the request's last query
                Qb = qI_f[qb].astype(np.float64)                    # [HI,128]
                s = np.sign(w[qb]).astype(np.float64)
                s[s == 0] = 1.0
                u = Qb.T @ np.linalg.solve(Qb @ Qb.T, s)
                u /= np.linalg.norm(u)
                n = planted[b]
                noise = pg.standard_normal((n.size, DI)).astype(np.float32)
                kv = (3.0 * math.sqrt(DI) * u[None, :] + 0.25 * noise).astype(np.float32)
                rows = page_table[b, n // PAGE].astype(np.int64) * PAGE + (n % PAGE)
                if scales is None:
                    codes[rows] = kv
                else:
                    quant = codec.quantize_fp4_e8m0_blocks if idx_dt == DT_FP4 else codec.quantize_fp8_e8m0_blocks
                    c, e = quant(kv, 32)
                    codes[rows] = c
                    scales[rows] = e

    ik_keys, ik_scales = _indexer_pool(ss[5], total_pages, idx_dt, key_override)
    kv_pool = _kv_rows(ss[6], total_pages * PAGE, kv_fmt)
    if planted_frac > 0:
        for b in range(B):
            n = planted[b]
            d = q_f[b * S + S - 1].astype(np.float64).sum(axis=0)
            d /= np.linalg.norm(d)
            # a planted row leans on the queries' summed direction (cosine about 0.89) and keeps the
            # scale of the N(0, 1) rows around it: (2 sqrt(512) d + N(0, I)) / sqrt(5) has the same
            # expected squared norm, 512, as an N(0, I) row
            x = ((2.0 * math.sqrt(512) * d[None, :] + g[8].standard_normal((n.size, 512))) / math.sqrt(5.0)).astype(np.float32)
            rows = page_table[b, n // PAGE].astype(np.int64) * PAGE + (n % PAGE)
            kv_pool[rows] = codec.pack_kv_rows(x, kv_fmt)
    kv_pool = kv_pool.reshape(total_pages, PAGE, -1)
    win = _kv_rows(ss[7], B * ring, win_fmt).reshape(B, ring, -1)

    return Workload(
        name=name, kind="decode", B=B, Q=Q, H=H, HI=HI, q_dt=q_dt, out_dt=out_dt, idx_dt=idx_dt,
        kv_fmt=kv_fmt, win_fmt=win_fmt, q=_encode_q(q_f, q_dt), sink=sink, qI=qI, qI_scale=qI_s,
        w=w, ik_keys=ik_keys, ik_scales=ik_scales, kv_pool=kv_pool, win_rows=win,
        page_table=page_table, q_req=(np.arange(Q) // S).astype(np.int32),
        n_vis=np.asarray(n_vis, dtype=np.int32), ctx_len=ctx_len, topk=topk, planted=planted, ratio=ratio,
        q_per_req=S, ring=ring)


def make_prefill(name: str, T: int, H: int, HI: int, *, q_dt=DT_BF16, out_dt=DT_BF16,
                 idx_dt=DT_FP8, kv_fmt=KV_BF16, seed: int = 0, q_start: int = 0,
                 q_count: int | None = None, topk: int = TOPK, ratio: int = COMPRESS) -> Workload:
    """Causal prefill of one request with ``T`` raw tokens; queries are positions
    ``q_start .. q_start+q_count-1``.  Query t sees compressed entries ``c < (t+1)//4`` and the raw
    window ``[t-127, t]``.

    Sub-streams, spawned in this order: page permutation, q, sink, indexer q, w, indexer key pool,
    compressed KV pool, raw KV rows.
    """
    q_count = T - q_start if q_count is None else q_count
    n_c = T // ratio
    ss = np.random.SeedSequence(seed).spawn(8)
    g = [np.random.Generator(np.random.PCG64(s)) for s in ss]
    page_table, total_pages = _page_table(g[0], [n_c])
    Q = q_count
    q = np.empty((Q, H * 512), dtype=np.float32 if q_dt == DT_F32 else np.uint16)
    _normal_rows(ss[1], Q, H * 512, lambda x, lo, hi: _encode_q(x, q_dt), q)
    q = q.reshape(Q, H, 512)
    sink = g[2].standard_normal(H, dtype=np.float32)
    _, qI, qI_s = _indexer_queries(g[3], Q, HI, idx_dt)
    w = (g[4].standard_normal((Q, HI), dtype=np.float32) * np.float32(DI ** -0.5 * HI ** -0.5)).astype(np.float32)
    ik_keys, ik_scales = _indexer_pool(ss[5], total_pages, idx_dt)
    kv_pool = _kv_rows(ss[6], total_pages * PAGE, kv_fmt).reshape(total_pages, PAGE, -1)
    raw = _kv_rows(ss[7], T, kv_fmt).reshape(1, T, -1)
    pos = np.arange(q_start, q_start + Q, dtype=np.int32)
    return Workload(
        name=name, kind="prefill", B=1, Q=Q, H=H, HI=HI, q_dt=q_dt, out_dt=out_dt, idx_dt=idx_dt,
        kv_fmt=kv_fmt, win_fmt=kv_fmt, q=q, sink=sink, qI=qI, qI_scale=qI_s, w=w,
        ik_keys=ik_keys, ik_scales=ik_scales, kv_pool=kv_pool, win_rows=raw,
        page_table=page_table, q_req=np.zeros(Q, dtype=np.int32),
        n_vis=((pos + 1) // ratio).astype(np.int32), positions=pos, topk=topk, ratio=ratio)


# ------------------------------------------------------------------------------------------------
# The five named workloads.  Sizes default to the full configurations; the parity tests pass
# smaller sizes of the same recipe.
# ------------------------------------------------------------------------------------------------

def tiny_decode(seed: int = 0) -> Workload:
    """B=1, T=4096 (1024 compressed entries, 128-token window), H=16, HI=16, everything fp32."""
    return make_decode("tiny_decode", [4096], H=16, HI=16, q_dt=DT_F32, out_dt=DT_F32,
                       idx_dt=DT_F32, kv_fmt=KV_F32, seed=seed)


def batched_decode(seed: int = 0, B: int = 32, T: int = 65536, H: int = 64, HI: int = 64,
                   idx_dt: int = DT_FP8, q_per_req: int = 1) -> Workload:
    """B=32 requests at T=65536 (16384 compressed entries in 256 pages of 64), FP8-nope/BF16-rope
    KV with per-64 fp32 scales, FP8 (or FP4) indexer with E8M0 per-32 scales, bf16 q, H=HI=64."""
    return make_decode("batched_decode", [T] * B, H=H, HI=HI, seed=seed, idx_dt=idx_dt, q_per_req=q_per_req)


def long_decode(seed: int = 0, B: int = 8, T: int = 1 << 20, H: int = 64, HI: int = 64,
                idx_dt: int = DT_FP8, q_per_req: int = 1) -> Workload:
    """B=8 requests at T=1,048,576 (262,144 compressed entries), formats as batched_decode, with 1%
    planted high-similarity entries per request."""
    return make_decode("long_decode", [T] * B, H=H, HI=HI, seed=seed, planted_frac=0.01, idx_dt=idx_dt,
                       q_per_req=q_per_req)


def causal_prefill(seed: int = 0, T: int = 8192, H: int = 64, HI: int = 64, q_start: int = 0,
                   q_count: int | None = None, idx_dt: int = DT_FP8) -> Workload:
    """One request, T=8192 query positions, bf16 q and KV rows, FP8 (or FP4) indexer."""
    return make_prefill("causal_prefill", T, H=H, HI=HI, seed=seed, q_start=q_start, q_count=q_count,
                        idx_dt=idx_dt)


def dense_decode(seed: int = 0, B: int = 8, T: int = 1 << 20, H: int = 64, ratio: int = 128) -> Workload:
    """A layer without an indexer (heavily compressed, ratio 128): B=8 requests at T=1,048,576, so
    each query attends 128 window rows and all 8,192 compressed rows; FP8-nope/BF16-rope rows, bf16
    q.  The indexer arrays the generator also draws are not used on this path."""
    return make_decode("dense_decode", [T] * B, H=H, HI=16, seed=seed, ratio=ratio)


RAGGED_EMPTY_ROWS = (3, 17, 42, 63)


def ragged_lengths(seed: int = 0, B: int = 64, empty=RAGGED_EMPTY_ROWS, lo: int = 512,
                   hi: int = 131072) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(10)[9]))
    T = np.clip(np.round(np.exp(g.normal(math.log(8192.0), 1.2, size=B))), lo, hi).astype(np.int32)
    for r in empty:
        if r < B:
            T[r] = 0
    return T


def ragged_decode(seed: int = 0, B: int = 64, H: int = 8, HI: int = 64, hi: int = 131072,
                  idx_dt: int = DT_FP8) -> Workload:
    """B=64 lognormal contexts in [512, 131072] (rows 3, 17, 42, 63 empty), H=8 (padded to 16
    inside the kernels), bf16 q and KV rows, FP8 (or FP4) indexer."""
    T = ragged_lengths(seed, B, hi=hi)
    return make_decode("ragged_decode", T, H=H, HI=HI, kv_fmt=KV_BF16, seed=seed, idx_dt=idx_dt)


# ------------------------------------------------------------------------------------------------
# Compressor inputs: token projections of one request and the compressor's parameters.
# ------------------------------------------------------------------------------------------------
COMPRESS_ROPE_THETA = 160000.0   # base frequency of the compressed entries' rotary embedding


@dataclass
class CompressorInputs:
    name: str
    T: int                    # raw tokens with projections (positions 0 .. T-1)
    ratio: int                # 4 (overlapping windows, two halves per token) or 128
    D: int                    # compressed row width: 512 (KV) or 128 (indexer keys)
    proj_dt: int              # DT_BF16 or DT_F32 projections
    kv_tok: np.ndarray        # [T, coff*D] (bf16 bits as uint16, or float32)
    score_tok: np.ndarray     # [T, coff*D]
    ape: np.ndarray           # [ratio, coff*D] float32
    norm_w: np.ndarray        # [D] float32
    eps: float
    rope_cos: np.ndarray      # [T // ratio, 32] float32: angles of entry c at position c * ratio
    rope_sin: np.ndarray

    @property
    def coff(self) -> int:
        return 2 if self.ratio == 4 else 1

    @property
    def n_entries(self) -> int:
        return self.T // self.ratio


def make_compressor(name: str, T: int, ratio: int, D: int = 512, proj_dt: int = DT_BF16,
                    seed: int = 0) -> CompressorInputs:
    """Seeded compressor inputs.  Sub-streams in this order: kv projections, gate projections, ape,
    norm weight.  Projections are N(0,1) (the gate scores also N(0,1), so the window softmax is
    neither flat nor one-hot); ape ~ N(0, 0.5); norm weight ~ 1 + N(0, 0.1).  The rotary angles of
    entry c are (c * ratio) * theta^(-2i/64), i < 32, in float32."""
    coff = 2 if ratio == 4 else 1
    ss = np.random.SeedSequence(seed).spawn(4)
    g = [np.random.Generator(np.random.PCG64(s)) for s in ss]
    kv = g[0].standard_normal((T, coff * D), dtype=np.float32)
    sc = g[1].standard_normal((T, coff * D), dtype=np.float32)
    ape = (g[2].standard_normal((ratio, coff * D), dtype=np.float32) * np.float32(0.5)).astype(np.float32)
    w = (1.0 + 0.1 * g[3].standard_normal(D, dtype=np.float32)).astype(np.float32)
    n_c = T // ratio
    freqs = (1.0 / (np.float32(COMPRESS_ROPE_THETA) ** (np.arange(0, 64, 2, dtype=np.float32) / np.float32(64))))
    ang = np.outer(np.arange(n_c, dtype=np.float32) * np.float32(ratio), freqs.astype(np.float32)).astype(np.float32)
    enc = codec.bf16_encode if proj_dt == DT_BF16 else (lambda x: x.astype(np.float32))
    return CompressorInputs(name=name, T=T, ratio=ratio, D=D, proj_dt=proj_dt, kv_tok=enc(kv), score_tok=enc(sc),
                            ape=ape, norm_w=w, eps=1e-6, rope_cos=np.cos(ang).astype(np.float32),
                            rope_sin=np.sin(ang).astype(np.float32))
