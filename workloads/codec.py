"""Encoders that turn real-valued synthetic data into the byte formats the CSA path consumes.

This module is input-generation plumbing.  It encodes; it never decodes and it holds none of the
attention, indexer or selection arithmetic.  The CPU oracle has its own decoders and the GPU
library uses the hardware conversions; both are checked against each other only through the bytes
produced here.

Formats (all little-endian):

* FP8 E4M3FN (OCP "fn" flavour, max finite 448, no infinities, 0x7F/0xFF are NaN).  The pages
  name ``float8_e4m3`` as the FP8 type of the kernels and clamp quantised values to +-448
  (page "DeepSeek-V4 全面解读", sections 3.2 and 3.4).  Rounding is round-to-nearest-even with
  saturation to +-448; the pages do not state the rounding mode, so the plainest reading is used.
* E8M0: one byte, value ``2**(e - 127)``; the power-of-two scale of "fast_round_scale"
  (same page, section 3.3): ``2**ceil(log2(max(amax, 1e-4) / 448))``.
* BF16: the upper 16 bits of an fp32, round-to-nearest-even.
* FP4 E2M1 (magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6), two per byte, element 2i in the low nibble
  ("float4_e2m1fn_x2"); block 32 with a power-of-two E8M0 scale ``2**ceil(log2(max(amax,
  6*2**-126) / 6))`` (page "DeepSeek-V4 全面解读", section 3.5, fp4_quant_kernel).  Rounding is
  round-to-nearest-even on the E2M1 grid with saturation to +-6; the pages do not state it.
"""
from __future__ import annotations

import numpy as np

FP8_MAX = 448.0
AMAX_FLOOR = 1e-4          # act_quant clamps the block amax to at least 1e-4 before dividing


def fp8_e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """Round float32 values to FP8 E4M3FN codes (RNE, saturating to +-448, NaN -> 0x7F)."""
    x = np.asarray(x, dtype=np.float32)
    nan = np.isnan(x)
    xc = np.clip(np.where(nan, np.float32(0), x), -FP8_MAX, FP8_MAX).astype(np.float32)
    sign = np.signbit(xc).astype(np.uint8) << np.uint8(7)
    a = np.abs(xc)
    bits = a.view(np.uint32)
    # normal range of e4m3 (|a| >= 2^-6): round the fp32 mantissa to 3 bits, keeping exponent carry
    lsb = (bits >> np.uint32(20)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFFF) + lsb) >> np.uint32(20)           # (exp8 << 3) | m3
    normal_code = rounded.astype(np.int64) - (120 << 3)                    # rebias 127 -> 7
    # subnormal range: multiples of 2^-9, exact scaling then round-half-even
    sub_code = np.rint(a.astype(np.float64) * 512.0).astype(np.int64)
    code = np.where(a >= np.float32(2.0 ** -6), normal_code, sub_code)
    out = (code.astype(np.uint8) & np.uint8(0x7F)) | sign
    out[nan] = np.uint8(0x7F)
    return out


def bf16_encode(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even; NaN kept quiet."""
    x = np.asarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    r = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((bits[nan] >> np.uint64(16)) | np.uint64(0x40)).astype(np.uint16)
    return r


def e8m0_exponent_for(amax: np.ndarray) -> np.ndarray:
    """Biased E8M0 code of the power-of-two scale ``2**ceil(log2(max(amax,1e-4)/448))``.

    Done on the fp32 bit pattern of ``amax * (1/448)`` the way the pages' fast_log2_ceil does it:
    exponent field minus 127, plus one when any mantissa bit is set.
    """
    a = np.maximum(np.asarray(amax, dtype=np.float32), np.float32(AMAX_FLOOR))
    v = (a * np.float32(1.0 / FP8_MAX)).astype(np.float32)
    bits = v.view(np.uint32)
    e = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int64) - 127
    e = e + ((bits & np.uint32(0x7FFFFF)) != 0)
    return (e + 127).astype(np.uint8)


def quantize_fp8_e8m0_blocks(x: np.ndarray, block: int = 32):
    """Quantise the last axis of ``x`` in blocks of ``block`` with E8M0 scales.

    Returns (codes uint8 same shape as x, scale codes uint8 [..., n_blocks]).
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    assert n % block == 0
    xb = x.reshape(*x.shape[:-1], n // block, block)
    e = e8m0_exponent_for(np.abs(xb).max(axis=-1))
    inv = np.ldexp(np.float32(1.0), 127 - e.astype(np.int32)).astype(np.float32)   # exact 1/scale
    codes = fp8_e4m3fn_encode(xb * inv[..., None])
    return codes.reshape(x.shape), e


FP4_MAX = 6.0
FP4_AMAX_FLOOR = 6.0 * 2.0 ** -126
_FP4_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)   # codes 0..7


def fp4_e2m1_encode(x: np.ndarray) -> np.ndarray:
    """Round values to FP4 E2M1 nibble codes (0..15): nearest grid magnitude, ties to the even code,
    saturating at 6."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), FP4_MAX)
    d = np.abs(a[..., None] - _FP4_GRID)                      # distance to every magnitude
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                          # one or two nearest codes
    even = cand & (np.arange(8) % 2 == 0)
    code = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1)).astype(np.uint8)
    sign = (np.signbit(x) & (code != 0)).astype(np.uint8) << np.uint8(3)
    return code | sign


def e8m0_exponent_fp4(amax: np.ndarray) -> np.ndarray:
    """Biased E8M0 code of ``2**ceil(log2(max(amax, 6*2**-126) / 6))`` (exact, on the fp32 bits)."""
    a = np.maximum(np.asarray(amax, dtype=np.float32), np.float32(FP4_AMAX_FLOOR))
    v = (a.astype(np.float64) / FP4_MAX).astype(np.float32)
    bits = v.view(np.uint32)
    e = ((bits >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int64) - 127
    e = e + ((bits & np.uint32(0x7FFFFF)) != 0)
    return (e + 127).astype(np.uint8)


def quantize_fp4_e8m0_blocks(x: np.ndarray, block: int = 32):
    """Quantise the last axis of ``x`` to FP4 E2M1 in blocks of ``block`` with E8M0 scales.

    Returns (packed codes uint8 [..., n/2], element 2i in the low nibble; scale codes uint8
    [..., n_blocks]).
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    assert n % block == 0 and n % 2 == 0
    xb = x.reshape(*x.shape[:-1], n // block, block)
    e = e8m0_exponent_fp4(np.abs(xb).max(axis=-1))
    inv = np.ldexp(1.0, 127 - e.astype(np.int64))           # exact 1/scale
    codes = fp4_e2m1_encode(xb.astype(np.float64) * inv[..., None]).reshape(*x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, e


def quantize_fp8_f32_blocks(x: np.ndarray, block: int = 64):
    """Quantise the last axis in blocks with an fp32 scale ``max(amax,1e-4) * (1/448)``.

    Returns (codes uint8, scales float32 [..., n_blocks]).
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-1]
    assert n % block == 0
    xb = x.reshape(*x.shape[:-1], n // block, block)
    amax = np.maximum(np.abs(xb).max(axis=-1), np.float32(AMAX_FLOOR)).astype(np.float32)
    s = (amax * np.float32(1.0 / FP8_MAX)).astype(np.float32)
    codes = fp8_e4m3fn_encode(xb / s[..., None])
    return codes.reshape(x.shape), s


# ----------------------------------------------------------------------------------------------
# KV row formats.  A compressed or raw KV row has 512 dims: 448 "nope" dims followed by 64 "rope"
# dims (the rope part is the last 64 dims of the head, page "DeepSeek-V4 全面解读" section 2.11
# step 8; SGLang packs nope as FP8 with a per-block scale and rope as BF16, page "DeepSeek-V4 in
# SGLang 深度理解分析", concept 5).
# ----------------------------------------------------------------------------------------------
HEAD_DIM = 512
NOPE_DIM = 448
ROPE_DIM = 64
KV_BLOCK = 64

KV_F32, KV_BF16, KV_FP8 = 0, 1, 2
ROW_BYTES = {KV_F32: 2048, KV_BF16: 1024, KV_FP8: 608}
# FP8 row: [0,448) e4m3fn nope | [448,576) 64 x bf16 rope | [576,604) 7 x fp32 scale | [604,608) 0
FP8_ROPE_OFF = 448
FP8_SCALE_OFF = 576


def pack_kv_rows(x: np.ndarray, fmt: int) -> np.ndarray:
    """Pack float32 rows [..., 512] into the byte rows of ``fmt``; returns uint8 [..., ROW_BYTES]."""
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] == HEAD_DIM
    lead = x.shape[:-1]
    if fmt == KV_F32:
        return np.ascontiguousarray(x).view(np.uint8).reshape(*lead, 2048)
    if fmt == KV_BF16:
        return bf16_encode(x).view(np.uint8).reshape(*lead, 1024)
    assert fmt == KV_FP8
    out = np.zeros((*lead, 608), dtype=np.uint8)
    codes, scales = quantize_fp8_f32_blocks(x[..., :NOPE_DIM], KV_BLOCK)
    out[..., :NOPE_DIM] = codes
    out[..., FP8_ROPE_OFF:FP8_SCALE_OFF] = bf16_encode(x[..., NOPE_DIM:]).view(np.uint8).reshape(*lead, 128)
    out[..., FP8_SCALE_OFF:FP8_SCALE_OFF + 28] = np.ascontiguousarray(scales).view(np.uint8).reshape(*lead, 28)
    return out
