"""Pins of the oracle's format decoders and of the input encoders (CPU only).

The oracle decodes FP8 E4M3FN, E8M0 and BF16 with its own code; here each decoder is checked
exhaustively against PyTorch's independent implementation of the same format and against values
the format definitions fix.  The generator's encoders are checked against PyTorch's conversions.
"""
import math

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from workloads import codec


def test_fp8_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2                      # 0x7F and 0xFF only: no infinities in e4m3fn
    assert np.array_equal(ours[~nan], ref[~nan])


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6),
    (0x38, 1.0), (0xB8, -1.0), (0x3C, 1.5), (0x7E, 448.0), (0xFE, -448.0), (0x77, 240.0),
])
def test_fp8_definition_points(code, value):
    assert O.fp8_e4m3fn_value(code) == value


def test_e8m0_decode():
    v = O.e8m0_decode(np.array([0, 1, 126, 127, 128, 254, 255], dtype=np.uint8))
    assert v[3] == 1.0 and v[2] == 0.5 and v[4] == 2.0
    assert v[0] == 2.0 ** -127 and v[5] == 2.0 ** 127
    assert math.isnan(v[6])


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=4096, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_decode(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def test_fp8_encoder_matches_torch_rounding():
    rng = np.random.default_rng(2)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 30,
        rng.standard_normal(5000).astype(np.float32) * 0.01,       # subnormal range
        np.array([0.0, -0.0, 448.0, -448.0, 2.0 ** -6, 2.0 ** -10, 3 * 2.0 ** -10], np.float32),
    ])
    x = np.clip(x, -448, 448).astype(np.float32)
    ours = codec.fp8_e4m3fn_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)
    # saturation beyond the finite range
    assert codec.fp8_e4m3fn_encode(np.array([1e6, -1e6], np.float32)).tolist() == [0x7E, 0xFE]


def test_bf16_encoder_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(20000) * 10.0 ** rng.uniform(-8, 8, 20000)).astype(np.float32)
    ours = codec.bf16_encode(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize("amax,code", [
    (448.0, 127),            # 448/448 = 1 = 2^0
    (449.0, 128),            # just above -> next power of two
    (224.0, 126),
    (1.0, 127 - 8),          # 1/448 -> ceil(log2) = -8
    (1e-5, 105),             # clamped to 1e-4 first: ceil(log2(1e-4/448)) = -22
])
def test_e8m0_scale_rule(amax, code):
    """The power-of-two scale rule (fast_round_scale) of [P1] section 3.3 with the 1e-4 amax floor
    of section 3.4; expected codes worked out by hand."""
    assert int(codec.e8m0_exponent_for(np.array([amax], np.float32))[0]) == code


def test_fp8_kv_row_hand_built():
    """A hand-built FP8 row: nope code 0x38 (1.0) in block 0 with scale 0.5, 0xC0 (-2.0) in block 6
    with scale 4; rope bf16 0x3F80 (1.0) and 0xC000 (-2.0)."""
    row = np.zeros(608, np.uint8)
    row[0] = 0x38
    row[447] = 0xC0
    rope = np.zeros(64, np.uint16)
    rope[0] = 0x3F80
    rope[63] = 0xC000
    row[448:576] = rope.view(np.uint8)
    sc = np.zeros(7, np.float32)
    sc[0] = 0.5
    sc[6] = 4.0
    row[576:604] = sc.view(np.uint8)
    v = O.kv_row_values(row, O.KV_FP8)
    expect = np.zeros(512)
    expect[0] = 0.5
    expect[447] = -8.0
    expect[448] = 1.0
    expect[511] = -2.0
    assert np.array_equal(v, expect)


def test_pack_rows_round_trip_error_bound():
    """Packed rows decode to within the format's rounding bound of the source values."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16, 512)).astype(np.float32)
    for fmt, tol in [(O.KV_F32, 0.0), (O.KV_BF16, 2.0 ** -8), (O.KV_FP8, None)]:
        v = O.kv_row_values(codec.pack_kv_rows(x, fmt), fmt)
        if fmt == O.KV_FP8:
            amax = np.abs(x[:, :448]).reshape(16, 7, 64).max(-1, keepdims=True)
            bound = np.broadcast_to(amax / 448.0 * 16, (16, 7, 64)).reshape(16, 448)   # half-ulp at 448 is 16
            assert np.all(np.abs(v[:, :448] - x[:, :448]) <= bound * 1.0001)
            assert np.all(np.abs(v[:, 448:] - x[:, 448:]) <= np.abs(x[:, 448:]) * 2.0 ** -8)
            # relative error of nope values above the subnormal range is at most 2^-4
            big = np.abs(x[:, :448]) >= amax.repeat(64, -1).reshape(16, 448) / 448 * 2.0 ** -6 * 1.001
            assert np.all(np.abs(v[:, :448] - x[:, :448])[big] <= np.abs(x[:, :448])[big] * 2.0 ** -4)
        else:
            assert np.all(np.abs(v - x) <= np.abs(x) * tol)


# ----------------------------------------------------------------------------- FP4 E2M1 (MXFP4)

# The eight E2M1 magnitudes of the OCP microscaling FP4 format, codes 0..7; code | 8 is the negation.
_E2M1_MAGNITUDES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_fp4_all_codes_match_format_table():
    for code in range(16):
        ref = _E2M1_MAGNITUDES[code & 7] * (-1.0 if code & 8 else 1.0)
        assert O.fp4_e2m1_value(code) == ref
    assert max(abs(O.fp4_e2m1_value(c)) for c in range(16)) == 6.0    # fp4_max of the quantiser


def test_fp4_packed_nibble_order():
    # byte 0x5A: low nibble 0xA = -1.0 (element 0), high nibble 0x5 = 3.0 (element 1)
    v = O.fp4_decode_packed(np.array([[0x5A, 0x0F, 0x70]], dtype=np.uint8))
    assert v.tolist() == [[-1.0, 3.0, -6.0, 0.0, 0.0, 6.0]]


def test_fp4_encoder_rounds_to_nearest_even_and_saturates():
    grid = np.array(_E2M1_MAGNITUDES + [-m for m in _E2M1_MAGNITUDES[1:]] + [0.0])   # 16 values
    codes = codec.fp4_e2m1_encode(grid)
    packed = (codes[0::2] | (codes[1::2] << np.uint8(4))).astype(np.uint8)
    assert np.array_equal(O.fp4_decode_packed(packed[None, :])[0], grid)
    # ties go to the even code: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0])
    got = [O.fp4_e2m1_value(c) for c in codec.fp4_e2m1_encode(ties)]
    assert got == [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, -4.0]
    # off-tie points go to the nearest value; beyond 6 saturates
    got = [O.fp4_e2m1_value(c) for c in codec.fp4_e2m1_encode(np.array([0.26, 2.6, 4.9, 5.1, 7.0, -100.0]))]
    assert got == [0.5, 3.0, 4.0, 6.0, 6.0, -6.0]


@pytest.mark.parametrize("amax,code", [(6.0, 127), (6.01, 128), (3.0, 126), (12.0, 128), (0.0, 1), (1e-40, 1)])
def test_fp4_scale_rule(amax, code):
    """Power-of-two scale 2^ceil(log2(max(amax, 6*2^-126) / 6)) (fp4_quant_kernel)."""
    assert int(codec.e8m0_exponent_fp4(np.array([amax], np.float32))[0]) == code


def test_fp4_block_quantiser_picks_nearest_grid_value():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((40, 128)) * rng.uniform(0.01, 50, size=(40, 1))).astype(np.float32)
    packed, e = codec.quantize_fp4_e8m0_blocks(x, 32)
    assert packed.shape == (40, 64) and e.shape == (40, 4)
    vals = O.fp4_decode_packed(packed) * np.repeat(O.e8m0_decode(e), 32, axis=1)
    scale = np.repeat(O.e8m0_decode(e), 32, axis=1)
    cand = np.array(_E2M1_MAGNITUDES + [-m for m in _E2M1_MAGNITUDES[1:]])
    nearest_err = np.abs(x[..., None] - cand * scale[..., None]).min(axis=-1)
    assert np.allclose(np.abs(vals - x), nearest_err, rtol=0, atol=1e-6 * np.abs(x).max())
    # the block maximum lands within one grid step of the top value
    assert np.all(np.abs(x).reshape(40, 4, 32).max(axis=-1) <= 6.0 * O.e8m0_decode(e) * (1 + 1e-7))
