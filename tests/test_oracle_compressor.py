"""Pins of the oracle's compressor functions ([P1] section 2.9) against closed forms, a library
routine and hand-built inputs whose pooled result is known (CPU only)."""
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import csa_oracle as O
from workloads import configs


def test_hadamard_matches_library_matrix():
    x = np.random.default_rng(0).standard_normal((5, 128))
    ref = x @ scipy.linalg.hadamard(128).T / math.sqrt(128)
    np.testing.assert_allclose(O.hadamard_rotate(x), ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(O.hadamard_rotate(O.hadamard_rotate(x)), x, atol=1e-13)   # H/sqrt(n) is an involution


def test_gated_pool_closed_forms():
    rng = np.random.default_rng(1)
    kv = rng.standard_normal((8, 16))
    np.testing.assert_allclose(O.gated_pool(kv, np.zeros((8, 16))), kv.mean(axis=0), atol=1e-15)
    s = np.zeros((8, 16))
    s[5] = 800.0                                     # one position dominates every feature
    np.testing.assert_allclose(O.gated_pool(kv, s), kv[5], atol=1e-12)
    s = rng.standard_normal((8, 16))
    w = np.exp(s) / np.exp(s).sum(axis=0)
    np.testing.assert_allclose(O.gated_pool(kv, s), (w * kv).sum(axis=0), rtol=1e-13)


def test_overlap_placement_by_halves():
    """Ratio 4: token t's overlapping half holds t, its normal half 1000 + t.  With flat scores,
    entry i pools the overlapping halves of window i-1 and the normal halves of window i (entry 0:
    its own normal halves only)."""
    T, D = 16, 8
    kv = np.zeros((T, 2 * D))
    kv[:, :D] = np.arange(T)[:, None]
    kv[:, D:] = 1000 + np.arange(T)[:, None]
    sc = np.zeros((T, 2 * D))
    ape = np.zeros((4, 2 * D))
    for i in range(4):
        k, s = O.compressor_window(kv, sc, ape, i, 4, True, D)
        expect = np.mean([1000 + t for t in range(4 * i, 4 * i + 4)] + [t for t in range(4 * i - 4, 4 * i) if i > 0])
        assert k.shape == ((8 if i else 4), D)
        np.testing.assert_allclose(O.gated_pool(k, s), expect, atol=1e-12)


def test_ape_shifts_scores_per_position():
    """The position embedding enters the softmax: a large ape at window position 2 selects token
    4i+2's normal half and (for the borrowed half) token 4(i-1)+2's overlapping half equally."""
    T, D = 12, 4
    kv = np.random.default_rng(2).standard_normal((T, 2 * D))
    ape = np.zeros((4, 2 * D))
    ape[2, :] = 900.0
    k, s = O.compressor_window(kv, np.zeros((T, 2 * D)), ape, 2, 4, True, D)
    np.testing.assert_allclose(O.gated_pool(k, s), 0.5 * (kv[10, D:] + kv[6, :D]), atol=1e-12)


def test_rms_norm_and_rope_closed_forms():
    x = np.full(512, 3.0)
    np.testing.assert_allclose(O.rms_norm(x, np.ones(512), 0.0), np.ones(512), atol=1e-15)
    y = O.rms_norm(np.arange(1.0, 9.0), np.full(8, 2.0), 1e-6)
    np.testing.assert_allclose(y, 2 * np.arange(1.0, 9.0) / math.sqrt(np.mean(np.arange(1.0, 9.0) ** 2) + 1e-6))
    v = np.zeros(64)
    v[1] = 1.0                                       # imaginary part of pair 0
    r = O.rope_pairs(v, np.cos(np.full(32, np.pi / 2)), np.sin(np.full(32, np.pi / 2)))
    np.testing.assert_allclose(r[:2], [-1.0, 0.0], atol=1e-15)   # i * i = -1, within the pair
    assert np.allclose(r[2:], 0)
    z = np.random.default_rng(3).standard_normal(64)
    ang = np.random.default_rng(4).uniform(-3, 3, 32)
    r = O.rope_pairs(z, np.cos(ang), np.sin(ang))
    np.testing.assert_allclose(np.hypot(r[0::2], r[1::2]), np.hypot(z[0::2], z[1::2]), rtol=1e-13)
    np.testing.assert_allclose(O.rope_pairs(z, np.ones(32), np.zeros(32)), z)


@pytest.mark.parametrize("ratio", [4, 128])
def test_compress_entries_flat_scores_is_normalised_mean(ratio):
    """With zero projections of the gate and zero ape the pooled row is the plain window mean; the
    entry is then RMS-normalised and its last 64 dims rotated by the entry's angles."""
    ci = configs.make_compressor("c", 4 * ratio, ratio, D=512, proj_dt=configs.DT_F32, seed=5)
    sc = np.zeros_like(ci.score_tok)
    ape = np.zeros_like(ci.ape)
    kv = ci.kv_tok.astype(np.float64)
    got = O.compress_entries(kv, sc, ape, ci.norm_w, ci.eps, ci.rope_cos[2:4], ci.rope_sin[2:4], 2, 2, ratio)
    for i, c in enumerate([2, 3]):
        if ratio == 4:
            m = np.concatenate([kv[4 * c - 4:4 * c, :512], kv[4 * c:4 * c + 4, 512:]]).mean(axis=0)
        else:
            m = kv[128 * c:128 * c + 128].mean(axis=0)
        y = m / np.sqrt(np.mean(m * m) + ci.eps) * ci.norm_w
        cs, sn = ci.rope_cos[c].astype(np.float64), ci.rope_sin[c].astype(np.float64)
        a, b = y[448::2].copy(), y[449::2].copy()
        y[448::2], y[449::2] = a * cs - b * sn, a * sn + b * cs
        np.testing.assert_allclose(got[i], y, rtol=1e-12, atol=1e-12)


def test_compressor_rope_angles_recipe():
    ci = configs.make_compressor("c", 64, 4, D=128, seed=0)
    ang = np.arctan2(ci.rope_sin[3].astype(np.float64), ci.rope_cos[3].astype(np.float64))
    expect = 12.0 * 160000.0 ** (-np.arange(0, 64, 2) / 64.0)
    np.testing.assert_allclose(ang, np.angle(np.exp(1j * expect)), atol=1e-5)
