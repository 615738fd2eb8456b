"""GPU parity of the compressor kernels against the oracle (csa_compress_kv, csa_compress_index_keys).

The cache formats are quantised, so the rows are compared after decoding: every element must lie
within half a quantisation step (at the scale the kernel chose) of the oracle's exact value plus the
fp32 rounding of the pooling chain, and every chosen scale must be the one the scale rule gives for
the oracle's block maximum, up to that rounding."""
import numpy as np
import pytest

from oracle import csa_oracle as O
from workloads import configs

pytestmark = pytest.mark.gpu

CHAIN = 2e-5          # relative fp32 error of pooling, RMSNorm and rotation (generous)


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.fixture(scope="module")
def dev():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return "cuda"


def _fp8_half_step(x_over_s):
    """Half the e4m3fn spacing around |x| (in units of the scale): 2^-4 relative for normals,
    2^-10 absolute below the smallest normal 2^-6."""
    a = np.abs(x_over_s)
    return np.maximum(a * 2.0 ** -4, 2.0 ** -10)


def _fp4_half_step(x_over_s):
    a = np.abs(x_over_s) * 1.001
    return np.where(a < 2.0, 0.25, np.where(a < 4.0, 0.5, 1.0))


def _check_kv_rows(ref, pool, page_row, c_begin, fmt, where):
    for i in range(ref.shape[0]):
        c = c_begin + i
        raw = pool[page_row[c // 64], c % 64]
        got = O.kv_row_values(raw, fmt)
        r = ref[i]
        if fmt == configs.KV_F32:
            bound = CHAIN * (np.abs(r) + np.sqrt(np.mean(r * r)))
        elif fmt == configs.KV_BF16:
            bound = 2.0 ** -8 * np.abs(r) + CHAIN * np.sqrt(np.mean(r * r))
        else:
            s = raw[576:604].copy().view(np.float32).astype(np.float64)
            amax = np.abs(r[:448]).reshape(7, 64).max(axis=1)
            expect = np.maximum(amax, 1e-4) / 448.0
            assert np.all(np.abs(s - expect) <= 1e-4 * expect), f"{where} entry {c}: scales {s} vs {expect}"
            sb = np.repeat(s, 64)
            bound = np.empty(512)
            bound[:448] = 1.01 * _fp8_half_step(r[:448] / sb) * sb + CHAIN * np.abs(r[:448]) + 1e-6 * sb
            bound[448:] = 2.0 ** -8 * np.abs(r[448:]) + CHAIN * np.sqrt(np.mean(r * r))
            assert np.all(raw[604:608] == 0)
        err = np.abs(got - r)
        assert np.all(err <= bound), f"{where} entry {c}: max err {err.max():.3e}, worst ratio {(err / bound).max():.3f}"


@pytest.mark.parametrize("ratio", [4, 128])
@pytest.mark.parametrize("fmt", [configs.KV_FP8, configs.KV_BF16, configs.KV_F32])
@pytest.mark.parametrize("proj_dt", [configs.DT_BF16, configs.DT_F32])
def test_compress_kv(dev, ratio, fmt, proj_dt):
    from workloads import run
    T = 260 * 4 if ratio == 4 else 9 * 128 + 17            # a ragged tail of tokens with no entry yet
    ci = configs.make_compressor("ckv", T, ratio, D=512, proj_dt=proj_dt, seed=ratio + fmt)
    n = ci.n_entries
    _say(f"compress_kv ratio={ratio} fmt={fmt} proj_dt={proj_dt} entries={n}")
    page_row, pool = run.compress(ci, "kv", fmt, 0, n, dev, seed=1)
    ref = O.compressor_reference(ci, 0, n)
    _check_kv_rows(ref, pool, page_row, 0, fmt, f"ratio {ratio}")


def test_compress_kv_decode_step_window(dev):
    """A decode step: only entry 70's own tokens and the previous window's are passed (tok0 > 0),
    and an unmapped page (-1) is skipped."""
    from workloads import run
    ci = configs.make_compressor("ckv_step", 4 * 200, 4, D=512, seed=7)
    c = 70
    page_row = np.array([5, 2, -1, 0], np.int32)
    _say("compress_kv one entry from 8 projection rows")
    _, pool = run.compress(ci, "kv", configs.KV_FP8, c, 1, dev, tok0=4 * (c - 1), n_tok=8, num_pages=6,
                           page_row=page_row)
    _check_kv_rows(O.compressor_reference(ci, c, 1), pool, page_row, c, configs.KV_FP8, "step")
    _, pool = run.compress(ci, "kv", configs.KV_FP8, 128, 64, dev, tok0=4 * 127, n_tok=4 * 65, num_pages=6,
                           page_row=page_row)
    assert not pool.any(), "entries on an unmapped page must not be written"


@pytest.mark.parametrize("key_dt", [configs.DT_FP8, configs.DT_FP4])
@pytest.mark.parametrize("ratio", [4, 128])
def test_compress_index_keys(dev, key_dt, ratio):
    from workloads import run
    T = 300 * 4 if ratio == 4 else 10 * 128
    ci = configs.make_compressor("ckeys", T, ratio, D=128, seed=3 + key_dt)
    n = ci.n_entries
    _say(f"compress_index_keys ratio={ratio} key_dt={key_dt} entries={n}")
    page_row, (keys, scales) = run.compress(ci, "keys", key_dt, 0, n, dev, seed=2)
    ref = O.compressor_reference(ci, 0, n, rotate=True)
    fmax, floor = (448.0, 1e-4) if key_dt == configs.DT_FP8 else (6.0, 6.0 * 2.0 ** -126)
    for c in range(n):
        p, sl = int(page_row[c // 64]), c % 64
        got = O.indexer_key_values(keys, scales, key_dt, p, np.array([sl]))[0]
        s = O.e8m0_decode(scales[p, :, sl]).astype(np.float64)
        r = ref[c]
        amax = np.maximum(np.abs(r).reshape(4, 32).max(axis=1), floor) / fmax
        assert np.all(s >= amax * (1 - 1e-4)) and np.all(s < 2 * amax * (1 + 1e-4)), f"entry {c}: scales {s}"
        sb = np.repeat(s, 32)
        half = _fp8_half_step(r / sb) if key_dt == configs.DT_FP8 else _fp4_half_step(r / sb)
        bound = 1.01 * half * sb + CHAIN * np.abs(r) + 1e-6 * sb
        err = np.abs(got - r)
        assert np.all(err <= bound), f"entry {c}: max err {err.max():.3e}, worst ratio {(err / bound).max():.3f}"
