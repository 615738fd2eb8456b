"""GPU parity of the HIP path against the CPU oracle, at sizes the oracle finishes in seconds that
still span several tiles, pages and blocks with ragged tails.  Every call goes through the C ABI."""
import dataclasses
import math

import numpy as np
import pytest

from oracle import csa_oracle as O
from tests.helpers import BF16_TOL, F32_TOL, check_attention, check_topk_row
from workloads import configs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sparse_csa_amd as csa
    csa.lib()
    return "cuda"


def _run():
    from workloads import run, torch_io
    return run, torch_io


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


# ------------------------------------------------------------------------------------ indexer
@pytest.mark.parametrize("HI,idx_dt", [(64, configs.DT_FP8), (40, configs.DT_FP8), (16, configs.DT_FP8),
                                        (64, configs.DT_FP4), (40, configs.DT_FP4), (16, configs.DT_FP4),
                                        (16, configs.DT_F32), (64, configs.DT_F32)])
def test_indexer_scores(dev, HI, idx_dt):
    run, tio = _run()
    ctx = [4096, 1000, 257, 0, 6000, 3]
    wl = configs.make_decode("idx", ctx, H=16, HI=HI, idx_dt=idx_dt, seed=11)
    _say(f"indexer HI={HI} dt={idx_dt} ctx={ctx}")
    d = tio.to_device(wl, dev)
    logits = run.indexer(wl, d).cpu().numpy()
    for qi in range(wl.Q):
        nv = int(wl.n_vis[qi])
        ref = O.query_scores(wl, qi)
        got = logits[qi, :nv].astype(np.float64)
        bound = _fp32_score_bound(wl, qi)
        err = np.abs(got - ref)
        assert np.all(err <= bound), f"query {qi}: max err {err.max():.3e}, worst ratio {(err / bound).max():.2f}"
        if nv:
            _say(f"query {qi}: max err {err.max():.2e}, max err/bound {(err / bound).max():.3f}")
        assert np.all(np.isneginf(logits[qi, nv:wl.max_n_vis])), f"query {qi}: tail not -inf"


def test_indexer_fp8_products_exact_under_cancellation(dev):
    """FP8 operands whose products cancel inside one run of eight elements: 448*448 + v and
    448*448 - 448*448 + v for small v, in the same 32-element scale block and across blocks.  A
    matrix core that sums each run of products on a grid tied to the largest of them returns
    448*448 and 0 here; the scores must instead meet the fp32 bound of exact products."""
    run, tio = _run()
    base = configs.make_decode("idx_cancel", [256], H=16, HI=16, seed=1)
    qI = np.zeros_like(base.qI)
    keys = base.ik_keys.copy()
    w = np.zeros_like(base.w)
    w[0, 0] = 1.0
    E448, N448, ONE = 0x7E, 0xFE, 0x38      # e4m3fn codes of 448, -448 and 1
    qI[0, 0, [0, 2]] = E448
    qI[0, 0, [1, 65]] = ONE
    pg = int(base.page_table[0, 0])
    keys[pg] = 0
    for c in range(64):
        code = 0x20 + 2 * (c % 16)          # 0.125 ... 0.84
        keys[pg, c, 0] = E448
        if c < 16:
            keys[pg, c, 1] = code            # 448^2 + v, one run of eight
        elif c < 32:
            keys[pg, c, 65] = code           # 448^2 + v, v in another scale block
        elif c < 48:
            keys[pg, c, [1, 2]] = [code, N448]   # 448^2 - 448^2 + v
        else:
            keys[pg, c, [2, 1, 3]] = [N448, code, code]
    wl = dataclasses.replace(base, qI=qI, qI_scale=np.full_like(base.qI_scale, 127), ik_keys=keys,
                             ik_scales=np.full_like(base.ik_scales, 127), w=w)
    logits = run.indexer(wl, tio.to_device(wl, dev)).cpu().numpy()[0, :64].astype(np.float64)
    ref = O.query_scores(wl, 0)
    assert ref[32] == 0.125 and ref[0] == 448.0 ** 2 + 0.125
    err = np.abs(logits - ref)
    bound = _fp32_score_bound(wl, 0)
    _say(f"cancelling fp8 products: max err {err.max():.3e}")
    assert np.all(err <= bound), f"max err {err.max():.3e} at entry {int(err.argmax())}"
    # every v is a multiple of 2^-6, so each exact sum is an fp32 value: exact products and fp32
    # accumulation reproduce them bit for bit
    assert np.all(logits == ref), f"inexact at entries {np.nonzero(logits != ref)[0][:8].tolist()}"


@pytest.mark.parametrize("key_dt", [configs.DT_FP8, configs.DT_FP4])
def test_indexer_reads_compressor_pages(dev, key_dt):
    """Key pages as csa_compress_index_keys leaves them on the device feed csa_indexer_logits
    unchanged, so the writer and the reader agree on the page order; the oracle scores the same
    pages read back and unpacked to rows."""
    import dataclasses
    import long_context_sparse_csa_amd as csa
    run, tio = _run()
    ci = configs.make_compressor("keys_to_indexer", 300 * 4, 4, D=128, seed=7 + key_dt)
    n = ci.n_entries
    _say(f"compressor pages -> indexer key_dt={key_dt} entries={n}")
    page_row, (keys_d, scales_d) = run.compress(ci, "keys", key_dt, 0, n, dev, seed=4, device_out=True)
    base = configs.make_decode("idx_from_compressor", [4 * n + 3], H=16, HI=64, idx_dt=key_dt, seed=12)
    wl = dataclasses.replace(base, ik_keys=csa.unpack_index_keys(keys_d.cpu().numpy()),
                             ik_scales=scales_d.cpu().numpy(), page_table=page_row[None, :].astype(np.int32))
    assert int(wl.n_vis[0]) == n and wl.page_table.shape == base.page_table.shape
    d = tio.to_device(wl, dev)
    d.ik_keys, d.ik_scales = keys_d, scales_d          # the compressor's own device pages
    logits = run.indexer(wl, d).cpu().numpy()
    ref = O.query_scores(wl, 0)
    err = np.abs(logits[0, :n].astype(np.float64) - ref)
    bound = _fp32_score_bound(wl, 0)
    assert np.all(err <= bound), f"max err {err.max():.3e}, worst ratio {(err / bound).max():.2f}"
    _say(f"max err {err.max():.2e}, max err/bound {(err / bound).max():.3f}")


def _fp32_score_bound(wl, qi):
    """Forward error bound of the score computed in fp32 from exact fp8 products: each head logit sums
    128 products (error <= 128 u sum|q_d k_d|), the weighted head sum adds HI more roundings.  u=2^-24."""
    nv = int(wl.n_vis[qi])
    if nv == 0:
        return np.zeros(0)
    u = 2.0 ** -24
    qh = O.indexer_q_values(wl.qI[qi], None if wl.qI_scale is None else wl.qI_scale[qi], wl.idx_dt)
    r = int(wl.q_req[qi])
    ent = np.arange(nv)
    pages = wl.page_table[r][ent // 64]
    k = np.empty((nv, 128))
    for p in np.unique(pages):
        sel = pages == p
        k[sel] = O.indexer_key_values(wl.ik_keys, wl.ik_scales, wl.idx_dt, int(p), (ent % 64)[sel])
    absdot = np.abs(k) @ np.abs(qh).T                       # [nv, HI]
    logit = k @ qh.T
    w = np.abs(wl.w[qi].astype(np.float64))
    return 2 * (128 * u * (absdot @ w) + (wl.HI + 2) * u * (np.maximum(logit, 0) @ w)) + 1e-30


# ------------------------------------------------------------------------------------ top-k
# Row lengths per selection path: rows longer than 32,768 entries take the multi-launch selection;
# shorter rows take one block per query: 1024 threads of 32 entries for rows of up to 32,768, and
# of 16 entries with 1024, 256 or 128 threads for rows of up to 16,384, 4,096 or 2,048 entries
# (the longest row of the call decides).
_TOPK_LENGTHS = {
    "multi_block": ([0, 1, 511, 512, 513, 777, 5000, 70000], 9000),
    "single_1024x32": ([0, 1, 511, 512, 513, 777, 16385, 32768], 20000),
    "single_1024": ([0, 1, 511, 512, 513, 777, 5000, 16384], 9000),
    "single_256": ([0, 1, 511, 512, 513, 777, 2049, 4096], 4000),
    "single_128": ([0, 1, 511, 512, 513, 777, 1500, 2048], 2000),
}


def _topk_cases(rng, size_class, k=None):
    lengths, m = _TOPK_LENGTHS[size_class]
    cases = [rng.standard_normal(n_vis).astype(np.float32) for n_vis in lengths]
    if k is not None and k < m:
        # a pair tied at the k-th largest score in a spread row (the value-range level resolves the
        # threshold bin; only the lower-index one of the pair is taken), and a pair tied at the k-1-th
        # and k-th (both taken: the selection is exactly the entries at or above the threshold)
        near = rng.standard_normal(m).astype(np.float32)
        order = np.argsort(-near.astype(np.float64), kind="stable")
        at = near.copy()
        at[order[k]] = at[order[k - 1]]
        cases.append(at)
        if k >= 2:
            above = near.copy()
            above[order[k - 1]] = above[order[k - 2]]
            cases.append(above)
    ties = rng.integers(0, 7, size=m).astype(np.float32)                   # heavy ties at the threshold
    cases.append(ties)
    flat = np.full(m * 2 // 3, 1.5, np.float32)                             # every score equal
    cases.append(flat)
    mixed = rng.standard_normal(m // 3).astype(np.float32)
    mixed[::7] = -np.inf
    mixed[5::11] = np.nan
    mixed[3::13] = -0.0
    mixed[4::17] = 0.0
    cases.append(mixed)
    few = np.full(2000, -np.inf, np.float32)                                # fewer finite than k
    few[rng.choice(2000, 100, replace=False)] = rng.standard_normal(100).astype(np.float32)
    cases.append(few)
    return cases


@pytest.mark.parametrize("size_class", list(_TOPK_LENGTHS))
@pytest.mark.parametrize("k", [512, 1, 100, 2048])
def test_topk_exact(dev, k, size_class):
    """Exact selection on ties, NaN, -inf, +-0 and all-equal rows, for every selection path.  In the
    one-block-per-query paths the threshold bin is resolved by one wave when it holds at most 2,048
    entries (the tied rows) and block-wide otherwise (the all-equal rows)."""
    run, _ = _run()
    rng = np.random.default_rng(5 + k)
    cases = _topk_cases(rng, size_class, k)
    n = [len(c) for c in cases]
    max_n = max(n)
    ld = (max_n + 63) // 64 * 64
    L = np.full((len(cases), ld), 7.0, np.float32)      # junk beyond n_vis must be ignored
    for i, c in enumerate(cases):
        L[i, :len(c)] = c
    _say(f"topk k={k} n_vis={n}")
    idx = run.topk(torch.from_numpy(L).to(dev), torch.tensor(n, dtype=torch.int32, device=dev), max_n, k)
    idx = idx.cpu().numpy()
    for i, c in enumerate(cases):
        ref = O.topk_select(c.astype(np.float64), len(c), k)
        if len(c) > k:
            ref = np.sort(ref)
        assert idx[i].tolist() == ref.tolist(), f"case {i} (n_vis={len(c)}) differs"


# ------------------------------------------------------------------------------------ sparse attention
@pytest.mark.parametrize("kv_fmt,q_dt", [(configs.KV_FP8, configs.DT_BF16), (configs.KV_BF16, configs.DT_BF16),
                                          (configs.KV_F32, configs.DT_F32), (configs.KV_FP8, configs.DT_F32)])
@pytest.mark.parametrize("H", [64, 8, 80])
@pytest.mark.parametrize("batch", ["q4", "q24"])
def test_sparse_attn_explicit_indices(dev, kv_fmt, q_dt, H, batch):
    """Explicit index lists with invalid, duplicate and out-of-range slots.  Four queries take the
    16-head blocks; 24 queries with 64 or 80 heads take the 64-head blocks with the key range
    split across blocks and merged by the combine kernel (80 heads: a second, mostly padded, head
    block)."""
    run, tio = _run()
    ctx = [3000, 700, 0, 5000]
    if batch == "q24":
        ctx += [64, 1, 128, 4096, 9000, 256, 2048, 333, 0, 7000, 1500, 640, 12000, 5, 900, 4000, 2500, 60,
                10000, 800]
    out_dt = configs.DT_F32 if q_dt == configs.DT_F32 else configs.DT_BF16
    wl = configs.make_decode("attn", ctx, H=H, HI=16, q_dt=q_dt, out_dt=out_dt, kv_fmt=kv_fmt, seed=21)
    rng = np.random.default_rng(H + kv_fmt)
    n_win, n_comp = 128, 300
    limit = wl.max_pages * 64
    idx = np.empty((wl.Q, n_win + n_comp), np.int32)
    idx[:, :n_win] = rng.integers(-5, 140, size=(wl.Q, n_win))
    idx[:, n_win:] = rng.integers(-3, limit + 10, size=(wl.Q, n_comp))
    idx[0, n_win + 5] = idx[0, n_win + 6]           # duplicate slot
    idx[1, :] = -1                                  # a query with no valid slot
    idx[1, 3] = 200                                 # out-of-range window index
    _say(f"sparse_attn kv_fmt={kv_fmt} q_dt={q_dt} H={H}")
    d = tio.to_device(wl, dev)
    out = tio.out_to_numpy(run.sparse_attn(wl, d, torch.from_numpy(idx).to(dev), n_win, n_comp))
    tol = F32_TOL if q_dt == configs.DT_F32 else BF16_TOL
    for qi in range(wl.Q):
        ref = O.attend(wl, qi, idx[qi, :n_win], idx[qi, n_win:])
        check_attention(out[qi], ref, tol, f"query {qi}")
    assert np.all(out[1] == 0.0)


# ------------------------------------------------------------------------------------ whole path
def _check_decode(wl, out, idx, tol, empty_rows=()):
    k = wl.topk
    errs = []
    for qi in range(wl.Q):
        nv = int(wl.n_vis[qi])
        scores = O.query_scores(wl, qi)
        win = O.query_window(wl, qi)
        assert idx[qi, :128].tolist() == win.tolist(), f"query {qi}: window indices differ"
        check_topk_row(idx[qi, 128:], scores, nv, k, f"query {qi}")
        ref = O.attend(wl, qi, idx[qi, :128], idx[qi, 128:])   # oracle on the GPU's own index set
        errs.append(check_attention(out[qi], ref, tol, f"query {qi}"))
    for r in empty_rows:
        assert np.all(out[r] == 0.0), f"row {r} must be exact zero"
    return max(errs)


def test_decode_tiny_fp32(dev):
    run, tio = _run()
    wl = configs.tiny_decode()
    _say("decode tiny fp32 (B=1, T=4096, H=16)")
    out, idx = run.decode(wl, tio.to_device(wl, dev))
    err = _check_decode(wl, tio.out_to_numpy(out), idx.cpu().numpy(), F32_TOL)
    _say(f"max err {err:.2e}")


def test_decode_batched_small(dev):
    run, tio = _run()
    wl = configs.batched_decode(B=4, T=65536)
    _say("decode batched small (B=4, T=65536, H=64, fp8)")
    out, idx = run.decode(wl, tio.to_device(wl, dev))
    err = _check_decode(wl, tio.out_to_numpy(out), idx.cpu().numpy(), BF16_TOL)
    _say(f"max err {err:.2e}")


def test_decode_batched_full(dev):
    """The batched decode workload at its full size (B=32, 65,536-token contexts, 64 heads, FP8 KV),
    in the launch configuration the benchmark times; three queries are checked against the oracle."""
    run, tio = _run()
    wl = configs.batched_decode()
    _say("decode batched full (B=32, T=65536, H=64, fp8)")
    out, idx = run.decode(wl, tio.to_device(wl, dev))
    out, idx = tio.out_to_numpy(out), idx.cpu().numpy()
    for qi in (0, 13, 31):
        nv = int(wl.n_vis[qi])
        assert idx[qi, :128].tolist() == O.query_window(wl, qi).tolist()
        check_topk_row(idx[qi, 128:], O.query_scores(wl, qi), nv, wl.topk, f"query {qi}")
        ref = O.attend(wl, qi, idx[qi, :128], idx[qi, 128:])
        check_attention(out[qi], ref, BF16_TOL, f"query {qi}")


def test_decode_selection_in_attention_short_and_long_rows(dev):
    """More than 16 requests at 64 heads: the attention blocks select their own rows.  Contexts mix
    rows with fewer visible entries than k (the list is every visible entry, then -1), rows at and
    around 4k (k entries exactly), rows ending mid-page and rows of the full 16,384 entries; every
    query's selection and output are checked against the oracle."""
    run, tio = _run()
    ctx = [0, 3, 700, 2047, 2048, 2052, 3001, 9000, 65536, 40000, 65535, 4100,
           1, 130, 2600, 60000, 17, 33333, 5000, 64000]
    wl = configs.make_decode("sel_attn", ctx, H=64, HI=64, seed=23)
    _say(f"decode, selection inside the attention blocks (B={len(ctx)}, H=64, fp8)")
    out, idx = run.decode(wl, tio.to_device(wl, dev))
    err = _check_decode(wl, tio.out_to_numpy(out), idx.cpu().numpy(), BF16_TOL, empty_rows=(0,))
    _say(f"max err {err:.2e}")


def test_decode_fp4_indexer(dev):
    """Whole decode path with the MXFP4 indexer (E2M1 pairs, E8M0 per 32): 4 requests at 65,536
    tokens plus a ragged batch whose contexts end mid-page, with 40 indexer heads."""
    run, tio = _run()
    wl = configs.batched_decode(B=4, T=65536, idx_dt=configs.DT_FP4)
    _say("decode batched small, fp4 indexer (B=4, T=65536, H=64)")
    out, idx = run.decode(wl, tio.to_device(wl, dev))
    err = _check_decode(wl, tio.out_to_numpy(out), idx.cpu().numpy(), BF16_TOL)
    _say(f"max err {err:.2e}")
    ctx = [0, 100, 2000, 2047, 2052, 9000, 131, 4]
    wl = configs.make_decode("ragged_fp4", ctx, H=8, HI=40, kv_fmt=configs.KV_BF16, idx_dt=configs.DT_FP4,
                             seed=6)
    _say(f"decode ragged, fp4 indexer ctx={ctx}")
    out, idx = run.decode(wl, tio.to_device(wl, dev))
    _check_decode(wl, tio.out_to_numpy(out), idx.cpu().numpy(), BF16_TOL, empty_rows=(0,))


@pytest.mark.parametrize("idx_dt", [configs.DT_FP8, configs.DT_FP4])
def test_decode_multi_query(dev, idx_dt):
    """Three queries per request (the last three tokens decoded together): contexts shorter than
    the query count, around the 512-entry selection threshold and past the 128-token window."""
    run, tio = _run()
    ctx = [65536, 4099, 2, 2049, 20000, 130]
    wl = configs.make_decode("multi", ctx, H=64, HI=64, seed=31, q_per_req=3, idx_dt=idx_dt)
    _say(f"decode multi-query S=3 ctx={ctx} idx_dt={idx_dt}")
    out, idx = run.decode(wl, tio.to_device(wl, dev))
    err = _check_decode(wl, tio.out_to_numpy(out), idx.cpu().numpy(), BF16_TOL)
    _say(f"max err {err:.2e}")


def test_decode_multi_query_unshared_blocks(dev):
    """Five queries per request: more than one indexer block shares, so each query takes its own
    blocks (the per-query path with the request mapping q / S)."""
    run, tio = _run()
    ctx = [9000, 4, 600]
    wl = configs.make_decode("multi5", ctx, H=16, HI=40, seed=33, q_per_req=5)
    _say(f"decode multi-query S=5 ctx={ctx}")
    out, idx = run.decode(wl, tio.to_device(wl, dev))
    err = _check_decode(wl, tio.out_to_numpy(out), idx.cpu().numpy(), BF16_TOL)
    _say(f"max err {err:.2e}")


def test_hca_decode_fp32(dev):
    """A layer without an indexer in fp32 (q, rows and output): the fp32 attention over dense
    lists of 128 + 300 slots."""
    run, tio = _run()
    ctx = [128 * 300 + 77, 128 * 5]
    wl = configs.make_decode("hca_f32", ctx, H=8, HI=4, q_dt=configs.DT_F32, out_dt=configs.DT_F32,
                             kv_fmt=configs.KV_F32, seed=14, ratio=128)
    _say(f"hca decode fp32 ctx={ctx}")
    out = tio.out_to_numpy(run.hca_decode(wl, tio.to_device(wl, dev)))
    for qi in range(wl.Q):
        check_attention(out[qi], O.run_query_dense(wl, qi), F32_TOL, f"query {qi}")


def test_decode_multi_query_long_rows(dev):
    """Two queries per request on rows longer than the one-block selection takes (the histogram /
    collect / finish path and its preparation launch)."""
    run, tio = _run()
    ctx = [262144, 100003]
    wl = configs.make_decode("multi_long", ctx, H=16, HI=64, seed=32, q_per_req=2)
    _say(f"decode multi-query S=2 ctx={ctx}")
    out, idx = run.decode(wl, tio.to_device(wl, dev))
    err = _check_decode(wl, tio.out_to_numpy(out), idx.cpu().numpy(), BF16_TOL)
    _say(f"max err {err:.2e}")


def test_decode_long_planted_small(dev):
    run, tio = _run()
    wl = configs.make_decode("long_small", [262144, 262144], H=64, HI=64, seed=0, planted_frac=0.01)
    _say("decode long planted small (B=2, T=262144)")
    out, idx = run.decode(wl, tio.to_device(wl, dev))
    idx = idx.cpu().numpy()
    _check_decode(wl, tio.out_to_numpy(out), idx, BF16_TOL)
    for b in range(wl.B):
        assert set(idx[b, 128:].tolist()) <= set(wl.planted[b].tolist())


def test_decode_ragged_small(dev):
    run, tio = _run()
    ctx = [0, 100, 2000, 2047, 2048, 2052, 9000, 0, 131, 4]
    wl = configs.make_decode("ragged_small", ctx, H=8, HI=64, kv_fmt=configs.KV_BF16, seed=4)
    _say(f"decode ragged small ctx={ctx}")
    out, idx = run.decode(wl, tio.to_device(wl, dev))
    _check_decode(wl, tio.out_to_numpy(out), idx.cpu().numpy(), BF16_TOL, empty_rows=(0, 7))


def test_prefill_small(dev):
    run, tio = _run()
    wl = configs.causal_prefill(T=2560)
    _say("prefill small (T=2560, H=64)")
    out, idx = run.prefill(wl, tio.to_device(wl, dev))
    out, idx = tio.out_to_numpy(out), idx.cpu().numpy()
    sample = sorted(set([0, 1, 2, 3, 4, 127, 128, 129, 2045, 2046, 2047, 2048, 2049, 2559] +
                        np.random.default_rng(0).choice(2560, 24, replace=False).tolist()))
    for t in sample:
        nv = int(wl.n_vis[t])
        scores = O.query_scores(wl, t)
        assert idx[t, :128].tolist() == O.window_prefill(t).tolist()
        check_topk_row(idx[t, 128:], scores, nv, wl.topk, f"t={t}")
        ref = O.attend(wl, t, idx[t, :128], idx[t, 128:])
        check_attention(out[t], ref, BF16_TOL, f"t={t}")


@pytest.mark.parametrize("idx_dt", [configs.DT_FP8, configs.DT_FP4])
def test_prefill_chunk_ragged(dev, idx_dt):
    """A prefill chunk that starts mid-sequence, with a query count that is not a multiple of the
    indexer's query block, a visible prefix that ends mid-page, and 40 indexer heads (padded to
    48 inside the matrix-core kernels); FP8 and MXFP4 indexer operands."""
    run, tio = _run()
    wl = configs.causal_prefill(T=4100, HI=40, q_start=2003, q_count=1013, seed=5, idx_dt=idx_dt)
    _say(f"prefill chunk (T=4100, q 2003..3015, HI=40, idx_dt={idx_dt})")
    out, idx = run.prefill(wl, tio.to_device(wl, dev))
    out, idx = tio.out_to_numpy(out), idx.cpu().numpy()
    sample = sorted(set([0, 1, 2, 3, 14, 15, 16, 17, 252, 253, 1008, 1009, 1010, 1011, 1012] +
                        np.random.default_rng(1).choice(wl.Q, 16, replace=False).tolist()))
    for i in sample:
        t = int(wl.positions[i])
        nv = int(wl.n_vis[i])
        scores = O.query_scores(wl, i)
        assert idx[i, :128].tolist() == O.window_prefill(t).tolist()
        check_topk_row(idx[i, 128:], scores, nv, wl.topk, f"t={t}")
        ref = O.attend(wl, i, idx[i, :128], idx[i, 128:])
        check_attention(out[i], ref, BF16_TOL, f"t={t}")


# ------------------------------------------------------------------------------------ no indexer
def test_hca_decode_ragged(dev):
    """Layers without an indexer at ratio 128: window ring ++ every visible compressed entry, over
    contexts with 0, 37, 130 and 512 visible entries, an empty context and a context shorter than
    the window."""
    run, tio = _run()
    ctx = [128 * 37 + 5, 0, 100, 128 * 130 + 127, 1 << 16]
    wl = configs.make_decode("hca_ragged", ctx, H=64, HI=4, seed=12, ratio=128)
    _say(f"hca decode ragged ctx={ctx} ratio=128")
    out = tio.out_to_numpy(run.hca_decode(wl, tio.to_device(wl, dev)))
    for qi in range(wl.Q):
        err = check_attention(out[qi], O.run_query_dense(wl, qi), BF16_TOL, f"query {qi}")
        _say(f"query {qi} (n_vis {int(wl.n_vis[qi])}): max err {err:.2e}")
    assert np.all(out[1] == 0.0)


def test_hca_decode_million_tokens(dev):
    """Two requests at 1,048,576 tokens (8,192 compressed entries each): 8,320-slot lists, split over
    more key ranges than one merge group holds."""
    run, tio = _run()
    wl = configs.dense_decode(B=2)
    _say("hca decode (B=2, T=1048576, ratio 128, fp8 rows)")
    out = tio.out_to_numpy(run.hca_decode(wl, tio.to_device(wl, dev)))
    for qi in range(wl.Q):
        err = check_attention(out[qi], O.run_query_dense(wl, qi), BF16_TOL, f"query {qi}")
        _say(f"query {qi}: max err {err:.2e}")


def test_hca_prefill_chunk(dev):
    """Prefill without an indexer at ratio 128: a chunk starting mid-sequence; query t attends raw
    rows [t-127, t] and compressed entries c < (t+1)/128."""
    run, tio = _run()
    wl = configs.make_prefill("hca_prefill", 4100, H=64, HI=4, seed=13, q_start=2003, q_count=1013, ratio=128)
    _say("hca prefill chunk (T=4100, q 2003..3015, ratio 128)")
    out = tio.out_to_numpy(run.hca_prefill(wl, tio.to_device(wl, dev)))
    sample = sorted(set([0, 1, 45, 46, 47, 172, 173, 174, 1012] +
                        np.random.default_rng(2).choice(wl.Q, 12, replace=False).tolist()))
    for i in sample:
        check_attention(out[i], O.run_query_dense(wl, i), BF16_TOL, f"t={int(wl.positions[i])}")


@pytest.mark.parametrize("H", [64, 8])
def test_sparse_attn_long_lists(dev, H):
    """Explicit index lists of 9,128 slots (invalid, out-of-range and duplicate slots included):
    enough key ranges that the split partials merge in several groups."""
    run, tio = _run()
    wl = configs.make_decode("attn_long", [1 << 20, 40000, 3 << 18], H=H, HI=4, seed=23, ratio=32)
    rng = np.random.default_rng(H)
    n_win, n_comp = 128, 9000
    limit = wl.max_pages * 64
    idx = np.empty((wl.Q, n_win + n_comp), np.int32)
    idx[:, :n_win] = rng.integers(-5, 140, size=(wl.Q, n_win))
    idx[:, n_win:] = rng.integers(-3, limit + 10, size=(wl.Q, n_comp))
    idx[0, n_win + 7] = idx[0, n_win + 8000]
    _say(f"sparse_attn long lists H={H} n_comp={n_comp}")
    d = tio.to_device(wl, dev)
    out = tio.out_to_numpy(run.sparse_attn(wl, d, torch.from_numpy(idx).to(dev), n_win, n_comp))
    for qi in range(wl.Q):
        ref = O.attend(wl, qi, idx[qi, :n_win], idx[qi, n_win:])
        err = check_attention(out[qi], ref, BF16_TOL, f"query {qi}")
        _say(f"query {qi}: max err {err:.2e}")

