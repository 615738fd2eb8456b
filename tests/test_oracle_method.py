"""Pins of the oracle's method functions against brute force, closed forms, library routines and
invariants (CPU only).  Each check is built so that a plausible slip in the oracle (a dropped
ReLU, a wrong sign, a transposed operand, a missing sink term, an off-by-one window) fails it.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import csa_oracle as O
from workloads import configs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- indexer

def _indexer_loops(q, k, w):
    HI, d = len(q), len(q[0])
    out = []
    for c in range(len(k)):
        tot = 0.0
        for h in range(HI):
            dot = 0.0
            for i in range(d):
                dot += q[h][i] * k[c][i]
            tot += w[h] * (dot if dot > 0 else 0.0)
        out.append(tot)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_indexer_matches_triple_loop(seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((3, 8))
    k = rng.standard_normal((7, 8))
    w = rng.standard_normal(3)
    ref = _indexer_loops(q.tolist(), k.tolist(), w.tolist())
    np.testing.assert_allclose(O.indexer_scores(q, k, w), ref, rtol=1e-13, atol=1e-13)


def test_indexer_single_head_is_relu_dot():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 16))
    k = rng.standard_normal((50, 16))
    s = O.indexer_scores(q, k, np.ones(1))
    for c in range(50):
        dot = sum(float(a) * float(b) for a, b in zip(q[0], k[c]))
        assert s[c] == pytest.approx(max(dot, 0.0), rel=1e-12, abs=1e-12)
    assert np.all(s >= 0) and np.any(s == 0)


def test_indexer_golden_hand_example():
    """Integer example worked by hand in tests/golden/indexer_hand.json."""
    g = json.load(open(os.path.join(GOLDEN, "indexer_hand.json")))
    s = O.indexer_scores(np.array(g["q"], float), np.array(g["k"], float), np.array(g["w"], float))
    assert s.tolist() == g["expected_scores"]


# ----------------------------------------------------------------------------- top-k

def test_topk_matches_python_sort_with_ties():
    rng = np.random.default_rng(6)
    s = rng.integers(0, 40, size=3000).astype(np.float64)      # many exact ties
    for n_vis, k in [(3000, 512), (2999, 100), (513, 512), (1000, 1)]:
        got = O.topk_select(s, n_vis, k)
        ref = sorted(range(n_vis), key=lambda c: (-s[c], c))[:k]
        assert got.tolist() == ref


@pytest.mark.parametrize("n_vis", [0, 1, 5, 511, 512])
def test_topk_short_context_takes_all(n_vis):
    s = np.random.default_rng(7).standard_normal(max(n_vis, 1))
    got = O.topk_select(s, n_vis, 512)
    assert got.tolist() == list(range(n_vis)) + [-1] * (512 - n_vis)


def test_topk_masks_invisible_entries():
    s = np.arange(100, dtype=float)          # the largest scores are the invisible tail
    got = O.topk_select(s, 60, 10)
    assert got.tolist() == list(range(59, 49, -1))


def test_topk_set_invariant_to_positive_weight_scale():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((4, 16))
    k = rng.standard_normal((2000, 16))
    w = rng.standard_normal(4)
    a = O.topk_select(O.indexer_scores(q, k, w), 2000, 64)
    b = O.topk_select(O.indexer_scores(q, k, 7.5 * w), 2000, 64)
    assert set(a.tolist()) == set(b.tolist())


# ----------------------------------------------------------------------------- windows

def test_window_decode_closed_forms():
    assert O.window_decode(0).tolist() == [-1] * 128
    assert O.window_decode(5).tolist() == [-1] * 123 + [0, 1, 2, 3, 4]
    assert O.window_decode(128).tolist() == list(range(128))
    w = O.window_decode(300)
    assert w.tolist() == [p % 128 for p in range(172, 300)]
    assert sorted(w.tolist()) == list(range(128))


def test_window_prefill_closed_forms():
    assert O.window_prefill(0).tolist() == [-1] * 127 + [0]
    assert O.window_prefill(127).tolist() == list(range(128))
    assert O.window_prefill(1000).tolist() == list(range(873, 1001))


# ----------------------------------------------------------------------------- sparse attention

def _sdpa_with_sink(q, rows, sink, scale):
    """Dense attention through torch's scaled_dot_product_attention in fp64, the sink being one
    extra key of value zero whose logit is the sink (added as a float mask on a zero key)."""
    H, D = q.shape
    J = rows.shape[0]
    qt = torch.from_numpy(q).reshape(1, H, 1, D)
    k = torch.from_numpy(np.concatenate([rows, np.zeros((1, D))])).reshape(1, 1, J + 1, D).expand(1, H, J + 1, D)
    v = k.clone()
    mask = torch.zeros(1, H, 1, J + 1, dtype=torch.float64)
    mask[0, :, 0, J] = torch.from_numpy(sink)
    out = torch.nn.functional.scaled_dot_product_attention(qt, k, v, attn_mask=mask, scale=scale)
    return out.reshape(H, D).numpy()


@pytest.mark.parametrize("seed,H,J", [(0, 4, 30), (1, 16, 200), (2, 1, 1)])
def test_attention_all_positions_equals_dense_sdpa(seed, H, J):
    rng = np.random.default_rng(seed)
    D = 512
    q = rng.standard_normal((H, D))
    rows = rng.standard_normal((J, D))
    sink = rng.standard_normal(H)
    scale = 1 / math.sqrt(D)
    ours = O.sparse_attention(q, rows, np.ones(J, bool), sink, scale)
    np.testing.assert_allclose(ours, _sdpa_with_sink(q, rows, sink, scale), rtol=1e-12, atol=1e-13)


def test_attention_invalid_slots_are_dropped():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((8, 512))
    rows = rng.standard_normal((40, 512))
    valid = rng.random(40) < 0.5
    sink = rng.standard_normal(8)
    a = O.sparse_attention(q, rows, valid, sink, 0.05)
    b = _sdpa_with_sink(q, rows[valid], sink, 0.05)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_attention_closed_forms():
    D = 512
    v = np.zeros((1, D))
    v[0, 3] = 2.0
    # one key: out = v e^S / (e^S + e^sink); with S = sink the output is v/2
    q = np.zeros((1, D))
    q[0, 3] = 0.75                                    # S = q . v = 0.75 * 2 = 1.5 (scale 1)
    out = O.sparse_attention(q, v, np.array([True]), np.array([1.5]), 1.0)
    assert out[0, 3] == pytest.approx(1.0, rel=1e-15)
    out = O.sparse_attention(q, v, np.array([True]), np.array([0.0]), 1.0)
    assert out[0, 3] == pytest.approx(2.0 * math.exp(1.5) / (math.exp(1.5) + 1.0), rel=1e-14)
    # n identical keys: n e^S v / (n e^S + e^sink)
    rows = np.repeat(v, 5, axis=0)
    out = O.sparse_attention(q, rows, np.ones(5, bool), np.array([0.25]), 1.0)
    assert out[0, 3] == pytest.approx(2.0 * 5 * math.exp(1.5) / (5 * math.exp(1.5) + math.exp(0.25)), rel=1e-14)
    # sink -> -inf: plain softmax
    rng = np.random.default_rng(10)
    qq = rng.standard_normal((2, D))
    rr = rng.standard_normal((6, D))
    out = O.sparse_attention(qq, rr, np.ones(6, bool), np.array([-1e4, -1e4]), 0.1)
    S = 0.1 * qq @ rr.T
    p = np.exp(S - S.max(1, keepdims=True))
    np.testing.assert_allclose(out, (p / p.sum(1, keepdims=True)) @ rr, rtol=1e-12)


def test_attention_empty_row_is_exact_zero():
    q = np.random.default_rng(11).standard_normal((16, 512))
    rows = np.random.default_rng(12).standard_normal((640, 512))
    out = O.sparse_attention(q, rows, np.zeros(640, bool), np.full(16, 3.0), 0.04)
    assert np.all(out == 0.0)


def test_attention_permutation_invariant():
    rng = np.random.default_rng(13)
    q = rng.standard_normal((4, 512))
    rows = rng.standard_normal((64, 512))
    valid = rng.random(64) < 0.8
    sink = rng.standard_normal(4)
    perm = rng.permutation(64)
    a = O.sparse_attention(q, rows, valid, sink, 0.044)
    b = O.sparse_attention(q, rows[perm], valid[perm], sink, 0.044)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_attention_golden_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "attention_hand.json")))
    for case in g["cases"]:
        D = 512
        q = np.zeros((1, D))
        for i, x in case["q"]:
            q[0, i] = x
        rows = np.zeros((len(case["rows"]), D))
        for j, r in enumerate(case["rows"]):
            for i, x in r:
                rows[j, i] = x
        out = O.sparse_attention(q, rows, np.array(case["valid"], bool), np.array([case["sink"]]), case["scale"])
        exp = np.zeros(D)
        for i, x in case["expected"]:
            exp[i] = x
        np.testing.assert_allclose(out[0], exp, rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------------------- whole path

def test_decode_path_top_equals_all_when_short():
    """A context shorter than 4*512 tokens selects every compressed entry, so the path equals dense
    attention over [window rows ++ all compressed rows]."""
    wl = configs.make_decode("t", [1200], H=4, HI=4, seed=3)
    out, top, _ = O.run_query(wl, 0)
    assert top.tolist() == list(range(300)) + [-1] * 212
    rows, valid = O.gather_rows(wl, 0, O.window_decode(1200), np.arange(300))
    assert valid.all()
    ref = _sdpa_with_sink(O.q_values(wl.q[0], wl.q_dt), rows, wl.sink.astype(np.float64), wl.softmax_scale)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("ratio", [1, 3, 4, 128])
def test_compressed_visible_brute_force(ratio):
    """Entry c is visible when every raw token it summarises ([c*ratio, (c+1)*ratio)) is among the
    first n tokens; counted token by token."""
    for n in list(range(0, 300, 7)) + [ratio * 5 - 1, ratio * 5, ratio * 5 + 1]:
        brute = sum(1 for c in range(n + 1) if all(c * ratio + i < n for i in range(ratio)))
        assert O.compressed_visible(n, ratio) == brute


def test_dense_compressed_layer_equals_dense_sdpa():
    """A layer without an indexer at ratio 128: the query attends the window ring and all 37 visible
    compressed entries, which equals dense attention over rows read straight from the pool."""
    T = 128 * 37 + 5
    wl = configs.make_decode("hca", [T], H=4, HI=4, seed=9, ratio=128)
    assert int(wl.n_vis[0]) == O.compressed_visible(T, 128) == 37
    out = O.run_query_dense(wl, 0)
    rows = [O.kv_row_values(wl.win_rows[0, p % 128], wl.win_fmt) for p in range(T - 128, T)]
    rows += [O.kv_row_values(wl.kv_pool[wl.page_table[0, c // 64], c % 64], wl.kv_fmt) for c in range(37)]
    ref = _sdpa_with_sink(O.q_values(wl.q[0], wl.q_dt), np.array(rows), wl.sink.astype(np.float64),
                          wl.softmax_scale)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)


def test_dense_compressed_prefill_is_causal():
    """Prefill at ratio 128: query t sees floor((t+1)/128) entries, so the query at the last token of
    a block sees that block's entry and the one before it does not."""
    wl = configs.make_prefill("hca_p", 1024, H=2, HI=2, seed=1, q_start=120, q_count=300, ratio=128)
    for i, t in enumerate(wl.positions):
        assert int(wl.n_vis[i]) == O.compressed_visible(int(t) + 1, 128)
    i = int(np.nonzero(wl.positions == 255)[0][0])
    assert int(wl.n_vis[i]) == 2 and int(wl.n_vis[i - 1]) == 1
    np.testing.assert_array_equal(O.dense_compressed_indices(2), [0, 1])


@pytest.mark.parametrize("T,S", [(5000, 2), (5000, 4), (130, 3), (3, 4), (128, 2), (129, 4)])
def test_multi_query_window_against_simulated_ring(T, S):
    """S queries per request (the last S of T tokens): write tokens 0..T-1 one by one into a ring of
    128 + S - 1 slots, then every valid slot of query j's window must hold exactly the positions
    [p-127, p] (p = T - S + j), in order, with -1 for positions before 0."""
    R = 128 + S - 1
    ring = np.full(R, -1)
    for pos in range(T):
        ring[pos % R] = pos
    for j in range(S):
        p = T - S + j
        win = O.window_decode(O.decode_tokens_seen(T, S, j), 128, R)
        expect = np.arange(p - 127, p + 1)
        for slot, e in zip(win, expect):
            if e < 0:
                assert slot == -1
            else:
                assert slot >= 0 and ring[slot] == e


def test_multi_query_visibility_and_single_query_reduction():
    """Query j of S sees the compressed entries whose 4 tokens are all at or before position
    T - S + j; with S = 1 the workload is the plain one-query decode."""
    wl = configs.make_decode("mq", [4099, 7, 20000], H=2, HI=2, seed=4, q_per_req=3)
    assert wl.Q == 9 and wl.win_rows.shape[1] == 130
    for q in range(wl.Q):
        T = int(wl.ctx_len[q // 3])
        p = T - 3 + q % 3
        assert int(wl.q_req[q]) == q // 3
        assert int(wl.n_vis[q]) == sum(1 for c in range(p + 2) if 4 * c + 3 <= p)
    one = configs.make_decode("mq1", [4099, 7], H=2, HI=2, seed=4, q_per_req=1)
    ref = configs.make_decode("mq1", [4099, 7], H=2, HI=2, seed=4)
    assert one.Q == 2 and np.array_equal(one.q, ref.q) and np.array_equal(one.n_vis, [1024, 1])
    np.testing.assert_array_equal(O.query_window(one, 0), O.window_decode(4099))


def test_scores_use_page_table_and_block_scales():
    """Scores computed from the paged byte layout equal scores from keys decoded entry by entry with
    the scale bytes read at [page][block][slot]."""
    wl = configs.make_decode("t", [1000], H=4, HI=8, seed=4)
    s = O.query_scores(wl, 0)
    qh = O.indexer_q_values(wl.qI[0], wl.qI_scale[0], wl.idx_dt)
    for c in [0, 63, 64, 130, 249]:
        p = wl.page_table[0, c // 64]
        slot = c % 64
        k = np.array([O.fp8_e4m3fn_value(x) for x in wl.ik_keys[p, slot]])
        scl = [2.0 ** (int(wl.ik_scales[p, b, slot]) - 127) for b in range(4)]
        k = k * np.repeat(scl, 32)
        ref = sum(float(wl.w[0, h]) * max(0.0, float(qh[h] @ k)) for h in range(8))
        assert s[c] == pytest.approx(ref, rel=1e-12, abs=1e-12)


def test_fp4_scores_use_page_table_nibbles_and_block_scales():
    """FP4 indexer (two E2M1 values per byte, element 2i in the low nibble, E8M0 per 32): scores from
    the paged byte layout equal scores from keys and queries unpacked nibble by nibble here."""
    wl = configs.make_decode("t4", [1000], H=4, HI=8, idx_dt=configs.DT_FP4, seed=4)
    assert wl.ik_keys.shape[-1] == 64 and wl.qI.shape[-1] == 64
    s = O.query_scores(wl, 0)

    def unpack(row):
        out = []
        for byte in row:
            out += [O.fp4_e2m1_value(int(byte) & 0xF), O.fp4_e2m1_value(int(byte) >> 4)]
        return np.array(out)

    qh = np.stack([unpack(wl.qI[0, h]) * np.repeat([2.0 ** (int(x) - 127) for x in wl.qI_scale[0, h]], 32)
                   for h in range(8)])
    for c in [0, 63, 64, 130, 249]:
        p = wl.page_table[0, c // 64]
        slot = c % 64
        k = unpack(wl.ik_keys[p, slot]) * np.repeat([2.0 ** (int(wl.ik_scales[p, b, slot]) - 127) for b in range(4)], 32)
        ref = sum(float(wl.w[0, h]) * max(0.0, float(qh[h] @ k)) for h in range(8))
        assert s[c] == pytest.approx(ref, rel=1e-12, abs=1e-12)


def test_long_context_planted_entries_win():
    """Reduced long-context recipe (T=262144, 655 planted entries): every planted entry outscores every other entry, so
    the top-512 set is a subset of the planted set."""
    wl = configs.make_decode("t", [262144], H=4, HI=64, seed=0, planted_frac=0.01)
    assert wl.planted[0].size == 655
    s = O.query_scores(wl, 0)
    planted = wl.planted[0]
    mask = np.zeros(s.size, bool)
    mask[planted] = True
    assert s[mask].min() > s[~mask].max()
    top = O.topk_select(s, s.size, 512)
    assert set(top.tolist()) <= set(planted.tolist())


def test_ragged_lengths_recipe():
    T = configs.ragged_lengths(0)
    assert T.shape == (64,)
    assert [int(T[r]) for r in configs.RAGGED_EMPTY_ROWS] == [0, 0, 0, 0]
    rest = np.delete(T, configs.RAGGED_EMPTY_ROWS)
    assert rest.min() >= 512 and rest.max() <= 131072
    assert (rest // 4 < 512).sum() >= 1


def test_gather_rows_drops_negative_out_of_range_and_unmapped_slots():
    """The oracle's reading of slots the pages leave open ([P1] section 3.7 masks only -1): a
    negative index, an index at or past its source's length, or a compressed index on a page the
    page table leaves unmapped (-1) or maps past the pool is dropped (zero row, not valid).  Valid
    slots hold the stored bf16 row, decoded here by torch, with duplicates kept."""
    wl = configs.make_decode("gather", [300, 1000], H=2, HI=2, kv_fmt=configs.KV_BF16, seed=8)
    r = 1
    pt = wl.page_table.copy()
    assert pt.shape[1] >= 4 and pt[r, :4].min() >= 0
    pt[r, 2] = -1                       # an unmapped page
    pt[r, 3] = wl.num_pages + 5         # a page id past the pool
    wl.page_table = pt
    wr = wl.win_rows.shape[1]
    limit = pt.shape[1] * 64
    win = np.array([-1, -7, 0, 5, 5, wr - 1, wr, wr + 10])
    comp = np.array([-1, -3, 0, 70, 70, 2 * 64 + 1, 3 * 64 + 9, limit, limit + 5, 63])
    rows, valid = O.gather_rows(wl, r, win, comp)      # one query per request: query r is request r's
    expect = [False, False, True, True, True, True, False, False,
              False, False, True, True, True, False, False, False, False, True]
    assert valid.tolist() == expect

    def bf16_row(raw):
        return torch.from_numpy(raw.view(np.int16).copy()).view(torch.bfloat16).double().numpy()

    for j, ok in enumerate(expect):
        if not ok:
            assert np.all(rows[j] == 0.0)
            continue
        if j < win.size:
            ref = bf16_row(wl.win_rows[r, win[j]])
        else:
            c = comp[j - win.size]
            ref = bf16_row(wl.kv_pool[pt[r, c // 64], c % 64])
        np.testing.assert_array_equal(rows[j], ref)
    # an all-dropped list attends to nothing: exact zeros
    out = O.attend(wl, r, np.array([-1, wr]), np.array([-2, limit, 2 * 64]))
    assert np.all(out == 0.0)


def test_long_context_planted_rows_keep_the_row_scale():
    """Planted KV rows lean on the queries' summed direction yet keep the scale of the N(0, 1) rows
    around them (expected squared norm 512), so outputs stay of order one as with unplanted rows."""
    from workloads import codec
    wl = configs.make_decode("t", [65536], H=8, HI=16, seed=2, planted_frac=0.01, kv_fmt=configs.KV_F32)
    n = wl.planted[0]
    rows = np.stack([O.kv_row_values(wl.kv_pool[wl.page_table[0, c // 64], c % 64], wl.kv_fmt) for c in n])
    others = np.stack([O.kv_row_values(wl.kv_pool[wl.page_table[0, c // 64], c % 64], wl.kv_fmt)
                       for c in np.setdiff1d(np.arange(2000), n)[:200]])
    d = O.q_values(wl.q[0], wl.q_dt).sum(axis=0)
    d /= np.linalg.norm(d)
    assert codec.ROW_BYTES[wl.kv_fmt] == 2048
    assert abs(np.mean(np.sum(rows ** 2, axis=1)) / 512 - 1.0) < 0.05
    assert abs(np.mean(np.sum(others ** 2, axis=1)) / 512 - 1.0) < 0.05
    cos = rows @ d / np.linalg.norm(rows, axis=1)
    assert 0.85 < cos.mean() < 0.93
