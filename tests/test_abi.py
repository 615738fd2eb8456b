"""The C ABI library loads, exports every function include/csa.h declares, and rejects bad arguments
on the host before touching the GPU (CPU only: no call here reaches a kernel launch).

The rejection tests pass fake device addresses, so host validation is all that stands between them
and a kernel launch: they run only where no GPU is visible."""
import ctypes

import pytest

import long_context_sparse_csa_amd as csa
from long_context_sparse_csa_amd import binding as B

FAKE = 1 << 20          # a 16-byte aligned non-null address; never dereferenced by validation
MISALIGNED = FAKE + 4


def _gpu_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0      # counts devices without initialising HIP
    except Exception:  # noqa: BLE001
        return False


fake_pointers = pytest.mark.skipif(_gpu_visible(), reason="fake device addresses: run only where no GPU is visible")


def test_library_exports_every_declared_symbol():
    L = csa.lib()
    names = B.header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), f"missing export {n}"
    assert set(names) == set(B._SIGS), "binding signatures and header declarations diverge"


def test_status_strings():
    for s in range(-8, 1):
        assert csa.csa_status_string(s) != "unknown status"
    assert csa.csa_status_string(5) == "unknown status"
    assert csa.csa_last_hip_error() == 0


def test_workspace_queries():
    assert csa.csa_topk_workspace_bytes(0, 10, 512) == 0
    assert csa.csa_topk_workspace_bytes(8, 262144, 512) >= 8 * 262144 * 8
    assert csa.csa_decode_workspace_bytes(32, 64, 64, 65536, 512) > 32 * 16384 * 4
    assert csa.csa_sparse_attn_workspace_bytes(1, 16, 0) == 0
    assert csa.csa_prefill_workspace_bytes(8192, 64, 64, 8192, 512) > 8192 * 2048 * 4


def _idx(**kw):
    d = dict(keys=FAKE, scales=FAKE, dt=B.CSA_FP8_E4M3FN, num_pages=4, page_table=FAKE, max_pages=4)
    d.update(kw)
    return B.PagedIdx(d["keys"], d["scales"], d["dt"], d["num_pages"], d["page_table"], d["max_pages"], 0)


def _kv(**kw):
    d = dict(rows=FAKE, fmt=B.CSA_KV_FP8NOPE_BF16ROPE, num_pages=4, page_table=FAKE, max_pages=4)
    d.update(kw)
    return B.PagedKV(d["rows"], d["fmt"], d["num_pages"], d["page_table"], d["max_pages"], 0)


def _indexer(**kw):
    a = dict(qI=FAKE, qs=FAKE, dt=B.CSA_FP8_E4M3FN, w=FAKE, keys=_idx(), q_req=FAKE, n_req=1, n_vis=FAKE, Q=1,
             HI=64, max_n_vis=256, logits=FAKE, ld=256)
    a.update(kw)
    return csa.lib().csa_indexer_logits(a["qI"], a["qs"], a["dt"], a["w"], ctypes.byref(a["keys"]), a["q_req"],
                                        a["n_req"], a["n_vis"], a["Q"], a["HI"], a["max_n_vis"], a["logits"], a["ld"],
                                        None)


@pytest.mark.parametrize("kw,status", [
    (dict(qI=None), -1), (dict(w=None), -1), (dict(qs=None), -1), (dict(logits=None), -1),
    (dict(keys=_idx(keys=None)), -1), (dict(keys=_idx(scales=None)), -1),
    (dict(dt=1), -3), (dict(keys=_idx(dt=0)), -3), (dict(dt=0, keys=_idx(dt=0)), -3),   # f32 keys with scales
    (dict(dt=4, keys=_idx(dt=4)), -3), (dict(dt=B.CSA_FP4_E2M1), -3),                   # unknown / key dtype differs
    (dict(dt=B.CSA_FP4_E2M1, keys=_idx(dt=B.CSA_FP4_E2M1), qs=None), -1),
    (dict(dt=B.CSA_FP4_E2M1, keys=_idx(dt=B.CSA_FP4_E2M1, scales=None)), -1),
    (dict(HI=0), -2), (dict(HI=65), -2), (dict(Q=0), -2), (dict(n_req=0), -2), (dict(ld=100), -2),
    (dict(max_n_vis=-1), -2), (dict(keys=_idx(num_pages=0)), -2),
    (dict(qI=MISALIGNED), -4), (dict(logits=FAKE + 2), -4), (dict(keys=_idx(keys=MISALIGNED)), -4),
])
@fake_pointers
def test_indexer_rejects(kw, status):
    assert _indexer(**kw) == status


def _topk(**kw):
    a = dict(logits=FAKE, ld=1024, n_vis=FAKE, Q=2, max_n_vis=1000, k=512, idx=FAKE, ld_idx=512, ws=FAKE,
             ws_bytes=1 << 40)
    a.update(kw)
    return csa.lib().csa_topk(a["logits"], a["ld"], a["n_vis"], a["Q"], a["max_n_vis"], a["k"], a["idx"], a["ld_idx"],
                              a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(logits=None), -1), (dict(idx=None), -1), (dict(n_vis=None), -1),
    (dict(k=0), -2), (dict(k=2049), -2), (dict(ld_idx=100), -2), (dict(ld=999), -2), (dict(Q=0), -2),
    (dict(ws=None), -5), (dict(ws_bytes=10), -5), (dict(ws=FAKE + 8), -4), (dict(idx=FAKE + 1), -4),
])
@fake_pointers
def test_topk_rejects(kw, status):
    assert _topk(**kw) == status


def _attn(**kw):
    a = dict(q=FAKE, q_dt=B.CSA_BF16, Q=2, H=64, sink=FAKE, win=FAKE, win_fmt=2, wr=128, comp=_kv(), q_req=FAKE,
             n_req=2, idx=FAKE, ld_idx=640, n_win=128, n_comp=512, scale=0.044, out=FAKE, out_dt=1, ws=FAKE,
             ws_bytes=1 << 40)
    a.update(kw)
    comp = ctypes.byref(a["comp"]) if a["comp"] is not None else None
    return csa.lib().csa_sparse_attn(a["q"], a["q_dt"], a["Q"], a["H"], a["sink"], a["win"], a["win_fmt"], a["wr"],
                                     comp, a["q_req"], a["n_req"], a["idx"], a["ld_idx"], a["n_win"], a["n_comp"],
                                     a["scale"], a["out"], a["out_dt"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(sink=None), -1), (dict(out=None), -1), (dict(idx=None), -1),
    (dict(win=None), -1), (dict(comp=None), -1), (dict(comp=_kv(rows=None)), -1),
    (dict(q_dt=2), -3), (dict(out_dt=2), -3), (dict(win_fmt=7), -3), (dict(comp=_kv(fmt=9)), -3),
    (dict(H=0), -2), (dict(H=129), -2), (dict(n_win=0, n_comp=0), -2), (dict(n_comp=5000), -2),
    (dict(ld_idx=600), -2), (dict(scale=float("inf")), -2), (dict(n_win=-1), -2),
    (dict(q=MISALIGNED), -4), (dict(out=FAKE + 8), -4), (dict(win=MISALIGNED), -4),
    (dict(ws=None), -5), (dict(ws_bytes=0), -5),
])
@fake_pointers
def test_sparse_attn_rejects(kw, status):
    assert _attn(**kw) == status


@fake_pointers
def test_sparse_attn_allows_null_window_without_window_slots():
    # n_win == 0 with a NULL window source passes validation; only the workspace check remains, so
    # the call is refused for a workspace one byte short of what it needs (never launched)
    need = csa.csa_sparse_attn_workspace_bytes(2, 64, 512)
    if need == 0:
        pytest.skip("this shape needs no workspace: the call would pass validation and launch")
    assert _attn(win=None, n_win=0, ld_idx=512, ws_bytes=need - 1) == -5


def _decode(**kw):
    a = dict(B=2, H=64, HI=64, k=512, q=FAKE, q_dt=1, sink=FAKE, qI=FAKE, qs=FAKE, qI_dt=2, w=FAKE, keys=_idx(),
             comp=_kv(), win=FAKE, win_fmt=2, ctx=FAKE, max_ctx=65536, scale=0.044, out=FAKE, out_dt=1, idx_out=None,
             ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return csa.lib().csa_decode(a["B"], a["H"], a["HI"], a["k"], a["q"], a["q_dt"], a["sink"], a["qI"], a["qs"],
                                a["qI_dt"], a["w"], ctypes.byref(a["keys"]), ctypes.byref(a["comp"]), a["win"],
                                a["win_fmt"], a["ctx"], a["max_ctx"], a["scale"], a["out"], a["out_dt"], a["idx_out"],
                                a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(ctx=None), -1), (dict(win=None), -1), (dict(qI=None), -1),
    (dict(keys=_idx(page_table=None)), -1),
    (dict(qI_dt=0), -3), (dict(win_fmt=5), -3),
    (dict(B=0), -2), (dict(k=0), -2), (dict(HI=65), -2), (dict(max_ctx=-5), -2),
    (dict(comp=_kv(max_pages=3)), -2),
    (dict(ws=None), -5), (dict(ws_bytes=100), -5), (dict(idx_out=FAKE + 2), -4),
])
@fake_pointers
def test_decode_rejects(kw, status):
    assert _decode(**kw) == status


def _decode_multi(**kw):
    a = dict(B=2, S=3, H=64, HI=64, k=512, q=FAKE, q_dt=1, sink=FAKE, qI=FAKE, qs=FAKE, qI_dt=2, w=FAKE, keys=_idx(),
             comp=_kv(), win=FAKE, win_fmt=2, ring=130, ctx=FAKE, max_ctx=65536, scale=0.044, out=FAKE, out_dt=1,
             idx_out=None, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return csa.lib().csa_decode_multi(a["B"], a["S"], a["H"], a["HI"], a["k"], a["q"], a["q_dt"], a["sink"], a["qI"],
                                      a["qs"], a["qI_dt"], a["w"], ctypes.byref(a["keys"]), ctypes.byref(a["comp"]),
                                      a["win"], a["win_fmt"], a["ring"], a["ctx"], a["max_ctx"], a["scale"], a["out"],
                                      a["out_dt"], a["idx_out"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(ctx=None), -1), (dict(win=None), -1), (dict(qI_dt=0), -3),
    (dict(S=0), -2), (dict(S=17), -2), (dict(ring=129), -2), (dict(S=1, ring=127), -2), (dict(B=30000), -2),
    (dict(max_ctx=-1), -2), (dict(k=0), -2), (dict(ws=None), -5), (dict(ws_bytes=64), -5),
    (dict(ctx=FAKE + 1), -4),
])
@fake_pointers
def test_decode_multi_rejects(kw, status):
    assert _decode_multi(**kw) == status


def test_decode_multi_workspace_matches_one_query_decode():
    assert csa.csa_decode_multi_workspace_bytes(32, 1, 64, 64, 65536, 512) == \
        csa.csa_decode_workspace_bytes(32, 64, 64, 65536, 512)
    assert csa.csa_decode_multi_workspace_bytes(8, 4, 64, 64, 65536, 512) == \
        csa.csa_decode_workspace_bytes(32, 64, 64, 65536, 512)
    assert csa.csa_decode_multi_workspace_bytes(8, 0, 64, 64, 65536, 512) == 0


def _prefill(**kw):
    a = dict(Q=16, H=64, HI=64, k=512, q=FAKE, q_dt=1, sink=FAKE, qI=FAKE, qs=FAKE, qI_dt=2, w=FAKE, keys=_idx(),
             comp=_kv(), raw=FAKE, raw_fmt=1, T=256, pos0=0, scale=0.044, out=FAKE, out_dt=1, idx_out=None,
             ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return csa.lib().csa_prefill(a["Q"], a["H"], a["HI"], a["k"], a["q"], a["q_dt"], a["sink"], a["qI"], a["qs"],
                                 a["qI_dt"], a["w"], ctypes.byref(a["keys"]), ctypes.byref(a["comp"]), a["raw"],
                                 a["raw_fmt"], a["T"], a["pos0"], a["scale"], a["out"], a["out_dt"], a["idx_out"],
                                 a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(raw=None), -1), (dict(pos0=250), -2), (dict(T=0), -2), (dict(pos0=-1), -2), (dict(ws_bytes=8), -5),
])
@fake_pointers
def test_prefill_rejects(kw, status):
    assert _prefill(**kw) == status


def _hca_decode(**kw):
    a = dict(B=2, H=64, q=FAKE, q_dt=1, sink=FAKE, comp=_kv(), win=FAKE, win_fmt=2, ctx=FAKE, max_ctx=65536,
             ratio=128, scale=0.044, out=FAKE, out_dt=1, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return csa.lib().csa_hca_decode(a["B"], a["H"], a["q"], a["q_dt"], a["sink"], ctypes.byref(a["comp"]), a["win"],
                                    a["win_fmt"], a["ctx"], a["max_ctx"], a["ratio"], a["scale"], a["out"],
                                    a["out_dt"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), -1), (dict(ctx=None), -1), (dict(win=None), -1), (dict(sink=None), -1),
    (dict(comp=_kv(page_table=None)), -1), (dict(win_fmt=5), -3), (dict(q_dt=2), -3),
    (dict(B=0), -2), (dict(H=129), -2), (dict(ratio=0), -2), (dict(max_ctx=-1), -2),
    (dict(ratio=4, comp=_kv(max_pages=1024), max_ctx=1 << 20), -2),        # 128 + 65,536 slots per query
    (dict(ws=None), -5), (dict(ws_bytes=100), -5), (dict(ws=FAKE + 8), -4), (dict(ctx=FAKE + 2), -4),
])
@fake_pointers
def test_hca_decode_rejects(kw, status):
    assert _hca_decode(**kw) == status


def _hca_prefill(**kw):
    a = dict(Q=16, H=64, q=FAKE, q_dt=1, sink=FAKE, comp=_kv(), raw=FAKE, raw_fmt=1, T=4096, pos0=0, ratio=128,
             scale=0.044, out=FAKE, out_dt=1, ws=FAKE, ws_bytes=1 << 40)
    a.update(kw)
    return csa.lib().csa_hca_prefill(a["Q"], a["H"], a["q"], a["q_dt"], a["sink"], ctypes.byref(a["comp"]), a["raw"],
                                     a["raw_fmt"], a["T"], a["pos0"], a["ratio"], a["scale"], a["out"], a["out_dt"],
                                     a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(raw=None), -1), (dict(out=None), -1), (dict(pos0=4090), -2), (dict(T=0), -2), (dict(ratio=-3), -2),
    (dict(ws_bytes=8), -5), (dict(scale=float("inf")), -2),
])
@fake_pointers
def test_hca_prefill_rejects(kw, status):
    assert _hca_prefill(**kw) == status


def test_hca_workspace_queries():
    n = csa.csa_hca_decode_workspace_bytes(8, 64, 1 << 20, 128)
    assert n >= 8 * (128 + 8192) * 4                                   # the index lists
    assert csa.csa_hca_decode_workspace_bytes(8, 64, 1 << 20, 4) == 0   # 262,144 slots: out of range
    assert csa.csa_hca_decode_workspace_bytes(8, 64, 1 << 20, 0) == 0
    assert csa.csa_hca_prefill_workspace_bytes(8192, 64, 8192, 128) >= 8192 * (128 + 64) * 4


def test_profile_toggle_without_launches():
    csa.csa_profile_enable(True)
    assert csa.csa_profile_collect("indexer_fp8") == (0.0, 0)
    csa.csa_profile_enable(False)
    csa.csa_profile_reset()


def test_debug_counter_is_a_debug_build_feature():
    import ctypes
    n = ctypes.c_uint64(7)
    assert csa.lib().csa_debug_violations(ctypes.byref(n)) == -6 and n.value == 0
    assert csa.lib().csa_debug_violations(None) == -1
