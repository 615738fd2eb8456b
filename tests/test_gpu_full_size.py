"""Parity at the full sizes of the causal prefill (8,192 query positions) and the ragged decode batch
(64 requests, lognormal contexts, four empty rows), through the fused entries in the launch
configuration the benchmark times.  Acceptance as everywhere: band-tolerant top-k against the
oracle's scores, then the oracle evaluated on the GPU's own index set."""
import numpy as np
import pytest

from oracle import csa_oracle as O
from tests.helpers import BF16_TOL, check_attention, check_topk_row
from workloads import configs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

# Prefill rows checked: every boundary the visibility and window rules have, then a stratified
# draw of the rest (four rows from every 32-position stratum), 1,036 rows in all
PREFILL_EDGES = [0, 1, 2, 3, 4, 5, 6, 7, 126, 127, 128, 129, 2044, 2045, 2046, 2047, 2048, 2049, 2050, 2051,
                 4095, 4096, 8188, 8189, 8190, 8191]


def prefill_rows(T=8192, per_stratum=4, stratum=32, seed=0):
    rng = np.random.default_rng(seed)
    picks = set(PREFILL_EDGES)
    for s0 in range(0, T, stratum):
        picks.update(int(x) for x in rng.choice(np.arange(s0, min(T, s0 + stratum)), per_stratum, replace=False))
    return sorted(picks)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sparse_csa_amd as csa
    csa.lib()
    return "cuda"


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


def test_prefill_full_size(dev):
    from workloads import run, torch_io
    wl = configs.causal_prefill()
    rows = prefill_rows()
    assert len(rows) >= 1024 and all(t in rows for t in PREFILL_EDGES)
    _say(f"prefill full size (T=8192, H=64), {len(rows)} rows checked")
    out, idx = run.prefill(wl, torch_io.to_device(wl, dev))
    out, idx = torch_io.out_to_numpy(out), idx.cpu().numpy()
    errs = []
    for n, t in enumerate(rows):
        nv = int(wl.n_vis[t])
        assert idx[t, :128].tolist() == O.window_prefill(t).tolist(), f"t={t}: window"
        check_topk_row(idx[t, 128:], O.query_scores(wl, t), nv, wl.topk, f"t={t}")
        errs.append(check_attention(out[t], O.attend(wl, t, idx[t, :128], idx[t, 128:]), BF16_TOL, f"t={t}"))
        if n % 256 == 0:
            _say(f"{n} rows checked, max err so far {max(errs):.2e}")
    _say(f"max err {max(errs):.2e}")


def test_ragged_decode_full_size(dev):
    from workloads import run, torch_io
    wl = configs.ragged_decode()
    assert wl.B == 64
    _say(f"ragged decode full size (B=64, contexts {int(wl.ctx_len.min())}..{int(wl.ctx_len.max())}, H=8)")
    out, idx = run.decode(wl, torch_io.to_device(wl, dev))
    out, idx = torch_io.out_to_numpy(out), idx.cpu().numpy()
    errs = []
    for qi in range(wl.Q):
        nv = int(wl.n_vis[qi])
        assert idx[qi, :128].tolist() == O.query_window(wl, qi).tolist(), f"query {qi}: window"
        check_topk_row(idx[qi, 128:], O.query_scores(wl, qi), nv, wl.topk, f"query {qi}")
        errs.append(check_attention(out[qi], O.attend(wl, qi, idx[qi, :128], idx[qi, 128:]), BF16_TOL,
                                    f"query {qi}"))
    for r in configs.RAGGED_EMPTY_ROWS:
        assert int(wl.ctx_len[r]) == 0 and np.all(idx[r] == -1)
        assert np.all(out[r] == 0.0), f"row {r} must be exact zero"
    _say(f"all 64 rows checked, max err {max(errs):.2e}")
