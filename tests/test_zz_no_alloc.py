"""csa_decode_noalloc (the decode step with its workspace in the library's static scratch array)
against csa_decode with a caller workspace, through the C ABI: two calls in a row, the second with
a smaller input, each compared with csa_decode on the same inputs (selected indices equal, outputs
within the bf16 bar).  Also: a call needing more than the scratch holds is refused."""
import numpy as np
import pytest

from tests.helpers import BF16_TOL
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


def _both(wl, dev):
    import long_context_sparse_csa_amd as csa
    from workloads import run, torch_io
    d = torch_io.to_device(wl, dev)
    out_ref, idx_ref = run.decode(wl, d)
    out = torch_io.empty_out(wl, dev)
    idx = torch.full((wl.Q, 128 + wl.topk), -7, dtype=torch.int32, device=dev)
    csa.csa_decode_noalloc(wl.B, wl.H, wl.HI, wl.topk, d.q, wl.q_dt, d.sink, d.qI, d.qI_scale, wl.idx_dt, d.w,
                           run._keys(wl, d), run._comp(wl, d), d.win_rows, wl.win_fmt, d.ctx_len,
                           int(wl.ctx_len.max()), wl.softmax_scale, out, wl.out_dt, idx, None)
    torch.cuda.synchronize()
    return (torch_io.out_to_numpy(out), idx.cpu().numpy()), (torch_io.out_to_numpy(out_ref), idx_ref.cpu().numpy())


def test_noalloc_matches_decode_twice(dev):
    import long_context_sparse_csa_amd as csa
    big = configs.long_decode(B=2, T=1 << 19)          # long rows: the sketch selection
    small = configs.make_decode("noalloc_small", [20000, 3, 0, 9000], H=16, HI=64, seed=9)
    assert csa.csa_decode_workspace_bytes(big.B, big.H, big.HI, int(big.ctx_len.max()), big.topk) > \
        csa.csa_decode_workspace_bytes(small.B, small.H, small.HI, int(small.ctx_len.max()), small.topk)
    for wl in (big, small):
        print(f"[gpu] noalloc vs decode: {wl.name} B={wl.B} max ctx={int(wl.ctx_len.max())}", flush=True)
        (out, idx), (out_ref, idx_ref) = _both(wl, dev)
        assert np.array_equal(idx, idx_ref), f"{wl.name}: selected indices differ"
        err = float(np.abs(out - out_ref).max())
        assert np.all(np.isfinite(out)) and err <= BF16_TOL, f"{wl.name}: max-abs {err:.3e}"
        print(f"[gpu] max-abs vs csa_decode {err:.2e}", flush=True)


def test_noalloc_refuses_calls_beyond_scratch(dev):
    import long_context_sparse_csa_amd as csa
    from long_context_sparse_csa_amd import binding as B
    # 64 requests at 1M tokens need far more than the scratch: refused before any launch
    need = csa.csa_decode_workspace_bytes(64, 64, 64, 1 << 20, 512)
    assert need > B.NOALLOC_SCRATCH_BYTES
    wl = configs.make_decode("noalloc_tiny", [300], H=16, HI=16, seed=2)
    from workloads import run, torch_io
    d = torch_io.to_device(wl, dev)
    out = torch_io.empty_out(wl, dev)
    with pytest.raises(csa.CsaError) as e:
        csa.csa_decode_noalloc(64, wl.H, wl.HI, wl.topk, d.q, wl.q_dt, d.sink, d.qI, d.qI_scale, wl.idx_dt, d.w,
                               run._keys(wl, d), run._comp(wl, d), d.win_rows, wl.win_fmt, d.ctx_len, 1 << 20,
                               wl.softmax_scale, out, wl.out_dt, None, None)
    assert e.value.status == -8
