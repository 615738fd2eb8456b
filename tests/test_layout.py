"""Host-side index-key page order: pack/unpack against the byte formula the C header states."""
import numpy as np
import pytest

from long_context_sparse_csa_amd import pack_index_keys, unpack_index_keys


@pytest.mark.parametrize("R", [128, 64])
def test_pack_matches_header_formula(R):
    x = np.random.default_rng(R).integers(0, 256, (2, 64, R), dtype=np.uint8)
    flat = pack_index_keys(x).reshape(2, -1)
    halves = R // 64
    s, b = np.meshgrid(np.arange(64), np.arange(R), indexing="ij")
    off = ((s % 4) * halves + b // 64) * 1024 + (s // 4 + 16 * ((b % 64) // 16)) * 16 + b % 16
    for p in range(2):
        assert (flat[p, off] == x[p]).all()
    assert sorted(off.ravel().tolist()) == list(range(64 * R))   # a permutation of the page


@pytest.mark.parametrize("R", [128, 64])
def test_unpack_inverts_pack(R):
    x = np.random.default_rng(1).integers(0, 256, (5, 64, R), dtype=np.uint8)
    assert (unpack_index_keys(pack_index_keys(x)) == x).all()
    assert (unpack_index_keys(pack_index_keys(x).reshape(5, -1)) == x).all()


def test_lane_chunks():
    # kilobyte 1 of an FP8 page is key group 0's second half: lane L = n + 16g holds slot 4n,
    # bytes [64 + 16g, 80 + 16g)
    x = np.random.default_rng(2).integers(0, 256, (1, 64, 128), dtype=np.uint8)
    kb = pack_index_keys(x).reshape(8, 64, 16)[1]
    for L in range(64):
        n, g = L % 16, L // 16
        assert (kb[L] == x[0, 4 * n, 64 + 16 * g: 80 + 16 * g]).all()


def test_rejects_bad_rows():
    with pytest.raises(ValueError):
        pack_index_keys(np.zeros((1, 64, 96), np.uint8))
    with pytest.raises(ValueError):
        pack_index_keys(np.zeros((1, 32, 128), np.uint8))
