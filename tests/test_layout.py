"""The folded weight's tile layout, as the C header defines it element by
element, against the vectorised unpacking the GPU tests use (CPU only)."""

import numpy as np

from parity import unpack_folded


def pack_by_definition(Wf: np.ndarray) -> np.ndarray:
    """Element (k, n) of W' [3d, d] at ((n/16)*(3d/32) + k/32)*512 +
    8*(16*((k%32)/8) + n%16) + k%8, one element at a time."""
    K, d = Wf.shape
    out = np.full(K * d, np.nan)
    for k in range(K):
        for n in range(d):
            off = ((n // 16) * (K // 32) + k // 32) * 512 + 8 * (16 * ((k % 32) // 8) + n % 16) + k % 8
            assert np.isnan(out[off])
            out[off] = Wf[k, n]
    assert not np.isnan(out).any()
    return out


def test_unpack_matches_header_definition():
    for d in (64, 128):
        Wf = np.arange(3 * d * d, dtype=np.float64).reshape(3 * d, d)
        tiles = pack_by_definition(Wf)
        assert np.array_equal(unpack_folded(tiles, d), Wf)


def test_column_block_is_one_contiguous_run():
    d = 64
    Wf = np.arange(3 * d * d, dtype=np.float64).reshape(3 * d, d)
    tiles = pack_by_definition(Wf)
    run = tiles[: 3 * d * 16]  # the first 16-column block
    assert set(run.astype(np.int64) % d) == set(range(16))
    # lane 0 of the first tile: column 0, k = 0..7
    assert np.array_equal(tiles[:8], Wf[:8, 0])
    # lane 17 of the first tile: column 1, k = 8..15
    assert np.array_equal(tiles[8 * 17: 8 * 18], Wf[8:16, 1])
