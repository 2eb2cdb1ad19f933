"""The tile-packed weight order (host reference used by the GPU layout test)
against the block formula stated for DG_LAYOUT_TILED in include/dg.h, element
by element on small stacks: a single matrix keeps a 16-row tile's 64-k chunks
together, a stack of G > 1 keeps the k chunk of every matrix's tiles together."""

import numpy as np
import pytest

from tests.util import pack_tiled


def _offset(g, n, k, G, N, K, itemsize):
    t, c, r, q = n // 16, k // 64, n % 16, (k % 64) // 16
    blk = (t * (K // 64) + c) if G == 1 else ((c * G + g) * (N // 16) + t)
    lane = r + 16 * q
    if itemsize == 1:
        return blk * 1024 + lane * 16 + k % 16
    h = (k % 16) // 8
    return blk * 1024 + h * 512 + lane * 8 + k % 8


@pytest.mark.parametrize("G,N,K", [(1, 32, 128), (1, 16, 64), (3, 32, 128), (2, 48, 192)])
@pytest.mark.parametrize("dtype", [np.uint8, np.int16])
def test_pack_tiled_matches_documented_order(G, N, K, dtype):
    rng = np.random.default_rng(G * 1000 + N + K)
    w = rng.integers(0, 120, (G, N, K)).astype(dtype)
    flat = pack_tiled(w if G > 1 else w[0]).reshape(-1)
    isz = np.dtype(dtype).itemsize
    gi, ni, ki = np.meshgrid(np.arange(G), np.arange(N), np.arange(K), indexing="ij")
    off = np.vectorize(lambda g, n, k: _offset(g, n, k, G, N, K, isz))(gi, ni, ki)
    assert np.array_equal(flat[off], w)
    # a permutation: every packed slot is filled exactly once
    assert np.array_equal(np.sort(off.reshape(-1)), np.arange(G * N * K))
