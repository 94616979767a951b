"""Pins of the token-order oracle (CPU only) and bit-exact agreement of the library's host-side
order builder with it.

The Hilbert index is pinned by what defines a Hilbert curve on the 2^b cube, not by its own
formula: the order-1 square is the textbook U (0,0) -> (0,1) -> (1,1) -> (1,0); the index is a
bijection onto 0 .. 2^(n b) - 1 starting at the origin; consecutive indices are neighbouring cells
(the curve is continuous); and every aligned run of 2^(n L) indices fills one aligned sub-cube of
side 2^L (the curve finishes each sub-cube before it moves on).
"""
import ctypes
import itertools

import numpy as np
import pytest

from oracle import token_order as tor


def test_order_one_square_is_the_textbook_u():
    cells = sorted(itertools.product(range(2), range(2)), key=lambda c: tor.hilbert_index(list(c), 1))
    assert cells == [(0, 0), (0, 1), (1, 1), (1, 0)]


@pytest.mark.parametrize("n,bits", [(2, 1), (2, 2), (2, 3), (2, 4), (3, 1), (3, 2), (3, 3)])
def test_hilbert_curve_defining_properties(n, bits):
    side = 1 << bits
    cells = list(itertools.product(range(side), repeat=n))
    idx = {c: tor.hilbert_index(list(c), bits) for c in cells}
    assert sorted(idx.values()) == list(range(side ** n))          # bijection
    assert idx[(0,) * n] == 0                                       # starts at the origin
    by_index = sorted(cells, key=lambda c: idx[c])
    for a, b in zip(by_index, by_index[1:]):                       # continuity
        assert sum(abs(x - y) for x, y in zip(a, b)) == 1, (a, b)
    for level in range(1, bits):                                   # sub-cube at every level
        run = 1 << (n * level)
        for k in range(0, side ** n, run):
            chunk = np.array(by_index[k:k + run])
            lo = chunk.min(axis=0)
            assert np.all(chunk.max(axis=0) - lo == (1 << level) - 1)
            assert np.all(lo % (1 << level) == 0)


def test_grid_order_is_a_permutation_with_mostly_adjacent_steps():
    T, H, W = 3, 5, 6
    order = tor.hilbert_order(T, H, W)
    assert sorted(order.tolist()) == list(range(T * H * W))
    coords = np.stack(np.unravel_index(order, (T, H, W)), axis=1)
    steps = np.abs(np.diff(coords, axis=0)).sum(axis=1)
    assert np.mean(steps == 1) > 0.8
    full = tor.hilbert_order(4, 4, 4)
    coords = np.stack(np.unravel_index(full, (4, 4, 4)), axis=1)
    assert np.all(np.abs(np.diff(coords, axis=0)).sum(axis=1) == 1)


def test_reorder_and_restore_are_inverse_gathers():
    r = np.random.default_rng(3)
    order = tor.hilbert_order(2, 3, 5)
    X = r.standard_normal((1, 2, 32, 4))              # 30 valid tokens + 2 padding rows
    Xr = tor.reorder(X, order)
    for n in range(30):
        assert np.array_equal(Xr[:, :, n], X[:, :, order[n]])
    assert np.array_equal(Xr[:, :, 30:], X[:, :, 30:])
    assert np.array_equal(tor.restore(Xr, order), X)


def test_blocks_are_more_compact_along_the_curve():
    """The effect the pages describe, on the wan13b latent grid: the 64-token blocks of the Hilbert
    order span much smaller boxes of the (t, h, w) grid than row-major blocks."""
    T, H, W = 21, 30, 52
    order = tor.hilbert_order(T, H, W)
    def mean_extent(seq):
        c = np.stack(np.unravel_index(seq, (T, H, W)), axis=1)
        n = len(seq) // 64 * 64
        blocks = c[:n].reshape(-1, 64, 3)
        return float(np.mean(np.sum(blocks.max(axis=1) - blocks.min(axis=1) + 1, axis=1)))
    assert mean_extent(order) < 0.5 * mean_extent(np.arange(T * H * W))


@pytest.mark.parametrize("grid", [(1, 1, 1), (2, 3, 5), (3, 5, 6), (4, 4, 4), (21, 30, 52), (7, 1, 64)])
def test_library_order_matches_oracle(grid):
    from block_sparse_linear_mean_amd import _lib
    T, H, W = grid
    out = (ctypes.c_int32 * (T * H * W))()
    assert _lib.lib().sla_hilbert_order(T, H, W, out) == 0
    assert np.array_equal(np.frombuffer(out, dtype=np.int32), tor.hilbert_order(T, H, W))


def test_library_order_validation():
    from block_sparse_linear_mean_amd import _lib
    L = _lib.lib()
    out = (ctypes.c_int32 * 8)()
    assert L.sla_hilbert_order(0, 2, 2, out) == 2
    assert L.sla_hilbert_order(2, 2, 2, None) == 1
    assert L.sla_hilbert_order(1 << 12, 1 << 12, 1 << 12, out) == 4     # more than 2^31 tokens
