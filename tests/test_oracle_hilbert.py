"""Pins of the oracle's 3D Hilbert token order (DFSAttn page, trick 1).

The page asks for a reordering along a 3D Hilbert curve so that tokens next
to each other in the sequence are next to each other in space and time.
The pins check the defining properties of the curve, not the oracle's own
formula: every step of the curve moves to a face neighbour, the curve visits
every cell once, its coarsest level is the reflected Gray code, and the
first quarter of the 64-cube is the 32x32x64 box the latent grid is padded to.
"""
import numpy as np
import pytest

import oracle
from conftest import golden


def _curve_cells(bits):
    """Cube cells listed in curve order (brute force over the whole cube)."""
    s = 1 << bits
    g = np.indices((s, s, s)).reshape(3, -1)
    idx = oracle.hilbert_index_3d(g[0], g[1], g[2], bits)
    order = np.argsort(idx)
    return idx, g[:, order].T


def test_order1_is_reflected_gray_code():
    rows = golden("hilbert_order1_corners.txt")
    _, cells = _curve_cells(1)
    want = np.array([[int(r[1]), int(r[2]), int(r[3])] for r in rows])
    assert np.array_equal(cells, want)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
def test_curve_is_bijective_and_face_adjacent(bits):
    idx, cells = _curve_cells(bits)
    s = 1 << bits
    assert np.array_equal(np.sort(idx), np.arange(s ** 3))
    steps = np.abs(np.diff(cells, axis=0)).sum(axis=1)
    assert np.all(steps == 1)
    assert np.array_equal(cells[0], [0, 0, 0])


def test_first_quarter_of_64_cube_is_32x32x64_box_and_contiguous():
    idx, cells = _curve_cells(6)
    at, ay, ax = oracle.hilbert_axis_map(6)
    first = cells[: 65536]
    # the box t<32, y<32, x<64 in curve-axis coordinates
    assert first[:, at].max() == 31 and first[:, ay].max() == 31
    assert first[:, ax].max() == 63
    assert len({tuple(c) for c in first}) == 65536
    steps = np.abs(np.diff(first, axis=0)).sum(axis=1)
    assert np.all(steps == 1)


def test_axis_map_is_natural_order():
    # x on the first-step axis (axis 2), t and y on axes 0 and 1
    for bits in range(1, 7):
        assert oracle.hilbert_axis_map(bits) == (0, 1, 2)


@pytest.mark.parametrize("grid", [(21, 30, 52), (4, 8, 8), (3, 5, 7), (1, 1, 1),
                                  (2, 3, 1), (9, 1, 17)])
def test_perm_is_bijection_starting_at_origin(grid):
    T, Hg, W = grid
    perm, inv = oracle.hilbert_perm(T, Hg, W)
    N = T * Hg * W
    assert np.array_equal(np.sort(perm), np.arange(N))
    assert np.array_equal(inv[perm], np.arange(N))
    assert perm[0] == 0


def test_perm_is_cropped_curve_order():
    # brute force: walk the padded 32x32x64 box in curve order, drop cells
    # outside the 21x30x52 grid, and compare with the oracle's permutation
    T, Hg, W = 21, 30, 52
    _, cells = _curve_cells(6)
    at, ay, ax = oracle.hilbert_axis_map(6)
    t, y, x = cells[:, at], cells[:, ay], cells[:, ax]
    inside = (t < T) & (y < Hg) & (x < W)
    want = ((t * Hg + y) * W + x)[inside]
    perm, _ = oracle.hilbert_perm(T, Hg, W)
    assert np.array_equal(perm, want)


def test_permute_unpermute_identity():
    rng = np.random.default_rng(0)
    X = rng.integers(0, 1 << 16, size=(2, 3, 390, 8), dtype=np.uint16)
    perm, _ = oracle.hilbert_perm(3, 10, 13)
    Y = oracle.permute_tokens(X, perm)
    assert np.array_equal(Y[..., 5, :], X[..., perm[5], :])
    assert np.array_equal(oracle.unpermute_tokens(Y, perm), X)


def test_hilbert_blocks_are_more_compact_than_raster():
    """Diagnostic behind the reordering: 64-token blocks span a smaller
    space-time box in Hilbert order than in raster order."""
    T, Hg, W = 21, 30, 52
    perm, _ = oracle.hilbert_perm(T, Hg, W)
    raster = np.arange(T * Hg * W)

    def mean_box(order):
        t, r = np.divmod(order, Hg * W)
        y, x = np.divmod(r, W)
        vols = []
        for s in range(0, order.size - 63, 64):
            sl = slice(s, s + 64)
            vols.append((np.ptp(t[sl]) + 1) * (np.ptp(y[sl]) + 1) * (np.ptp(x[sl]) + 1))
        return np.mean(vols)

    assert mean_box(perm) < 0.5 * mean_box(raster)
