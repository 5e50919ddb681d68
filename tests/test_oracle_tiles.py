"""Pins of the oracle's SICS scheme generation over shaped 3D tiles (SPADE
parts 1 and 2): tile geometry against brute-force enumeration, SICS against
the closed form and an explicit pairwise loop, and the shape choice against
planted fields whose coherent axis is known."""
import itertools

import numpy as np
import pytest

from oracle import clusters as OC
from oracle import tiles as OT

MENU = [(1, 4, 32), (1, 8, 16), (2, 8, 8), (8, 4, 4)]


@pytest.mark.parametrize("grid,shape", [((3, 10, 13), (1, 4, 32)), ((3, 10, 13), (2, 8, 8)),
                                        ((21, 30, 52), (8, 4, 4)), ((5, 7, 9), (2, 3, 4)),
                                        ((4, 8, 8), (4, 8, 8))])
def test_tiles_partition_the_grid_in_raster_tile_order(grid, shape):
    T, Hg, W = grid
    ts, ys, xs = shape
    a = OT.tile_assign(T, Hg, W, shape)
    nt = OT.n_tiles(T, Hg, W, shape)
    want = np.full(T * Hg * W, -1)
    c = 0
    for tt, ty, tx in itertools.product(range(-(-T // ts)), range(-(-Hg // ys)), range(-(-W // xs))):
        for t in range(tt * ts, min(T, (tt + 1) * ts)):
            for y in range(ty * ys, min(Hg, (ty + 1) * ys)):
                for x in range(tx * xs, min(W, (tx + 1) * xs)):
                    want[(t * Hg + y) * W + x] = c
        c += 1
    assert c == nt
    assert np.array_equal(a, want)


def _pairwise_cos_sum(X):
    s = 0.0
    for i in range(len(X)):
        for j in range(len(X)):
            if i != j:
                ni, nj = np.linalg.norm(X[i]), np.linalg.norm(X[j])
                if ni > 0 and nj > 0:
                    s += float(X[i] @ X[j]) / (ni * nj)
    return s


def test_sics_equals_pairwise_cosines_and_the_closed_form():
    rng = np.random.default_rng(3)
    X = rng.normal(size=(30, 8))
    X[4] = 0.0                                        # zero row: cosine 0 with everything
    a = rng.integers(0, 4, size=30)
    got = OT.sics_per_tile(X, a, 5)
    for c in range(5):
        rows = X[a == c]
        assert got[c] == pytest.approx(_pairwise_cos_sum(rows), rel=1e-12, abs=1e-12)
        # closed form: |sum of unit rows|^2 - (number of non-zero rows)
        U = OT.unit_rows(rows)
        u = U.sum(axis=0)
        assert got[c] == pytest.approx(float(u @ u) - int((np.abs(rows).sum(1) > 0).sum()),
                                       rel=1e-12, abs=1e-12)
    assert got[4] == 0.0                              # empty tile


def test_sics_score_limits():
    grid = (2, 4, 8)
    N = 64
    same = np.tile(np.array([[1.0, -2.0, 0.5]]), (N, 1))
    assert OT.sics_score(same, same, grid, (1, 2, 4)) == pytest.approx(1.0)
    # alternating antipodal rows along x: a tile of xs = 2 has cosine -1 pairs
    alt = np.array([[1.0, 0.0] if n % 2 == 0 else [-1.0, 0.0] for n in range(N)])
    assert OT.sics_score(alt, alt, grid, (1, 1, 2)) == pytest.approx(-1.0)
    # one-token tiles have no pairs: score 0
    assert OT.sics_score(alt, alt, grid, (1, 1, 1)) == 0.0


def _field(grid, axes, d=16, seed=0):
    """Random unit-scale vectors that depend only on the given grid axes."""
    T, Hg, W = grid
    rng = np.random.default_rng(seed)
    shape = [T if 0 in axes else 1, Hg if 1 in axes else 1, W if 2 in axes else 1]
    base = rng.normal(size=shape + [d])
    F = np.broadcast_to(base, (T, Hg, W, d))
    return np.ascontiguousarray(F).reshape(T * Hg * W, d)


def test_shape_choice_follows_the_coherent_axis():
    grid = (8, 8, 32)
    # depends on t only: every shape with ts = 1 is perfectly coherent; the
    # first of them in the menu wins the tie
    X = _field(grid, (0,))
    pick, scores = OT.choose_shape(X, X, grid, MENU)
    assert pick == 0 and scores[0] == pytest.approx(1.0) and scores[1] == pytest.approx(1.0)
    assert scores[3] < 0.5
    # depends on x only: the thinnest tiles along x are the most coherent
    X = _field(grid, (2,), seed=1)
    pick, scores = OT.choose_shape(X, X, grid, MENU)
    assert pick == 3
    assert scores[3] > scores[2] > scores[1] > scores[0]
    # depends on (t, y): tiles one frame deep and short along y win
    X = _field(grid, (0, 1), seed=2)
    pick, scores = OT.choose_shape(X, X, grid, MENU)
    assert pick == 0
    # queries and keys both count: keys coherent along x flip the choice
    # only when they outweigh the queries
    Q = _field(grid, (0,), seed=3)
    K = _field(grid, (2,), seed=4)
    pick, scores = OT.choose_shape(Q, K, grid, MENU)
    ref = [(OT.sics_score(Q, Q, grid, s) + OT.sics_score(K, K, grid, s)) / 2 for s in MENU]
    assert np.allclose(scores, ref)
    assert pick == int(np.argmax(ref))


class _WL:
    T, Hg, W, block = 3, 10, 13, 128
    tile_shapes = MENU
    scale = float(np.float32(1 / np.sqrt(16)))
    rule, mass, diag = "topk", 0.9, False

    def densities(self):
        return np.full(2, 0.25, np.float32)


def test_tiles_workload_head_layout_is_one_block_per_tile():
    wl = _WL()
    rng = np.random.default_rng(5)
    N = wl.T * wl.Hg * wl.W
    Q, K = rng.normal(size=(N, 16)), rng.normal(size=(N, 16))
    ref = OT.tiles_workload_head(wl, Q, K)
    C = OT.max_tiles((wl.T, wl.Hg, wl.W), MENU)
    a = OT.tile_assign(wl.T, wl.Hg, wl.W, MENU[ref["pick"]])
    nt = OT.n_tiles(wl.T, wl.Hg, wl.W, MENU[ref["pick"]])
    assert ref["q_order"].size == C * wl.block
    used = ref["q_blk"] >= 0
    assert used.sum() == nt
    # block j holds tile j (tiles in index order, each one block)
    assert np.array_equal(ref["q_blk"][:nt], np.arange(nt))
    assert np.array_equal(ref["q_cnt"][:nt], np.bincount(a, minlength=nt))
    for j in range(nt):
        toks = ref["q_order"][j * wl.block: (j + 1) * wl.block]
        assert np.array_equal(toks[toks >= 0], np.nonzero(a == j)[0])
    # the means are the tiles' exact means
    assert np.array_equal(ref["cq"], OC.cluster_means(Q, a, C))


def test_key_coherence_against_pairwise_cosines_and_limits():
    rng = np.random.default_rng(11)
    X = rng.normal(size=(40, 8))
    X[7] = 0.0                                        # a zero key: cosine 0 with everything
    a = rng.integers(0, 5, size=40)
    a[3] = 5                                          # tile 5 holds one token
    coh = OT.key_coherence(X, a, 7)
    for c in range(5):
        rows = X[a == c]
        n = len(rows)
        assert coh[c] == pytest.approx(_pairwise_cos_sum(rows) / (n * (n - 1)), rel=1e-12,
                                       abs=1e-12)
    assert coh[5] == 1.0 and coh[6] == 1.0            # one token, no token
    # identical keys agree fully; alternating antipodal pairs disagree fully
    same = np.tile(np.array([[0.5, -1.0, 2.0]]), (6, 1))
    assert OT.key_coherence(same, np.zeros(6, dtype=np.int64), 1)[0] == pytest.approx(1.0)
    alt = np.array([[1.0, 2.0], [-1.0, -2.0]])
    assert OT.key_coherence(alt, np.zeros(2, dtype=np.int64), 1)[0] == pytest.approx(-1.0)
    # a key and a zero key: the one pair has cosine 0
    half = np.array([[1.0, 2.0], [0.0, 0.0]])
    assert OT.key_coherence(half, np.zeros(2, dtype=np.int64), 1)[0] == 0.0


def _ticket_field(grid, noisy_tiles, shape, d=16, seed=0):
    """Keys constant within every tile of `shape` except the tiles listed,
    whose keys are independent noise; queries random."""
    T, Hg, W = grid
    rng = np.random.default_rng(seed)
    a = OT.tile_assign(T, Hg, W, shape)
    nt = OT.n_tiles(T, Hg, W, shape)
    base = rng.normal(size=(nt, d))
    K = base[a].copy()
    for t in noisy_tiles:
        K[a == t] = rng.normal(size=((a == t).sum(), d))
    return rng.normal(size=(T * Hg * W, d)), K


class _TicketWL(_WL):
    T, Hg, W, block = 2, 8, 16, 64
    tile_shapes = [(1, 4, 16)]
    scale = float(np.float32(1 / np.sqrt(16)))


@pytest.mark.parametrize("rule,diag", [("topk", False), ("mass", False), ("topk", True)])
def test_ticket_ignores_incoherent_tiles(rule, diag):
    grid = (2, 8, 16)
    noisy = [1, 2]
    Q, K = _ticket_field(grid, noisy, (1, 4, 16), seed=7)
    wl = _TicketWL()
    wl.rule, wl.diag, wl.mass = rule, diag, 0.95
    wl.densities = lambda: np.full(1, 0.2, np.float32)
    base = OT.tiles_workload_head(wl, Q, K)
    assert base["pick"] == 0
    assert np.all(base["eligible"])                   # no ticket: every tile
    wl.sics_ticket = 0.5
    ref = OT.tiles_workload_head(wl, Q, K)
    assert np.allclose(ref["coh"][[0, 3]], 1.0) and np.all(ref["coh"][noisy] < 0.2)
    assert np.array_equal(ref["eligible"], [True, False, False, True])
    keep = ref["keepC"]
    for a_ in range(4):
        for t in noisy:
            # a noisy tile is never kept, except as a row's own diagonal
            assert keep[a_, t] == (diag and a_ == t)
    # brute force: every row's selection equals the one made over the
    # admitted tiles alone (re-indexed), plus its own tile with the diagonal
    adm = [0, 3]
    S, nk = base["S"], base["nk"]
    for a_ in range(4):
        row = S[a_:a_ + 1][:, adm]
        want = OC.cluster_select(np.vstack([row, row]), nk[adm], Q.shape[0], rule,
                                 density=0.2, tau=0.95)[0]
        if diag and a_ in adm:
            want[adm.index(a_)] = True
        assert np.array_equal(keep[a_, adm], want), a_
    # a ticket of -1 admits every tile and leaves the selection as it was
    wl.sics_ticket = -1.0
    same = OT.tiles_workload_head(wl, Q, K)
    assert np.array_equal(same["keepC"], base["keepC"])


def test_ticket_admitting_nothing_keeps_nothing_but_the_diagonal():
    rng = np.random.default_rng(2)
    S = rng.normal(size=(4, 4)).astype(np.float32)
    nk = np.array([5, 5, 5, 0])
    none = np.zeros(4, dtype=bool)
    for rule in ("topk", "mass"):
        assert not OC.cluster_select(S, nk, 15, rule, density=0.5, tau=0.9,
                                     eligible=none).any()
        k = OC.cluster_select(S, nk, 15, rule, density=0.5, tau=0.9, diag=True, eligible=none)
        assert np.array_equal(k, np.diag([True, True, True, False]))
