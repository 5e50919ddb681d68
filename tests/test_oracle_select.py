"""Pins of the oracle's block selection.

Rules (all per query block and per head, as the SPADE page, part 2 decides
per head):
* top-k under a fixed density budget (SVG-EAR page, section 2B);
* the smallest set reaching a share of the cumulative attention mass
  (SVG-EAR page, section 4 "top-p"; SVOO page, section 2A);
* a structured window plus rotating global anchors (LVSA abstract).

The pins are brute force over all subsets, the limit cases of the rules,
monotonicity, ties, and a token-level restatement of the window rule.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from conftest import golden


def _brute_topk(s, k):
    """Max-sum k-subset; among equal sums the lexicographically smallest."""
    best = None
    for sub in itertools.combinations(range(len(s)), k):
        key = (-sum(float(s[j]) for j in sub), sub)
        if best is None or key < best:
            best = key
    return set(best[1])


def _brute_mass(s, tau):
    """Minimal-cardinality subset reaching tau of the total mass; among those
    the largest mass, then the lexicographically smallest."""
    p = np.exp(s.astype(np.float64) - float(s.max()))
    Z = math.fsum(p)
    thr = float(np.float32(tau)) * Z
    for m in range(1, len(s) + 1):
        cands = []
        for sub in itertools.combinations(range(len(s)), m):
            mass = math.fsum(p[list(sub)])
            if mass >= thr:
                cands.append((-mass, sub))
        if cands:
            return set(min(cands)[1])
    raise AssertionError


def _row_sets(keep):
    return [set(np.nonzero(r)[0]) for r in keep]


@pytest.mark.parametrize("nb", [1, 2, 5, 9, 12])
def test_topk_matches_brute_force(nb):
    rng = np.random.default_rng(nb)
    S = rng.standard_normal((6, nb)).astype(np.float32)
    S[0, :] = 0.0                                     # all tied
    if nb > 3:
        S[1, 1] = S[1, 3] = S[1].max()                # tie at the top
        S[2, 0] = -0.0
        S[2, 2] = 0.0                                 # signed zeros tie
    for k in range(1, nb + 1):
        got = _row_sets(oracle.topk_keep(S, k))
        for r in range(S.shape[0]):
            assert got[r] == _brute_topk(S[r], k), (r, k)


@pytest.mark.parametrize("nb", [1, 3, 7, 11])
@pytest.mark.parametrize("tau", [0.5, 0.9, 0.95, 1.0])
def test_mass_matches_brute_force(nb, tau):
    rng = np.random.default_rng(100 + nb)
    S = (rng.standard_normal((5, nb)) * rng.uniform(0.5, 4.0, size=(5, 1))).astype(np.float32)
    got = _row_sets(oracle.mass_keep(S, tau))
    for r in range(S.shape[0]):
        want = _brute_mass(S[r], tau)
        assert len(got[r]) == len(want)
        assert got[r] == want


def test_full_budget_keeps_everything():
    rng = np.random.default_rng(5)
    S = rng.standard_normal((8, 10)).astype(np.float32) * 5
    assert oracle.topk_keep(S, 10).all()
    assert oracle.mass_keep(S, 1.0).all()
    assert oracle.k_from_density(1.0, 10) == 10


def test_masks_are_nested():
    rng = np.random.default_rng(6)
    S = rng.standard_normal((16, 24)).astype(np.float32) * 3
    prev = np.zeros_like(S, dtype=bool)
    for k in range(1, 25):
        cur = oracle.topk_keep(S, k)
        assert np.all(cur >= prev) and np.all(cur.sum(1) == k)
        prev = cur
    prev = np.zeros_like(S, dtype=bool)
    for tau in np.linspace(0.05, 1.0, 20):
        cur = oracle.mass_keep(S, tau)
        assert np.all(cur >= prev)
        prev = cur


def test_zero_scores_tie_break_and_mass_count():
    # Q = 0 gives every pooled score 0: ties broken by lower block index, and
    # the mass rule needs ceil(tau*nb) equal blocks (tau a float32)
    nb = 20
    Qh = np.zeros((nb * 64, 64))
    Kh = np.random.default_rng(0).standard_normal((nb * 64, 64))
    keep, S = oracle.select_head(Qh, Kh, N=nb * 64, block=64, HgW=64, sigma=0.125,
                                 rule="topk", k=7)
    assert np.all(S == 0)
    assert all(s == set(range(7)) for s in _row_sets(keep))
    keep, _ = oracle.select_head(Qh, Kh, N=nb * 64, block=64, HgW=64, sigma=0.125,
                                 rule="mass", tau=0.9)
    m = math.ceil(float(np.float32(0.9)) * nb)
    assert all(s == set(range(m)) for s in _row_sets(keep))


def test_k_from_density_golden():
    rows = {r[0]: r for r in golden("block_geometry.txt")}
    nb = int(rows["wan14b_720p"][6])
    assert oracle.k_from_density(0.15, nb) == int(rows["wan14b_720p"][8])
    assert oracle.k_from_density(0.15, 600) == 90      # 90.000001 must not round up
    assert oracle.k_from_density(0.0, 100) == 1
    assert oracle.k_from_density(0.05, 512) == 26
    assert oracle.k_from_density(0.5, 512) == 256


def test_window_matches_token_level_definition():
    """Block j is in block i's window iff some token of j lies within r latent
    frames of some token of i."""
    for (T, Hg, W, block, r) in [(6, 5, 7, 16, 1), (126, 30, 52, 128, 1),
                                 (9, 3, 3, 4, 0), (5, 4, 4, 64, 2)]:
        N, HgW = T * Hg * W, Hg * W
        nb = -(-N // block)
        frame = np.arange(N) // HgW
        if nb > 200:                      # sample rows of the long grid
            rows = np.random.default_rng(0).choice(nb, 40, replace=False)
        else:
            rows = np.arange(nb)
        got = oracle.window_keep(N, block, HgW, r)
        for i in rows:
            fi = frame[i * block: min(N, (i + 1) * block)]
            for j in range(nb):
                fj = frame[j * block: min(N, (j + 1) * block)]
                near = (np.abs(fi[:, None] - fj[None, :]) <= r).any()
                assert got[i, j] == near, (T, Hg, W, i, j)


def test_window_and_anchor_density_of_long_horizon_grid():
    N, block, HgW = 196560, 128, 1560
    nb = N // block + 1
    win = oracle.window_keep(N, block, HgW, 1)
    assert win.shape == (nb, nb) and np.all(np.diag(win))
    assert np.array_equal(win, win.T)                   # non-causal, symmetric
    assert 0.02 < win.mean() < 0.03
    anchors = oracle.anchor_blocks(nb, 4, 1000)
    assert list(anchors) == [1000, 1384, 232, 616]      # (1000 + m*384) mod 1536


def test_anchor_rotation():
    for nb, A in [(10, 3), (1536, 4), (7, 7), (5, 8)]:
        for off in (0, 3, 123456789):
            a = oracle.anchor_blocks(nb, A, off)
            assert len(a) == A
            assert a[0] == off % nb
            assert all(0 <= x < nb for x in a)
            step = nb // A
            assert all((a[m] - a[0]) % nb == (m * step) % nb for m in range(A))


def test_csr_round_trip_and_ascending():
    rng = np.random.default_rng(9)
    keep = rng.random((30, 17)) < 0.3
    keep[3] = False
    row_ptr, col_idx = oracle.keep_to_csr(keep)
    assert row_ptr[0] == 0 and row_ptr[-1] == keep.sum()
    back = np.zeros_like(keep)
    for r in range(30):
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        assert np.all(np.diff(cols) > 0)
        back[r, cols] = True
    assert np.array_equal(back, keep)


def test_tiny_selection_keeps_topk_union_diagonal():
    import workloads as W
    wl = W.WORKLOADS[1]
    Q, K, V = W.make_qkv(wl)
    keep, S = oracle.select_workload(wl, Q, K)
    for h in range(wl.H):
        for i in range(wl.nb):
            top = _brute_topk(S[0, h, i], 2)
            assert set(np.nonzero(keep[0, h, i])[0]) == top | {i}
