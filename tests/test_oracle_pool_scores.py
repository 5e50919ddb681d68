"""Pins of the oracle's block means and pooled scores.

Block means: the DFSAttn page (trick 2) and the SVG-EAR page (section 2A)
summarise a block by its mean ("media", the centroid).  Scores: the block
score is the scaled dot product of the means.  The pins below compare the
oracle with exact rational arithmetic and with special cases, never with a
retyped copy of its own formula.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as W


def _round_f32(x: Fraction) -> Fraction:
    """Exact round-to-nearest-even of a rational to IEEE binary32."""
    if x == 0:
        return Fraction(0)
    neg = x < 0
    a = -x if neg else x
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e - 23, -149)
    scaled = a / Fraction(2) ** q
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * Fraction(2) ** q
    return -r if neg else r


def _exact_fma_chain(a, b):
    acc = Fraction(0)
    for x, y in zip(a, b):
        acc = _round_f32(Fraction(float(x)) * Fraction(float(y)) + acc)
    return acc


@pytest.mark.parametrize("d", [1, 8, 64, 128])
def test_seqfma_dot_matches_exact_rounding_chain(d):
    rng = np.random.default_rng(d)
    for trial in range(12):
        scale = np.float32(10.0) ** rng.integers(-3, 4, size=d).astype(np.float32)
        a = (rng.standard_normal(d) * scale).astype(np.float32)
        b = (rng.standard_normal(d) * scale[::-1]).astype(np.float32)
        if trial % 3 == 0:          # heavy cancellation
            b[: d // 2] = -a[: d // 2]
        got = oracle.seqfma_dot(a, b)
        assert Fraction(got) == _exact_fma_chain(a, b)


def test_block_scores_layout_and_scale():
    rng = np.random.default_rng(1)
    qm = rng.standard_normal((5, 64)).astype(np.float32)
    km = rng.standard_normal((7, 64)).astype(np.float32)
    sigma = float(np.float32(1 / 8))
    S = oracle.block_scores(qm, km, sigma)
    assert S.shape == (5, 7) and S.dtype == np.float32
    for i in range(5):
        for j in range(7):
            want = _round_f32(Fraction(sigma) * _exact_fma_chain(qm[i], km[j]))
            assert Fraction(float(S[i, j])) == want


def test_constant_vectors_closed_form():
    # q = 0.5 * ones, k = 0.25 * ones, d = 128: every partial sum is exact,
    # dot = 16, scaled by 1/8 -> 2
    qm = np.full((1, 128), 0.5, np.float32)
    km = np.full((1, 128), 0.25, np.float32)
    assert oracle.block_scores(qm, km, 0.125)[0, 0] == np.float32(2.0)


@pytest.mark.parametrize("N,block", [(56, 64), (80, 128), (120, 128), (248, 128),
                                     (32760, 64)])
def test_constant_block_mean_is_exact(N, block):
    rng = np.random.default_rng(N)
    nb = -(-N // block)
    vals = W.bf16_bits_to_f32(W.f32_to_bf16_bits(
        rng.standard_normal((nb, 4)).astype(np.float32) * 3)).astype(np.float64)
    blk = np.minimum(np.arange(N) // block, nb - 1)
    X = vals[blk]                                     # block-constant
    m = oracle.block_means(X, block)
    assert np.array_equal(m.astype(np.float64), vals)


def test_block_sums_exact_and_mean_uses_true_count():
    rng = np.random.default_rng(7)
    N, block, d = 390, 128, 16                       # last block: 6 tokens
    X = W.bf16_bits_to_f32(W.f32_to_bf16_bits(
        rng.standard_normal((N, d)).astype(np.float32))).astype(np.float64)
    S = oracle.block_sums_f64(X, block)
    M = oracle.block_means(X, block)
    bounds = [0, 128, 256, 384, 390]
    for i in range(4):
        for c in range(d):
            exact = sum(Fraction(float(v)) for v in X[bounds[i]:bounds[i + 1], c])
            assert Fraction(float(S[i, c])) == exact
            n = bounds[i + 1] - bounds[i]
            err = abs(Fraction(float(M[i, c])) - exact / n)
            ulp = Fraction(float(np.spacing(np.float32(abs(M[i, c])))))
            assert err <= ulp / 2 + ulp / 2 ** 20


def _brute_subblock_max(Qh, Kh, block, sub, sigma):
    N = Qh.shape[0]
    nb = -(-N // block)
    qs = oracle.block_means(Qh, sub)
    ks = oracle.block_means(Kh, sub)
    out = np.empty((nb, nb), np.float32)
    for i in range(nb):
        a_sub = [a for a in range(i * block // sub, (i + 1) * block // sub) if a * sub < N]
        for j in range(nb):
            b_sub = [b for b in range(j * block // sub, (j + 1) * block // sub) if b * sub < N]
            best = -np.inf
            for a in a_sub:
                for b in b_sub:
                    s = np.float32(sigma) * np.float32(oracle.seqfma_dot(qs[a], ks[b]))
                    best = max(best, float(s))
            out[i, j] = best
    return out


@pytest.mark.parametrize("N,block,sub", [(100, 32, 8), (256, 64, 16), (200, 64, 16)])
def test_subblock_max_matches_brute_force(N, block, sub):
    rng = np.random.default_rng(N + sub)
    Qh = rng.standard_normal((N, 16))
    Kh = rng.standard_normal((N, 16))
    sigma = 0.25
    got = oracle.subblock_max_scores(Qh, Kh, block, sub, sigma)
    assert np.array_equal(got, _brute_subblock_max(Qh, Kh, block, sub, sigma))


def test_subblock_equal_to_block_reduces_to_block_scores():
    rng = np.random.default_rng(3)
    Qh = rng.standard_normal((300, 32))
    Kh = rng.standard_normal((300, 32))
    a = oracle.subblock_max_scores(Qh, Kh, 64, 64, 0.5)
    b = oracle.block_scores(oracle.block_means(Qh, 64), oracle.block_means(Kh, 64), 0.5)
    assert np.array_equal(a, b)


def test_subblock_mean_mode_is_block_mean_pooling():
    """The page's "sum of sub-block scores" equals block-mean pooling (up to
    rounding); the max of sub-pairs is never below their average."""
    rng = np.random.default_rng(4)
    Qh = rng.standard_normal((256, 32))
    Kh = rng.standard_normal((256, 32))
    mean_mode = oracle.subblock_max_scores(Qh, Kh, 64, 16, 0.5, mode="mean")
    blk = oracle.block_scores(oracle.block_means(Qh, 64), oracle.block_means(Kh, 64), 0.5)
    np.testing.assert_allclose(mean_mode, blk, rtol=1e-5, atol=1e-6)
    mx = oracle.subblock_max_scores(Qh, Kh, 64, 16, 0.5)
    assert np.all(mx >= mean_mode - 1e-6)
