"""Pins of the oracle's error-aware routing key (SVG-EAR page, section 2B).

The key of (query block i, KV block j) is the log of the compensation error of
block j probed with query block i's mean, per unit of block size, on one scale
per row.  Pins: a hand-evaluated two-token case (tests/golden), the identity
with the attention oracle's compensation (for query blocks whose tokens are
equal, the mean *is* every query, so the error is exactly the change of the
softmax numerator when block j alone is replaced by its centroid), exact
scaling with V, invariance under token order inside a block, a vanishing error
for constant-key blocks, and the page's claim that routing by error lowers the
output error of compensated attention against routing by score at equal
density.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W
from conftest import golden


def _bf16(x):
    return oracle.bf16_to_f64(W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32).copy()))


def test_two_token_block_hand_values():
    for x, y, err, key in golden("error_routing_two_token.txt"):
        Q = np.array([[1.0], [1.0]])
        K = np.array([[0.0], [1.0]])
        V = np.array([[float(x)], [float(y)]])
        k = oracle.error_keys(Q, K, V, block=2, sigma=1.0)
        assert k.shape == (1, 1)
        assert k[0, 0] == pytest.approx(float(key), abs=2e-7)


def _numerator(O, lse):
    return O * np.exp(lse)[:, None]


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_error_is_the_numerator_change_of_compensating_one_block(seed):
    rng = np.random.default_rng(seed)
    block, nb, d, sigma = 4, 6, 8, 0.4
    N = block * nb - 1                                 # ragged last block
    Q = _bf16(np.repeat(rng.normal(size=(nb, d)), block, axis=0)[:N])
    K = _bf16(rng.normal(size=(N, d)))
    V = _bf16(rng.normal(size=(N, d)))
    keys = oracle.error_keys(Q, K, V, block, sigma)
    n = np.diff(oracle.block_bounds(N, block)).astype(np.float64)
    dense = np.ones((nb, nb), dtype=bool)
    Od, ld = oracle.attention_head(Q, K, V, dense, block, sigma)
    Nd = _numerator(Od, ld)
    b = oracle.block_bounds(N, block)
    for j in range(nb):
        keep = dense.copy()
        keep[:, j] = False
        Oc, lc = oracle.attention_head(Q, K, V, keep, block, sigma, comp=True)
        diff = np.linalg.norm(_numerator(Oc, lc) - Nd, axis=1)      # per query token
        for i in range(nb):
            want = diff[b[i]]                                        # any token of block i
            got = math.exp(keys[i, j] + math.log(n[j]))
            assert got == pytest.approx(want, rel=1e-5)


def test_scaling_values_shifts_keys_by_log_factor():
    rng = np.random.default_rng(3)
    Q, K, V = (_bf16(rng.normal(size=(40, 8))) for _ in range(3))
    a = oracle.error_keys(Q, K, V, 8, 0.35)
    b = oracle.error_keys(Q, K, 2.0 * V, 8, 0.35)
    assert np.allclose(b - a, math.log(2.0), atol=1e-12)


def test_token_order_inside_a_block_does_not_matter():
    rng = np.random.default_rng(4)
    Q, K, V = (_bf16(rng.normal(size=(32, 8))) for _ in range(3))
    perm = np.concatenate([rng.permutation(8) + 8 * j for j in range(4)])
    a = oracle.error_keys(Q, K, V, 8, 0.35)
    b = oracle.error_keys(Q, K[perm], V[perm], 8, 0.35)
    assert np.allclose(a, b, atol=1e-9)


def test_constant_key_block_has_no_error():
    rng = np.random.default_rng(5)
    Q = _bf16(rng.normal(size=(16, 8)))
    K = _bf16(np.repeat(rng.normal(size=(2, 8)), 8, axis=0))       # each block one key
    V = _bf16(rng.normal(size=(16, 8)))
    keys = oracle.error_keys(Q, K, V, 8, 0.35)
    # the centroid is exact up to the float32 rounding of its logit and of the
    # value sum: relative error below 1e-6 of the block's own contribution
    b = oracle.block_bounds(16, 8)
    for j in range(2):
        a_norm = np.linalg.norm(V[b[j]:b[j + 1]].sum(axis=0))
        assert np.all(np.exp(keys[:, j] + math.log(8)) <= 1e-6 * a_norm)


def test_routing_by_error_beats_routing_by_score():
    """SVG-EAR 2B / 4: at equal density, compensated attention with blocks kept
    by error is closer to dense attention than with blocks kept by score."""
    wl = W.WORKLOADS[2].replace(T=3, Hg=10, W=26, H=4, block=64, rule="topk", density=0.2)
    Q, K, V = W.make_qkv(wl)
    n_better = 0
    for h in range(wl.H):
        q, k, v = (oracle.bf16_to_f64(x[0, h]) for x in (Q, K, V))
        kk = oracle.head_k(wl, h)
        common = dict(N=wl.N, block=wl.block, HgW=wl.Hg * wl.W, sigma=wl.scale, k=kk)
        keep_s, _ = oracle.select_head(q, k, rule="topk", **common)
        keep_e, _ = oracle.select_head(q, k, rule="err", Vh=v, **common)
        assert keep_s.sum() == keep_e.sum()
        dense, _ = oracle.attention_head(q, k, v, np.ones_like(keep_s), wl.block, wl.scale)
        Os, _ = oracle.attention_head(q, k, v, keep_s, wl.block, wl.scale, comp=True)
        Oe, _ = oracle.attention_head(q, k, v, keep_e, wl.block, wl.scale, comp=True)
        mse_s = float(((Os - dense) ** 2).mean())
        mse_e = float(((Oe - dense) ** 2).mean())
        assert (keep_s != keep_e).any()                 # the two rules do differ
        n_better += mse_e < mse_s
    assert n_better == wl.H
