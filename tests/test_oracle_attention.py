"""Pins of the oracle's block-sparse attention (float64).

What is pinned, and against what:
* every block kept -> dense softmax attention (torch's scaled_dot_product_
  attention in float64 on the CPU, a library routine) and torch.logsumexp;
* compensation with nothing skipped -> the same dense result;
* block-constant keys -> compensated output equals dense attention for any
  mask (the centroid replacement of the SVG-EAR page, section 2A, is exact
  when every key of a block equals the block mean);
* nothing kept, everything compensated -> dense attention over inputs whose
  keys and values are replaced by their block means (torch again);
* constant values -> output equals that value (a convex combination);
* the block-skipping loop -> the literal dense N x N softmax with a -inf mask;
* Hilbert reordering -> dense attention is unchanged (permutation equivariance);
* hand-computed closed forms under tests/golden/.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from conftest import golden


def _sdpa(Q, K, V, sigma):
    q = torch.from_numpy(Q)[None, None]
    k = torch.from_numpy(K)[None, None]
    v = torch.from_numpy(V)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=sigma)
    lse = torch.logsumexp(sigma * (q[0, 0] @ k[0, 0].T), dim=-1)
    return out[0, 0].numpy(), lse.numpy()


def _rand(N, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, d)) * scale, rng.standard_normal((N, d)) * scale,
            rng.standard_normal((N, d)))


@pytest.mark.parametrize("N,block,d", [(256, 64, 64), (390, 128, 32), (100, 64, 16)])
def test_full_mask_is_dense_attention(N, block, d):
    Q, K, V = _rand(N, d, N)
    nb = -(-N // block)
    sigma = 1 / math.sqrt(d)
    O, lse = oracle.attention_head(Q, K, V, np.ones((nb, nb), bool), block, sigma)
    Od, lsed = _sdpa(Q, K, V, sigma)
    np.testing.assert_allclose(O, Od, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lsed, atol=1e-12, rtol=0)


def test_compensation_with_nothing_skipped_is_dense():
    Q, K, V = _rand(390, 32, 1)
    nb = 4
    O, lse = oracle.attention_head(Q, K, V, np.ones((nb, nb), bool), 128, 0.2, comp=True)
    Od, lsed = _sdpa(Q, K, V, 0.2)
    np.testing.assert_allclose(O, Od, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_block_constant_keys_make_compensation_exact(seed):
    N, block, d = 330, 64, 16
    nb = -(-N // block)
    rng = np.random.default_rng(seed)
    Q, _, V = _rand(N, d, seed + 10)
    kb = rng.standard_normal((nb, d))
    K = kb[np.minimum(np.arange(N) // block, nb - 1)]
    keep = rng.random((nb, nb)) < 0.4
    O, lse = oracle.attention_head(Q, K, V, keep, block, 0.3, comp=True)
    Od, lsed = _sdpa(Q, K, V, 0.3)
    np.testing.assert_allclose(O, Od, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, atol=1e-12)


def test_nothing_kept_is_attention_over_centroids():
    N, block, d = 300, 64, 16
    nb = -(-N // block)
    Q, K, V = _rand(N, d, 5)
    blk = np.minimum(np.arange(N) // block, nb - 1)
    counts = np.bincount(blk)
    Kbar = np.stack([K[blk == j].mean(0) for j in range(nb)])[blk]
    Vbar = np.stack([V[blk == j].mean(0) for j in range(nb)])[blk]
    O, lse = oracle.attention_head(Q, K, V, np.zeros((nb, nb), bool), block, 0.25, comp=True)
    Od, lsed = _sdpa(Q, Kbar, Vbar, 0.25)
    np.testing.assert_allclose(O, Od, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, atol=1e-12)
    assert counts[-1] == 300 - 4 * 64


@pytest.mark.parametrize("comp", [False, True])
def test_constant_values_give_that_value(comp):
    N, block, d = 256, 64, 8
    nb = 4
    Q, K, _ = _rand(N, d, 3, scale=2.0)
    v = np.linspace(-1, 1, d)
    V = np.tile(v, (N, 1))
    keep = np.random.default_rng(3).random((nb, nb)) < 0.5
    keep[np.arange(nb), np.arange(nb)] = True
    O, _ = oracle.attention_head(Q, K, V, keep, block, 0.5, comp=comp)
    np.testing.assert_allclose(O, np.tile(v, (N, 1)), atol=1e-13)


def test_single_kept_block_is_softmax_over_that_block():
    N, block, d = 256, 64, 8
    Q, K, V = _rand(N, d, 4)
    keep = np.zeros((4, 4), bool)
    keep[:, 2] = True
    O, lse = oracle.attention_head(Q, K, V, keep, block, 0.5)
    Od, lsed = _sdpa(Q, K[128:192], V[128:192], 0.5)
    np.testing.assert_allclose(O, Od, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, atol=1e-12)


@pytest.mark.parametrize("comp", [False, True])
@pytest.mark.parametrize("N,block", [(256, 64), (1000, 128)])
def test_block_skipping_equals_dense_minus_inf(comp, N, block):
    Q, K, V = _rand(N, 16, N, scale=1.5)
    nb = -(-N // block)
    keep = np.random.default_rng(N).random((nb, nb)) < 0.35
    keep[0] = False                          # an empty row (compensation only)
    if not comp:
        keep[0, 0] = True
    O, lse = oracle.attention_head(Q, K, V, keep, block, 0.25, comp=comp)
    Od, lsed = oracle.dense_masked_attention_head(Q, K, V, keep, block, 0.25, comp=comp)
    np.testing.assert_allclose(O, Od, atol=1e-12)
    np.testing.assert_allclose(lse, lsed, atol=1e-12)


def test_empty_row_without_compensation():
    Q, K, V = _rand(128, 8, 0)
    keep = np.array([[False, True], [True, True]])
    O, lse = oracle.attention_head(Q, K, V, keep, 64, 0.5)
    keep[0, :] = False
    O, lse = oracle.attention_head(Q, K, V, keep, 64, 0.5)
    assert np.all(O[:64] == 0) and np.all(np.isneginf(lse[:64]))


def test_hilbert_order_is_equivariant_for_dense_attention():
    T, Hg, Wd = 3, 5, 7
    N, d = T * Hg * Wd, 16
    Q, K, V = _rand(N, d, 11)
    perm, _ = oracle.hilbert_perm(T, Hg, Wd)
    nb = -(-N // 16)
    full = np.ones((nb, nb), bool)
    Op, lsep = oracle.attention_head(oracle.permute_tokens(Q, perm),
                                     oracle.permute_tokens(K, perm),
                                     oracle.permute_tokens(V, perm), full, 16, 0.25)
    O = oracle.unpermute_tokens(Op, perm)
    Od, lsed = _sdpa(Q, K, V, 0.25)
    np.testing.assert_allclose(O, Od, atol=1e-12)
    np.testing.assert_allclose(lsep[np.argsort(perm)], lsed, atol=1e-12)


def test_closed_forms():
    rows = {r[0]: [float(x) for x in r[1:]] for r in golden("softmax_closed_forms.txt")}
    l3 = math.log(3.0)
    q = np.array([[1.0, 0.0], [1.0, 0.0]])
    K = np.array([[0.0, 0.0], [l3, 0.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0]])
    O, lse = oracle.attention_head(q, K, V, np.ones((1, 1), bool), 2, 1.0)
    np.testing.assert_allclose(O[0], rows["A"][:2], atol=1e-15)
    np.testing.assert_allclose(lse[0], rows["A"][2], atol=1e-15)
    O, lse = oracle.attention_head(q, K, V, np.zeros((1, 1), bool), 2, 1.0, comp=True)
    np.testing.assert_allclose(O[0], rows["B"][:2], atol=1e-15)
    np.testing.assert_allclose(lse[0], rows["B"][2], atol=1e-15)
    q4 = np.array([[1.0, 0.0]] * 4)
    K4 = np.array([[0.0, 0.0], [l3, 0.0], [0.0, 0.0], [0.0, 0.0]])
    V4 = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0], [-1.0, 1.0]])
    keep = np.array([[True, False], [True, False]])
    O, lse = oracle.attention_head(q4, K4, V4, keep, 2, 1.0, comp=True)
    np.testing.assert_allclose(O[0], rows["C"][:2], atol=1e-15)
    np.testing.assert_allclose(lse[0], rows["C"][2], atol=1e-15)


def test_kept_flops_counts_true_block_sizes():
    keep = np.ones((4, 4), bool)
    assert oracle.kept_flops(keep, 256, 64, 64) == 4 * 64 * 256 * 256
    keep = np.zeros((3, 3), bool)
    keep[2, 2] = True                         # 6-token last block of N = 134
    assert oracle.kept_flops(keep, 134, 64, 8) == 4 * 8 * 6 * 6


def test_pipeline_on_tiny_workload_runs():
    wl = W.WORKLOADS[1]
    Q, K, V = W.make_qkv(wl)
    keep, S = oracle.select_workload(wl, Q, K)
    assert keep.shape == (1, 2, 4, 4)
    assert np.all(keep.sum(-1) >= 2) and np.all(keep.sum(-1) <= 3)
    O, lse = oracle.attention_head(oracle.bf16_to_f64(Q[0, 0]), oracle.bf16_to_f64(K[0, 0]),
                                   oracle.bf16_to_f64(V[0, 0]), keep[0, 0], 64, wl.scale)
    assert np.all(np.isfinite(O))
