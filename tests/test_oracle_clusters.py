"""Pins of the oracle's data-dependent block formation (SVOO 2B co-clustering,
SVG-EAR 2A k-means, the padded cluster layout, cluster-level selection and
attention) against brute force, planted structure and dense restatements."""
import numpy as np
import pytest

import oracle
from oracle import clusters as OC


def _bf16(x):
    """Round float64 data to bf16 values (as the inputs are), returned as float64."""
    import workloads as W
    return oracle.bf16_to_f64(W.f32_to_bf16_bits(np.asarray(x, np.float32)))


def test_chunk_bounds_and_initial_centroids():
    b = OC.chunk_bounds(390, 7)
    assert b[0] == 0 and b[-1] == 390 and np.all(np.diff(b) >= 55) and np.all(np.diff(b) <= 56)
    rng = np.random.default_rng(0)
    X = _bf16(rng.normal(size=(390, 8)))
    c1 = OC.initial_centroids(X, 1)
    assert np.array_equal(c1[0], (X.sum(axis=0) / 390).astype(np.float32))
    c7 = OC.initial_centroids(X, 7)
    for c in range(7):
        assert np.array_equal(c7[c], (X[b[c]:b[c + 1]].sum(axis=0) / (b[c + 1] - b[c])).astype(np.float32))


def test_cluster_means_exact_and_empty_keeps_previous():
    X = np.array([[1.0, 2.0], [3.0, 5.0], [-1.0, 0.5]])
    a = np.array([0, 0, 2])
    prev = np.array([[9, 9], [7, 7], [8, 8]], np.float32)
    m = OC.cluster_means(X, a, 3, prev=prev)
    assert np.array_equal(m, np.array([[2.0, 3.5], [7, 7], [-1.0, 0.5]], np.float32))


def test_assignment_is_the_nearest_centroid_up_to_fp32_ties():
    rng = np.random.default_rng(1)
    X = _bf16(rng.normal(size=(600, 32)))
    cent = rng.normal(size=(9, 32)).astype(np.float32)
    a = OC.assign_tokens(X, cent, kmeans=True)
    d2 = ((X[:, None, :] - cent.astype(np.float64)[None]) ** 2).sum(-1)      # float64
    best = d2.min(axis=1)
    # the chosen centroid is the nearest one, or within fp32 rounding of it
    assert np.all(d2[np.arange(600), a] - best <= 1e-4 * (1 + best))
    assert np.mean(a == d2.argmin(axis=1)) > 0.99
    aff = OC.assign_tokens(X, cent, kmeans=False)
    dots = X @ cent.astype(np.float64).T
    assert np.all(dots.max(axis=1) - dots[np.arange(600), aff] <= 1e-4 * (1 + np.abs(dots).max(axis=1)))


def test_assignment_ties_go_to_the_lower_index():
    X = np.ones((3, 4))
    cent = np.ones((3, 4), np.float32)
    assert np.array_equal(OC.assign_tokens(X, cent, kmeans=False), [0, 0, 0])
    assert np.array_equal(OC.assign_tokens(X, cent, kmeans=True), [0, 0, 0])


def _planted(rng, sizes, d, sep=8.0, noise=0.3):
    """Tokens of len(sizes) groups in raster order, group g around sep * e_g."""
    X = []
    for g, n in enumerate(sizes):
        c = np.zeros(d); c[g] = sep
        X.append(c + noise * rng.normal(size=(n, d)))
    return _bf16(np.concatenate(X))


def _labels_match(a, truth):
    """a is truth up to a relabelling (a bijection between used labels)."""
    pairs = set(zip(a.tolist(), truth.tolist()))
    return len(pairs) == len(set(a.tolist())) == len(set(truth.tolist()))


def test_kmeans_moves_chunk_boundaries_onto_planted_groups():
    rng = np.random.default_rng(2)
    # groups do not align with the equal chunks of the initial partition, but
    # each chunk is dominated by a different group (Lloyd from that start
    # reaches the planted partition; from a start that merges groups it would not)
    sizes = [55, 75, 60, 80, 60]
    X = _planted(rng, sizes, 16)
    truth = np.repeat(np.arange(5), sizes)
    aq, ak, cq, ck = OC.kmeans_head(X, X, 5, iters=8)
    assert _labels_match(aq, truth) and np.array_equal(aq, ak)
    # Lloyd: the objective never increases
    c = OC.initial_centroids(X, 5)
    obj = []
    for _ in range(6):
        a = OC.assign_tokens(X, c, kmeans=True)
        obj.append(((X - c.astype(np.float64)[a]) ** 2).sum())
        c = OC.cluster_means(X, a, 5, prev=c)
    assert all(obj[i + 1] <= obj[i] * (1 + 1e-9) for i in range(len(obj) - 1))


def test_coclustering_pairs_query_and_key_groups():
    rng = np.random.default_rng(3)
    sizes_q = [60, 25, 100, 45]
    sizes_k = [30, 80, 50, 70]
    Q = _planted(rng, sizes_q, 12)
    K = _planted(rng, sizes_k, 12)
    aq, ak, cq, ck = OC.cocluster_head(Q, K, 4, iters=5)
    tq = np.repeat(np.arange(4), sizes_q)
    tk = np.repeat(np.arange(4), sizes_k)
    assert _labels_match(aq, tq) and _labels_match(ak, tk)
    # key cluster c is the partner of query cluster c: the same planted group
    for c in range(4):
        gq = set(tq[aq == c].tolist())
        gk = set(tk[ak == c].tolist())
        assert gq == gk and len(gq) == 1


def test_layout_is_a_stable_padded_bijection():
    rng = np.random.default_rng(4)
    a = rng.integers(0, 6, size=390)
    a[a == 4] = 5                                   # cluster 4 empty
    order, bc, cnt = OC.cluster_layout(a, 6, 64)
    assert order.size == OC.padded_blocks(390, 64, 6) * 64
    valid = order[order >= 0]
    assert np.array_equal(np.sort(valid), np.arange(390))
    for c in range(6):
        blocks = np.nonzero(bc == c)[0]
        n = int((a == c).sum())
        assert blocks.size == -(-n // 64)
        if blocks.size:
            assert np.array_equal(blocks, np.arange(blocks[0], blocks[0] + blocks.size))
            toks = order[blocks[0] * 64: blocks[0] * 64 + n]
            assert np.array_equal(toks, np.nonzero(a == c)[0])     # ascending
            assert cnt[blocks].sum() == n and np.all(cnt[blocks[:-1]] == 64)
    assert np.all(cnt[bc < 0] == 0)
    assert np.all(order.reshape(-1, 64)[bc < 0] == -1)


def _brute_prefix(S_row, nk, weight, target):
    """Smallest prefix of the ranking (S desc, index asc) over live clusters
    whose weight reaches target, checked against every prefix length."""
    live = [b for b in range(S_row.size) if nk[b] > 0]
    ranked = sorted(live, key=lambda b: (-float(S_row[b]), b))
    for m in range(1, len(ranked) + 1):
        if sum(weight[b] for b in ranked[:m]) >= target:
            return set(ranked[:m])
    return set(ranked)


@pytest.mark.parametrize("seed", range(6))
def test_cluster_selection_brute_force(seed):
    rng = np.random.default_rng(seed)
    C, N = 7, 500
    S = rng.normal(size=(C, C)).astype(np.float32)
    S[0, 3] = S[0, 5]                               # a tie
    nk = rng.integers(0, 150, size=C)
    nk[2] = 0                                       # an empty key cluster
    for dens in (0.05, 0.3, 0.9):
        keep = OC.cluster_select(S, nk, N, "topk", density=dens)
        budget = max(1, int(np.ceil(float(np.float32(dens)) * N * (1 - 1e-6))))
        for a in range(C):
            want = _brute_prefix(S[a], nk, nk, budget)
            assert set(np.nonzero(keep[a])[0].tolist()) == want
    for tau in (0.5, 0.9, 1.0):
        keep = OC.cluster_select(S, nk, N, "mass", tau=tau, diag=True)
        for a in range(C):
            live = nk > 0
            smax = S[a][live].max()
            w = {b: nk[b] * np.exp(float(S[a, b]) - float(smax)) for b in range(C)}
            target = float(np.float32(tau)) * sum(w[b] for b in range(C) if nk[b] > 0)
            want = _brute_prefix(S[a], nk, w, target * (1 - 1e-12))
            if nk[a] > 0:
                want.add(a)
            assert set(np.nonzero(keep[a])[0].tolist()) == want
            assert not keep[a, 2]


def test_block_keep_expands_cluster_keep():
    keepC = np.array([[True, False], [False, True]])
    qblk = np.array([0, 0, 1, -1])
    kblk = np.array([1, 0, 0, -1])
    keep = OC.cluster_block_keep(keepC, qblk, kblk)
    assert np.array_equal(keep, [[0, 1, 1, 0], [0, 1, 1, 0], [1, 0, 0, 0], [0, 0, 0, 0]])


def _dense_token_mask_attention(Q, K, V, aq, ak, keepC, sigma, comp):
    """The same attention as one dense softmax: -inf bias on keys of unkept
    clusters, plus one centroid column per cluster (masked where kept)."""
    C = keepC.shape[0]
    M = keepC[aq][:, ak]                                       # [N, N]
    L = np.where(M, sigma * (Q @ K.T), -np.inf)
    Vv = V
    if comp:
        n = np.bincount(ak, minlength=C).astype(np.float64)
        kb = np.stack([K[ak == c].mean(axis=0) if n[c] else np.zeros(K.shape[1]) for c in range(C)])
        vb = np.stack([V[ak == c].mean(axis=0) if n[c] else np.zeros(V.shape[1]) for c in range(C)])
        with np.errstate(divide="ignore"):
            Lc = sigma * (Q @ kb.T) + np.log(n)[None, :]
        Lc = np.where(keepC[aq] | (n == 0)[None, :], -np.inf, Lc)
        L = np.concatenate([L, Lc], axis=1)
        Vv = np.concatenate([V, vb])
    m = L.max(axis=1, keepdims=True)
    e = np.exp(L - m)
    return (e @ Vv) / e.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("comp", [False, True])
def test_cluster_attention_equals_dense_token_mask(comp):
    rng = np.random.default_rng(5)
    N, d, C = 150, 16, 5
    Q, K, V = (_bf16(rng.normal(size=(N, d))) for _ in range(3))
    aq = rng.integers(0, C, size=N)
    ak = rng.integers(0, C, size=N)
    ak[ak == 3] = 1                                           # empty key cluster 3
    keepC = rng.random((C, C)) < 0.4
    keepC[:, 0] = True                                        # every row attends somewhere
    O, lse = OC.cluster_attention_head(Q, K, V, aq, ak, keepC, 0.25, comp=comp)
    ref = _dense_token_mask_attention(Q, K, V, aq, ak, keepC, 0.25, comp)
    assert np.allclose(O, ref, rtol=1e-12, atol=1e-12)


def test_cluster_attention_limits():
    rng = np.random.default_rng(6)
    N, d, C = 120, 8, 4
    Q, K, V = (_bf16(rng.normal(size=(N, d))) for _ in range(3))
    aq = rng.integers(0, C, size=N)
    ak = rng.integers(0, C, size=N)
    dense = oracle.attention_head(Q, K, V, np.ones((1, 1), bool), N, 0.3)[0]
    full = np.ones((C, C), bool)
    for comp in (False, True):       # nothing skipped: dense attention
        O, _ = OC.cluster_attention_head(Q, K, V, aq, ak, full, 0.3, comp=comp)
        assert np.allclose(O, dense, rtol=1e-12, atol=1e-12)
    # every key cluster made of one repeated key: compensation is exact
    Kc = rng.normal(size=(C, d))[ak]
    dense_c = oracle.attention_head(Q, Kc, V, np.ones((1, 1), bool), N, 0.3)[0]
    keepC = rng.random((C, C)) < 0.5
    O, _ = OC.cluster_attention_head(Q, Kc, V, aq, ak, keepC, 0.3, comp=True)
    assert np.allclose(O, dense_c, rtol=1e-10, atol=1e-10)
