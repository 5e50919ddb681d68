"""Oracle, data-dependent block formation -- TEST INFRASTRUCTURE ONLY.

Plain CPU restatement of how the pages form attention blocks from the
content of Q and K instead of from token positions.  Only the tests, the
package smoke check and the benchmark's CPU-baseline leg may import it.

Sources:

* "SVOO: Training-Free Sparse Attention ... Online Bidirectional
  Co-Clustering" -- section 2B: keys are grouped by their affinity to the
  current query centroids, then queries by their affinity to the updated key
  centroids, alternately; the partitions are reused for several steps.
* "SVG-EAR: Parameter-Free Linear Compensation ..." -- section 2A: queries and
  keys are grouped with k-means and permuted so that every cluster is
  contiguous; a skipped cluster is replaced by its centroid.

Readings (the pages leave these open; each is stated where it is used):

* affinity = dot product of a token with a centroid; k-means distance =
  squared Euclidean distance, i.e. the largest x.c - |c|^2 / 2;
* initial centroids = means of C equal chunks of the raster token order
  (the partition a fixed block layout would give), ties go to the lower
  cluster index, an empty cluster keeps its previous centroid;
* a cluster occupies whole attention blocks of the padded layout: its
  tokens, in ascending token order, then zero padding up to a multiple of
  the block size; the layout has ceil(N / block) + C blocks (an upper bound
  for every head) and the blocks past the last cluster are empty;
* selection over clusters: pooled scores of the centroids; a budget of
  ``density * N`` key tokens (shortest prefix of the ranked clusters whose
  token count reaches it) or a cumulative mass where a cluster of n tokens
  weighs n exp(S); the kept clusters of a query cluster are kept for every
  block of it.

Arithmetic that decides an integer (an assignment, the ranking) is the
one both sides share: float32 dot products as sequential fused
multiply-add chains (``oracle_scores.c``), k-means bias fl32(-0.5 * |c|^2)
added in float32, exact float64 sums rounded once for the means.
Attention is float64.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import block_scores, seqfma_dot


def chunk_bounds(N: int, C: int) -> np.ndarray:
    """Token bounds of C equal chunks of the raster order: floor(c N / C)."""
    return (np.arange(C + 1, dtype=np.int64) * N) // C


def cluster_means(X: np.ndarray, assign: np.ndarray, C: int,
                  prev: Optional[np.ndarray] = None) -> np.ndarray:
    """fp32 means of the tokens of each cluster: fl32(exact sum / n_c).

    X: float64 [N, d] (exact widening of bf16).  Sums of bf16 values are exact
    in float64 as long as their significands span fewer than 53 bits, so the
    order of the additions does not matter.  An empty cluster keeps ``prev``
    (zeros when none is given).
    """
    d = X.shape[1]
    sums = np.zeros((C, d), dtype=np.float64)
    np.add.at(sums, assign, X)
    n = np.bincount(assign, minlength=C).astype(np.float64)
    out = np.zeros((C, d), dtype=np.float32) if prev is None else np.array(prev, np.float32)
    nz = n > 0
    out[nz] = (sums[nz] / n[nz, None]).astype(np.float32)
    return out


def assign_tokens(X: np.ndarray, cent: np.ndarray, kmeans: bool) -> np.ndarray:
    """Cluster of every token: the largest score, the lowest index on ties.

    score(x, c) = seqfma(x, c)                       (affinity, co-clustering)
                = fl32(seqfma(x, c) + fl32(-0.5 * seqfma(c, c)))   (k-means)
    """
    X32 = np.ascontiguousarray(X, dtype=np.float32)
    c32 = np.ascontiguousarray(cent, dtype=np.float32)
    s = block_scores(X32, c32, 1.0)                           # [N, C] fp32
    if kmeans:
        bias = np.array([np.float32(-0.5) * np.float32(seqfma_dot(c, c)) for c in c32],
                        dtype=np.float32)
        s = (s + bias[None, :]).astype(np.float32)
    return np.argmax(s, axis=1).astype(np.int64)


def initial_centroids(X: np.ndarray, C: int) -> np.ndarray:
    b = chunk_bounds(X.shape[0], C)
    assign = np.repeat(np.arange(C), np.diff(b))
    return cluster_means(X, assign, C)


def cocluster_head(Qh: np.ndarray, Kh: np.ndarray, C: int, iters: int):
    """SVOO bidirectional co-clustering of one head (section 2B).

    Each round: keys go to the query centroid they are most affine to and the
    key centroids are updated; then queries go to the key centroid they are
    most affine to and the query centroids are updated.  Key cluster c is the
    partner of query cluster c.  Returns (query clusters, key clusters,
    query centroids, key centroids).
    """
    cq = initial_centroids(Qh, C)
    ck = initial_centroids(Kh, C)
    aq = ak = None
    for _ in range(iters):
        ak = assign_tokens(Kh, cq, kmeans=False)
        ck = cluster_means(Kh, ak, C, prev=ck)
        aq = assign_tokens(Qh, ck, kmeans=False)
        cq = cluster_means(Qh, aq, C, prev=cq)
    return aq, ak, cq, ck


def kmeans_head(Qh: np.ndarray, Kh: np.ndarray, C: int, iters: int):
    """SVG-EAR semantic k-means of one head (section 2A): Lloyd's iterations
    on Q and on K separately.  Returns (aq, ak, cq, ck) as cocluster_head."""
    out = []
    for X in (Qh, Kh):
        c = initial_centroids(X, C)
        a = None
        for _ in range(iters):
            a = assign_tokens(X, c, kmeans=True)
            c = cluster_means(X, a, C, prev=c)
        out.append((a, c))
    (aq, cq), (ak, ck) = out
    return aq, ak, cq, ck


def padded_blocks(N: int, block: int, C: int) -> int:
    """Blocks of the padded clustered layout (an upper bound for any head)."""
    return -(-N // block) + C


def cluster_layout(assign: np.ndarray, C: int, block: int, nbp: int = None):
    """Padded layout of one side of one head.

    Returns (order, blk_cluster, blk_count): order[p] = token at slot p or -1
    (padding), for nbp * block slots; blk_cluster[j] = cluster of block j or -1;
    blk_count[j] = tokens (not padding) in block j.  ``nbp`` defaults to the
    bound ceil(N / block) + C; clusters of at most ``block`` tokens each fit in
    nbp = C blocks.
    """
    N = assign.size
    if nbp is None:
        nbp = padded_blocks(N, block, C)
    n = np.bincount(assign, minlength=C)
    nblk = -(-n // block)
    order = np.full(nbp * block, -1, dtype=np.int64)
    blk_cluster = np.full(nbp, -1, dtype=np.int64)
    blk_count = np.zeros(nbp, dtype=np.int64)
    start = 0
    for c in range(C):
        toks = np.nonzero(assign == c)[0]                 # ascending token order
        order[start * block: start * block + toks.size] = toks
        for k in range(nblk[c]):
            blk_cluster[start + k] = c
            blk_count[start + k] = min(block, toks.size - k * block)
        start += nblk[c]
    return order, blk_cluster, blk_count


def cluster_scores(cq: np.ndarray, ck: np.ndarray, sigma: float) -> np.ndarray:
    """S[a, b] = fl32(sigma * seqfma(cq[a], ck[b])), as for block means."""
    return block_scores(cq, ck, sigma)


def cluster_select(S: np.ndarray, nk: np.ndarray, N: int, rule: str,
                   density: float = 0.0, tau: float = 1.0, diag: bool = False,
                   eligible=None) -> np.ndarray:
    """Kept key clusters of every query cluster, bool [C, C].

    Empty key clusters, and those ``eligible`` (bool [C], optional) rules out,
    are never kept.  The others are ranked by S
    (descending, lower index on ties); "topk" keeps the shortest prefix whose
    token count reaches B = max(1, ceil(density * N * (1 - 1e-6))) (density a
    float32); "mass" keeps the shortest prefix whose weight sum_{prefix}
    n_b exp(S_b - S_max) (float64, accumulated in rank order) reaches tau times
    the total (tau a float32).  diag adds b = a when cluster a has keys.
    """
    C = S.shape[0]
    keep = np.zeros((C, C), dtype=bool)
    ok = nk > 0
    if eligible is not None:
        ok = ok & np.asarray(eligible, dtype=bool)
    live = np.nonzero(ok)[0]
    if rule == "topk":
        budget = max(1, int(np.ceil(float(np.float32(density)) * N * (1.0 - 1e-6))))
    for a in range(C):
        if diag and nk[a] > 0:
            keep[a, a] = True
        if live.size == 0:
            continue
        s = S[a, live]
        order = live[np.argsort(-s.astype(np.float64), kind="stable")]
        if rule == "topk":
            cum = np.cumsum(nk[order])
            m = int(np.searchsorted(cum, budget) + 1)
        elif rule == "mass":
            w = nk[order].astype(np.float64) * np.exp(S[a, order].astype(np.float64)
                                                      - float(S[a, order[0]]))
            cum = np.cumsum(w)
            thr = float(np.float32(tau)) * cum[-1]
            m = int(np.nonzero(cum >= thr)[0][0] + 1)
        else:
            raise ValueError(rule)
        keep[a, order[:min(m, order.size)]] = True
    return keep


def cluster_block_keep(keepC: np.ndarray, qblk: np.ndarray, kblk: np.ndarray) -> np.ndarray:
    """Block-level keep of the padded layout: row i keeps every block of the
    key clusters its query cluster keeps; blocks of no cluster keep nothing."""
    nbp = qblk.size
    keep = np.zeros((nbp, kblk.size), dtype=bool)
    for i in range(nbp):
        if qblk[i] < 0:
            continue
        kc = keepC[qblk[i]]
        keep[i] = (kblk >= 0) & kc[np.maximum(kblk, 0)]
    return keep


def cluster_attention_head(Qh, Kh, Vh, aq, ak, keepC, sigma: float, comp: bool = False,
                           q_clusters=None):
    """Attention of one head over the clustered partition, float64, raster order.

    A query of cluster a attends to every key of the key clusters a keeps;
    with ``comp`` every other non-empty key cluster b adds one centroid term
    (key = exact mean of its keys, value = exact mean of its values, weight
    n_b) -- SVG-EAR 2A, with clusters in place of blocks.  Rows of query
    clusters not in ``q_clusters`` are NaN.
    """
    N, d = Qh.shape
    C = keepC.shape[0]
    nk = np.bincount(ak, minlength=C).astype(np.float64)
    O = np.full((N, Vh.shape[1]), np.nan)
    lse = np.full(N, np.nan)
    if comp:
        ksum = np.zeros((C, d)); np.add.at(ksum, ak, Kh)
        vsum = np.zeros((C, Vh.shape[1])); np.add.at(vsum, ak, Vh)
        nz = nk > 0
        kbar = np.zeros_like(ksum); kbar[nz] = ksum[nz] / nk[nz, None]
        vbar = np.zeros_like(vsum); vbar[nz] = vsum[nz] / nk[nz, None]
    for a in (range(C) if q_clusters is None else q_clusters):
        qt = np.nonzero(aq == a)[0]
        if qt.size == 0:
            continue
        q = Qh[qt]
        kt = np.nonzero(keepC[a][ak])[0]
        logits = [sigma * (q @ Kh[kt].T)]
        values = [Vh[kt]]
        if comp:
            skip = np.nonzero(~keepC[a] & (nk > 0))[0]
            logits.append(sigma * (q @ kbar[skip].T) + np.log(nk[skip])[None, :])
            values.append(vbar[skip])
        L = np.concatenate(logits, axis=1)
        Vv = np.concatenate(values, axis=0)
        if L.shape[1] == 0:
            O[qt] = 0.0
            lse[qt] = -np.inf
            continue
        m = L.max(axis=1, keepdims=True)
        e = np.exp(L - m)
        s = e.sum(axis=1, keepdims=True)
        O[qt] = (e @ Vv) / s
        lse[qt] = (m + np.log(s))[:, 0]
    return O, lse


def cluster_head(Qh, Kh, mode: str, C: int, iters: int):
    if mode == "cocluster":
        return cocluster_head(Qh, Kh, C, iters)
    if mode == "kmeans":
        return kmeans_head(Qh, Kh, C, iters)
    raise ValueError(mode)


def cluster_workload_head(wl, Qh, Kh, Vh=None):
    """The clustered path of one head of a workload description (duck-typed:
    cluster, n_clusters, cluster_iters, block, scale, rule, density, mass,
    diag).  Returns a dict with the clusters, centroids, both layouts, the
    cluster-level and block-level keep and the cluster scores."""
    C = wl.n_clusters
    aq, ak, cq, ck = cluster_head(Qh, Kh, wl.cluster, C, wl.cluster_iters)
    N = Qh.shape[0]
    nk = np.bincount(ak, minlength=C)
    S = cluster_scores(cq, ck, wl.scale)
    dens = 0.0
    if wl.rule == "topk":
        dens = float(wl.densities()[0]) if wl.densities() is not None else 0.0
    keepC = cluster_select(S, nk, N, wl.rule, density=dens, tau=wl.mass, diag=wl.diag)
    qo, qb, qc = cluster_layout(aq, C, wl.block)
    ko, kb, kc = cluster_layout(ak, C, wl.block)
    return dict(aq=aq, ak=ak, cq=cq, ck=ck, S=S, keepC=keepC, nq=np.bincount(aq, minlength=C),
                nk=nk, q_order=qo, q_blk=qb, q_cnt=qc, k_order=ko, k_blk=kb, k_cnt=kc,
                keep=cluster_block_keep(keepC, qb, kb))

