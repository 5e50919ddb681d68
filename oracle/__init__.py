"""Oracle for block-sparse video attention -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation of what the hot path
computes.  Only the tests, the package smoke check and the benchmark's
CPU-baseline leg may import it; the product library never does, and it
shares no code with the HIP path (no kernels, headers, helpers or tables).

Sources (titles of the pages the method is taken from):

* "DFSAttn: Dynamic Fine-grained Sparse Attention for Efficient Video
  Generation" -- trick 1 (3D Hilbert curve token reordering), trick 2
  (sub-block scoring from block means).
* "SVG-EAR: Parameter-Free Linear Compensation for Sparse Video Generation
  via Error-aware Routing" -- section 2A (centroid = mean of the keys and
  values of a cluster replaces the skipped ones), section 1 / 2B (selection
  on attention scores under a fixed density budget), section 4 (top-p
  selection), section 2B (streaming update, no materialised logits).
* "SVG-EAR" again -- section 2B (error-aware routing: the compensation
  error of every block, probed with the query-cluster centroids standing in
  for the individual queries, ranks the blocks by error per unit cost under
  the density budget).
* "SVOO: Training-Free Sparse Attention ... Bidirectional Co-Clustering" --
  section 2A (density that covers a share of the cumulative attention mass).
* "LVSA: Training-Free Sparse Attention for Long Video Diffusion" -- abstract
  (structured window pattern plus rotating global anchors, block-sparse).
* "SPADE: An Input-Adaptive Sparse Attention Engine ..." -- part 2 (the keep
  decision is taken per head).

Precision.  The pages fix none.  Attention is computed in float64 from the
exact float32 widening of the bf16 inputs.  Selection is decided on float32
block scores with the numeric definition of ``oracle_scores.c`` (sequential
fused multiply-add), block means are exact float64 sums rounded once to
float32, and the cumulative-mass rule works in float64 -- the decision
precision both sides must share.

Functions with no independent pin: none; every function is pinned by the
``not gpu`` tests (brute force, closed forms, library special cases).
Agreement with the papers' own (unpublished) implementations is parity
unpinned: the pages print no mask, score or output value.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle_scores.c")
_lib = None


def build_oracle_lib() -> str:
    """Compile the oracle's C part with gcc (no HIP, no shared code)."""
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", _SRC, "-o", _LIB_PATH, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build_oracle_lib()
        lib = ctypes.CDLL(_LIB_PATH)
        fp = ctypes.POINTER(ctypes.c_float)
        lib.oracle_block_scores.argtypes = [fp, fp, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_float, fp]
        lib.oracle_block_scores.restype = None
        lib.oracle_seqfma_dot.argtypes = [fp, fp, ctypes.c_int64]
        lib.oracle_seqfma_dot.restype = ctypes.c_float
        _lib = lib
    return _lib


def _fptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


# ---------------------------------------------------------------------------
# inputs
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns, as float64."""
    u = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def block_bounds(N: int, block: int) -> np.ndarray:
    """Token ranges of the contiguous equal-size blocks; the last may be short.

    Returns int64 [nb+1] with block i = tokens [b[i], b[i+1]).
    """
    nb = -(-N // block)
    b = np.arange(nb + 1, dtype=np.int64) * block
    b[-1] = N
    return b


# ---------------------------------------------------------------------------
# O1. 3D Hilbert token order (DFSAttn, trick 1)
# ---------------------------------------------------------------------------

def hilbert_index_3d(a0, a1, a2, bits: int) -> np.ndarray:
    """Hilbert-curve index of cells (a0, a1, a2) in a cube of side 2**bits.

    Skilling's method (J. Skilling, "Programming the Hilbert curve", AIP Conf.
    Proc. 707, 2004): undo the curve's rotations/reflections from the top bit
    down, Gray-encode the coordinates (the "transpose" form of the index), and
    read the index by interleaving the bits with axis 0 most significant.
    """
    X = [np.array(a, dtype=np.int64, copy=True) for a in (a0, a1, a2)]
    Q = 1 << (bits - 1)
    while Q > 1:
        P = Q - 1
        for i in range(3):
            bit = (X[i] & Q) != 0
            t = np.where(bit, 0, (X[0] ^ X[i]) & P)        # exchange low bits
            X[0] = np.where(bit, X[0] ^ P, X[0] ^ t)        # or invert them
            if i:
                X[i] = X[i] ^ t
        Q >>= 1
    for i in (1, 2):                                        # Gray encode
        X[i] = X[i] ^ X[i - 1]
    t = np.zeros_like(X[0])
    Q = 1 << (bits - 1)
    while Q > 1:
        t = np.where((X[2] & Q) != 0, t ^ (Q - 1), t)
        Q >>= 1
    X = [x ^ t for x in X]
    idx = np.zeros_like(X[0])
    for b in range(bits - 1, -1, -1):
        for i in range(3):
            idx = (idx << 1) | ((X[i] >> b) & 1)
    return idx


def hilbert_first_step_axis(bits: int) -> int:
    """Curve axis along which the first two octants of the cube are stacked.

    Found by brute force over the whole cube: the first quarter of the curve
    (two octants) must be exactly the box that is 2**bits long on that axis
    and 2**(bits-1) on the other two.
    """
    s = 1 << bits
    g = np.indices((s, s, s)).reshape(3, -1)
    idx = hilbert_index_3d(g[0], g[1], g[2], bits)
    first = idx < (s ** 3) // 4
    found = [ax for ax in range(3)
             if np.array_equal(first, np.all(np.delete(g, ax, axis=0) < s // 2, axis=0))]
    if len(found) != 1:
        raise AssertionError(f"no unique first-step axis: {found}")
    return found[0]


def hilbert_axis_map(bits: int):
    """Curve axes assigned to (t, y, x).

    Reading: x (the longest side of the latent grids) goes on the curve's
    first-step axis, so that a 2^(b-1) x 2^(b-1) x 2^b box is one contiguous
    stretch of the curve; t and y take the two remaining axes in increasing
    order.
    """
    ax_x = hilbert_first_step_axis(bits)
    rest = [a for a in range(3) if a != ax_x]
    return rest[0], rest[1], ax_x


def hilbert_bits(T: int, Hg: int, W: int) -> int:
    return max(1, int(math.ceil(math.log2(max(T, Hg, W)))))


def hilbert_perm(T: int, Hg: int, W: int):
    """perm[r] = raster index of the r-th latent cell in Hilbert order; inv = perm^-1.

    The grid (t, y, x) is placed in the cube of side 2^b (b = ceil(log2 of the
    largest side)), every cube cell outside the grid is dropped, and the
    remaining cells are sorted by curve index.
    """
    bits = hilbert_bits(T, Hg, W)
    at, ay, ax = hilbert_axis_map(bits)
    t, y, x = np.indices((T, Hg, W)).reshape(3, -1)
    coords = [None, None, None]
    coords[at], coords[ay], coords[ax] = t, y, x
    idx = hilbert_index_3d(coords[0], coords[1], coords[2], bits)
    perm = np.argsort(idx, kind="stable").astype(np.int64)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(perm.size)
    return perm, inv


def permute_tokens(X: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """X'[..., n, :] = X[..., perm[n], :]."""
    return np.take(X, perm, axis=-2)


def unpermute_tokens(X: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """X[..., perm[n], :] = X'[..., n, :]."""
    out = np.empty_like(X)
    out[..., perm, :] = X
    return out


# ---------------------------------------------------------------------------
# O2. block means (DFSAttn trick 2 "media"; SVG-EAR 2A centroid)
# ---------------------------------------------------------------------------

def block_sums_f64(X: np.ndarray, block: int) -> np.ndarray:
    """Exact float64 sums of each block of tokens: [..., N, d] -> [..., nb, d].

    Sums of at most a few hundred bf16 values are exact in float64 (their
    significands span far fewer than 53 bits), so the order of the additions
    does not matter.
    """
    X = np.asarray(X, dtype=np.float64)
    N, d = X.shape[-2], X.shape[-1]
    nfull = N // block
    lead = X.shape[:-2]
    parts = [X[..., : nfull * block, :].reshape(*lead, nfull, block, d).sum(axis=-2)]
    if nfull * block < N:
        parts.append(X[..., nfull * block:, :].sum(axis=-2, keepdims=True))
    return np.concatenate(parts, axis=-2)


def block_means(X: np.ndarray, block: int) -> np.ndarray:
    """fp32 block means: fl32( (exact sum) / n_i ), n_i = true token count."""
    N = X.shape[-2]
    n = np.diff(block_bounds(N, block)).astype(np.float64)
    return (block_sums_f64(X, block) / n[:, None]).astype(np.float32)


def block_sums_f32(X: np.ndarray, block: int) -> np.ndarray:
    """fp32 block sums: fl32(exact sum)."""
    return block_sums_f64(X, block).astype(np.float32)


# ---------------------------------------------------------------------------
# O3. pooled scores
# ---------------------------------------------------------------------------

def block_scores(qm: np.ndarray, km: np.ndarray, sigma: float) -> np.ndarray:
    """S[i, j] = fl32(sigma * seqfma_dot(qm[i], km[j])) for one head."""
    qm = np.ascontiguousarray(qm, dtype=np.float32)
    km = np.ascontiguousarray(km, dtype=np.float32)
    out = np.empty((qm.shape[0], km.shape[0]), dtype=np.float32)
    _load().oracle_block_scores(_fptr(qm), _fptr(km), qm.shape[0], km.shape[0],
                                qm.shape[1], ctypes.c_float(sigma), _fptr(out))
    return out


def seqfma_dot(a: np.ndarray, b: np.ndarray) -> float:
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    return float(_load().oracle_seqfma_dot(_fptr(a), _fptr(b), a.size))


def subblock_max_scores(Qh: np.ndarray, Kh: np.ndarray, block: int, sub: int,
                        sigma: float, mode: str = "max") -> np.ndarray:
    """Block scores from sub-block scores (DFSAttn trick 2), one head.

    Each block is cut into sub-blocks of ``sub`` tokens (the last one of the
    sequence may be short); every sub-block pair is scored like O3 on its
    sub-block means, and the block score is the max over the sub-block pairs
    that exist.  ``mode="mean"`` averages the sub-pair dot products instead
    (equal to plain block-mean pooling in exact arithmetic; a regression
    check of the sub-block indexing only).
    """
    N = Qh.shape[0]
    qs = block_means(Qh, sub)
    ks = block_means(Kh, sub)
    nb = -(-N // block)
    spb = block // sub
    nsub = qs.shape[0]
    if mode == "max":
        s = block_scores(qs, ks, sigma).astype(np.float64)
        pad = np.full((nb * spb, nb * spb), -np.inf)
        pad[:nsub, :nsub] = s
        return pad.reshape(nb, spb, nb, spb).max(axis=(1, 3)).astype(np.float32)
    # "mean": count-weighted average of sub-pair dot products (float64)
    cnt = np.diff(block_bounds(N, sub)).astype(np.float64)
    dots = (qs.astype(np.float64) * cnt[:, None]) @ (ks.astype(np.float64) * cnt[:, None]).T
    blk = np.arange(nsub) // spb
    acc = np.zeros((nb, nb))
    np.add.at(acc, (blk[:, None], blk[None, :]), dots)
    n = np.diff(block_bounds(N, block)).astype(np.float64)
    return sigma * acc / np.outer(n, n)


# ---------------------------------------------------------------------------
# O4. selection
# ---------------------------------------------------------------------------

def k_from_density(rho, nb: int) -> int:
    """k = clamp(ceil(rho*nb*(1 - 1e-6)), 1, nb), rho a float32 widened to double.

    The fixed density budget (SVG-EAR page, section 2B) gives at least the
    requested share of the blocks; the 1e-6 relative slack absorbs the float32
    representation error of rho (0.15f * 600 = 90.0000036 keeps 90 blocks).
    """
    k = math.ceil(float(np.float32(rho)) * nb * (1.0 - 1e-6))
    return int(min(max(k, 1), nb))


def rank_order(S: np.ndarray) -> np.ndarray:
    """Column order per row: score descending, block index ascending on ties."""
    return np.argsort(-S, axis=-1, kind="stable")


def topk_keep(S: np.ndarray, k: int) -> np.ndarray:
    order = rank_order(S)
    keep = np.zeros(S.shape, dtype=bool)
    np.put_along_axis(keep, order[:, :k], True, axis=1)
    return keep


def mass_cutoff(S: np.ndarray, tau: float) -> np.ndarray:
    """Number of blocks m the cumulative-mass rule keeps in each row.

    p_j = exp(S_j - S_max) in float64, accumulated in rank order; keep the
    shortest prefix whose sum reaches tau * (sum of all p), tau a float32.
    """
    order = rank_order(S)
    s = np.take_along_axis(S, order, axis=1).astype(np.float64)
    p = np.exp(s - s[:, :1])
    cum = np.cumsum(p, axis=1)
    thr = float(np.float32(tau)) * cum[:, -1:]
    return np.argmax(cum >= thr, axis=1) + 1


def mass_keep(S: np.ndarray, tau: float) -> np.ndarray:
    order = rank_order(S)
    m = mass_cutoff(S, tau)
    keep = np.zeros(S.shape, dtype=bool)
    cols = np.arange(S.shape[1])[None, :] < m[:, None]
    rows = np.broadcast_to(np.arange(S.shape[0])[:, None], S.shape)
    keep[rows[cols], order[cols]] = True
    return keep


def block_frames(N: int, block: int, HgW: int):
    """First and last latent frame covered by each block (raster order)."""
    b = block_bounds(N, block)
    return b[:-1] // HgW, (b[1:] - 1) // HgW


def window_keep(N: int, block: int, HgW: int, r: int) -> np.ndarray:
    """LVSA structured window: KV block j is kept for query block i when the
    frames it covers come within r latent frames of those block i covers."""
    lo, hi = block_frames(N, block, HgW)
    return (lo[None, :] <= hi[:, None] + r) & (hi[None, :] >= lo[:, None] - r)


def anchor_blocks(nb: int, A: int, offset: int) -> np.ndarray:
    """LVSA rotating global anchors: a_m = (offset + m*floor(nb/A)) mod nb."""
    if A <= 0:
        return np.zeros(0, dtype=np.int64)
    return (int(offset) + np.arange(A, dtype=np.int64) * (nb // A)) % nb


# ---------------------------------------------------------------------------
# O4b. error-aware routing (SVG-EAR 2B)
# ---------------------------------------------------------------------------

def error_keys(Qh: np.ndarray, Kh: np.ndarray, Vh: np.ndarray, block: int,
               sigma: float) -> np.ndarray:
    """Routing key of every (query block i, KV block j) of one head, float64 [nb, nb].

    The query block's mean qbar_i stands in for its queries (the page's query
    centroids; cost O(C_q N_k d) instead of O(N_q N_k d)).  With the logits
    l_t = sigma * qbar_i . k_t of the tokens t of block j and m = max_t l_t:

      exact contribution     A = sum_t exp(l_t - m) v_t
      centroid replacement   Ahat = n_j exp(S_ij - m) vbar_j

    where S_ij is the pooled score fl32(sigma * qbar_i . kbar_j) of the
    score-based rules (the centroid's logit) and vbar_j = fl32(sum_t v_t) / n_j
    (the block sum the compensation uses).  The key is the log of the
    compensation error per unit of cost, on one scale for the whole row:

      key = ln ||A - Ahat||_2 + m - ln n_j          (-inf when A == Ahat)

    qbar, kbar are the fp32 block means of the score-based rules; every other
    step is float64.
    """
    b = block_bounds(Qh.shape[0], block)
    nb = b.size - 1
    n = np.diff(b).astype(np.float64)
    qm = block_means(Qh, block).astype(np.float64)
    S = block_scores(block_means(Qh, block), block_means(Kh, block), sigma).astype(np.float64)
    vbar = block_sums_f32(Vh, block).astype(np.float64) / n[:, None]
    keys = np.empty((nb, nb), dtype=np.float64)
    for j in range(nb):
        Kj = np.asarray(Kh[b[j]:b[j + 1]], dtype=np.float64)
        Vj = np.asarray(Vh[b[j]:b[j + 1]], dtype=np.float64)
        L = sigma * (qm @ Kj.T)                         # [nb, n_j]
        m = L.max(axis=1)
        A = np.exp(L - m[:, None]) @ Vj                 # [nb, d]
        Ahat = (n[j] * np.exp(S[:, j] - m))[:, None] * vbar[j][None, :]
        err = np.sqrt(((A - Ahat) ** 2).sum(axis=1))
        with np.errstate(divide="ignore"):
            keys[:, j] = np.log(err) + m - np.log(n[j])
    return keys


def select_head(Qh: Optional[np.ndarray], Kh: Optional[np.ndarray], *, N: int,
                block: int, HgW: int, sigma: float, rule: str, k: int = 0,
                tau: float = 1.0, sub_block: int = 0, diag: bool = False,
                window_frames: int = -1, n_anchors: int = 0,
                anchor_offset: int = 0, Vh: Optional[np.ndarray] = None):
    """Keep mask [nb, nb] of one (batch, head) and the scores it was decided on.

    Qh, Kh (and Vh for the error rule): exact token values [N, d] (already in
    the order blocks are formed in).  Returns (keep bool [nb, nb], ranking
    keys [nb, nb] or None): float32 pooled scores for "topk" / "mass", the
    float64 error keys for "err" (top-k by error per block size, SVG-EAR 2B).
    """
    nb = -(-N // block)
    keep = np.zeros((nb, nb), dtype=bool)
    S = None
    if rule in ("topk", "mass"):
        if sub_block:
            S = subblock_max_scores(Qh, Kh, block, sub_block, sigma)
        else:
            S = block_scores(block_means(Qh, block), block_means(Kh, block), sigma)
        keep |= topk_keep(S, k) if rule == "topk" else mass_keep(S, tau)
    elif rule == "err":
        if sub_block:
            raise ValueError("the error rule works on whole blocks")
        S = error_keys(Qh, Kh, Vh, block, sigma)
        keep |= topk_keep(S, k)
    elif rule != "none":
        raise ValueError(rule)
    if diag:
        keep |= np.eye(nb, dtype=bool)
    if window_frames >= 0:
        keep |= window_keep(N, block, HgW, window_frames)
    if n_anchors > 0:
        keep[:, anchor_blocks(nb, n_anchors, anchor_offset)] = True
    return keep, S


def keep_to_csr(keep: np.ndarray):
    """Rows of a [R, nb] keep mask -> (row_ptr int32 [R+1], col_idx int32), ascending."""
    counts = keep.sum(axis=1)
    row_ptr = np.zeros(keep.shape[0] + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    col_idx = np.nonzero(keep)[1]
    return row_ptr.astype(np.int32), col_idx.astype(np.int32)


# ---------------------------------------------------------------------------
# O5. attention (plain definition, float64)
# ---------------------------------------------------------------------------

def attention_head(Qh, Kh, Vh, keep, block: int, sigma: float, comp: bool = False,
                   q_blocks=None):
    """Block-sparse softmax attention of one head, float64.

    For a query token of block i the logits are sigma*q.k_t over the tokens of
    the kept KV blocks (every other logit is -inf and contributes exp(-inf) =
    0).  With ``comp`` every skipped KV block j adds one centroid pseudo-token:
    key = mean of K over block j, value = mean of V over block j, weight n_j
    (SVG-EAR 2A: the keys and values of a skipped cluster are replaced by
    their centroid, so the block contributes n_j*exp(sigma*q.kbar_j)*vbar_j).

    Qh, Kh, Vh: float64 [N, d].  keep: bool [nb, nb].
    Returns (O float64 [N, d], lse float64 [N]); rows of Q blocks not in
    ``q_blocks`` are NaN.
    """
    N, d = Qh.shape
    b = block_bounds(N, block)
    nb = b.size - 1
    n = np.diff(b).astype(np.float64)
    O = np.full((N, Vh.shape[1]), np.nan)
    lse = np.full(N, np.nan)
    if comp:
        kbar = block_sums_f64(Kh, block) / n[:, None]
        vbar = block_sums_f64(Vh, block) / n[:, None]
    for i in (range(nb) if q_blocks is None else q_blocks):
        q = Qh[b[i]:b[i + 1]]
        kept = np.nonzero(keep[i])[0]
        tok = np.concatenate([np.arange(b[j], b[j + 1]) for j in kept]) if kept.size else \
            np.zeros(0, dtype=np.int64)
        logits = [sigma * (q @ Kh[tok].T)]
        values = [Vh[tok]]
        if comp:
            skip = np.nonzero(~keep[i])[0]
            logits.append(sigma * (q @ kbar[skip].T) + np.log(n[skip])[None, :])
            values.append(vbar[skip])
        L = np.concatenate(logits, axis=1)
        Vv = np.concatenate(values, axis=0)
        if L.shape[1] == 0:
            O[b[i]:b[i + 1]] = 0.0
            lse[b[i]:b[i + 1]] = -np.inf
            continue
        m = L.max(axis=1, keepdims=True)
        e = np.exp(L - m)
        s = e.sum(axis=1, keepdims=True)
        O[b[i]:b[i + 1]] = (e @ Vv) / s
        lse[b[i]:b[i + 1]] = (m + np.log(s))[:, 0]
    return O, lse


def dense_masked_attention_head(Qh, Kh, Vh, keep, block: int, sigma: float,
                                comp: bool = False):
    """The same attention written as one dense N x N softmax with -inf bias.

    softmax(sigma*Q K^T + M) V with M = 0 on tokens of kept blocks and -inf
    elsewhere; with ``comp`` the nb centroid columns (logit sigma*q.kbar_j +
    ln n_j, value vbar_j) are appended, masked to -inf where j is kept.
    """
    N, d = Qh.shape
    b = block_bounds(N, block)
    n = np.diff(b).astype(np.float64)
    blk = np.repeat(np.arange(b.size - 1), np.diff(b))
    tok_keep = keep[blk][:, blk]                    # [N, N]
    L = sigma * (Qh @ Kh.T)
    L = np.where(tok_keep, L, -np.inf)
    Vv = Vh
    if comp:
        kbar = block_sums_f64(Kh, block) / n[:, None]
        vbar = block_sums_f64(Vh, block) / n[:, None]
        C = sigma * (Qh @ kbar.T) + np.log(n)[None, :]
        C = np.where(keep[blk], -np.inf, C)
        L = np.concatenate([L, C], axis=1)
        Vv = np.concatenate([Vh, vbar], axis=0)
    m = L.max(axis=1, keepdims=True)
    empty = np.isneginf(m[:, 0])              # a row that attends to nothing
    m[empty] = 0.0
    e = np.exp(L - m)
    s = e.sum(axis=1, keepdims=True)
    s[empty] = 1.0
    O = (e @ Vv) / s
    lse = (m + np.log(s))[:, 0]
    O[empty] = 0.0
    lse[empty] = -np.inf
    return O, lse


# ---------------------------------------------------------------------------
# the whole path for one workload
# ---------------------------------------------------------------------------

def head_k(wl, h: int) -> int:
    nb = wl.nb
    if wl.topk is not None:
        return int(min(max(wl.topk, 1), nb))
    dens = wl.densities()
    if dens is not None:
        return k_from_density(dens[h], nb)
    return 0


def select_workload(wl, Q, K, heads=None, anchor_offset: int = 0, perm=None, V=None):
    """Keep masks [B, len(heads), nb, nb] and ranking keys for bf16-bit inputs.

    Q, K (and V for the error rule): uint16 [B, nh, N, d] in raster order;
    ``perm`` (Hilbert order) is applied first when given.
    """
    heads = list(range(wl.H)) if heads is None else list(heads)
    B, nh = Q.shape[0], Q.shape[1]
    keep = np.zeros((B, nh, wl.nb, wl.nb), dtype=bool)
    scores = np.zeros((B, nh, wl.nb, wl.nb), dtype=np.float64 if wl.rule == "err" else np.float32)
    for bi in range(B):
        for hi, h in enumerate(heads):
            q = bf16_to_f64(Q[bi, hi]) if wl.rule != "none" else None
            k = bf16_to_f64(K[bi, hi]) if wl.rule != "none" else None
            v = bf16_to_f64(V[bi, hi]) if wl.rule == "err" else None
            if perm is not None and q is not None:
                q, k = permute_tokens(q, perm), permute_tokens(k, perm)
                if v is not None:
                    v = permute_tokens(v, perm)
            kk, S = select_head(q, k, N=wl.N, block=wl.block, HgW=wl.Hg * wl.W,
                                sigma=wl.scale, rule=wl.rule, k=head_k(wl, h),
                                tau=wl.mass, sub_block=wl.sub_block, diag=wl.diag,
                                window_frames=wl.window_frames,
                                n_anchors=wl.n_anchors, anchor_offset=anchor_offset, Vh=v)
            keep[bi, hi] = kk
            if S is not None:
                scores[bi, hi] = S
    return keep, scores


def kept_flops(keep: np.ndarray, N: int, block: int, d: int) -> float:
    """4*d*sum over kept (i, j) of n_i*n_j (QK^T and PV multiply-adds)."""
    n = np.diff(block_bounds(N, block)).astype(np.float64)
    w = np.outer(n, n)
    return float(4.0 * d * (keep * w).sum())
