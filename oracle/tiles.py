"""Oracle, SICS scheme generation over shaped 3D tiles -- TEST INFRASTRUCTURE ONLY.

Plain CPU restatement of the page "SPADE: An Input-Adaptive Sparse Attention
Engine for Fast Video Diffusion Models Inference": part 1 (vDiT-SSR, a menu
of ways to cut the latent video cube into blocks -- wide and flat, tall and
thin, mixed) and part 2 (scheme generation by SICS, the sum of intra-block
cosine similarities, decided per head and per step).  Only the tests, the
package smoke check and the benchmark's CPU-baseline leg may import it.

Readings (the page describes the scheme only by analogy; each is stated
where it is used):

* a tile shape (ts, ys, xs) cuts the (T, Hg, W) grid into tiles
  [tt*ts, (tt+1)*ts) x [ty*ys, ...) x [tx*xs, ...) clipped at the grid's
  end; tiles are numbered in raster order of (tt, ty, tx) and each tile is
  one attention block (its volume is at most the block size);
* SICS of a tile = the sum over ordered pairs of distinct tokens of their
  cosine similarity (a zero vector has cosine 0 with everything); the scheme
  of a head is the menu shape with the largest mean intra-tile cosine of its
  queries and keys together, (SICS_Q + SICS_K) / (2 * sum_tiles n (n - 1)),
  the first shape of the menu on ties;
* the blocks of the chosen shape then go through the same selection as
  data-dependent blocks (scores of tile means, token budget or
  count-weighted cumulative mass) -- ``oracle.clusters`` with the tile index
  as the cluster;
* the optional SICS ticket theta (part 2's admission test): a key tile may
  be kept only if the mean cosine of its keys' ordered pairs,
  SICS_K / (n (n - 1)), is at least theta (a tile of one token counts as 1);
  the other tiles are ignored by the selection, i.e. treated like empty
  clusters (the explicit diagonal still adds a query tile's own keys);
  without a ticket (the default) every tile is admitted, as with theta = -1.

The shape choice is float64 on both sides; the scores of two shapes closer
than a relative 1e-9 are a near tie.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from . import clusters as OC

Shape = Tuple[int, int, int]


def tile_counts(T: int, Hg: int, W: int, shape: Shape) -> Tuple[int, int, int]:
    ts, ys, xs = shape
    return -(-T // ts), -(-Hg // ys), -(-W // xs)


def n_tiles(T: int, Hg: int, W: int, shape: Shape) -> int:
    a, b, c = tile_counts(T, Hg, W, shape)
    return a * b * c


def tile_assign(T: int, Hg: int, W: int, shape: Shape) -> np.ndarray:
    """Tile index of every token (raster order n = (t*Hg + y)*W + x)."""
    ts, ys, xs = shape
    _, nty, ntx = tile_counts(T, Hg, W, shape)
    t, y, x = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(W), indexing="ij")
    return (((t // ts) * nty + (y // ys)) * ntx + (x // xs)).reshape(-1).astype(np.int64)


def unit_rows(X: np.ndarray) -> np.ndarray:
    """Rows scaled to unit length (float64); zero rows stay zero."""
    X = np.asarray(X, dtype=np.float64)
    nrm = np.sqrt((X * X).sum(axis=1))
    out = np.zeros_like(X)
    nz = nrm > 0
    out[nz] = X[nz] / nrm[nz, None]
    return out


def sics_per_tile(X: np.ndarray, assign: np.ndarray, ntiles: int) -> np.ndarray:
    """SICS of every tile: sum over ordered pairs a != b of cos(x_a, x_b),
    from the Gram matrix of the tile's unit rows (its off-diagonal sum)."""
    U = unit_rows(X)
    out = np.zeros(ntiles)
    for c in range(ntiles):
        rows = U[assign == c]
        if rows.shape[0] < 2:
            continue
        G = rows @ rows.T
        out[c] = G.sum() - np.trace(G)
    return out


def sics_score(Qh: np.ndarray, Kh: np.ndarray, grid, shape: Shape) -> float:
    """Mean intra-tile cosine of queries and keys for one shape."""
    T, Hg, W = grid
    a = tile_assign(T, Hg, W, shape)
    nt = n_tiles(T, Hg, W, shape)
    n = np.bincount(a, minlength=nt).astype(np.float64)
    pairs = float((n * (n - 1)).sum())
    if pairs == 0:
        return 0.0
    s = sics_per_tile(Qh, a, nt).sum() + sics_per_tile(Kh, a, nt).sum()
    return s / (2.0 * pairs)


def choose_shape(Qh, Kh, grid, shapes: Sequence[Shape]):
    """(index of the chosen shape, scores of every shape): the largest score,
    the first of the menu on ties."""
    scores = np.array([sics_score(Qh, Kh, grid, s) for s in shapes])
    return int(np.argmax(scores)), scores


def key_coherence(Kh: np.ndarray, assign: np.ndarray, ntiles: int) -> np.ndarray:
    """Mean cosine over the ordered pairs of distinct keys of every tile,
    SICS_K / (n (n - 1)); 1 for a tile of fewer than two tokens."""
    n = np.bincount(assign, minlength=ntiles).astype(np.float64)
    out = np.ones(ntiles)
    many = n >= 2
    out[many] = sics_per_tile(Kh, assign, ntiles)[many] / (n[many] * (n[many] - 1.0))
    return out


def max_tiles(grid, shapes: Sequence[Shape]) -> int:
    return max(n_tiles(*grid, s) for s in shapes)


def tiles_workload_head(wl, Qh, Kh):
    """The tiled path of one head (duck-typed workload: T, Hg, W, block,
    tile_shapes, scale, rule, density, mass, diag, optionally sics_ticket).
    Returns the same dict as ``clusters.cluster_workload_head`` plus the
    shape scores, the chosen shape, the key coherence of its tiles and which
    of them the ticket admits."""
    grid = (wl.T, wl.Hg, wl.W)
    shapes = [tuple(s) for s in wl.tile_shapes]
    pick, scores = choose_shape(Qh, Kh, grid, shapes)
    C = max_tiles(grid, shapes)
    a = tile_assign(*grid, shapes[pick])
    N = Qh.shape[0]
    cq = OC.cluster_means(Qh, a, C)
    ck = OC.cluster_means(Kh, a, C)
    nk = np.bincount(a, minlength=C)
    S = OC.cluster_scores(cq, ck, wl.scale)
    dens = 0.0
    if wl.rule == "topk":
        dens = float(wl.densities()[0])
    # the ticket is a float32 compared in float64 with the fp64 coherence
    ticket = getattr(wl, "sics_ticket", None)
    coh = key_coherence(Kh, a, C)
    eligible = np.ones(C, dtype=bool)
    if ticket is not None:
        ticket = float(np.float32(ticket))
        eligible = coh >= ticket
    keepC = OC.cluster_select(S, nk, N, wl.rule, density=dens, tau=wl.mass, diag=wl.diag,
                              eligible=eligible)
    order, blk, cnt = OC.cluster_layout(a, C, wl.block, nbp=C)
    return dict(pick=pick, scores=scores, coh=coh, eligible=eligible, ticket=ticket,
                aq=a, ak=a, cq=cq, ck=ck, S=S, keepC=keepC, nq=nk,
                nk=nk, q_order=order, q_blk=blk, q_cnt=cnt, k_order=order, k_blk=blk, k_cnt=cnt,
                keep=OC.cluster_block_keep(keepC, blk, blk))
