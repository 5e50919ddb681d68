"""One block-sparse attention call with preallocated buffers.

The call is the whole hot path: block selection (pooling, scores, keep lists
as CSR) and block-sparse attention with optional centroid compensation
(SVG-EAR page, section 2A), over blocks of raster tokens or of the 3D Hilbert
order (DFSAttn page, trick 1).  The Hilbert order is folded into the kernels
(the problem's token order): pooling and the V re-layout read rows through
it, the attention kernel reads its queries and writes O and lse through it,
and only K is gathered into block order once, inside the attention call; Q,
V and O are never reordered as whole tensors.  Every step is one or more HIP
kernels of libsparse_attn.so enqueued on the current stream; this class only
owns the buffers so that repeated calls allocate nothing.

Mask reuse (DFSAttn page, trick 3: the previous step's mask is cached; SVOO
page, section 2B: the clustering is refreshed only every few diffusion steps):
with ``refresh_every = r`` the selection runs on calls 0, r, 2r, ... and the
calls in between keep its CSR.  A reusing call still attends over its own
inputs and, with compensation, recomputes the centroids of the skipped blocks
from its own K and V (sparse_attn_centroids); only the keep decision is reused.

:class:`ClusteredAttention` is the same call with data-dependent blocks
(SVOO page, section 2B: bidirectional Q/K co-clustering; SVG-EAR page,
section 2A: k-means clusters made contiguous by a permutation): cluster Q and
K, gather them (and V) into the padded clustered layout, select over
clusters, attend with per-block token counts, scatter O back to token order.
With ``refresh_every = r`` it clusters and selects on calls 0, r, 2r, ...
(SVOO keeps its partition for ~20 diffusion steps); the calls in between keep
the partition and the keep lists, gather their own Q, K, V into the layout and,
with compensation, take the cluster centroids from their own K and V.
With a ``tiles`` cluster spec (SPADE parts 1-2) the partition of every head is
the tile grid of the menu shape that SICS picks for it on the refreshing call;
with a SICS ticket only the tiles whose keys agree (mean pairwise key cosine
at least the ticket) may be kept, the others are ignored.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import (Clusters, ClusterSpec, Problem, Selection, SelectSpec, alloc_workspace,
               centroids, cluster, cluster_centroids, cluster_gather,
               cluster_fwd_prepare, cluster_fwd_run, cluster_select, sics,
               cluster_size, fwd, fwd_prepare, fwd_prepare_counts, fwd_run,
               hilbert_perm_build, padded_problem, select, workspace_size)


class BlockSparseAttention:
    def __init__(self, prob: Problem, spec: SelectSpec, hilbert: bool = False,
                 device="cuda", want_scores: bool = False, want_lse: bool = False,
                 refresh_every: int = 1):
        if refresh_every < 1:
            raise ValueError("refresh_every must be >= 1")
        if hilbert and spec.window_frames >= 0:
            # the window is a range of latent frames over raster-ordered blocks;
            # blocks of Hilbert-ordered tokens span frames in no such order
            raise ValueError("a latent-frame window needs raster token order (hilbert=False)")
        self.spec, self.hilbert = spec, hilbert
        self.refresh_every = int(refresh_every)
        self.calls = 0              # calls made so far (the reuse policy counts them)
        self.have_mask = False
        self.device = torch.device(device)
        self.perm = self.perm_dev = None
        if hilbert:
            # blocks of the Hilbert order: the problem's token order
            perm, _ = hilbert_perm_build(prob.T, prob.Hg, prob.W)
            self.perm = perm
            self.perm_dev = torch.from_numpy(perm).to(self.device)
            prob = Problem(**{**prob.__dict__, "token_order": self.perm_dev})
        self.prob = prob
        nb, rows = prob.nb, prob.rows
        shape = (prob.B, prob.H, prob.N, prob.d)
        self.sel = Selection(torch.empty(rows + 1, dtype=torch.int32, device=self.device),
                             torch.empty(rows * nb, dtype=torch.int32, device=self.device))
        if want_scores:
            self.sel.scores = torch.empty(rows * nb, dtype=torch.float32, device=self.device)
        if spec.want_comp:
            self.sel.k_mean = torch.empty(prob.B, prob.H, nb, prob.d, dtype=torch.float32,
                                          device=self.device)
            self.sel.v_sum = torch.empty_like(self.sel.k_mean)
        # the error rule's selection writes V in block layout straight into the
        # forward workspace, so the forward call does not lay it out again
        self.share_v = spec.rule == "err"
        self.v_ready = False       # the forward workspace holds V of the last selection
        self.ws_select = alloc_workspace(workspace_size(prob, spec, v_blocks=self.share_v), self.device)
        self.ws_fwd = alloc_workspace(workspace_size(prob, None), self.device)
        # O and lse in the caller's token order (also with Hilbert blocks)
        self.O = torch.empty(shape, dtype=torch.bfloat16, device=self.device)
        self.lse = torch.empty(prob.B, prob.H, prob.N, dtype=torch.float32,
                               device=self.device) if want_lse else None

    def run_select(self, Q, K, V, anchor_offset: Optional[int] = None) -> Selection:
        """The selection.  With the error rule it also leaves this V in block
        layout in the forward workspace, and the next run_fwd /
        run_fwd_prepare use that layout instead of laying out their V again:
        pass them the same V (run_centroids, the mask-reuse path, drops it)."""
        spec = self.spec
        if anchor_offset is not None:
            spec = SelectSpec(**{**spec.__dict__, "anchor_offset": int(anchor_offset)})
        sel = select(self.prob, spec, Q, K, V if spec.want_comp else None,
                     out=self.sel, workspace=self.ws_select,
                     v_blocks=self.ws_fwd if self.share_v else None)
        self.have_mask = True
        self.v_ready = self.share_v
        return sel

    def run_centroids(self, K, V):
        """Compensation statistics of the current K, V for a reused mask (the
        forward call then lays out this V itself)."""
        self.v_ready = False
        if self.spec.want_comp:
            centroids(self.prob, K, V, self.sel.k_mean, self.sel.v_sum)

    def reuses_next(self) -> bool:
        """Whether the next call keeps the current mask under the refresh policy."""
        return self.have_mask and self.calls % self.refresh_every != 0

    def run_fwd(self, Q, K, V, row_ptr=None, col_idx=None):
        if self.v_ready:
            # V is already in the workspace (written by the selection)
            self.run_fwd_prepare(V, row_ptr)
            return self.run_fwd_attention(Q, K, row_ptr, col_idx)
        rp = self.sel.row_ptr if row_ptr is None else row_ptr
        ci = self.sel.col_idx if col_idx is None else col_idx
        fwd(self.prob, Q, K, V, rp, ci, self.sel.k_mean, self.sel.v_sum, O=self.O, lse=self.lse,
            workspace=self.ws_fwd)
        return self.O

    def run_fwd_prepare(self, V, row_ptr=None):
        """First half of run_fwd: V (and the centroids) laid out in the workspace
        (V only if the last selection has not already put it there)."""
        rp = self.sel.row_ptr if row_ptr is None else row_ptr
        fwd_prepare(self.prob, None if self.v_ready else V, rp, self.sel.k_mean, self.sel.v_sum,
                    workspace=self.ws_fwd)

    def run_fwd_attention(self, Q, K, row_ptr=None, col_idx=None):
        """Second half of run_fwd: the attention kernel (with Hilbert blocks,
        K gathered into block order first)."""
        rp = self.sel.row_ptr if row_ptr is None else row_ptr
        ci = self.sel.col_idx if col_idx is None else col_idx
        fwd_run(self.prob, Q, K, rp, ci, self.spec.want_comp, O=self.O, lse=self.lse,
                workspace=self.ws_fwd)
        return self.O

    def __call__(self, Q, K, V, anchor_offset: Optional[int] = None,
                 reuse_mask: Optional[bool] = None) -> torch.Tensor:
        """One call.  ``reuse_mask``: keep the last selection (True), select
        anew (False) or follow the refresh policy (None)."""
        if reuse_mask is None:
            reuse_mask = self.reuses_next()
        if reuse_mask and not self.have_mask:
            raise RuntimeError("no mask to reuse: the first call must select")
        if reuse_mask:
            self.run_centroids(K, V)
        else:
            self.run_select(Q, K, V, anchor_offset)
        self.run_fwd(Q, K, V)
        self.calls += 1
        return self.O

    def keep_mask(self) -> np.ndarray:
        """Kept-block mask [B, H, nb, nb] of the last selection (host copy)."""
        p = self.prob
        rp = self.sel.row_ptr.cpu().numpy()
        ci = self.sel.col_idx[: int(rp[-1])].cpu().numpy()
        keep = np.zeros((p.rows, p.nb), dtype=bool)
        rows = np.repeat(np.arange(p.rows), np.diff(rp))
        keep[rows, ci] = True
        return keep.reshape(p.B, p.H, p.nb, p.nb)


class ClusteredAttention:
    """One attention call over data-dependent blocks, preallocated buffers.

    prob: the problem in token order; cspec: clustering; spec: selection over
    clusters (SA_RULE_TOPK with density, or SA_RULE_MASS; diag; want_comp).
    """

    def __init__(self, prob: Problem, cspec: ClusterSpec, spec: SelectSpec, device="cuda",
                 want_scores: bool = False, want_lse: bool = False, refresh_every: int = 1):
        if refresh_every < 1:
            raise ValueError("refresh_every must be >= 1")
        self.prob, self.spec = prob, spec
        self.device = torch.device(device)
        self.shape_idx = self.shape_scores = None
        self.tile_coherence = None
        if cspec.mode == "tiles":
            BH = prob.B * prob.H
            self.shape_idx = torch.zeros(BH, dtype=torch.int32, device=self.device)
            self.shape_scores = torch.zeros(BH, len(cspec.shapes), dtype=torch.float64,
                                            device=self.device)
            if cspec.ticket is not None:
                # every tile's key coherence, for the SICS ticket
                self.tile_coherence = torch.zeros(BH, len(cspec.shapes), cspec.n_clusters,
                                                  dtype=torch.float64, device=self.device)
            cspec = ClusterSpec(cspec.mode, cspec.n_clusters, cspec.iters, list(cspec.shapes),
                                self.shape_idx, cspec.ticket, self.tile_coherence)
        self.cspec = cspec
        self.refresh_every = int(refresh_every)
        self.calls = 0
        self.have_partition = False
        self.nbp, ws_c, ws_s = cluster_size(prob, cspec)
        self.pprob = padded_problem(prob, self.nbp)
        pp = self.pprob
        self.cl = Clusters.empty(prob, cspec, self.nbp, spec.want_comp, self.device)
        rows = pp.rows
        self.sel = Selection(torch.empty(rows + 1, dtype=torch.int32, device=self.device),
                             torch.empty(rows * self.nbp, dtype=torch.int32, device=self.device))
        if want_scores:
            self.sel.scores = torch.empty(prob.B * prob.H, cspec.n_clusters, cspec.n_clusters,
                                          dtype=torch.float32, device=self.device)
        if spec.want_comp:
            self.sel.k_mean = torch.empty(pp.B, pp.H, self.nbp, pp.d, dtype=torch.float32,
                                          device=self.device)
            self.sel.v_sum = torch.empty_like(self.sel.k_mean)
        self.ws_cluster = alloc_workspace(ws_c, self.device)
        self.ws_select = alloc_workspace(ws_s, self.device)
        self.ws_fwd = alloc_workspace(workspace_size(pp, None), self.device)
        # K is gathered into the padded layout (V too when a kept partition's
        # centroids are recomputed); V is laid out and Q read, O and lse
        # written in token order by the forward calls themselves
        pshape = (pp.B, pp.H, pp.N, pp.d)
        self.Kp = torch.empty(pshape, dtype=torch.bfloat16, device=self.device)
        self.Vp = torch.empty_like(self.Kp)
        self.O = torch.empty(prob.B, prob.H, prob.N, prob.d, dtype=torch.bfloat16,
                             device=self.device)
        self.lse = None
        if want_lse:
            self.lse = torch.empty(prob.B, prob.H, prob.N, dtype=torch.float32,
                                   device=self.device)
        self._Q = self._V = None   # this call's Q and V (read by the forward calls)

    def run_cluster(self, Q, K, V, choose_shapes: bool = True):
        """Form the partition.  In tile mode SICS first picks each head's tile
        shape, unless ``choose_shapes`` is False: then the shapes already in
        ``self.shape_idx`` (set by the caller) are used."""
        if self.cspec.mode == "tiles" and choose_shapes:
            sics(self.prob, self.cspec, Q, K, self.shape_idx, self.shape_scores,
                 workspace=self.ws_cluster)
        cluster(self.prob, self.cspec, Q, K, V if self.spec.want_comp else None, out=self.cl,
                workspace=self.ws_cluster)
        self.have_partition = True
        return self.cl

    def reuses_next(self) -> bool:
        """Whether the next call keeps the current partition and selection."""
        return self.have_partition and self.calls % self.refresh_every != 0

    def run_centroids(self):
        """Compensation statistics of this call's K, V for a kept partition
        (V gathered into the padded layout for them)."""
        if self.spec.want_comp:
            cluster_gather(self.prob, self.cspec, self.cl.k_order, self._V, self.Vp)
            cluster_centroids(self.prob, self.cspec, self.Kp, self.Vp, self.cl, self.sel.k_mean,
                              self.sel.v_sum)

    def run_gather(self, Q, K, V):
        """K into the padded layout (Q and V stay in token order: the forward
        calls read them through q_order and k_order)."""
        self._Q, self._V = Q, V
        cluster_gather(self.prob, self.cspec, self.cl.k_order, K, self.Kp)

    def run_select(self) -> Selection:
        return cluster_select(self.prob, self.cspec, self.spec, self.cl, out=self.sel,
                              workspace=self.ws_select)

    def run_fwd_prepare(self):
        cluster_fwd_prepare(self.prob, self.cspec, self.cl.k_order, self._V, self.sel.row_ptr,
                            self.cl.k_cnt, self.sel.k_mean, self.sel.v_sum, workspace=self.ws_fwd)

    def run_fwd_attention(self):
        """The attention over the padded layout, Q read and O, lse written in
        token order (this call's Q, from run_gather)."""
        cluster_fwd_run(self.prob, self.cspec, self.cl.q_order, self._Q, self.Kp,
                        self.sel.row_ptr, self.sel.col_idx, self.spec.want_comp, O=self.O,
                        lse=self.lse, workspace=self.ws_fwd)
        return self.O

    def run_scatter(self):
        """O (and lse) in token order: written there by run_fwd_attention."""
        return self.O

    def __call__(self, Q, K, V, reuse: Optional[bool] = None,
                 choose_shapes: bool = True) -> torch.Tensor:
        """One call.  ``reuse``: keep the partition and selection (True), form
        them anew (False) or follow the refresh policy (None).
        ``choose_shapes``: in tile mode, False keeps the caller's per-head
        shapes in ``self.shape_idx`` instead of running SICS."""
        if reuse is None:
            reuse = self.reuses_next()
        if reuse and not self.have_partition:
            raise RuntimeError("no partition to reuse: the first call must cluster")
        if not reuse:
            self.run_cluster(Q, K, V, choose_shapes=choose_shapes)
        self.run_gather(Q, K, V)
        if reuse:
            self.run_centroids()
        else:
            self.run_select()
        self.run_fwd_prepare()
        self.run_fwd_attention()
        self.calls += 1
        return self.run_scatter()

    def kept_tokens(self) -> torch.Tensor:
        """Key tokens each query block attends to exactly, [B*H*nbp] (device)."""
        pp = self.pprob
        rp = self.sel.row_ptr.long()
        ci = self.sel.col_idx[: int(rp[-1])].long()
        cnt = self.cl.k_cnt.reshape(-1).long()
        bh = torch.repeat_interleave(torch.arange(pp.rows, device=rp.device) // self.nbp,
                                     rp[1:] - rp[:-1])
        per = cnt[bh * self.nbp + ci]
        out = torch.zeros(pp.rows, dtype=torch.long, device=rp.device)
        rows = torch.repeat_interleave(torch.arange(pp.rows, device=rp.device), rp[1:] - rp[:-1])
        out.index_add_(0, rows, per)
        return out


class GraphedCall:
    """A pipeline's call captured as HIP graphs and replayed.

    One graph per variant of the call: forming the selection (or partition)
    anew and keeping it.  A replay enqueues every kernel of the call with one
    host launch instead of one per kernel.  It reads the input tensors given
    here (the caller copies each step's data into them) and writes the
    pipeline's own output buffers (``pipe.O``, ``pipe.lse``).  Each variant is
    first run once eagerly on a side stream, so the library's one-time set-up
    (kernel attributes, occupancy queries) happens outside the capture; the
    library enqueues no memset, copy, allocation or host synchronisation, so
    the whole call is capturable.  Calls through the graphs and eager calls of
    the same pipeline can be mixed: both follow ``pipe.calls``.
    """

    def __init__(self, pipe, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor):
        if getattr(pipe.spec, "n_anchors", 0) > 0:
            # the selection takes the anchor offset by value at launch, so a
            # replay would repeat the captured call's anchors instead of
            # rotating them
            raise ValueError("rotating anchors change on every call; run them eagerly, "
                             "not as graph replays")
        self.pipe = pipe
        self.inputs = (Q, K, V)
        kw = "reuse" if isinstance(pipe, ClusteredAttention) else "reuse_mask"
        self._run = lambda keep: pipe(Q, K, V, **{kw: keep})
        calls = pipe.calls
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for keep in (False, True):        # forming first: keeping needs a selection
                self._run(keep)
        torch.cuda.current_stream().wait_stream(side)
        self.graphs = {}
        for keep in (False, True):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._run(keep)
            self.graphs[keep] = g
        pipe.calls = calls

    def __call__(self, keep: Optional[bool] = None) -> torch.Tensor:
        """One call: ``keep`` the last selection / partition (True), form it
        anew (False) or follow the pipeline's refresh policy (None)."""
        p = self.pipe
        if keep is None:
            keep = p.reuses_next()
        self.graphs[bool(keep)].replay()
        p.calls += 1
        return p.O
