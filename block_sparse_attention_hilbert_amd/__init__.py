"""Python binding of libsparse_attn.so: block-sparse video attention on MI355X.

Argument marshalling only.  Every step of the path (pooling, scoring,
selection, CSR construction, attention, Hilbert reordering) runs in the HIP
kernels of the C library; PyTorch provides device memory and the current
stream.  The functions mirror the C ABI in ``include/sparse_attn.h``:

* :func:`hilbert_perm_build` -- host Hilbert order of a latent grid
* :func:`hilbert_permute`, :func:`hilbert_unpermute` -- token reordering
* :func:`select` -- ``sparse_attn_select``: keep lists as CSR
* :func:`fwd` -- ``sparse_attn_fwd``: block-sparse attention (+ compensation)
* :func:`fwd_prepare`, :func:`fwd_run` -- its two halves
  (:func:`fwd_prepare_counts`: with a token count per KV block)
* :func:`centroids` -- compensation statistics alone (mask reuse)
* :func:`cluster_size`, :func:`cluster`, :func:`cluster_gather`,
  :func:`cluster_scatter`, :func:`cluster_select`, :func:`cluster_centroids` --
  data-dependent block formation (co-clustering / k-means / tiles) and
  selection over clusters
* :func:`sics` -- per-head choice of a tile shape (SICS scheme generation)
* :func:`workspace_size`

If the shared library is missing the import fails loudly; there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsparse_attn.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE, SA_ERR_HIP = range(5)
SA_RULE_NONE, SA_RULE_TOPK, SA_RULE_MASS, SA_RULE_ERR = range(4)
RULES = {"none": SA_RULE_NONE, "topk": SA_RULE_TOPK, "mass": SA_RULE_MASS, "err": SA_RULE_ERR}
SA_CLUSTER_COCLUSTER, SA_CLUSTER_KMEANS, SA_CLUSTER_TILES = 1, 2, 3
CLUSTER_MODES = {"cocluster": SA_CLUSTER_COCLUSTER, "kmeans": SA_CLUSTER_KMEANS,
                 "tiles": SA_CLUSTER_TILES}

EXPORTS = ("sparse_attn_workspace_size", "hilbert_perm_build", "hilbert_permute",
           "hilbert_unpermute", "sparse_attn_select", "sparse_attn_fwd",
           "sparse_attn_fwd_prepare", "sparse_attn_fwd_run", "sparse_attn_centroids",
           "sparse_attn_fwd_prepare_counts", "sparse_attn_cluster_size", "sparse_attn_cluster",
           "sparse_attn_cluster_gather", "sparse_attn_cluster_scatter",
           "sparse_attn_cluster_select", "sparse_attn_cluster_centroids", "sparse_attn_sics",
           "sparse_attn_last_error")


class SaProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("T", ctypes.c_int32), ("Hg", ctypes.c_int32),
                ("W", ctypes.c_int32), ("block", ctypes.c_int32), ("scale", ctypes.c_float)]


class SaSelectSpec(ctypes.Structure):
    _fields_ = [("rule", ctypes.c_int32), ("sub_block", ctypes.c_int32),
                ("topk", ctypes.POINTER(ctypes.c_int32)),
                ("density", ctypes.POINTER(ctypes.c_float)),
                ("mass", ctypes.c_float), ("diag", ctypes.c_int32),
                ("window_frames", ctypes.c_int32), ("n_anchors", ctypes.c_int32),
                ("anchor_offset", ctypes.c_int64), ("want_comp", ctypes.c_int32)]


class SaTileShape(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("y", ctypes.c_int32), ("x", ctypes.c_int32)]


class SaClusterSpec(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("n_clusters", ctypes.c_int32),
                ("iters", ctypes.c_int32), ("n_shapes", ctypes.c_int32),
                ("shapes", ctypes.POINTER(SaTileShape)), ("shape_idx", ctypes.c_void_p)]


class SparseAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sparse_attn status {status}: {msg}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python block_sparse_attention_hilbert_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    missing = [name for name in EXPORTS if not hasattr(lib, name)]
    if missing:
        raise ImportError(f"{LIB_PATH} is out of date (no {', '.join(missing)}); rebuild it "
                          "with `python block_sparse_attention_hilbert_amd/build.py`")
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER
    lib.sparse_attn_workspace_size.argtypes = [P(SaProblem), P(SaSelectSpec), P(sz)]
    lib.hilbert_perm_build.argtypes = [ctypes.c_int32] * 3 + [vp, vp]
    lib.hilbert_permute.argtypes = [P(SaProblem), vp, vp, vp, vp]
    lib.hilbert_unpermute.argtypes = [P(SaProblem), vp, vp, vp, vp]
    lib.sparse_attn_select.argtypes = [P(SaProblem), P(SaSelectSpec), vp, vp, vp, vp, vp, vp,
                                       vp, vp, vp, sz, vp]
    lib.sparse_attn_fwd.argtypes = [P(SaProblem), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sparse_attn_fwd_prepare.argtypes = [P(SaProblem), vp, vp, vp, vp, vp, sz, vp]
    lib.sparse_attn_centroids.argtypes = [P(SaProblem), vp, vp, vp, vp, vp]
    lib.sparse_attn_fwd_run.argtypes = [P(SaProblem), vp, vp, vp, vp, ctypes.c_int32, vp, vp, vp,
                                        sz, vp]
    lib.sparse_attn_fwd_prepare_counts.argtypes = [P(SaProblem), vp, vp, vp, vp, vp, vp, sz, vp]
    lib.sparse_attn_cluster_size.argtypes = [P(SaProblem), P(SaClusterSpec), vp, vp, vp]
    lib.sparse_attn_cluster.argtypes = [P(SaProblem), P(SaClusterSpec)] + [vp] * 15 + [sz, vp]
    lib.sparse_attn_cluster_gather.argtypes = [P(SaProblem), P(SaClusterSpec), vp, vp, vp, vp]
    lib.sparse_attn_cluster_scatter.argtypes = [P(SaProblem), P(SaClusterSpec)] + [vp] * 6
    lib.sparse_attn_cluster_select.argtypes = ([P(SaProblem), P(SaClusterSpec), P(SaSelectSpec)]
                                               + [vp] * 13 + [sz, vp])
    lib.sparse_attn_cluster_centroids.argtypes = [P(SaProblem), P(SaClusterSpec)] + [vp] * 10
    lib.sparse_attn_sics.argtypes = [P(SaProblem), P(SaClusterSpec), vp, vp, vp, vp, vp, sz, vp]
    for name in EXPORTS[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    lib.sparse_attn_last_error.argtypes = []
    lib.sparse_attn_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def _check(status: int):
    if status != SA_OK:
        raise SparseAttnError(status, lib.sparse_attn_last_error().decode())


@dataclass
class Problem:
    B: int
    H: int
    N: int
    d: int
    T: int
    Hg: int
    W: int
    block: int
    scale: float = 0.0

    @property
    def nb(self) -> int:
        return -(-self.N // self.block)

    @property
    def rows(self) -> int:
        return self.B * self.H * self.nb

    def c(self) -> SaProblem:
        return SaProblem(self.B, self.H, self.N, self.d, self.T, self.Hg, self.W, self.block,
                         self.scale)


@dataclass
class SelectSpec:
    rule: str = "topk"
    sub_block: int = 0
    topk: Optional[Sequence[int]] = None
    density: Optional[Sequence[float]] = None
    mass: float = 0.9
    diag: bool = False
    window_frames: int = -1
    n_anchors: int = 0
    anchor_offset: int = 0
    want_comp: bool = False

    def c(self):
        """ctypes struct plus the host arrays it points to (kept alive by the caller)."""
        keep = []
        topk = density = None
        if self.topk is not None:
            arr = np.ascontiguousarray(self.topk, dtype=np.int32)
            keep.append(arr)
            topk = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        if self.density is not None:
            arr = np.ascontiguousarray(self.density, dtype=np.float32)
            keep.append(arr)
            density = arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float))
        s = SaSelectSpec(RULES[self.rule], self.sub_block, topk, density, self.mass,
                         int(self.diag), self.window_frames, self.n_anchors,
                         int(self.anchor_offset), int(self.want_comp))
        return s, keep


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def workspace_size(prob: Problem, spec: Optional[SelectSpec] = None) -> int:
    n = ctypes.c_size_t(0)
    if spec is None:
        _check(lib.sparse_attn_workspace_size(ctypes.byref(prob.c()), None, ctypes.byref(n)))
    else:
        cs, keep = spec.c()
        _check(lib.sparse_attn_workspace_size(ctypes.byref(prob.c()), ctypes.byref(cs),
                                              ctypes.byref(n)))
    return int(n.value)


def alloc_workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """A 256-byte aligned device buffer (torch's caching allocator aligns to 512)."""
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def hilbert_perm_build(T: int, Hg: int, W: int):
    """(perm, inv) int32 numpy arrays of the 3D Hilbert order of a T x Hg x W grid."""
    N = T * Hg * W
    perm = np.empty(N, np.int32)
    inv = np.empty(N, np.int32)
    _check(lib.hilbert_perm_build(T, Hg, W, perm.ctypes.data, inv.ctypes.data))
    return perm, inv


def hilbert_permute(prob: Problem, src: torch.Tensor, perm_dev: torch.Tensor,
                    dst: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    dst = torch.empty_like(src) if dst is None else dst
    _check(lib.hilbert_permute(ctypes.byref(prob.c()), _ptr(src), _ptr(dst), _ptr(perm_dev),
                               _stream(stream)))
    return dst


def hilbert_unpermute(prob: Problem, src: torch.Tensor, perm_dev: torch.Tensor,
                      dst: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    dst = torch.empty_like(src) if dst is None else dst
    _check(lib.hilbert_unpermute(ctypes.byref(prob.c()), _ptr(src), _ptr(dst), _ptr(perm_dev),
                                 _stream(stream)))
    return dst


@dataclass
class Selection:
    row_ptr: torch.Tensor
    col_idx: torch.Tensor
    scores: Optional[torch.Tensor] = None
    k_mean: Optional[torch.Tensor] = None
    v_sum: Optional[torch.Tensor] = None


def select(prob: Problem, spec: SelectSpec, Q: torch.Tensor, K: torch.Tensor,
           V: Optional[torch.Tensor] = None, *, want_scores: bool = False,
           out: Optional[Selection] = None, workspace: Optional[torch.Tensor] = None,
           stream=None) -> Selection:
    """sparse_attn_select.  Output buffers are allocated unless ``out`` is given."""
    dev = (Q if Q is not None else K).device
    nb, rows = prob.nb, prob.rows
    if out is None:
        out = Selection(torch.empty(rows + 1, dtype=torch.int32, device=dev),
                        torch.empty(rows * nb, dtype=torch.int32, device=dev))
        if want_scores:
            out.scores = torch.empty(rows * nb, dtype=torch.float32, device=dev)
        if spec.want_comp:
            out.k_mean = torch.empty(prob.B, prob.H, nb, prob.d, dtype=torch.float32, device=dev)
            out.v_sum = torch.empty_like(out.k_mean)
    if workspace is None:
        workspace = alloc_workspace(workspace_size(prob, spec), dev)
    cs, keep = spec.c()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.sparse_attn_select(ctypes.byref(prob.c()), ctypes.byref(cs), _ptr(Q), _ptr(K),
                                  _ptr(V), _ptr(out.row_ptr), _ptr(out.col_idx),
                                  _ptr(out.scores), _ptr(out.k_mean), _ptr(out.v_sum),
                                  _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def centroids(prob: Problem, K: torch.Tensor, V: torch.Tensor, k_mean: torch.Tensor,
              v_sum: torch.Tensor, stream=None) -> None:
    """sparse_attn_centroids: block means of K and block sums of V (no selection)."""
    _check(lib.sparse_attn_centroids(ctypes.byref(prob.c()), _ptr(K), _ptr(V), _ptr(k_mean),
                                     _ptr(v_sum), _stream(stream)))


def fwd(prob: Problem, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
        row_ptr: torch.Tensor, col_idx: torch.Tensor, k_mean: Optional[torch.Tensor] = None,
        v_sum: Optional[torch.Tensor] = None, *, O: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None, want_lse: bool = False,
        workspace: Optional[torch.Tensor] = None, stream=None):
    """sparse_attn_fwd.  Returns O (and lse when requested or given)."""
    O = torch.empty_like(Q) if O is None else O
    if want_lse and lse is None:
        lse = torch.empty(prob.B, prob.H, prob.N, dtype=torch.float32, device=Q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_size(prob, None), Q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.sparse_attn_fwd(ctypes.byref(prob.c()), _ptr(Q), _ptr(K), _ptr(V), _ptr(row_ptr),
                               _ptr(col_idx), _ptr(k_mean), _ptr(v_sum), _ptr(O), _ptr(lse),
                               _ptr(workspace), ws_bytes, _stream(stream)))
    return (O, lse) if lse is not None else O


def fwd_prepare(prob: Problem, V: torch.Tensor, row_ptr: torch.Tensor,
                k_mean: Optional[torch.Tensor] = None, v_sum: Optional[torch.Tensor] = None, *,
                workspace: torch.Tensor, stream=None) -> None:
    """sparse_attn_fwd_prepare: V (and the centroids) laid out in ``workspace``."""
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.sparse_attn_fwd_prepare(ctypes.byref(prob.c()), _ptr(V), _ptr(row_ptr),
                                       _ptr(k_mean), _ptr(v_sum), _ptr(workspace), ws_bytes,
                                       _stream(stream)))


def fwd_run(prob: Problem, Q: torch.Tensor, K: torch.Tensor, row_ptr: torch.Tensor,
            col_idx: torch.Tensor, with_comp: bool, *, O: torch.Tensor,
            lse: Optional[torch.Tensor] = None, workspace: torch.Tensor, stream=None) -> None:
    """sparse_attn_fwd_run: the attention kernel on a prepared workspace."""
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.sparse_attn_fwd_run(ctypes.byref(prob.c()), _ptr(Q), _ptr(K), _ptr(row_ptr),
                                   _ptr(col_idx), int(bool(with_comp)), _ptr(O), _ptr(lse),
                                   _ptr(workspace), ws_bytes, _stream(stream)))


def problem_for(wl, scale: float = 0.0) -> Problem:
    """Problem statement of a workload description (duck-typed: B, H, N, d, T, Hg, W, block)."""
    return Problem(wl.B, wl.H, wl.N, wl.d, wl.T, wl.Hg, wl.W, wl.block, scale)


def spec_for(wl, anchor_offset: int = 0) -> SelectSpec:
    """Selection spec of a workload description."""
    dens = wl.densities()
    topk = wl.topks()
    return SelectSpec(rule=wl.rule, sub_block=wl.sub_block,
                      topk=None if topk is None else list(topk),
                      density=None if dens is None or topk is not None else list(dens),
                      mass=wl.mass, diag=wl.diag, window_frames=wl.window_frames,
                      n_anchors=wl.n_anchors, anchor_offset=anchor_offset,
                      want_comp=wl.comp)


def fwd_prepare_counts(prob: Problem, V: torch.Tensor, row_ptr: torch.Tensor,
                       kv_count: torch.Tensor, k_mean: Optional[torch.Tensor] = None,
                       v_sum: Optional[torch.Tensor] = None, *, workspace: torch.Tensor,
                       stream=None) -> None:
    """sparse_attn_fwd_prepare_counts: as fwd_prepare, with int32 [B*H, nb] token
    counts per KV block (keys past a block's count take no part)."""
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.sparse_attn_fwd_prepare_counts(ctypes.byref(prob.c()), _ptr(V), _ptr(row_ptr),
                                              _ptr(k_mean), _ptr(v_sum), _ptr(kv_count),
                                              _ptr(workspace), ws_bytes, _stream(stream)))


# ---------------------------------------------------------------------------
# data-dependent block formation
# ---------------------------------------------------------------------------

@dataclass
class ClusterSpec:
    mode: str = "kmeans"          # "cocluster" | "kmeans" | "tiles"
    n_clusters: int = 64          # tiles: the menu's largest tile count
    iters: int = 3
    shapes: Optional[Sequence] = None          # tiles: menu of (t, y, x)
    shape_idx: Optional[torch.Tensor] = None   # tiles: device int32 [B*H]

    def c(self) -> SaClusterSpec:
        n, sp = 0, None
        if self.shapes:
            arr = (SaTileShape * len(self.shapes))(*[SaTileShape(*map(int, s)) for s in self.shapes])
            self._shape_arr = arr                  # lives as long as the spec
            sp = ctypes.cast(arr, ctypes.POINTER(SaTileShape))
            n = len(self.shapes)
        return SaClusterSpec(CLUSTER_MODES[self.mode], self.n_clusters, self.iters, n, sp,
                             None if self.shape_idx is None else self.shape_idx.data_ptr())


def cluster_size(prob: Problem, cspec: ClusterSpec):
    """(nbp, ws_cluster, ws_select): blocks of the padded clustered layout and
    the workspace bytes of cluster() and cluster_select()."""
    nbp = ctypes.c_int32(0)
    w1, w2 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib.sparse_attn_cluster_size(ctypes.byref(prob.c()), ctypes.byref(cspec.c()),
                                        ctypes.byref(nbp), ctypes.byref(w1), ctypes.byref(w2)))
    return int(nbp.value), int(w1.value), int(w2.value)


def padded_problem(prob: Problem, nbp: int) -> Problem:
    """The attention problem on the padded clustered layout (one flat frame)."""
    Np = nbp * prob.block
    return Problem(prob.B, prob.H, Np, prob.d, 1, 1, Np, prob.block, prob.scale)


@dataclass
class Clusters:
    """Output of cluster(): layouts (int32) and centroids (fp32) of both sides."""
    q_order: torch.Tensor     # [B*H, Np] token at each padded slot, -1 = padding
    k_order: torch.Tensor
    q_blk: torch.Tensor       # [B*H, nbp] cluster of each padded block, -1 = none
    k_blk: torch.Tensor
    q_cnt: torch.Tensor       # [B*H, nbp] tokens in each padded block
    k_cnt: torch.Tensor
    q_cent: torch.Tensor      # [B*H, C, d]
    k_cent: torch.Tensor
    q_count: torch.Tensor     # [B*H, C] cluster sizes
    k_count: torch.Tensor
    v_cent: Optional[torch.Tensor] = None

    @staticmethod
    def empty(prob: Problem, cspec: ClusterSpec, nbp: int, with_v: bool, device) -> "Clusters":
        BH, C, Np = prob.B * prob.H, cspec.n_clusters, nbp * prob.block
        i32 = dict(dtype=torch.int32, device=device)
        f32 = dict(dtype=torch.float32, device=device)
        return Clusters(torch.empty(BH, Np, **i32), torch.empty(BH, Np, **i32),
                        torch.empty(BH, nbp, **i32), torch.empty(BH, nbp, **i32),
                        torch.empty(BH, nbp, **i32), torch.empty(BH, nbp, **i32),
                        torch.empty(BH, C, prob.d, **f32), torch.empty(BH, C, prob.d, **f32),
                        torch.empty(BH, C, **i32), torch.empty(BH, C, **i32),
                        torch.empty(BH, C, prob.d, **f32) if with_v else None)


def cluster(prob: Problem, cspec: ClusterSpec, Q: torch.Tensor, K: torch.Tensor,
            V: Optional[torch.Tensor] = None, *, out: Optional[Clusters] = None,
            workspace: Optional[torch.Tensor] = None, stream=None) -> Clusters:
    """sparse_attn_cluster: clusters of Q and K per (b, h) and their padded
    layouts; with V also the value means of the key clusters."""
    nbp, ws_c, _ = cluster_size(prob, cspec)
    if out is None:
        out = Clusters.empty(prob, cspec, nbp, V is not None, Q.device)
    if workspace is None:
        workspace = alloc_workspace(ws_c, Q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.sparse_attn_cluster(ctypes.byref(prob.c()), ctypes.byref(cspec.c()), _ptr(Q),
                                   _ptr(K), _ptr(V), _ptr(out.q_order), _ptr(out.k_order),
                                   _ptr(out.q_blk), _ptr(out.k_blk), _ptr(out.q_cnt),
                                   _ptr(out.k_cnt), _ptr(out.q_cent), _ptr(out.k_cent),
                                   _ptr(out.v_cent if V is not None else None),
                                   _ptr(out.q_count), _ptr(out.k_count), _ptr(workspace),
                                   ws_bytes, _stream(stream)))
    return out


def cluster_gather(prob: Problem, cspec: ClusterSpec, order: torch.Tensor, src: torch.Tensor,
                   dst: torch.Tensor, stream=None) -> torch.Tensor:
    """sparse_attn_cluster_gather: rows of src [B,H,N,d] into the padded layout dst
    [B,H,Np,d] (zero rows for padding)."""
    _check(lib.sparse_attn_cluster_gather(ctypes.byref(prob.c()), ctypes.byref(cspec.c()),
                                          _ptr(order), _ptr(src), _ptr(dst), _stream(stream)))
    return dst


def cluster_scatter(prob: Problem, cspec: ClusterSpec, order: torch.Tensor, src: torch.Tensor,
                    dst: torch.Tensor, lse_src: Optional[torch.Tensor] = None,
                    lse_dst: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """sparse_attn_cluster_scatter: rows of the padded layout back to token order."""
    _check(lib.sparse_attn_cluster_scatter(ctypes.byref(prob.c()), ctypes.byref(cspec.c()),
                                           _ptr(order), _ptr(src), _ptr(dst), _ptr(lse_src),
                                           _ptr(lse_dst), _stream(stream)))
    return dst


def cluster_select(prob: Problem, cspec: ClusterSpec, spec: SelectSpec, cl: Clusters, *,
                   out: Optional[Selection] = None, want_scores: bool = False,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> Selection:
    """sparse_attn_cluster_select: keep decision over clusters as CSR over the
    padded blocks (+ per-block compensation statistics with want_comp)."""
    nbp, _, ws_s = cluster_size(prob, cspec)
    dev = cl.q_cent.device
    BH, C = prob.B * prob.H, cspec.n_clusters
    rows = BH * nbp
    if out is None:
        out = Selection(torch.empty(rows + 1, dtype=torch.int32, device=dev),
                        torch.empty(rows * nbp, dtype=torch.int32, device=dev))
        if want_scores:
            out.scores = torch.empty(BH, C, C, dtype=torch.float32, device=dev)
        if spec.want_comp:
            out.k_mean = torch.empty(prob.B, prob.H, nbp, prob.d, dtype=torch.float32, device=dev)
            out.v_sum = torch.empty_like(out.k_mean)
    if workspace is None:
        workspace = alloc_workspace(ws_s, dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    cs, keep = spec.c()
    _check(lib.sparse_attn_cluster_select(
        ctypes.byref(prob.c()), ctypes.byref(cspec.c()), ctypes.byref(cs), _ptr(cl.q_cent),
        _ptr(cl.k_cent), _ptr(cl.v_cent), _ptr(cl.k_count), _ptr(cl.q_blk), _ptr(cl.k_blk),
        _ptr(cl.k_cnt), _ptr(out.row_ptr), _ptr(out.col_idx), _ptr(out.scores),
        _ptr(out.k_mean), _ptr(out.v_sum), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def cluster_centroids(prob: Problem, cspec: ClusterSpec, Kp: torch.Tensor, Vp: torch.Tensor,
                      cl: Clusters, k_mean: torch.Tensor, v_sum: torch.Tensor,
                      stream=None) -> None:
    """sparse_attn_cluster_centroids: key / value means of the kept partition
    from this call's K, V in the padded layout (into cl.k_cent, cl.v_cent) and
    the per-block compensation statistics."""
    _check(lib.sparse_attn_cluster_centroids(ctypes.byref(prob.c()), ctypes.byref(cspec.c()),
                                             _ptr(Kp), _ptr(Vp), _ptr(cl.k_count), _ptr(cl.k_blk),
                                             _ptr(cl.k_cnt), _ptr(cl.k_cent), _ptr(cl.v_cent),
                                             _ptr(k_mean), _ptr(v_sum), _stream(stream)))


def sics(prob: Problem, cspec: ClusterSpec, Q: torch.Tensor, K: torch.Tensor,
         shape_idx: torch.Tensor, scores: Optional[torch.Tensor] = None, *,
         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """sparse_attn_sics: per (b, h) the tile shape of the menu with the most
    coherent tiles (mean intra-tile cosine of Q and K) into shape_idx (device
    int32 [B*H]); scores (device fp64 [B*H, n_shapes]) if given."""
    if workspace is None:
        workspace = alloc_workspace(cluster_size(prob, cspec)[1], Q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.sparse_attn_sics(ctypes.byref(prob.c()), ctypes.byref(cspec.c()), _ptr(Q), _ptr(K),
                                _ptr(scores), _ptr(shape_idx), _ptr(workspace), ws_bytes,
                                _stream(stream)))
    return shape_idx


def cluster_spec_for(wl) -> ClusterSpec:
    """Cluster spec of a workload description (cluster, n_clusters, cluster_iters,
    tile_shapes)."""
    if wl.cluster == "tiles":
        return ClusterSpec("tiles", wl.n_clusters, 0, shapes=[tuple(s) for s in wl.tile_shapes])
    return ClusterSpec(wl.cluster, wl.n_clusters, wl.cluster_iters)
