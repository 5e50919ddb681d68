"""Python binding of libsparse_attn.so: block-sparse video attention on MI355X.

Argument marshalling only.  Every step of the path (pooling, scoring,
selection, CSR construction, attention, Hilbert reordering) runs in the HIP
kernels of the C library; PyTorch provides device memory and the current
stream.  The functions mirror the C ABI in ``include/sparse_attn.h``:

* :func:`hilbert_perm_build` -- host Hilbert order of a latent grid
* :func:`hilbert_permute`, :func:`hilbert_unpermute` -- token reordering
* :func:`select` -- ``sparse_attn_select``: keep lists as CSR
  (:func:`select_noalloc`: the same with the library's fixed scratch)
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
           "sparse_attn_select_noalloc", "sparse_attn_cluster_fwd_run",
           "sparse_attn_cluster_fwd_prepare", "sparse_attn_last_error")


class SaProblem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("T", ctypes.c_int32), ("Hg", ctypes.c_int32),
                ("W", ctypes.c_int32), ("block", ctypes.c_int32), ("scale", ctypes.c_float),
                ("token_order", ctypes.c_void_p)]


class SaSelectSpec(ctypes.Structure):
    _fields_ = [("rule", ctypes.c_int32), ("sub_block", ctypes.c_int32),
                ("topk", ctypes.POINTER(ctypes.c_int32)),
                ("density", ctypes.POINTER(ctypes.c_float)),
                ("mass", ctypes.c_float), ("diag", ctypes.c_int32),
                ("window_frames", ctypes.c_int32), ("n_anchors", ctypes.c_int32),
                ("anchor_offset", ctypes.c_int64), ("want_comp", ctypes.c_int32),
                ("v_blocks", ctypes.c_void_p)]


class SaTileShape(ctypes.Structure):
    _fields_ = [("t", ctypes.c_int32), ("y", ctypes.c_int32), ("x", ctypes.c_int32)]


class SaClusterSpec(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("n_clusters", ctypes.c_int32),
                ("iters", ctypes.c_int32), ("n_shapes", ctypes.c_int32),
                ("shapes", ctypes.POINTER(SaTileShape)), ("shape_idx", ctypes.c_void_p),
                ("ticket", ctypes.c_float), ("tile_coherence", ctypes.c_void_p)]


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
    lib.sparse_attn_select_noalloc.argtypes = [P(SaProblem), P(SaSelectSpec), vp, vp, vp, vp, vp,
                                               vp, vp, vp, vp]
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
    lib.sparse_attn_cluster_fwd_run.argtypes = ([P(SaProblem), P(SaClusterSpec), vp, vp, vp, vp, vp,
                                                 ctypes.c_int32, vp, vp, vp, sz, vp])
    lib.sparse_attn_cluster_fwd_prepare.argtypes = ([P(SaProblem), P(SaClusterSpec)] + [vp] * 7 +
                                                    [sz, vp])
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
    # device int32 [N]: blocks are runs of the tokens in this order (Q, K, V,
    # O and lse stay in the caller's order), or None: as given
    token_order: Optional[torch.Tensor] = None

    @property
    def nb(self) -> int:
        return -(-self.N // self.block)

    @property
    def rows(self) -> int:
        return self.B * self.H * self.nb

    def c(self) -> SaProblem:
        order = None
        if self.token_order is not None:
            t = self.token_order
            if t.dtype != torch.int32 or tuple(t.shape) != (self.N,) or not t.is_contiguous():
                raise ValueError(f"token_order must be a contiguous int32 tensor of shape ({self.N},)")
            if t.device.type != "cuda":
                raise ValueError("token_order must be a GPU tensor")
            order = t.data_ptr()
        return SaProblem(self.B, self.H, self.N, self.d, self.T, self.Hg, self.W, self.block,
                         self.scale, order)


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

    def c(self, v_blocks: int = 0):
        """ctypes struct plus the host arrays it points to (kept alive by the
        caller); ``v_blocks``: device address for the error rule's V layout (0: none)."""
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
                         int(self.anchor_offset), int(self.want_comp), v_blocks or None)
        return s, keep


_BF16, _I32, _F32, _U8 = torch.bfloat16, torch.int32, torch.float32, torch.uint8


class _Args:
    """Checked device pointers of one call's tensor arguments.  The C library
    sees only addresses and sizes, so everything it cannot check is checked
    here, before the call: each tensor's dtype, exact shape or minimum element
    count and contiguity (the kernels index dense row-major buffers) as it is
    marshalled, then that all of them live on one GPU."""

    def __init__(self):
        self.seen = []

    def __call__(self, t: Optional[torch.Tensor], name: str, dtype: torch.dtype, *, shape=None,
                 numel: Optional[int] = None, optional: bool = False):
        if t is None:
            if optional:
                return None
            raise ValueError(f"{name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor (got {type(t).__name__})")
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
        if numel is not None and t.numel() < numel:
            raise ValueError(f"{name} holds {t.numel()} elements; at least {numel} are needed")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        self.seen.append((name, t))
        return ctypes.c_void_p(t.data_ptr())

    def call(self, fn, *args):
        """fn(*args) once every tensor seen is on the same GPU."""
        dev = None
        for name, t in self.seen:
            if t.device.type != "cuda":
                raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{name} is on {t.device}, the call's other tensors on {dev}")
        return fn(*[a.handle() if isinstance(a, _Stream) else a for a in args])


def _ws(A: _Args, workspace: Optional[torch.Tensor]):
    """(pointer, bytes) of a workspace buffer (uint8, contiguous, same GPU)."""
    if workspace is None:
        return None, 0
    return A(workspace, "workspace", _U8), workspace.numel()


def _tokens(prob: "Problem", N: Optional[int] = None):
    return (prob.B, prob.H, prob.N if N is None else N, prob.d)


class _Stream:
    """The HIP stream of a call (the current one unless given), looked up
    when the call is made, after its arguments are checked."""

    def __init__(self, stream=None):
        self.stream = stream

    def handle(self):
        s = torch.cuda.current_stream() if self.stream is None else self.stream
        return ctypes.c_void_p(s.cuda_stream)


def workspace_size(prob: Problem, spec: Optional[SelectSpec] = None, *, v_blocks: bool = False) -> int:
    """sparse_attn_workspace_size; ``v_blocks``: the error rule's V layout goes
    to the caller's buffer (the size query reads only whether it is given)."""
    n = ctypes.c_size_t(0)
    if spec is None:
        _check(lib.sparse_attn_workspace_size(ctypes.byref(prob.c()), None, ctypes.byref(n)))
    else:
        cs, keep = spec.c(256 if v_blocks else 0)
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


def _permute_args(A: "_Args", prob: Problem, src, perm_dev, dst):
    ps = A(src, "src", _BF16, shape=_tokens(prob))
    dev = src.device
    if dst is None:
        dst = torch.empty(_tokens(prob), dtype=_BF16, device=dev)
    pd = A(dst, "dst", _BF16, shape=_tokens(prob))
    pp = A(perm_dev, "perm_dev", _I32, shape=(prob.N,))
    return ps, pd, pp, dst


def hilbert_permute(prob: Problem, src: torch.Tensor, perm_dev: torch.Tensor,
                    dst: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    A = _Args()
    ps, pd, pp, dst = _permute_args(A, prob, src, perm_dev, dst)
    _check(A.call(lib.hilbert_permute, ctypes.byref(prob.c()), ps, pd, pp, _Stream(stream)))
    return dst


def hilbert_unpermute(prob: Problem, src: torch.Tensor, perm_dev: torch.Tensor,
                      dst: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    A = _Args()
    ps, pd, pp, dst = _permute_args(A, prob, src, perm_dev, dst)
    _check(A.call(lib.hilbert_unpermute, ctypes.byref(prob.c()), ps, pd, pp, _Stream(stream)))
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
           v_blocks: Optional[torch.Tensor] = None, stream=None) -> Selection:
    """sparse_attn_select.  Output buffers are allocated unless ``out`` is given.
    ``v_blocks`` (error rule): a forward workspace whose start receives V in
    block layout, for a following ``fwd_prepare(V=None)``."""
    A = _Args()
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
    vb = 0
    if v_blocks is not None:
        need = prob.B * prob.H * nb * prob.d * prob.block * 2
        vb = A(v_blocks, "v_blocks", _U8, numel=need).value
    cs, keep = spec.c(vb)
    if workspace is None:
        workspace = alloc_workspace(workspace_size(prob, spec, v_blocks=vb != 0), dev)
    tok, stat = _tokens(prob), (prob.B, prob.H, nb, prob.d)
    args = [A(Q, "Q", _BF16, shape=tok, optional=True),
            A(K, "K", _BF16, shape=tok, optional=True),
            A(V, "V", _BF16, shape=tok, optional=True),
            A(out.row_ptr, "row_ptr", _I32, numel=rows + 1),
            A(out.col_idx, "col_idx", _I32, numel=rows * nb),
            A(out.scores, "scores", _F32, numel=rows * nb, optional=True),
            A(out.k_mean, "k_mean", _F32, shape=stat, optional=True),
            A(out.v_sum, "v_sum", _F32, shape=stat, optional=True)]
    wp, ws_bytes = _ws(A, workspace)
    _check(A.call(lib.sparse_attn_select, ctypes.byref(prob.c()), ctypes.byref(cs), *args, wp, ws_bytes,
                                  _Stream(stream)))
    return out


def select_noalloc(prob: Problem, spec: SelectSpec, Q: torch.Tensor, K: torch.Tensor,
                   V: Optional[torch.Tensor] = None, *, out: Selection, stream=None) -> Selection:
    """sparse_attn_select_noalloc: sparse_attn_select with the library's own
    fixed scratch instead of a workspace (for callers that cannot allocate;
    the output buffers in ``out`` are the caller's)."""
    A = _Args()
    nb, rows = prob.nb, prob.rows
    cs, keep = spec.c()
    tok, stat = _tokens(prob), (prob.B, prob.H, nb, prob.d)
    args = [A(Q, "Q", _BF16, shape=tok, optional=True),
            A(K, "K", _BF16, shape=tok, optional=True),
            A(V, "V", _BF16, shape=tok, optional=True),
            A(out.row_ptr, "row_ptr", _I32, numel=rows + 1),
            A(out.col_idx, "col_idx", _I32, numel=rows * nb),
            A(out.scores, "scores", _F32, numel=rows * nb, optional=True),
            A(out.k_mean, "k_mean", _F32, shape=stat, optional=True),
            A(out.v_sum, "v_sum", _F32, shape=stat, optional=True)]
    _check(A.call(lib.sparse_attn_select_noalloc, ctypes.byref(prob.c()), ctypes.byref(cs), *args,
                  _Stream(stream)))
    return out


def centroids(prob: Problem, K: torch.Tensor, V: torch.Tensor, k_mean: torch.Tensor,
              v_sum: torch.Tensor, stream=None) -> None:
    """sparse_attn_centroids: block means of K and block sums of V (no selection)."""
    A = _Args()
    dev, tok, stat = K.device, _tokens(prob), (prob.B, prob.H, prob.nb, prob.d)
    _check(A.call(lib.sparse_attn_centroids, ctypes.byref(prob.c()), A(K, "K", _BF16, shape=tok),
                                     A(V, "V", _BF16, shape=tok),
                                     A(k_mean, "k_mean", _F32, shape=stat),
                                     A(v_sum, "v_sum", _F32, shape=stat),
                                     _Stream(stream)))


def _comp_args(A: "_Args", prob: Problem, k_mean, v_sum):
    stat = (prob.B, prob.H, prob.nb, prob.d)
    return (A(k_mean, "k_mean", _F32, shape=stat, optional=True),
            A(v_sum, "v_sum", _F32, shape=stat, optional=True))


def fwd(prob: Problem, Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor,
        row_ptr: torch.Tensor, col_idx: torch.Tensor, k_mean: Optional[torch.Tensor] = None,
        v_sum: Optional[torch.Tensor] = None, *, O: Optional[torch.Tensor] = None,
        lse: Optional[torch.Tensor] = None, want_lse: bool = False,
        workspace: Optional[torch.Tensor] = None, stream=None):
    """sparse_attn_fwd.  Returns O (and lse when requested or given)."""
    A = _Args()
    tok = _tokens(prob)
    pq = A(Q, "Q", _BF16, shape=tok)
    dev = Q.device
    O = torch.empty(tok, dtype=_BF16, device=dev) if O is None else O
    if want_lse and lse is None:
        lse = torch.empty(prob.B, prob.H, prob.N, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = alloc_workspace(workspace_size(prob, None), dev)
    wp, ws_bytes = _ws(A, workspace)
    _check(A.call(lib.sparse_attn_fwd, ctypes.byref(prob.c()), pq, A(K, "K", _BF16, shape=tok),
                               A(V, "V", _BF16, shape=tok),
                               A(row_ptr, "row_ptr", _I32, numel=prob.rows + 1),
                               A(col_idx, "col_idx", _I32),
                               *_comp_args(A, prob, k_mean, v_sum),
                               A(O, "O", _BF16, shape=tok),
                               A(lse, "lse", _F32, shape=tok[:3], optional=True),
                               wp, ws_bytes, _Stream(stream)))
    return (O, lse) if lse is not None else O


def fwd_prepare(prob: Problem, V: torch.Tensor, row_ptr: torch.Tensor,
                k_mean: Optional[torch.Tensor] = None, v_sum: Optional[torch.Tensor] = None, *,
                workspace: torch.Tensor, stream=None) -> None:
    """sparse_attn_fwd_prepare: V (and the centroids) laid out in ``workspace``.
    V = None: the workspace already starts with V in block layout (written by
    an error-rule ``select`` with ``v_blocks=workspace``)."""
    A = _Args()
    pv = A(V, "V", _BF16, shape=_tokens(prob), optional=True)
    wp, ws_bytes = _ws(A, workspace)
    _check(A.call(lib.sparse_attn_fwd_prepare, ctypes.byref(prob.c()), pv,
                                       A(row_ptr, "row_ptr", _I32, numel=prob.rows + 1),
                                       *_comp_args(A, prob, k_mean, v_sum), wp, ws_bytes,
                                       _Stream(stream)))


def fwd_run(prob: Problem, Q: torch.Tensor, K: torch.Tensor, row_ptr: torch.Tensor,
            col_idx: torch.Tensor, with_comp: bool, *, O: torch.Tensor,
            lse: Optional[torch.Tensor] = None, workspace: torch.Tensor, stream=None) -> None:
    """sparse_attn_fwd_run: the attention kernel on a prepared workspace."""
    A = _Args()
    tok = _tokens(prob)
    pq = A(Q, "Q", _BF16, shape=tok)
    dev = Q.device
    wp, ws_bytes = _ws(A, workspace)
    _check(A.call(lib.sparse_attn_fwd_run, ctypes.byref(prob.c()), pq, A(K, "K", _BF16, shape=tok),
                                   A(row_ptr, "row_ptr", _I32, numel=prob.rows + 1),
                                   A(col_idx, "col_idx", _I32), int(bool(with_comp)),
                                   A(O, "O", _BF16, shape=tok),
                                   A(lse, "lse", _F32, shape=tok[:3], optional=True),
                                   wp, ws_bytes, _Stream(stream)))


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
    A = _Args()
    pv = A(V, "V", _BF16, shape=_tokens(prob))
    dev = V.device
    wp, ws_bytes = _ws(A, workspace)
    _check(A.call(lib.sparse_attn_fwd_prepare_counts, ctypes.byref(prob.c()), pv, A(row_ptr, "row_ptr", _I32, numel=prob.rows + 1),
        *_comp_args(A, prob, k_mean, v_sum),
        A(kv_count, "kv_count", _I32, numel=prob.B * prob.H * prob.nb),
        wp, ws_bytes, _Stream(stream)))


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
    ticket: Optional[float] = None             # tiles: SICS ticket in [-1, 1], or none
    tile_coherence: Optional[torch.Tensor] = None  # tiles + ticket: fp64 [B*H, n_shapes, C]

    def c(self) -> SaClusterSpec:
        if self.shape_idx is not None:
            _Args()(self.shape_idx, "shape_idx", _I32)
        if (self.ticket is None) != (self.tile_coherence is None):
            raise ValueError("a SICS ticket and tile_coherence go together")
        if self.tile_coherence is not None:
            _Args()(self.tile_coherence, "tile_coherence", torch.float64)
        n, sp = 0, None
        if self.shapes:
            arr = (SaTileShape * len(self.shapes))(*[SaTileShape(*map(int, s)) for s in self.shapes])
            self._shape_arr = arr                  # lives as long as the spec
            sp = ctypes.cast(arr, ctypes.POINTER(SaTileShape))
            n = len(self.shapes)
        return SaClusterSpec(CLUSTER_MODES[self.mode], self.n_clusters, self.iters, n, sp,
                             None if self.shape_idx is None else self.shape_idx.data_ptr(),
                             0.0 if self.ticket is None else float(self.ticket),
                             None if self.tile_coherence is None else self.tile_coherence.data_ptr())


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
    A = _Args()
    nbp, ws_c, _ = cluster_size(prob, cspec)
    if out is None:
        out = Clusters.empty(prob, cspec, nbp, V is not None, Q.device)
    if workspace is None:
        workspace = alloc_workspace(ws_c, Q.device)
    dev, tok = Q.device, _tokens(prob)
    BH, C, Np = prob.B * prob.H, cspec.n_clusters, nbp * prob.block
    if cspec.shape_idx is not None:
        A(cspec.shape_idx, "shape_idx", _I32, shape=(BH,))
    args = [A(Q, "Q", _BF16, shape=tok), A(K, "K", _BF16, shape=tok),
            A(V, "V", _BF16, shape=tok, optional=True)]
    args += [A(getattr(out, f), f, _I32, shape=(BH, Np)) for f in ("q_order", "k_order")]
    args += [A(getattr(out, f), f, _I32, shape=(BH, nbp))
             for f in ("q_blk", "k_blk", "q_cnt", "k_cnt")]
    args += [A(getattr(out, f), f, _F32, shape=(BH, C, prob.d)) for f in ("q_cent", "k_cent")]
    args += [A(out.v_cent if V is not None else None, "v_cent", _F32, shape=(BH, C, prob.d), optional=V is None)]
    args += [A(getattr(out, f), f, _I32, shape=(BH, C)) for f in ("q_count", "k_count")]
    wp, ws_bytes = _ws(A, workspace)
    _check(A.call(lib.sparse_attn_cluster, ctypes.byref(prob.c()), ctypes.byref(cspec.c()), *args, wp,
                                   ws_bytes, _Stream(stream)))
    return out


def _padded_rows(prob: Problem, cspec: ClusterSpec) -> int:
    return cluster_size(prob, cspec)[0] * prob.block


def cluster_gather(prob: Problem, cspec: ClusterSpec, order: torch.Tensor, src: torch.Tensor,
                   dst: torch.Tensor, stream=None) -> torch.Tensor:
    """sparse_attn_cluster_gather: rows of src [B,H,N,d] into the padded layout dst
    [B,H,Np,d] (zero rows for padding)."""
    A = _Args()
    Np, dev = _padded_rows(prob, cspec), src.device
    _check(A.call(lib.sparse_attn_cluster_gather, ctypes.byref(prob.c()), ctypes.byref(cspec.c()),
        A(order, "order", _I32, shape=(prob.B * prob.H, Np)),
        A(src, "src", _BF16, shape=_tokens(prob)),
        A(dst, "dst", _BF16, shape=_tokens(prob, Np)), _Stream(stream)))
    return dst


def cluster_scatter(prob: Problem, cspec: ClusterSpec, order: torch.Tensor, src: torch.Tensor,
                    dst: torch.Tensor, lse_src: Optional[torch.Tensor] = None,
                    lse_dst: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """sparse_attn_cluster_scatter: rows of the padded layout back to token order."""
    A = _Args()
    Np, dev = _padded_rows(prob, cspec), src.device
    _check(A.call(lib.sparse_attn_cluster_scatter, ctypes.byref(prob.c()), ctypes.byref(cspec.c()),
        A(order, "order", _I32, shape=(prob.B * prob.H, Np)),
        A(src, "src", _BF16, shape=_tokens(prob, Np)),
        A(dst, "dst", _BF16, shape=_tokens(prob)),
        A(lse_src, "lse_src", _F32, shape=(prob.B, prob.H, Np), optional=True),
        A(lse_dst, "lse_dst", _F32, shape=(prob.B, prob.H, prob.N), optional=True),
        _Stream(stream)))
    return dst


def cluster_fwd_prepare(prob: Problem, cspec: ClusterSpec, k_order: torch.Tensor, V: torch.Tensor,
                        row_ptr: torch.Tensor, kv_count: torch.Tensor,
                        k_mean: Optional[torch.Tensor] = None, v_sum: Optional[torch.Tensor] = None,
                        *, workspace: torch.Tensor, stream=None) -> None:
    """sparse_attn_cluster_fwd_prepare: fwd_prepare_counts over the padded
    clustered layout with V read in token order through k_order."""
    A = _Args()
    Np = _padded_rows(prob, cspec)
    pp = padded_problem(prob, Np // prob.block)
    wp, ws_bytes = _ws(A, workspace)
    _check(A.call(lib.sparse_attn_cluster_fwd_prepare, ctypes.byref(prob.c()), ctypes.byref(cspec.c()),
        A(k_order, "k_order", _I32, shape=(prob.B * prob.H, Np)),
        A(V, "V", _BF16, shape=_tokens(prob)),
        A(row_ptr, "row_ptr", _I32, numel=pp.rows + 1),
        *_comp_args(A, pp, k_mean, v_sum),
        A(kv_count, "kv_count", _I32, numel=pp.B * pp.H * pp.nb),
        wp, ws_bytes, _Stream(stream)))


def cluster_fwd_run(prob: Problem, cspec: ClusterSpec, q_order: torch.Tensor, Q: torch.Tensor,
                    Kp: torch.Tensor, row_ptr: torch.Tensor, col_idx: torch.Tensor,
                    with_comp: bool, *, O: torch.Tensor, lse: Optional[torch.Tensor] = None,
                    workspace: torch.Tensor, stream=None) -> torch.Tensor:
    """sparse_attn_cluster_fwd_run: the attention over the padded clustered
    layout (Kp gathered, the workspace prepared for the padded problem) with Q
    read and O, lse written in token order through q_order."""
    A = _Args()
    Np = _padded_rows(prob, cspec)
    tok = _tokens(prob)
    wp, ws_bytes = _ws(A, workspace)
    _check(A.call(lib.sparse_attn_cluster_fwd_run, ctypes.byref(prob.c()), ctypes.byref(cspec.c()),
        A(q_order, "q_order", _I32, shape=(prob.B * prob.H, Np)),
        A(Q, "Q", _BF16, shape=tok), A(Kp, "Kp", _BF16, shape=_tokens(prob, Np)),
        A(row_ptr, "row_ptr", _I32, numel=prob.B * prob.H * (Np // prob.block) + 1),
        A(col_idx, "col_idx", _I32), int(bool(with_comp)),
        A(O, "O", _BF16, shape=tok), A(lse, "lse", _F32, shape=tok[:3], optional=True),
        wp, ws_bytes, _Stream(stream)))
    return O


def cluster_select(prob: Problem, cspec: ClusterSpec, spec: SelectSpec, cl: Clusters, *,
                   out: Optional[Selection] = None, want_scores: bool = False,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> Selection:
    """sparse_attn_cluster_select: keep decision over clusters as CSR over the
    padded blocks (+ per-block compensation statistics with want_comp)."""
    A = _Args()
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
    wp, ws_bytes = _ws(A, workspace)
    cs, keep = spec.c()
    cen, stat = (BH, C, prob.d), (prob.B, prob.H, nbp, prob.d)
    _check(A.call(lib.sparse_attn_cluster_select, ctypes.byref(prob.c()), ctypes.byref(cspec.c()), ctypes.byref(cs),
        A(cl.q_cent, "q_cent", _F32, shape=cen),
        A(cl.k_cent, "k_cent", _F32, shape=cen),
        A(cl.v_cent, "v_cent", _F32, shape=cen, optional=True),
        A(cl.k_count, "k_count", _I32, shape=(BH, C)),
        A(cl.q_blk, "q_blk", _I32, shape=(BH, nbp)),
        A(cl.k_blk, "k_blk", _I32, shape=(BH, nbp)),
        A(cl.k_cnt, "k_cnt", _I32, shape=(BH, nbp)),
        A(out.row_ptr, "row_ptr", _I32, numel=rows + 1),
        A(out.col_idx, "col_idx", _I32, numel=rows * nbp),
        A(out.scores, "scores", _F32, numel=BH * C * C, optional=True),
        A(out.k_mean, "k_mean", _F32, shape=stat, optional=True),
        A(out.v_sum, "v_sum", _F32, shape=stat, optional=True),
        wp, ws_bytes, _Stream(stream)))
    return out


def cluster_centroids(prob: Problem, cspec: ClusterSpec, Kp: torch.Tensor, Vp: torch.Tensor,
                      cl: Clusters, k_mean: torch.Tensor, v_sum: torch.Tensor,
                      stream=None) -> None:
    """sparse_attn_cluster_centroids: key / value means of the kept partition
    from this call's K, V in the padded layout (into cl.k_cent, cl.v_cent) and
    the per-block compensation statistics."""
    A = _Args()
    nbp = cluster_size(prob, cspec)[0]
    BH, C, dev = prob.B * prob.H, cspec.n_clusters, Kp.device
    ptok, cen, stat = _tokens(prob, nbp * prob.block), (BH, C, prob.d), (prob.B, prob.H, nbp, prob.d)
    _check(A.call(lib.sparse_attn_cluster_centroids, ctypes.byref(prob.c()), ctypes.byref(cspec.c()), A(Kp, "Kp", _BF16, shape=ptok),
        A(Vp, "Vp", _BF16, shape=ptok),
        A(cl.k_count, "k_count", _I32, shape=(BH, C)),
        A(cl.k_blk, "k_blk", _I32, shape=(BH, nbp)),
        A(cl.k_cnt, "k_cnt", _I32, shape=(BH, nbp)),
        A(cl.k_cent, "k_cent", _F32, shape=cen),
        A(cl.v_cent, "v_cent", _F32, shape=cen),
        A(k_mean, "k_mean", _F32, shape=stat),
        A(v_sum, "v_sum", _F32, shape=stat), _Stream(stream)))


def sics(prob: Problem, cspec: ClusterSpec, Q: torch.Tensor, K: torch.Tensor,
         shape_idx: torch.Tensor, scores: Optional[torch.Tensor] = None, *,
         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """sparse_attn_sics: per (b, h) the tile shape of the menu with the most
    coherent tiles (mean intra-tile cosine of Q and K) into shape_idx (device
    int32 [B*H]); scores (device fp64 [B*H, n_shapes]) if given."""
    A = _Args()
    if workspace is None:
        workspace = alloc_workspace(cluster_size(prob, cspec)[1], Q.device)
    dev, tok, BH = Q.device, _tokens(prob), prob.B * prob.H
    wp, ws_bytes = _ws(A, workspace)
    _check(A.call(lib.sparse_attn_sics, ctypes.byref(prob.c()), ctypes.byref(cspec.c()), A(Q, "Q", _BF16, shape=tok),
        A(K, "K", _BF16, shape=tok),
        A(scores, "scores", torch.float64, shape=(BH, len(cspec.shapes or ())),
             optional=True),
        A(shape_idx, "shape_idx", _I32, shape=(BH,)), wp, ws_bytes,
        _Stream(stream)))
    return shape_idx


def cluster_spec_for(wl) -> ClusterSpec:
    """Cluster spec of a workload description (cluster, n_clusters, cluster_iters,
    tile_shapes)."""
    if wl.cluster == "tiles":
        return ClusterSpec("tiles", wl.n_clusters, 0, shapes=[tuple(s) for s in wl.tile_shapes],
                           ticket=wl.sics_ticket)
    return ClusterSpec(wl.cluster, wl.n_clusters, wl.cluster_iters)
