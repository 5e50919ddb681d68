"""The C ABI on a host without a GPU: the library loads, exports every entry
point the header declares, rejects malformed calls before any HIP call, and
its host-side Hilbert order equals the oracle's."""
import ctypes
import os
import re

import numpy as np
import pytest

import block_sparse_attention_hilbert_amd as sa
import oracle
from conftest import ROOT


def _header_functions():
    text = open(os.path.join(ROOT, "include", "sparse_attn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:sa_status|const char\*)\s+(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    names = _header_functions()
    assert set(names) == set(sa.EXPORTS)
    lib = ctypes.CDLL(sa.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


@pytest.mark.parametrize("grid", [(21, 30, 52), (4, 8, 8), (3, 10, 13), (1, 1, 1),
                                  (126, 30, 52), (5, 1, 9), (21, 45, 80)])
def test_hilbert_order_matches_oracle(grid):
    perm, inv = sa.hilbert_perm_build(*grid)
    operm, oinv = oracle.hilbert_perm(*grid)
    assert np.array_equal(perm, operm) and np.array_equal(inv, oinv)


def _err(fn, *a, **k):
    with pytest.raises(sa.SparseAttnError) as e:
        fn(*a, **k)
    return e.value.status


GOOD = dict(B=1, H=2, N=390, d=128, T=3, Hg=10, W=13, block=128)


def _prob(**kw):
    p = dict(GOOD)
    p.update(kw)
    return sa.Problem(**p)


def test_problem_validation():
    assert _err(sa.workspace_size, _prob(d=96)) == sa.SA_ERR_UNSUPPORTED
    assert _err(sa.workspace_size, _prob(block=32)) == sa.SA_ERR_UNSUPPORTED
    assert _err(sa.workspace_size, _prob(N=391)) == sa.SA_ERR_INVALID_ARG
    assert _err(sa.workspace_size, _prob(B=0)) == sa.SA_ERR_INVALID_ARG
    assert _err(sa.workspace_size, _prob(T=0, N=0)) == sa.SA_ERR_INVALID_ARG
    assert _err(sa.workspace_size, _prob(scale=float("inf"))) == sa.SA_ERR_INVALID_ARG
    with pytest.raises(sa.SparseAttnError, match="d = 96"):
        sa.workspace_size(_prob(d=96))
    n = ctypes.c_size_t(0)
    assert sa.lib.sparse_attn_workspace_size(None, None, ctypes.byref(n)) == sa.SA_ERR_INVALID_ARG
    assert b"prob is NULL" in sa.lib.sparse_attn_last_error()


def test_spec_validation():
    p = _prob()
    bad = [sa.SelectSpec(rule="topk"),                               # no k, no density
           sa.SelectSpec(rule="topk", topk=[0, 1]),
           sa.SelectSpec(rule="topk", density=[0.0, 0.5]),
           sa.SelectSpec(rule="topk", density=[0.5, 1.5]),
           sa.SelectSpec(rule="mass", mass=0.0),
           sa.SelectSpec(rule="mass", mass=1.5),
           sa.SelectSpec(rule="mass", sub_block=48),
           sa.SelectSpec(rule="mass", sub_block=8),
           sa.SelectSpec(rule="mass", sub_block=256),
           sa.SelectSpec(rule="none", window_frames=-2),
           sa.SelectSpec(rule="none", n_anchors=5),               # nb = 4
           sa.SelectSpec(rule="none", n_anchors=1, anchor_offset=-1),
           sa.SelectSpec(rule="err", density=[0.5, 0.5]),                 # no compensation
           sa.SelectSpec(rule="err", want_comp=True),                     # no k, no density
           sa.SelectSpec(rule="err", density=[0.5, 0.5], want_comp=True, sub_block=16)]
    for s in bad:
        assert _err(sa.workspace_size, p, s) == sa.SA_ERR_INVALID_ARG, s
    big = sa.Problem(1, 1, 4097 * 64, 64, 4097, 1, 64, 64)
    assert _err(sa.workspace_size, big, sa.SelectSpec(rule="mass")) == sa.SA_ERR_UNSUPPORTED
    assert sa.workspace_size(big, sa.SelectSpec(rule="none", window_frames=1)) > 0


def test_workspace_sizes_are_consistent():
    p = _prob()
    a = sa.workspace_size(p, sa.SelectSpec(rule="mass"))
    b = sa.workspace_size(p, sa.SelectSpec(rule="mass", sub_block=16))
    c = sa.workspace_size(p, sa.SelectSpec(rule="none", window_frames=1))
    assert 0 < c < a < b
    # the error rule adds V re-laid out per block and its keys to the topk layout
    t = sa.workspace_size(p, sa.SelectSpec(rule="topk", topk=[1, 1], want_comp=True))
    e = sa.workspace_size(p, sa.SelectSpec(rule="err", topk=[1, 1], want_comp=True))
    assert e == t + 2 * 4 * 128 * 128 * 2 + 256           # keys: 128 bytes rounded up to 256
    # V re-laid out per block [B*H*nb*d*block] bf16 + centroid keys [B*H*nb*d]
    # + centroid values in tiles of `block` blocks [B*H*ceil(nb/block)*d*block]
    BH, nb, d, blk = 2, 4, 128, 128
    # (plus 256 bytes of row-schedule counters and 256 bytes of block token
    # counts, int16 [B*H*nb] rounded up)
    assert sa.workspace_size(p) == 512 + 2 * (BH * nb * d * blk + BH * nb * d + BH * 1 * d * blk)


def test_select_and_fwd_reject_before_any_launch():
    """Null / misaligned pointers and small workspaces fail on the host."""
    p = _prob().c()
    spec, keep = sa.SelectSpec(rule="mass").c()
    vp = ctypes.c_void_p
    fake = vp(1 << 20)                 # never dereferenced: validation fails first
    odd = vp((1 << 20) + 8)
    st = sa.lib.sparse_attn_select(ctypes.byref(p), ctypes.byref(spec), None, None, None,
                                   fake, fake, None, None, None, fake, 1 << 30, None)
    assert st == sa.SA_ERR_INVALID_ARG
    st = sa.lib.sparse_attn_select(ctypes.byref(p), ctypes.byref(spec), odd, fake, None,
                                   fake, fake, None, None, None, fake, 1 << 30, None)
    assert st == sa.SA_ERR_INVALID_ARG
    st = sa.lib.sparse_attn_select(ctypes.byref(p), ctypes.byref(spec), fake, fake, None,
                                   fake, fake, None, None, None, fake, 16, None)
    assert st == sa.SA_ERR_WORKSPACE
    st = sa.lib.sparse_attn_select(ctypes.byref(p), ctypes.byref(spec), fake, fake, None,
                                   fake, fake, None, None, None, vp((1 << 20) + 64), 1 << 30, None)
    assert st == sa.SA_ERR_WORKSPACE
    comp, keep2 = sa.SelectSpec(rule="mass", want_comp=True).c()
    st = sa.lib.sparse_attn_select(ctypes.byref(p), ctypes.byref(comp), fake, fake, None,
                                   fake, fake, None, None, None, fake, 1 << 30, None)
    assert st == sa.SA_ERR_INVALID_ARG
    # fwd
    st = sa.lib.sparse_attn_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None,
                                fake, None, fake, 1 << 30, None)
    assert st == sa.SA_ERR_INVALID_ARG                     # k_mean without v_sum
    st = sa.lib.sparse_attn_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake,
                                fake, None, None, 0, None)
    assert st == sa.SA_ERR_WORKSPACE
    st = sa.lib.sparse_attn_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, None, None,
                                fake, None, fake, 1024, None)
    assert st == sa.SA_ERR_WORKSPACE
    st = sa.lib.sparse_attn_fwd(ctypes.byref(p), fake, fake, fake, None, fake, None, None,
                                fake, None, None, 0, None)
    assert st == sa.SA_ERR_INVALID_ARG
    # permute: overlap
    st = sa.lib.hilbert_permute(ctypes.byref(p), fake, vp((1 << 20) + 16), fake, None)
    assert st == sa.SA_ERR_INVALID_ARG
    assert sa.lib.hilbert_perm_build(0, 1, 1, None, None) == sa.SA_ERR_INVALID_ARG
    assert sa.lib.hilbert_perm_build(300, 1, 1, None, None) == sa.SA_ERR_UNSUPPORTED


def test_fwd_halves_reject_before_any_launch():
    p = _prob().c()
    vp = ctypes.c_void_p
    fake = vp(1 << 20)
    odd = vp((1 << 20) + 8)
    prep, run = sa.lib.sparse_attn_fwd_prepare, sa.lib.sparse_attn_fwd_run
    # (V = NULL is accepted: the workspace then already holds V in block layout)
    assert prep(ctypes.byref(p), odd, fake, None, None, fake, 1 << 30, None) == sa.SA_ERR_INVALID_ARG
    assert prep(ctypes.byref(p), fake, None, None, None, fake, 1 << 30, None) == sa.SA_ERR_INVALID_ARG
    assert prep(ctypes.byref(p), fake, fake, fake, None, fake, 1 << 30, None) == sa.SA_ERR_INVALID_ARG
    assert prep(ctypes.byref(p), fake, fake, None, None, fake, 16, None) == sa.SA_ERR_WORKSPACE
    assert run(ctypes.byref(p), fake, fake, fake, fake, 2, fake, None, fake, 1 << 30,
               None) == sa.SA_ERR_INVALID_ARG
    assert run(ctypes.byref(p), None, fake, fake, fake, 0, fake, None, fake, 1 << 30,
               None) == sa.SA_ERR_INVALID_ARG
    assert run(ctypes.byref(p), fake, fake, fake, None, 0, fake, None, fake, 1 << 30,
               None) == sa.SA_ERR_INVALID_ARG
    # the compensation workspace is larger than the plain one
    need = sa.workspace_size(_prob())
    assert run(ctypes.byref(p), fake, fake, fake, fake, 1, fake, None, fake, need - 256,
               None) == sa.SA_ERR_WORKSPACE


def test_centroids_reject_before_any_launch():
    p = _prob().c()
    vp = ctypes.c_void_p
    fake, odd = vp(1 << 20), vp((1 << 20) + 8)
    assert sa.lib.sparse_attn_centroids(ctypes.byref(p), None, fake, fake, fake, None) == \
        sa.SA_ERR_INVALID_ARG
    assert b"required" in sa.lib.sparse_attn_last_error()
    assert sa.lib.sparse_attn_centroids(ctypes.byref(p), fake, fake, fake, None, None) == \
        sa.SA_ERR_INVALID_ARG
    assert sa.lib.sparse_attn_centroids(ctypes.byref(p), fake, odd, fake, fake, None) == \
        sa.SA_ERR_INVALID_ARG
    assert b"aligned" in sa.lib.sparse_attn_last_error()
    bad = _prob(N=391).c()
    assert sa.lib.sparse_attn_centroids(ctypes.byref(bad), fake, fake, fake, fake, None) == \
        sa.SA_ERR_INVALID_ARG


def test_reuse_policy_needs_a_first_selection():
    from block_sparse_attention_hilbert_amd.pipeline import BlockSparseAttention
    with pytest.raises(ValueError):
        BlockSparseAttention(_prob(), sa.SelectSpec(rule="mass"), device="cpu", refresh_every=0)



def test_cluster_sizes_and_validation():
    """Data-dependent block formation: sizes of the padded layout and the
    workspaces, and every malformed call rejected on the host."""
    p = sa.Problem(1, 12, 32760, 128, 21, 30, 52, 128)
    nbp, wc, ws = sa.cluster_size(p, sa.ClusterSpec("kmeans", 64, 3))
    assert nbp == 256 + 64
    # assignment + sorted order of both sides (int32 [BH, N]) dominate the workspace
    assert wc >= 4 * 12 * 32760 * 4
    assert ws >= 12 * 64 * 64 * 5
    small = _prob()
    for cs, code in [(sa.ClusterSpec("kmeans", 0, 1), sa.SA_ERR_INVALID_ARG),
                     (sa.ClusterSpec("kmeans", 391, 1), sa.SA_ERR_INVALID_ARG),   # > N
                     (sa.ClusterSpec("kmeans", 4, 0), sa.SA_ERR_INVALID_ARG),
                     (sa.ClusterSpec("kmeans", 4, 65), sa.SA_ERR_INVALID_ARG)]:
        assert _err(sa.cluster_size, small, cs) == code, cs
    bad_mode = sa.SaClusterSpec(7, 4, 1)
    assert sa.lib.sparse_attn_cluster_size(ctypes.byref(small.c()), ctypes.byref(bad_mode),
                                           None, None, None) == sa.SA_ERR_INVALID_ARG
    big = sa.Problem(1, 1, 4090 * 64, 64, 4090, 1, 64, 64)
    assert _err(sa.cluster_size, big, sa.ClusterSpec("kmeans", 16, 1)) == sa.SA_ERR_UNSUPPORTED


def test_select_v_blocks_validation_and_sizes():
    """The error rule's V layout can go to the caller's buffer (the start of a
    forward workspace): the selection workspace then shrinks by exactly that
    layout; v_blocks is rejected for the other rules and when misaligned, and
    the forward workspace starts with the layout."""
    p = _prob(N=1024, T=8, Hg=8, W=16, H=3)           # nb = 8
    err = sa.SelectSpec(rule="err", topk=[2, 2, 2], want_comp=True)
    layout = p.B * p.H * p.nb * p.d * p.block * 2
    full = sa.workspace_size(p, err)
    shared = sa.workspace_size(p, err, v_blocks=True)
    assert full - shared == layout
    # the forward workspace holds the layout first, so it is at least that big
    assert sa.workspace_size(p) >= layout
    vp = ctypes.c_void_p
    fake = vp(1 << 20)
    raw = p.c()
    n = ctypes.c_size_t(0)
    mass, keep = sa.SelectSpec(rule="mass").c(1 << 20)
    assert sa.lib.sparse_attn_workspace_size(ctypes.byref(raw), ctypes.byref(mass),
                                             ctypes.byref(n)) == sa.SA_ERR_INVALID_ARG
    odd, keep2 = err.c((1 << 20) + 128)
    assert sa.lib.sparse_attn_workspace_size(ctypes.byref(raw), ctypes.byref(odd),
                                             ctypes.byref(n)) == sa.SA_ERR_INVALID_ARG
    # the same checks on the selection call itself, before anything is launched
    st = sa.lib.sparse_attn_select(ctypes.byref(raw), ctypes.byref(odd), fake, fake, fake,
                                   fake, fake, None, fake, fake, fake, 1 << 30, None)
    assert st == sa.SA_ERR_INVALID_ARG
    st = sa.lib.sparse_attn_select(ctypes.byref(raw), ctypes.byref(mass), fake, fake, None,
                                   fake, fake, None, None, None, fake, 1 << 30, None)
    assert st == sa.SA_ERR_INVALID_ARG


def test_sics_ticket_validation():
    """The SICS ticket is opt-in through tile_coherence: without the buffer
    the ticket field is never read; with it the ticket must lie in [-1, 1],
    and the selection needs the chosen shapes."""
    small = _prob()                                   # grid 3 x 10 x 13
    menu = [(1, 4, 16), (1, 8, 8)]                    # 3*3*1 and 3*2*2 tiles
    spec = sa.ClusterSpec("tiles", 12, 0, shapes=menu)
    sa.cluster_size(small, spec)
    raw = spec.c()
    size = sa.lib.sparse_attn_cluster_size
    for t in (float("nan"), 1.5, -1.25, float("inf")):
        raw.ticket = t
        raw.tile_coherence = None                     # no buffer: no ticket, accepted
        assert size(ctypes.byref(small.c()), ctypes.byref(raw), None, None, None) == sa.SA_OK
        raw.tile_coherence = 1 << 20
        assert size(ctypes.byref(small.c()), ctypes.byref(raw), None, None, None) == \
            sa.SA_ERR_INVALID_ARG, t
    for t in (-1.0, 0.0, 0.72, 1.0):
        raw.ticket = t
        assert size(ctypes.byref(small.c()), ctypes.byref(raw), None, None, None) == sa.SA_OK, t
    raw.tile_coherence = (1 << 20) + 4                # not 8-byte aligned
    assert size(ctypes.byref(small.c()), ctypes.byref(raw), None, None, None) == sa.SA_ERR_INVALID_ARG
    raw.tile_coherence = 1 << 20
    # the selection with a ticket but no shape_idx is refused before any launch
    raw.ticket, raw.shape_idx = 0.5, None
    fake = ctypes.c_void_p(1 << 20)
    sel, _keep = sa.SelectSpec(rule="mass").c()
    call = sa.lib.sparse_attn_cluster_select
    args = [*([fake] * 9), None, None, None, fake, 1 << 30, None]
    assert call(ctypes.byref(small.c()), ctypes.byref(raw), ctypes.byref(sel), *args) == \
        sa.SA_ERR_INVALID_ARG
    assert b"shape_idx" in sa.lib.sparse_attn_last_error()
    # the binding wants both or neither
    with pytest.raises(ValueError):
        sa.ClusterSpec("tiles", 12, 0, shapes=menu, ticket=0.5).c()


def test_cluster_calls_reject_before_any_launch():
    p = _prob().c()
    cs = sa.ClusterSpec("cocluster", 4, 2).c()
    vp = ctypes.c_void_p
    fake, odd = vp(1 << 20), vp((1 << 20) + 8)
    outs = [fake] * 10
    cl = sa.lib.sparse_attn_cluster
    assert cl(ctypes.byref(p), ctypes.byref(cs), None, fake, None, *outs[:8], None, *outs[:2],
              fake, 1 << 30, None) == sa.SA_ERR_INVALID_ARG            # no Q
    assert cl(ctypes.byref(p), ctypes.byref(cs), odd, fake, None, *outs[:8], None, *outs[:2],
              fake, 1 << 30, None) == sa.SA_ERR_INVALID_ARG            # misaligned
    assert cl(ctypes.byref(p), ctypes.byref(cs), fake, fake, fake, *outs[:8], None, *outs[:2],
              fake, 1 << 30, None) == sa.SA_ERR_INVALID_ARG            # V without v_cent
    assert cl(ctypes.byref(p), ctypes.byref(cs), fake, fake, None, *outs[:8], None, *outs[:2],
              fake, 64, None) == sa.SA_ERR_WORKSPACE
    assert cl(ctypes.byref(p), ctypes.byref(cs), fake, fake, None, *outs[:8], None, *outs[:2],
              vp((1 << 20) + 64), 1 << 30, None) == sa.SA_ERR_WORKSPACE
    # gather / scatter: overlap, missing order, lse pairs
    g, s = sa.lib.sparse_attn_cluster_gather, sa.lib.sparse_attn_cluster_scatter
    assert g(ctypes.byref(p), ctypes.byref(cs), None, fake, vp(1 << 30), None) == \
        sa.SA_ERR_INVALID_ARG
    assert g(ctypes.byref(p), ctypes.byref(cs), fake, fake, vp((1 << 20) + 4096), None) == \
        sa.SA_ERR_INVALID_ARG
    assert b"overlap" in sa.lib.sparse_attn_last_error()
    assert s(ctypes.byref(p), ctypes.byref(cs), fake, fake, vp(1 << 30), fake, None, None) == \
        sa.SA_ERR_INVALID_ARG
    # selection over clusters: supported rules and structure only
    sel = sa.lib.sparse_attn_cluster_select
    ptrs = [fake] * 7 + [fake, fake]
    for spec, code in [(sa.SelectSpec(rule="none"), sa.SA_ERR_UNSUPPORTED),
                       (sa.SelectSpec(rule="err", density=[0.2, 0.2], want_comp=True),
                        sa.SA_ERR_UNSUPPORTED),
                       (sa.SelectSpec(rule="topk", topk=[1, 1]), sa.SA_ERR_UNSUPPORTED),
                       (sa.SelectSpec(rule="topk"), sa.SA_ERR_INVALID_ARG),
                       (sa.SelectSpec(rule="mass", sub_block=16), sa.SA_ERR_UNSUPPORTED),
                       (sa.SelectSpec(rule="mass", window_frames=1), sa.SA_ERR_UNSUPPORTED),
                       (sa.SelectSpec(rule="mass", n_anchors=1), sa.SA_ERR_UNSUPPORTED),
                       (sa.SelectSpec(rule="mass", mass=0.0), sa.SA_ERR_INVALID_ARG),
                       (sa.SelectSpec(rule="mass", want_comp=True), sa.SA_ERR_INVALID_ARG)]:
        c, keep = spec.c()
        st = sel(ctypes.byref(p), ctypes.byref(cs), ctypes.byref(c), *ptrs, None, None, None,
                 fake, 1 << 30, None)
        assert st == code, spec
    c, keep = sa.SelectSpec(rule="mass").c()
    assert sel(ctypes.byref(p), ctypes.byref(cs), ctypes.byref(c), *ptrs, None, None, None,
               fake, 8, None) == sa.SA_ERR_WORKSPACE
    # attention over the padded layout through q_order: map, operands, flags, workspace
    run = sa.lib.sparse_attn_cluster_fwd_run
    assert run(ctypes.byref(p), ctypes.byref(cs), None, fake, fake, fake, fake, 0, fake, None,
               fake, 1 << 30, None) == sa.SA_ERR_INVALID_ARG                 # no q_order
    assert run(ctypes.byref(p), ctypes.byref(cs), fake, odd, fake, fake, fake, 0, fake, None,
               fake, 1 << 30, None) == sa.SA_ERR_INVALID_ARG                 # misaligned Q
    assert run(ctypes.byref(p), ctypes.byref(cs), fake, fake, fake, fake, fake, 2, fake, None,
               fake, 1 << 30, None) == sa.SA_ERR_INVALID_ARG                 # with_comp
    assert run(ctypes.byref(p), ctypes.byref(cs), fake, fake, fake, fake, fake, 0, fake, None,
               fake, 16, None) == sa.SA_ERR_WORKSPACE
    # its preparation with V through k_order: map, V, counts, workspace
    cprep = sa.lib.sparse_attn_cluster_fwd_prepare
    assert cprep(ctypes.byref(p), ctypes.byref(cs), None, fake, fake, None, None, fake,
                 fake, 1 << 30, None) == sa.SA_ERR_INVALID_ARG               # no k_order
    assert cprep(ctypes.byref(p), ctypes.byref(cs), fake, odd, fake, None, None, fake,
                 fake, 1 << 30, None) == sa.SA_ERR_INVALID_ARG               # misaligned V
    assert cprep(ctypes.byref(p), ctypes.byref(cs), fake, fake, fake, None, None, None,
                 fake, 1 << 30, None) == sa.SA_ERR_INVALID_ARG               # no counts
    assert cprep(ctypes.byref(p), ctypes.byref(cs), fake, fake, fake, None, None, fake,
                 fake, 16, None) == sa.SA_ERR_WORKSPACE
    # prepare with counts needs the counts
    prep = sa.lib.sparse_attn_fwd_prepare_counts
    assert prep(ctypes.byref(p), fake, fake, None, None, None, fake, 1 << 30, None) == \
        sa.SA_ERR_INVALID_ARG
    assert b"kv_count" in sa.lib.sparse_attn_last_error()


def test_cluster_centroids_reject_before_any_launch():
    p = _prob().c()
    cs = sa.ClusterSpec("kmeans", 4, 2).c()
    vp = ctypes.c_void_p
    fake, odd = vp(1 << 20), vp((1 << 20) + 8)
    f = sa.lib.sparse_attn_cluster_centroids
    assert f(ctypes.byref(p), ctypes.byref(cs), fake, fake, fake, fake, fake, fake, fake, fake,
             None, None) == sa.SA_ERR_INVALID_ARG
    assert f(ctypes.byref(p), ctypes.byref(cs), odd, fake, fake, fake, fake, fake, fake, fake,
             fake, None) == sa.SA_ERR_INVALID_ARG
    assert b"aligned" in sa.lib.sparse_attn_last_error()
    bad = sa.ClusterSpec("kmeans", 0, 2).c()
    assert f(ctypes.byref(p), ctypes.byref(bad), fake, fake, fake, fake, fake, fake, fake, fake,
             fake, None) == sa.SA_ERR_INVALID_ARG


def test_sics_and_tile_mode_reject_before_any_launch():
    p = sa.Problem(1, 2, 390, 128, 3, 10, 13, 64)
    menu = [(1, 4, 16), (1, 8, 8), (2, 4, 8)]
    good = sa.ClusterSpec("tiles", 12, 0, shapes=menu)
    nbp, wc, ws = sa.cluster_size(p, good)
    assert nbp == 12                                   # one block per tile
    vp = ctypes.c_void_p
    fake = vp(1 << 20)
    f = sa.lib.sparse_attn_sics
    for cs, code in [(sa.ClusterSpec("kmeans", 4, 2), sa.SA_ERR_INVALID_ARG),      # not tiles
                     (sa.ClusterSpec("tiles", 11, 0, shapes=menu), sa.SA_ERR_INVALID_ARG),
                     (sa.ClusterSpec("tiles", 12, 0, shapes=menu + [(2, 8, 8)]),
                      sa.SA_ERR_INVALID_ARG),           # 128 tokens > block 64
                     (sa.ClusterSpec("tiles", 12, 0, shapes=[(0, 4, 16)]), sa.SA_ERR_INVALID_ARG),
                     (sa.ClusterSpec("tiles", 12, 0, shapes=[]), sa.SA_ERR_INVALID_ARG)]:
        st = f(ctypes.byref(p.c()), ctypes.byref(cs.c()), fake, fake, None, fake, fake, 1 << 30, None)
        assert st == code, cs
    st = f(ctypes.byref(p.c()), ctypes.byref(good.c()), fake, fake, None, None, fake, 1 << 30, None)
    assert st == sa.SA_ERR_INVALID_ARG                 # no shape_idx output
    st = f(ctypes.byref(p.c()), ctypes.byref(good.c()), fake, fake, None, fake, fake, 64, None)
    assert st == sa.SA_ERR_WORKSPACE
    # the partition call needs the per-head shapes
    outs = [fake] * 10
    st = sa.lib.sparse_attn_cluster(ctypes.byref(p.c()), ctypes.byref(good.c()), fake, fake, None,
                                    *outs[:8], None, *outs[:2], fake, 1 << 30, None)
    assert st == sa.SA_ERR_INVALID_ARG
    assert b"shape_idx" in sa.lib.sparse_attn_last_error()


def test_binding_checks_tensor_arguments():
    """The binding checks what the C library cannot see behind a pointer: the
    dtype, shape, contiguity and device of every tensor, before any call."""
    import torch
    p = _prob()
    tok = (p.B, p.H, p.N, p.d)
    bf = torch.zeros(tok, dtype=torch.bfloat16)
    rp = torch.zeros(p.rows + 1, dtype=torch.int32)
    ci = torch.zeros(p.rows * p.nb, dtype=torch.int32)
    # dtype: an fp16 Q, an int64 row_ptr
    with pytest.raises(TypeError, match="Q must be torch.bfloat16"):
        sa.fwd(p, bf.half(), bf, bf, rp, ci, O=bf, workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(TypeError, match="row_ptr must be torch.int32"):
        sa.fwd_run(p, bf, bf, rp.long(), ci, False, O=bf,
                   workspace=torch.zeros(16, dtype=torch.uint8))
    # shape: a [B,N,H,d] view, an output of the wrong size, a short lse
    with pytest.raises(ValueError, match="K must have shape"):
        sa.fwd_run(p, bf, bf.transpose(1, 2), rp, ci, False, O=bf,
                   workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="O must have shape"):
        sa.fwd_run(p, bf, bf, rp, ci, False, O=bf[:, :, :-1],
                   workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="lse must have shape"):
        sa.fwd_run(p, bf, bf, rp, ci, False, O=bf, lse=torch.zeros(p.B, p.H, p.N - 1),
                   workspace=torch.zeros(16, dtype=torch.uint8))
    # too few elements: row_ptr of rows entries, col_idx of the select output
    with pytest.raises(ValueError, match="row_ptr holds"):
        sa.fwd_run(p, bf, bf, rp[:-1], ci, False, O=bf,
                   workspace=torch.zeros(16, dtype=torch.uint8))
    out = sa.Selection(rp, ci[:-1])
    with pytest.raises(ValueError, match="col_idx holds"):
        sa.select(p, sa.SelectSpec(rule="mass"), bf, bf, out=out,
                  workspace=torch.zeros(16, dtype=torch.uint8))
    # contiguity: a permuted copy with the right shape
    nc = torch.zeros(p.B, p.H, p.d, p.N, dtype=torch.bfloat16).transpose(2, 3)
    assert tuple(nc.shape) == tok and not nc.is_contiguous()
    with pytest.raises(ValueError, match="V must be contiguous"):
        sa.fwd_prepare(p, nc, rp, workspace=torch.zeros(16, dtype=torch.uint8))
    # device: everything right but on the host
    with pytest.raises(ValueError, match="Q must be a GPU tensor"):
        sa.fwd_run(p, bf, bf, rp, ci, False, O=bf, workspace=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="src must be a GPU tensor"):
        sa.hilbert_permute(p, bf, torch.zeros(p.N, dtype=torch.int32), bf.clone())
    with pytest.raises(ValueError, match="perm_dev must have shape"):
        sa.hilbert_permute(p, bf, torch.zeros(p.N - 1, dtype=torch.int32), bf.clone())
    # the workspace is raw bytes
    with pytest.raises(TypeError, match="workspace must be torch.uint8"):
        sa.fwd_prepare(p, bf, rp, workspace=torch.zeros(16, dtype=torch.float32))


def test_pipeline_guards():
    """A latent-frame window needs raster order; graph replays cannot rotate
    the anchors the selection takes by value."""
    from types import SimpleNamespace

    from block_sparse_attention_hilbert_amd.pipeline import BlockSparseAttention, GraphedCall
    with pytest.raises(ValueError, match="raster token order"):
        BlockSparseAttention(_prob(), sa.SelectSpec(rule="none", window_frames=1), hilbert=True,
                             device="cpu")
    fake_pipe = SimpleNamespace(spec=sa.SelectSpec(rule="none", window_frames=1, n_anchors=4))
    with pytest.raises(ValueError, match="rotating anchors"):
        GraphedCall(fake_pipe, None, None, None)


def test_noalloc_select_rejects_beyond_its_scratch():
    """The allocation-free selection holds 64 MiB of scratch per GPU; a
    selection that needs more (the 40-head 720p layer: ~78 MiB) is refused on
    the host, before any HIP call, with a message naming both sizes."""
    import workloads as W
    wl = W.WORKLOADS[3]
    prob = sa.problem_for(wl)
    spec = sa.spec_for(wl)
    need = sa.workspace_size(prob, spec)
    assert need > 64 << 20
    cs, keep = spec.c()
    fake = ctypes.c_void_p(1 << 20)
    st = sa.lib.sparse_attn_select_noalloc(ctypes.byref(prob.c()), ctypes.byref(cs), fake, fake,
                                           None, fake, fake, None, None, None, None)
    assert st == sa.SA_ERR_UNSUPPORTED
    msg = sa.lib.sparse_attn_last_error().decode()
    assert str(need) in msg and str(64 << 20) in msg
    # malformed calls fail the same checks as sparse_attn_select
    st = sa.lib.sparse_attn_select_noalloc(ctypes.byref(_prob().c()), ctypes.byref(cs), None, None,
                                           None, fake, fake, None, None, None, None)
    assert st == sa.SA_ERR_INVALID_ARG


def test_token_order_is_refused_where_unsupported():
    """Only the selection, centroid and forward calls take a token order; the
    others refuse it before any launch, and so does a latent-frame window
    (frames are runs of raster blocks)."""
    p = _prob().c()
    p.token_order = ctypes.c_void_p(1 << 20)       # never dereferenced on the host
    vp = ctypes.c_void_p
    fake = vp(1 << 20)
    st = sa.lib.hilbert_permute(ctypes.byref(p), fake, vp(1 << 30), fake, None)
    assert st == sa.SA_ERR_UNSUPPORTED and b"token_order" in sa.lib.sparse_attn_last_error()
    cs = sa.ClusterSpec("kmeans", 4, 2).c()
    nbp, w1, w2 = ctypes.c_int32(0), ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = sa.lib.sparse_attn_cluster_size(ctypes.byref(p), ctypes.byref(cs), ctypes.byref(nbp),
                                         ctypes.byref(w1), ctypes.byref(w2))
    assert st == sa.SA_ERR_UNSUPPORTED
    spec, keep = sa.SelectSpec(rule="none", window_frames=1).c()
    n = ctypes.c_size_t(0)
    st = sa.lib.sparse_attn_workspace_size(ctypes.byref(p), ctypes.byref(spec), ctypes.byref(n))
    assert st == sa.SA_ERR_UNSUPPORTED and b"window" in sa.lib.sparse_attn_last_error()
    # the forward workspace grows by K in block order
    q = _prob().c()
    base = ctypes.c_size_t(0)
    assert sa.lib.sparse_attn_workspace_size(ctypes.byref(q), None, ctypes.byref(base)) == 0
    assert sa.lib.sparse_attn_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == 0
    g = GOOD
    assert n.value - base.value >= g["B"] * g["H"] * g["N"] * g["d"] * 2
