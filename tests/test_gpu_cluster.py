"""GPU parity of data-dependent block formation (SVOO section 2B co-clustering,
SVG-EAR section 2A k-means), through the C ABI, against the oracle.

Bar:
* cluster sizes, centroids (query, key, value means), the padded layouts
  (slot order, block cluster, block token count), the cluster scores and the
  per-block compensation statistics: bit-exact -- the assignment is a decision
  taken in the same fp32 arithmetic on both sides, means are fp32 roundings of
  exact sums;
* the block-level keep (CSR): bit-exact up to rows excused as near ties
  (cluster scores within 1e-6 of the row's largest |score|, or the cumulative
  weight at the cut within 1e-6 of mass x total), counted and reported;
* attention output in token order, given the oracle's clusters and keep:
  max |err| <= 2e-2, mean |err| <= 2e-3 against the float64 oracle; lse within
  2e-2.
"""
import numpy as np
import pytest

import oracle
from oracle import clusters as OC
from oracle import tiles as OT
import workloads as W
from parity_util import ATOL_MAX, ATOL_MEAN, LSE_ATOL, TIE_REL, from_dev, log, poison, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_hilbert_amd as sa  # noqa: F401  (fails loudly if unbuilt)
    yield


def _pipe(wl, want_lse=True):
    import block_sparse_attention_hilbert_amd as sa
    from block_sparse_attention_hilbert_amd.pipeline import ClusteredAttention
    spec = sa.spec_for(wl)
    if spec.topk is not None:
        raise ValueError("cluster selection takes a density")
    return ClusteredAttention(sa.problem_for(wl), sa.cluster_spec_for(wl), spec,
                              want_scores=True, want_lse=want_lse)


# several clusters, ragged cluster sizes, both head dims and block sizes
BASE = W.WORKLOADS[2].replace(T=3, Hg=10, W=13, H=2)          # N = 390
SMALL = {
    "cocluster_mass_d128_b128": BASE.replace(cluster="cocluster", n_clusters=3, cluster_iters=2),
    "kmeans_topk_comp_d128_b64": BASE.replace(block=64, cluster="kmeans", n_clusters=6,
                                              cluster_iters=3, rule="topk", density=0.3,
                                              comp=True),
    "cocluster_topk_comp_diag_d64_b64": BASE.replace(d=64, block=64, H=3, cluster="cocluster",
                                                     n_clusters=8, cluster_iters=4, rule="topk",
                                                     density=0.25, comp=True, diag=True),
    "kmeans_mass_d64_b128_wide": W.WORKLOADS[2].replace(T=5, Hg=9, W=29, H=2, d=64,
                                                      cluster="kmeans", n_clusters=10,
                                                      cluster_iters=2, mass=0.7),
    "kmeans_one_cluster": BASE.replace(block=64, cluster="kmeans", n_clusters=1,
                                       cluster_iters=1, rule="topk", density=0.5, comp=True),
    "cocluster_iid_many": W.WORKLOADS[1].replace(T=3, Hg=10, W=13, H=2, cluster="cocluster",
                                               n_clusters=40, cluster_iters=2, rule="mass",
                                               mass=0.8, diag=False, comp=True, topk=None),
    # SICS scheme generation over shaped tiles (SPADE parts 1-2), heads of
    # different anisotropy so that they pick different shapes
    "tiles_topk_d128_b64": BASE.replace(H=4, block=64, cluster="tiles", aniso=True,
                                        tile_shapes=((1, 4, 16), (1, 8, 8), (2, 4, 8), (3, 2, 8)),
                                        n_clusters=12, rule="topk", density=0.3),
    "tiles_mass_comp_diag_d64_b128": W.WORKLOADS[2].replace(
        T=5, Hg=9, W=29, H=4, d=64, cluster="tiles", aniso=True,
        tile_shapes=((1, 4, 32), (1, 8, 16), (2, 4, 16), (5, 3, 8)), n_clusters=20,
        mass=0.8, comp=True, diag=True),
    # 64 clusters (the most the matrix-core assignment and the partial-sum
    # means take) on a few hundred tokens: small and empty clusters, both
    # centroid tiles, both head dims
    "kmeans_c64_mass_comp_d64_iid": W.WORKLOADS[1].replace(T=3, Hg=10, W=13, H=2, d=64,
                                                         cluster="kmeans", n_clusters=64,
                                                         cluster_iters=3, rule="mass", mass=0.8,
                                                         diag=False, comp=True, topk=None),
    "cocluster_c64_topk_d128": BASE.replace(cluster="cocluster", n_clusters=64, cluster_iters=3,
                                            rule="topk", density=0.3),
    # fewer tokens than one 32-token group of the assignment (N = 21)
    "kmeans_tiny_d64": BASE.replace(T=1, Hg=3, W=7, H=3, d=64, block=64, cluster="kmeans",
                                    n_clusters=4, cluster_iters=2, rule="topk", density=0.5),
    "cocluster_tiny_d128": BASE.replace(T=1, Hg=3, W=7, H=2, cluster="cocluster", n_clusters=21,
                                        cluster_iters=2, mass=0.9),
    # more than 64 clusters: the assignment's vector-unit path
    "kmeans_c100_mass_comp": BASE.replace(block=64, cluster="kmeans", n_clusters=100,
                                          cluster_iters=2, mass=0.9, comp=True),
    # batches of two
    "kmeans_comp_batch2": BASE.replace(B=2, block=64, cluster="kmeans", n_clusters=6,
                                       cluster_iters=2, rule="topk", density=0.3, comp=True),
    "tiles_topk_batch2": BASE.replace(B=2, H=3, block=64, cluster="tiles", aniso=True,
                                      tile_shapes=((1, 4, 16), (1, 8, 8), (2, 4, 8)),
                                      n_clusters=12, rule="topk", density=0.3),
}
# the SICS ticket: at 0.3 one head admits every tile, two some and one none
# (its rows keep nothing, or only their own tile with the diagonal)
SMALL["tiles_ticket_topk_d128_b64"] = SMALL["tiles_topk_d128_b64"].replace(sics_ticket=0.3)
SMALL["tiles_ticket_mass_comp_diag"] = SMALL["tiles_mass_comp_diag_d64_b128"].replace(
    sics_ticket=0.3)


def _keep_from_csr(rp, ci, rows, nbp):
    keep = np.zeros((rows, nbp), dtype=bool)
    r = np.repeat(np.arange(rows), np.diff(rp))
    keep[r, ci[: rp[-1]]] = True
    return keep


def _excused(S_row, nk, wl, gk, ok):
    """A differing cluster-level row is excused by a near tie of the oracle's
    scores among the swapped clusters or a cumulative weight at the cut within
    1e-6 of the threshold."""
    only_g, only_o = np.nonzero(gk & ~ok)[0], np.nonzero(ok & ~gk)[0]
    s = S_row.astype(np.float64)
    live = np.nonzero(nk > 0)[0]
    tol = TIE_REL * np.max(np.abs(s[live]))
    if only_g.size and only_o.size and all(abs(s[x] - s[y]) <= tol for x in only_g for y in only_o):
        return True
    if wl.rule == "mass":
        order = live[np.argsort(-s[live], kind="stable")]
        w = nk[order] * np.exp(s[order] - s[order[0]])
        cum = np.cumsum(w)
        thr = float(np.float32(wl.mass)) * cum[-1]
        return bool(np.min(np.abs(cum - thr)) <= TIE_REL * cum[-1])
    return False


def check_case(wl, Q, K, V, heads, q_clusters_per_head=None, seed=0):
    """Runs the clustered call on the GPU and checks the heads `heads` (indices
    into b * H + h) against the oracle.  Returns the attention errors.

    In tile mode the oracle picks each head's shape first.  Where the GPU's
    pick differs -- allowed only as a near tie of the two shapes' fp64 scores
    (1e-9 relative) -- the call is run again on the GPU with the oracle's picks
    forced in, so the partition, selection and attention are checked against
    the oracle's own choice (the oracle never takes a value from the GPU)."""
    pipe = _pipe(wl)
    poison(pipe.O, pipe.lse)
    Qd, Kd, Vd = to_dev(Q), to_dev(K), to_dev(V)
    O = pipe(Qd, Kd, Vd)
    torch.cuda.synchronize()
    tiles = wl.cluster == "tiles"
    refs = {}
    excused = 0
    if tiles:
        pick_gpu = pipe.shape_idx.cpu().numpy()
        sc_gpu = pipe.shape_scores.cpu().numpy()
        forced = pick_gpu.copy()
        for bh in heads:
            b, h = divmod(bh, wl.H)
            q, k = oracle.bf16_to_f64(Q[b, h]), oracle.bf16_to_f64(K[b, h])
            ref = OT.tiles_workload_head(wl, q, k)
            tag = f"{wl.name} bh={bh}"
            assert np.allclose(sc_gpu[bh], ref["scores"], rtol=1e-9, atol=1e-12), tag
            if pick_gpu[bh] != ref["pick"]:
                top = ref["scores"]
                assert abs(top[pick_gpu[bh]] - top[ref["pick"]]) <= 1e-9 * np.abs(top).max(), tag
                excused += 1
                forced[bh] = ref["pick"]
            if ref["ticket"] is not None:
                # no tile's coherence may sit on the ticket: then the
                # admission is exact on both sides
                nt = int((ref["nk"] > 0).sum())
                assert np.all(np.abs(ref["coh"][:nt] - ref["ticket"]) > 1e-9), tag
            refs[bh] = ref
        if excused:
            log(f"[cluster] {wl.name}: {excused} near-tie shape picks; rerun with the oracle's")
            pipe.shape_idx.copy_(torch.from_numpy(forced))
            poison(pipe.O, pipe.lse)
            O = pipe(Qd, Kd, Vd, reuse=False, choose_shapes=False)
            torch.cuda.synchronize()
            assert np.array_equal(pipe.shape_idx.cpu().numpy(), forced)
    if tiles and wl.sics_ticket is not None:
        coh_gpu = pipe.tile_coherence.cpu().numpy()
        for bh in heads:
            ref = refs[bh]
            nt = int((ref["nk"] > 0).sum())
            got = coh_gpu[bh, ref["pick"], :nt]
            assert np.allclose(got, ref["coh"][:nt], rtol=1e-9, atol=1e-12), f"{wl.name} bh={bh}"
            log(f"[cluster] {wl.name} bh={bh}: {int(ref['eligible'][:nt].sum())} of {nt} "
                f"tiles admitted by the ticket {ref['ticket']:.3f}")
    assert not np.any((from_dev(O) & 0x7F80) == 0x7F80), "O holds NaN/Inf: rows not written"
    assert not np.any(np.isnan(pipe.lse.cpu().numpy())), "lse holds NaN: rows not written"
    C, nbp, blk = wl.n_clusters, pipe.nbp, wl.block
    cl, sel = pipe.cl, pipe.sel
    g = {k: getattr(cl, k).cpu().numpy() for k in
         ("q_order", "k_order", "q_blk", "k_blk", "q_cnt", "k_cnt", "q_cent", "k_cent",
          "q_count", "k_count")}
    v_cent = cl.v_cent.cpu().numpy() if cl.v_cent is not None else None
    S_gpu = sel.scores.cpu().numpy()
    rp = sel.row_ptr.cpu().numpy().astype(np.int64)
    ci = sel.col_idx.cpu().numpy()
    keep_gpu = _keep_from_csr(rp, ci, wl.B * wl.H * nbp, nbp).reshape(wl.B * wl.H, nbp, nbp)
    for r in range(keep_gpu.shape[0] * nbp):
        cols = ci[rp[r]: rp[r + 1]]
        assert np.all(np.diff(cols) > 0), "CSR rows must be ascending"
    Og = from_dev(O)
    lse_g = pipe.lse.cpu().numpy()
    km = sel.k_mean.cpu().numpy() if sel.k_mean is not None else None
    vs = sel.v_sum.cpu().numpy() if sel.v_sum is not None else None
    rng = np.random.default_rng(seed)
    errs, lse_errs = [], []
    picks = []
    for bh in heads:
        b, h = divmod(bh, wl.H)
        q = oracle.bf16_to_f64(Q[b, h])
        k = oracle.bf16_to_f64(K[b, h])
        v = oracle.bf16_to_f64(V[b, h])
        tag = f"{wl.name} bh={bh}"
        if tiles:
            ref = refs[bh]
            picks.append(int(ref["pick"]))
        else:
            ref = OC.cluster_workload_head(wl, q, k)
        assert np.array_equal(g["q_count"][bh], ref["nq"]), tag
        assert np.array_equal(g["k_count"][bh], ref["nk"]), tag
        assert np.array_equal(g["q_cent"][bh].view(np.uint32), ref["cq"].view(np.uint32)), tag
        assert np.array_equal(g["k_cent"][bh].view(np.uint32), ref["ck"].view(np.uint32)), tag
        for side in ("q", "k"):
            assert np.array_equal(g[f"{side}_order"][bh], ref[f"{side}_order"]), (tag, side)
            assert np.array_equal(g[f"{side}_blk"][bh], ref[f"{side}_blk"]), (tag, side)
            assert np.array_equal(g[f"{side}_cnt"][bh], ref[f"{side}_cnt"]), (tag, side)
        assert np.array_equal(S_gpu[bh].view(np.uint32), ref["S"].view(np.uint32)), tag
        if wl.comp:
            vref = OC.cluster_means(v, ref["ak"], C)
            live = ref["nk"] > 0
            assert np.array_equal(v_cent[bh][live].view(np.uint32), vref[live].view(np.uint32)), tag
            kb, kc = ref["k_blk"], ref["k_cnt"]
            for j in range(nbp):
                if kb[j] >= 0:
                    assert np.array_equal(km[b, h, j].view(np.uint32),
                                          ref["ck"][kb[j]].view(np.uint32)), (tag, j)
                    want = (np.float32(kc[j]) * vref[kb[j]]).astype(np.float32)
                    assert np.array_equal(vs[b, h, j].view(np.uint32), want.view(np.uint32)), (tag, j)
                else:
                    assert not km[b, h, j].any() and not vs[b, h, j].any(), (tag, j)
        # cluster-level keep read back from the block-level CSR
        keepC_gpu = np.zeros((C, C), dtype=bool)
        qb = ref["q_blk"]
        for i in range(nbp):
            if qb[i] >= 0:
                kept_blocks = np.nonzero(keep_gpu[bh, i])[0]
                keepC_gpu[qb[i], np.unique(ref["k_blk"][kept_blocks])] = True
        assert np.array_equal(keep_gpu[bh], OC.cluster_block_keep(keepC_gpu, qb, ref["k_blk"])), tag
        for a in np.nonzero(np.any(keepC_gpu != ref["keepC"], axis=1))[0]:
            if ref["nq"][a] == 0:
                continue
            nk_live = ref["nk"] * ref.get("eligible", True)
            assert _excused(ref["S"][a], nk_live, wl, keepC_gpu[a], ref["keepC"][a]), (tag, a)
            excused += 1
        # attention in token order, given the oracle's partition and keep
        qcs = list(range(C))
        if q_clusters_per_head is not None and q_clusters_per_head < C:
            qcs = sorted(rng.choice(C, q_clusters_per_head, replace=False).tolist())
        Oref, lref = OC.cluster_attention_head(q, k, v, ref["aq"], ref["ak"], ref["keepC"],
                                               wl.scale, comp=wl.comp, q_clusters=qcs)
        sel_tok = np.isin(ref["aq"], qcs)
        og = oracle.bf16_to_f64(Og[b, h])
        errs.append(np.abs(og[sel_tok] - Oref[sel_tok]).ravel())
        lg, lr = lse_g[b, h][sel_tok].astype(np.float64), lref[sel_tok]
        fin = np.isfinite(lr)
        assert np.array_equal(fin, np.isfinite(lg)), tag
        if fin.any():
            lse_errs.append(np.abs(lg[fin] - lr[fin]))
    e = np.concatenate(errs)
    le = np.concatenate(lse_errs) if lse_errs else np.zeros(1)
    if tiles:
        log(f"[cluster] {wl.name}: shapes picked per checked head {picks}")
    return float(e.max()), float(e.mean()), float(le.max()), excused


@pytest.mark.parametrize("name", list(SMALL))
def test_small_cluster_parity(name):
    wl = SMALL[name].replace(name=name)
    log(f"[cluster] {name}: N={wl.N} H={wl.H} d={wl.d} block={wl.block} C={wl.n_clusters} "
        f"mode={wl.cluster} rule={wl.rule} comp={wl.comp}")
    Q, K, V = W.make_qkv(wl)
    emax, emean, lmax, exc = check_case(wl, Q, K, V, heads=range(wl.B * wl.H))
    log(f"[cluster] {name}: max {emax:.2e} mean {emean:.2e} lse {lmax:.2e} excused rows {exc}")
    assert emax <= ATOL_MAX and emean <= ATOL_MEAN and lmax <= LSE_ATOL


@pytest.mark.parametrize("name", ["wan13b_cocluster", "wan13b_kmeans_comp", "wan13b_sics",
                                  "wan13b_sics_ticket"])
def test_full_size_cluster_parity(name):
    """The full 1.3B-sized layer (12 heads, N = 32,760): the whole call on the
    GPU; layouts, centroids, scores and keep of two heads checked exactly and
    the output of every query cluster of both checked heads."""
    wl = W.by_name(name)
    log(f"[cluster-full] {name}: N={wl.N} H={wl.H} C={wl.n_clusters}")
    Q, K, V = W.make_qkv(wl)
    emax, emean, lmax, exc = check_case(wl, Q, K, V, heads=[0, wl.H - 1], seed=1)
    log(f"[cluster-full] {name}: max {emax:.2e} mean {emean:.2e} lse {lmax:.2e} excused {exc}")
    assert emax <= ATOL_MAX and emean <= ATOL_MEAN and lmax <= LSE_ATOL


def test_counts_prepare_matches_fixed_layout():
    """fwd_prepare_counts with the fixed layout's own counts gives the same bits
    as fwd_prepare (with compensation), and counts below a block's extent mask
    exactly the keys past them (equal to attention on the shortened sequence)."""
    import block_sparse_attention_hilbert_amd as sa
    wl = W.WORKLOADS[2].replace(T=3, Hg=10, W=13, H=2, rule="topk", density=0.5, comp=True)
    prob = sa.problem_for(wl)
    Q, K, V = (to_dev(x) for x in W.make_qkv(wl))
    sel = sa.select(prob, sa.spec_for(wl), Q, K, V)
    ws = sa.alloc_workspace(sa.workspace_size(prob, None), Q.device)
    O1 = torch.empty_like(Q)
    O2 = torch.empty_like(Q)
    sa.fwd_prepare(prob, V, sel.row_ptr, sel.k_mean, sel.v_sum, workspace=ws)
    sa.fwd_run(prob, Q, K, sel.row_ptr, sel.col_idx, True, O=O1, workspace=ws)
    nb = prob.nb
    cnt = np.full((wl.B * wl.H, nb), wl.block, np.int32)
    cnt[:, -1] = wl.N - (nb - 1) * wl.block
    sa.fwd_prepare_counts(prob, V, sel.row_ptr, torch.from_numpy(cnt).cuda(), sel.k_mean,
                          sel.v_sum, workspace=ws)
    sa.fwd_run(prob, Q, K, sel.row_ptr, sel.col_idx, True, O=O2, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(O1.view(torch.int16), O2.view(torch.int16))


@pytest.mark.parametrize("name", ["kmeans_topk_comp_d128_b64", "cocluster_mass_d128_b128"])
def test_partition_reuse_across_steps(name):
    """Reuse of the clustering (SVOO 2B: kept for several diffusion steps): step
    0 clusters and selects, steps 1 and 2 keep its partition and keep lists.
    Every step must equal the oracle's cluster attention over step 0's
    partition and keep with that step's own Q, K, V (with compensation: the
    centroids of that step's K and V), and the recomputed centroids must be
    the exact means of the step's keys and values per kept cluster."""
    wl = SMALL[name].replace(name=name)
    log(f"[cluster-reuse] {name}")
    steps = W.make_step_qkv(wl, 3, drift=0.2)
    pipe = _pipe(wl)
    pipe.refresh_every = 3
    ref0 = []
    moved = 0
    for s, (Q, K, V) in enumerate(steps):
        assert pipe.reuses_next() == (s > 0)
        O = pipe(to_dev(Q), to_dev(K), to_dev(V))
        torch.cuda.synchronize()
        Og = from_dev(O)
        lse_g = pipe.lse.cpu().numpy()
        errs, lerrs = [], []
        for bh in range(wl.B * wl.H):
            b, h = divmod(bh, wl.H)
            q, k, v = (oracle.bf16_to_f64(x[b, h]) for x in (Q, K, V))
            if s == 0:
                ref0.append(OC.cluster_workload_head(wl, q, k))
            r = ref0[bh]
            assert np.array_equal(pipe.cl.k_order[bh].cpu().numpy(), r["k_order"])
            assert np.array_equal(pipe.cl.q_order[bh].cpu().numpy(), r["q_order"])
            if s > 0:
                fresh = OC.cluster_workload_head(wl, q, k)
                moved += int(np.sum(fresh["ak"] != r["ak"]) + np.sum(fresh["aq"] != r["aq"]))
            if wl.comp:
                live = r["nk"] > 0
                kc = OC.cluster_means(k, r["ak"], wl.n_clusters)
                vc = OC.cluster_means(v, r["ak"], wl.n_clusters)
                assert np.array_equal(pipe.cl.k_cent[bh].cpu().numpy()[live].view(np.uint32),
                                      kc[live].view(np.uint32))
                assert np.array_equal(pipe.cl.v_cent[bh].cpu().numpy()[live].view(np.uint32),
                                      vc[live].view(np.uint32))
            Oref, lref = OC.cluster_attention_head(q, k, v, r["aq"], r["ak"], r["keepC"],
                                                   wl.scale, comp=wl.comp)
            errs.append(np.abs(oracle.bf16_to_f64(Og[b, h]) - Oref).ravel())
            lerrs.append(np.abs(lse_g[b, h].astype(np.float64) - lref))
        e = np.concatenate(errs)
        le = np.concatenate(lerrs)
        log(f"[cluster-reuse] {name}: step {s}: max {e.max():.2e} mean {e.mean():.2e} "
            f"lse {le.max():.2e}")
        assert e.max() <= ATOL_MAX and e.mean() <= ATOL_MEAN and le.max() <= LSE_ATOL
    log(f"[cluster-reuse] {name}: tokens a fresh clustering would move: {moved}")
    assert moved > 0


@pytest.mark.parametrize("name", ["wan13b_cocluster", "wan13b_kmeans_comp"])
def test_full_size_cluster_runs_are_bitwise_identical(name):
    """Two clustered calls on the same inputs give the same bits.  The cluster
    sums are added up in LDS and across workgroups in an order that changes
    from launch to launch; they are exact, so the centroids, the partition,
    the keep lists and the output may not change."""
    wl = W.by_name(name)
    log(f"[cluster-det] {name}: N={wl.N} H={wl.H} C={wl.n_clusters}")
    pipe = _pipe(wl)
    Q, K, V = W.make_qkv(wl)
    Qd, Kd, Vd = to_dev(Q), to_dev(K), to_dev(V)
    runs = []
    for _ in range(2):
        poison(pipe.O, pipe.lse)
        O = pipe(Qd, Kd, Vd, reuse=False)
        torch.cuda.synchronize()
        cl = pipe.cl
        runs.append([from_dev(O).copy(), pipe.lse.cpu().numpy().view(np.uint32).copy()] +
                    [getattr(cl, f).cpu().numpy().copy() for f in
                     ("q_order", "k_order", "q_cnt", "k_cnt", "q_count", "k_count")] +
                    [getattr(cl, f).cpu().numpy().view(np.uint32).copy() for f in ("q_cent", "k_cent")] +
                    [pipe.sel.row_ptr.cpu().numpy().copy(), pipe.sel.col_idx.cpu().numpy().copy()])
    for k, (a, b) in enumerate(zip(*runs)):
        assert np.array_equal(a, b), f"output {k} differs between two identical calls"
    log(f"[cluster-det] {name}: identical")


def test_slot_maps_out_of_range_are_contained():
    """Slot maps with entries outside [0, N): the clustered forward calls clamp
    positive ones into range and skip (queries) or zero (values) negative
    ones, so they end normally; every token the clamped query map names gets
    its output row, tokens it never names keep what they held."""
    import block_sparse_attention_hilbert_amd as sa
    wl = SMALL["kmeans_topk_comp_d128_b64"].replace(name="kmeans_topk_comp_d128_b64")
    pipe = _pipe(wl)
    Q, K, V = (to_dev(x) for x in W.make_qkv(wl))
    pipe(Q, K, V)
    torch.cuda.synchronize()
    N = wl.N
    qo = pipe.cl.q_order.clone()
    ko = pipe.cl.k_order.clone()
    hit = (qo[0] >= 0).nonzero().flatten()[:3]
    moved = [int(qo[0, s]) for s in hit]
    qo[0, hit[0]] = N + 1000
    qo[0, hit[1]] = -7
    qo[0, hit[2]] = -(1 << 30)
    ko[0, (ko[0] >= 0).nonzero().flatten()[:2]] = N + 5
    sa.cluster_fwd_prepare(pipe.prob, pipe.cspec, ko, V, pipe.sel.row_ptr, pipe.cl.k_cnt,
                           pipe.sel.k_mean, pipe.sel.v_sum, workspace=pipe.ws_fwd)
    O = torch.empty_like(Q)
    poison(O)
    sa.cluster_fwd_run(pipe.prob, pipe.cspec, qo, Q, pipe.Kp, pipe.sel.row_ptr, pipe.sel.col_idx,
                       True, O=O, workspace=pipe.ws_fwd)
    torch.cuda.synchronize()
    Og = from_dev(O)
    named = np.zeros((wl.B * wl.H, N), dtype=bool)
    q = qo.cpu().numpy()
    for bh in range(wl.B * wl.H):
        t = q[bh][q[bh] >= 0]
        named[bh, np.minimum(t, N - 1)] = True
    nan_rows = np.any((Og & 0x7F80) == 0x7F80, axis=-1).reshape(wl.B * wl.H, N)
    assert not np.any(nan_rows & named), "a named row was not written"
    for t in moved[1:]:
        assert nan_rows[0, t], "a token no slot names was written"
    log(f"[cluster-maps] malformed slot maps contained ({int(named.sum())} rows written)")
