"""GPU parity: the HIP path (through the C ABI) against the oracle.

Bar (stated here, derived in the design notes):
* block means, block sums and pooled scores: bit-exact (same fp32 definition);
* keep masks: bit-exact, except rows excused as near ties (counted, reported);
* Hilbert order and token reordering: bit-exact;
* attention output given the oracle's mask: max |err| <= 2e-2 and mean |err|
  <= 2e-3 against the float64 oracle; lse within 2e-2.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from parity_util import (ATOL_MAX, ATOL_MEAN, ERR_KEY_ATOL, LSE_ATOL, OracleCase,
                         assert_outputs_written, compare_attention, compare_keys, from_dev, log,
                         mask_report, poison, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_hilbert_amd as sa  # noqa: F401  (fails loudly if unbuilt)
    yield


def _sa():
    import block_sparse_attention_hilbert_amd as sa
    return sa


def _pipeline(wl, want_scores=True, want_lse=True):
    sa = _sa()
    from block_sparse_attention_hilbert_amd.pipeline import BlockSparseAttention
    return BlockSparseAttention(sa.problem_for(wl), sa.spec_for(wl), hilbert=wl.hilbert,
                                want_scores=want_scores, want_lse=want_lse)


# small workloads: several tiles and a ragged last block (390 = 3*128 + 6 = 6*64 + 6)
SMALL = {
    "mass_d128_b128": W.WORKLOADS[2].replace(T=3, Hg=10, W=13, H=3),
    "topk_d128_b128": W.WORKLOADS[3].replace(T=3, Hg=10, W=13, H=4),
    "topk_diag_d64_b64": W.WORKLOADS[1].replace(T=3, Hg=10, W=13, H=2),
    "window_anchor_d128_b128": W.WORKLOADS[4].replace(T=6, Hg=10, W=13, H=2),
    "hilbert_comp_d128_b64": W.WORKLOADS[5].replace(T=3, Hg=10, W=13, H=3),
    "mass_sub32_d64_b128": W.WORKLOADS[2].replace(T=3, Hg=10, W=13, H=2, d=64, sub_block=32),
    "mass_comp_d64_b128": W.WORKLOADS[2].replace(T=5, Hg=7, W=11, H=2, d=64, comp=True, mass=0.5),
    "topk_d128_b64_wide": W.WORKLOADS[3].replace(T=5, Hg=9, W=29, H=2, block=64, density=0.3),
    # more heads than the per-head budgets passed inline with the launch
    "topk_70heads_d64_b64": W.WORKLOADS[5].replace(T=2, Hg=8, W=9, H=70, d=64, hilbert=False,
                                                 comp=False, sub_block=0),
    # error-aware routing (keys ranked top-k, compensation on)
    "err_d128_b128": W.WORKLOADS[2].replace(T=3, Hg=10, W=13, H=3, rule="err", density=0.2,
                                          comp=True),
    "err_hilbert_d128_b64": W.WORKLOADS[5].replace(T=3, Hg=10, W=13, H=3, rule="err",
                                                 sub_block=0),
    "err_d64_b64_wide": W.WORKLOADS[3].replace(T=5, Hg=9, W=29, H=2, d=64, block=64, rule="err",
                                             density=0.3, comp=True),
    "err_d64_b128_diag": W.WORKLOADS[1].replace(T=3, Hg=10, W=13, H=2, block=128, rule="err",
                                              comp=True, diag=True),
    # batches of two: every kernel indexes (batch, head) pairs
    "mass_batch2": W.WORKLOADS[2].replace(B=2, T=3, Hg=10, W=13, H=2),
    "hilbert_comp_batch2": W.WORKLOADS[5].replace(B=2, T=3, Hg=10, W=13, H=3),
    "window_anchor_batch2": W.WORKLOADS[4].replace(B=2, T=6, Hg=10, W=13, H=2),
    "err_batch2": W.WORKLOADS[2].replace(B=2, T=3, Hg=10, W=13, H=2, rule="err", density=0.3,
                                       comp=True),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_workload_parity(name):
    wl = SMALL[name]
    log(f"[parity] {name}: N={wl.N} nb={wl.nb} H={wl.H} d={wl.d} block={wl.block}")
    Q, K, V = W.make_qkv(wl)
    off = W.anchor_offset(wl.seed, 0, wl.nb)
    case = OracleCase(wl, Q, K, V, anchor_offset=off)
    pipe = _pipeline(wl)
    poison(pipe.O, pipe.lse)
    O = pipe(to_dev(Q), to_dev(K), to_dev(V), anchor_offset=off)
    torch.cuda.synchronize()
    assert_outputs_written(from_dev(O), pipe.lse.cpu().numpy(), wl, pipe.keep_mask(), perm=pipe.perm)

    if wl.rule == "err":
        S = pipe.sel.scores.view(wl.B, wl.H, wl.nb, wl.nb).cpu().numpy()
        kerr = compare_keys(S, case)
        log(f"[parity] {name}: routing keys max |err| = {kerr:.2e}")
        assert kerr <= ERR_KEY_ATOL
    elif wl.rule != "none":
        S = pipe.sel.scores.view(wl.B, wl.H, wl.nb, wl.nb).cpu().numpy()
        assert np.array_equal(S, case.S), "pooled scores differ"
    if wl.comp:
        km = pipe.sel.k_mean.cpu().numpy()
        vs = pipe.sel.v_sum.cpu().numpy()
        for b in range(wl.B):
            for h in range(wl.H):
                q, k, v = case.head_inputs(b, h)
                assert np.array_equal(km[b, h], oracle.block_means(k, wl.block))
                assert np.array_equal(vs[b, h], oracle.block_sums_f32(v, wl.block))
    keep = pipe.keep_mask()
    if wl.rule == "err":
        # the selection on the kernel's own keys is exact: top-k by key,
        # then the structured blocks
        for b in range(wl.B):
            for h in range(wl.H):
                want = oracle.topk_keep(S[b, h].astype(np.float64), oracle.head_k(wl, h))
                if wl.diag:
                    want |= np.eye(wl.nb, dtype=bool)
                if wl.window_frames >= 0:
                    want |= oracle.window_keep(wl.N, wl.block, wl.Hg * wl.W, wl.window_frames)
                if wl.n_anchors > 0:
                    want[:, oracle.anchor_blocks(wl.nb, wl.n_anchors, off)] = True
                assert np.array_equal(keep[b, h], want), (b, h)
    bad, excused, failures = mask_report(keep, case)
    log(f"[parity] {name}: density={keep.mean():.3f} mismatched rows={bad} near-ties={excused}")
    assert not failures, failures[:5]

    # attention given the oracle's mask
    rp, ci = oracle.keep_to_csr(case.keep.reshape(-1, wl.nb))
    poison(pipe.O, pipe.lse)
    O = pipe.run_fwd(to_dev(Q), to_dev(K), to_dev(V), torch.from_numpy(rp).cuda(),
                     torch.from_numpy(ci).cuda())
    torch.cuda.synchronize()
    assert_outputs_written(from_dev(O), pipe.lse.cpu().numpy(), wl, case.keep, perm=pipe.perm)
    lse = pipe.lse.cpu().numpy()                          # raster order
    emax, emean, lmax, n = compare_attention(from_dev(O), case, None, lse_gpu=lse)
    log(f"[parity] {name}: attention max={emax:.2e} mean={emean:.2e} lse={lmax:.2e}")
    assert emax <= ATOL_MAX and emean <= ATOL_MEAN and lmax <= LSE_ATOL


def test_hilbert_permute_kernels():
    sa = _sa()
    wl = W.WORKLOADS[5].replace(H=2)
    prob = sa.problem_for(wl)
    perm, _ = sa.hilbert_perm_build(wl.T, wl.Hg, wl.W)
    rng = np.random.default_rng(0)
    X = rng.integers(0, 1 << 16, size=(1, 2, wl.N, wl.d), dtype=np.uint16)
    pd = torch.from_numpy(perm).cuda()
    Xp = sa.hilbert_permute(prob, to_dev(X), pd)
    Xb = sa.hilbert_unpermute(prob, Xp, pd)
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(Xp), oracle.permute_tokens(X, oracle.hilbert_perm(wl.T, wl.Hg, wl.W)[0]))
    assert np.array_equal(from_dev(Xb), X)


def test_edge_single_token_and_empty_rows():
    sa = _sa()
    # N = 1: one block of one token; attention to itself is exactly v
    wl = W.WORKLOADS[1].replace(T=1, Hg=1, W=1, H=1, rule="topk", topk=1, diag=False)
    Q, K, V = W.make_qkv(wl)
    O = _pipeline(wl)(to_dev(Q), to_dev(K), to_dev(V))
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(O), V)
    # structural rule with no structure: every row empty -> O = 0, lse = -inf
    wl = W.WORKLOADS[4].replace(T=2, Hg=8, W=8, H=2, window_frames=-1, n_anchors=0)
    Q, K, V = W.make_qkv(wl)
    pipe = _pipeline(wl)
    O = pipe(to_dev(Q), to_dev(K), to_dev(V))
    torch.cuda.synchronize()
    assert int(pipe.sel.row_ptr[-1]) == 0
    assert np.all(from_dev(O) == 0) and np.all(np.isneginf(pipe.lse.cpu().numpy()))


def test_edge_full_budget_is_dense_attention():
    """mass = 1 and k = nb keep every block: the result is dense attention."""
    for wl in (SMALL["mass_d128_b128"].replace(mass=1.0),
               SMALL["topk_d128_b128"].replace(density=None, topk=10 ** 6)):
        Q, K, V = W.make_qkv(wl)
        pipe = _pipeline(wl)
        O = pipe(to_dev(Q), to_dev(K), to_dev(V))
        torch.cuda.synchronize()
        assert pipe.keep_mask().all()
        case = OracleCase(wl, Q, K, V)
        assert case.keep.all()
        emax, emean, _, _ = compare_attention(from_dev(O), case, None)
        assert emax <= ATOL_MAX and emean <= ATOL_MEAN


def test_edge_compensation_limits():
    """Compensation with every block kept adds nothing; with nothing kept the
    output is attention over the centroids (oracle, same mask)."""
    base = SMALL["hilbert_comp_d128_b64"]
    for wl in (base.replace(head_density=False, density=1.0),
               base.replace(rule="none", head_density=False, hilbert=False)):
        Q, K, V = W.make_qkv(wl)
        case = OracleCase(wl, Q, K, V)
        pipe = _pipeline(wl)
        O = pipe(to_dev(Q), to_dev(K), to_dev(V))
        torch.cuda.synchronize()
        assert np.array_equal(pipe.keep_mask(), case.keep)
        emax, emean, _, _ = compare_attention(from_dev(O), case, None)
        log(f"[parity] comp limit rule={wl.rule}: max={emax:.2e} mean={emean:.2e}")
        assert emax <= ATOL_MAX and emean <= ATOL_MEAN


def test_largest_sort_length():
    """nb = 4096 (the largest scored row) with the mass rule and sub-blocks."""
    wl = W.WORKLOADS[2].replace(T=64, Hg=64, W=64, H=1, block=64, d=64, sub_block=32, mass=0.5)
    assert wl.nb == 4096
    Q, K, V = W.make_qkv(wl)
    case = OracleCase(wl, Q, K, V)
    pipe = _pipeline(wl, want_lse=False)
    pipe.run_select(to_dev(Q), to_dev(K), None)
    torch.cuda.synchronize()
    S = pipe.sel.scores.view(1, 1, wl.nb, wl.nb).cpu().numpy()
    assert np.array_equal(S, case.S)
    bad, excused, failures = mask_report(pipe.keep_mask(), case)
    log(f"[parity] nb=4096: mismatched rows={bad} near-ties={excused}")
    assert not failures


def test_determinism():
    wl = SMALL["hilbert_comp_d128_b64"]
    Q, K, V = (to_dev(x) for x in W.make_qkv(wl))
    pipe = _pipeline(wl)
    a = pipe(Q, K, V).clone()
    b = pipe(Q, K, V).clone()
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", ["hilbert_comp_d128_b64", "mass_d128_b128"])
def test_fwd_halves_match_fwd(name):
    """sparse_attn_fwd == sparse_attn_fwd_prepare + sparse_attn_fwd_run (bit for bit), and a
    second run on the same preparation repeats the result."""
    wl = SMALL[name]
    Q, K, V = (to_dev(x) for x in W.make_qkv(wl))
    pipe = _pipeline(wl)
    pipe.run_select(Q, K, V, 0)
    ref = pipe.run_fwd(Q, K, V).clone()
    ref_lse = pipe.lse.clone()
    pipe.O.zero_()
    pipe.run_fwd_prepare(V)
    outs = []
    for _ in range(2):
        outs.append((pipe.run_fwd_attention(Q, K).clone(), pipe.lse.clone()))
    torch.cuda.synchronize()
    for o, lse in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(lse, ref_lse)


@pytest.mark.parametrize("name", ["err_d128_b128", "err_hilbert_d128_b64", "err_d64_b64_wide"])
def test_err_selection_shares_v_layout(name):
    """The error rule's selection writes V in block layout into the forward
    workspace (v_blocks), and the forward call then skips its own re-layout:
    keys, CSR, O and lse are bit-identical to a selection that keeps the layout
    in its own workspace followed by a forward call that lays V out again."""
    sa = _sa()
    wl = SMALL[name]
    Q, K, V = (to_dev(x) for x in W.make_qkv(wl))
    pipe = _pipeline(wl)
    assert pipe.share_v
    poison(pipe.O, pipe.lse)
    O = pipe(Q, K, V, anchor_offset=0).clone()
    lse = pipe.lse.clone()
    prob, spec = pipe.prob, sa.spec_for(wl)
    ref = sa.select(prob, spec, Q, K, V, want_scores=True)
    O2, lse2 = sa.fwd(prob, Q, K, V, ref.row_ptr, ref.col_idx, ref.k_mean, ref.v_sum, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(pipe.sel.row_ptr, ref.row_ptr)
    n = int(ref.row_ptr[-1])
    assert torch.equal(pipe.sel.col_idx[:n], ref.col_idx[:n])
    assert torch.equal(pipe.sel.scores, ref.scores)
    assert torch.equal(O.view(torch.int16), O2.view(torch.int16))
    assert torch.equal(lse, lse2)
    log(f"[share] {name}: shared V layout bit-identical ({n} kept blocks)")


@pytest.mark.parametrize("name", ["hilbert_comp_d128_b64", "mass_d128_b128", "err_d128_b128"])
def test_mask_reuse_across_steps(name):
    """Mask reuse (DFSAttn trick 3, SVOO 2B): step 0 selects, steps 1 and 2 keep
    its CSR.  Every step's output must equal the oracle's attention over step
    0's mask with that step's own inputs (and, with compensation, the
    centroids of that step's K and V)."""
    wl = SMALL[name]
    log(f"[reuse] {name}: N={wl.N} nb={wl.nb} H={wl.H}")
    steps = W.make_step_qkv(wl, 3, drift=0.2)
    pipe = _pipeline(wl)
    pipe.refresh_every = 3
    keep0 = None
    changed_total = 0
    for s, (Q, K, V) in enumerate(steps):
        case = OracleCase(wl, Q, K, V, anchor_offset=0)
        assert pipe.reuses_next() == (s > 0)
        O = pipe(to_dev(Q), to_dev(K), to_dev(V), anchor_offset=0)
        torch.cuda.synchronize()
        keep = pipe.keep_mask()
        if s == 0:
            keep0 = keep.copy()
            bad, excused, failures = mask_report(keep, case)
            assert not failures, failures[:5]
            case.keep = keep0
        else:
            assert np.array_equal(keep, keep0), "reused mask changed"
            changed = int((case.keep != keep0).any(axis=-1).sum())
            changed_total += changed
            log(f"[reuse] {name}: step {s}: rows whose fresh mask would differ: {changed}")
            case.keep = keep0
            if wl.comp:
                km = pipe.sel.k_mean.cpu().numpy()
                vs = pipe.sel.v_sum.cpu().numpy()
                for b in range(wl.B):
                    for h in range(wl.H):
                        q, k, v = case.head_inputs(b, h)
                        assert np.array_equal(km[b, h], oracle.block_means(k, wl.block))
                        assert np.array_equal(vs[b, h], oracle.block_sums_f32(v, wl.block))
        lse = pipe.lse.cpu().numpy()
        emax, emean, lmax, n = compare_attention(from_dev(O), case, None, lse_gpu=lse)
        log(f"[reuse] {name}: step {s}: attention max={emax:.2e} mean={emean:.2e} lse={lmax:.2e}")
        assert emax <= ATOL_MAX and emean <= ATOL_MEAN and lmax <= LSE_ATOL
    # the drift is large enough that a fresh selection would have differed
    assert changed_total > 0


def test_largest_attention_window():
    """The largest attention the interface admits: nb = 4096 blocks of 128
    tokens at d = 128 (the most LDS a workgroup takes), with a +-0-frame window
    (LVSA abstract: a temporal window) so that the oracle stays cheap: every
    row keeps the blocks of its own latent frame(s).  Every output row written;
    every 8th query block (and the first and last) against the oracle."""
    wl = W.WORKLOADS[4].replace(T=128, Hg=64, W=64, H=1, gen="iid", window_frames=0, n_anchors=0)
    assert wl.nb == 4096 and wl.d == 128 and wl.block == 128
    Q, K, V = W.make_qkv(wl)
    case = OracleCase(wl, Q, K, V)
    pipe = _pipeline(wl, want_scores=False)
    poison(pipe.O, pipe.lse)
    O = pipe(to_dev(Q), to_dev(K), to_dev(V))
    torch.cuda.synchronize()
    keep = pipe.keep_mask()
    assert np.array_equal(keep, case.keep)
    Og = from_dev(O)
    assert_outputs_written(Og, pipe.lse.cpu().numpy(), wl, keep)
    qb = sorted(set([0, wl.nb - 1] + list(range(0, wl.nb, 8))))
    O_ref, lse_ref = case.attention(0, 0, q_blocks=qb)
    bounds = oracle.block_bounds(wl.N, wl.block)
    og = oracle.bf16_to_f64(Og[0, 0])
    lg = pipe.lse.cpu().numpy()[0, 0].astype(np.float64)
    e = np.concatenate([np.abs(og[bounds[i]:bounds[i + 1]] - O_ref[bounds[i]:bounds[i + 1]]).ravel()
                        for i in qb])
    le = max(float(np.abs(lg[bounds[i]:bounds[i + 1]] - lse_ref[bounds[i]:bounds[i + 1]]).max())
             for i in qb)
    log(f"[parity] nb=4096 window: density={keep.mean():.4f} attention on {len(qb)} query blocks "
        f"max={e.max():.2e} mean={e.mean():.2e} lse={le:.2e}")
    assert e.max() <= ATOL_MAX and e.mean() <= ATOL_MEAN and le <= LSE_ATOL


def test_malformed_csr_is_contained():
    """A caller's CSR with a row longer than nb entries and a row whose end
    precedes its start: the kernel cuts the first to nb entries and takes the
    second as empty, ends normally and writes every other row as usual."""
    sa = _sa()
    wl = SMALL["mass_d128_b128"]
    prob = sa.problem_for(wl)
    Q, K, V = (to_dev(x) for x in W.make_qkv(wl))
    nb, rows = prob.nb, prob.rows
    keep = np.zeros((rows, nb), dtype=bool)
    keep[:, 0] = True
    keep[np.arange(rows), np.arange(rows) % nb] = True
    rp, ci = oracle.keep_to_csr(keep)
    # row 1: 3 nb entries (every block three times); row 2: end before start
    long_cols = np.tile(np.arange(nb, dtype=np.int32), 3)
    lens = np.diff(rp).astype(np.int64)
    lens[1] = long_cols.size
    rp2 = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    ci2 = np.concatenate([ci[: rp[1]], long_cols, ci[rp[2]:]]).astype(np.int32)
    rp2[3] = rp2[2] - 1                       # row 2 ends one entry before it starts
    ci2 = np.concatenate([ci2, np.zeros(4 * nb, np.int32)])
    O = torch.empty_like(Q)
    poison(O)
    out, lse = sa.fwd(prob, Q, K, V, torch.from_numpy(rp2).cuda(), torch.from_numpy(ci2).cuda(),
                      O=O, want_lse=True)
    torch.cuda.synchronize()
    Og = from_dev(out)
    assert not np.any((Og & 0x7F80) == 0x7F80), "every row written, no NaN"
    lse = lse.cpu().numpy()                    # [B, H, N]
    bounds = oracle.block_bounds(wl.N, wl.block)
    # row 2 (batch 0, head 0, query block 2) attended to nothing: O = 0, lse = -inf
    assert np.all(Og[0, 0, bounds[2]:bounds[3]] == 0)
    assert np.all(np.isneginf(lse[0, 0, bounds[2]:bounds[3]]))
    assert not np.any(np.isnan(lse))
    # row 1 attended to the first nb entries of its list: every block once
    case = OracleCase(wl, *W.make_qkv(wl))
    case.keep = np.ones((wl.B, wl.H, nb, nb), dtype=bool)
    O_ref, _ = case.attention(0, 0, q_blocks=[1])
    e = np.abs(oracle.bf16_to_f64(Og[0, 0, bounds[1]:bounds[2]]) - O_ref[bounds[1]:bounds[2]])
    assert e.max() <= ATOL_MAX


def test_token_order_out_of_range_is_contained():
    """A token order with entries outside [0, N): every gathered index is
    clamped into range, so the selection and the attention (with
    compensation) end normally and every row the clamped order names is
    written; rows it never names are left as they were."""
    import dataclasses
    sa = _sa()
    wl = SMALL["hilbert_comp_d128_b64"].replace(hilbert=False)
    N = wl.N
    order = np.arange(N, dtype=np.int32)
    order[[5, 77]] = [N + 1000, -3]                  # tokens 5 and 77 are never named
    clamped = np.clip(order, 0, N - 1)
    prob = dataclasses.replace(sa.problem_for(wl), token_order=torch.from_numpy(order).cuda())
    Q, K, V = (to_dev(x) for x in W.make_qkv(wl))
    spec = sa.spec_for(wl)
    sel = sa.select(prob, spec, Q, K, V)
    O = torch.empty_like(Q)
    poison(O)
    out, lse = sa.fwd(prob, Q, K, V, sel.row_ptr, sel.col_idx, O=O, want_lse=True,
                      k_mean=sel.k_mean, v_sum=sel.v_sum)
    torch.cuda.synchronize()
    Og = from_dev(out)
    named = np.zeros(N, dtype=bool)
    named[clamped] = True
    nan_rows = np.any((Og & 0x7F80) == 0x7F80, axis=-1)      # [B, H, N]
    assert not np.any(nan_rows[..., named]), "a named row was not written"
    assert np.all(~named[[5, 77]])
