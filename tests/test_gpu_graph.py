"""HIP graph replay of a whole call (pipeline.GraphedCall) against eager calls.

Every replay must equal, bit for bit, the eager call of a second pipeline on
the same inputs: both run the same deterministic kernels.  Between replays the
test runs that eager pipeline and synchronises, and it walks through calls
that form the selection (or partition) anew and calls that keep it.
"""
import pytest

import workloads as W
from parity_util import log, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_hilbert_amd as sa  # noqa: F401  (fails loudly if unbuilt)
    yield


BASE = W.WORKLOADS[2].replace(T=3, Hg=10, W=13, H=2)          # N = 390
CASES = {
    "fixed_mass_comp_b64": BASE.replace(block=64, comp=True),
    "fixed_hilbert_topk_b128": BASE.replace(hilbert=True, rule="topk", density=0.3),
    # error-aware routing: the selection writes V in block layout into the
    # forward workspace, and the forming graph skips the second re-layout
    "fixed_err_comp_b128": BASE.replace(rule="err", density=0.3, comp=True),
    "cocluster_mass_b128": BASE.replace(cluster="cocluster", n_clusters=3, cluster_iters=2),
    "kmeans_topk_comp_b64": BASE.replace(block=64, cluster="kmeans", n_clusters=6,
                                         cluster_iters=3, rule="topk", density=0.3, comp=True),
    "tiles_topk_b64": BASE.replace(H=3, block=64, cluster="tiles", aniso=True,
                                   tile_shapes=((1, 4, 16), (1, 8, 8), (2, 4, 8), (3, 2, 8)),
                                   n_clusters=12, rule="topk", density=0.3),
}


def _pipe(wl, refresh):
    import block_sparse_attention_hilbert_amd as sa
    from block_sparse_attention_hilbert_amd.pipeline import BlockSparseAttention, ClusteredAttention
    spec = sa.spec_for(wl)
    if wl.cluster:
        return ClusteredAttention(sa.problem_for(wl), sa.cluster_spec_for(wl), spec,
                                  want_lse=True, refresh_every=refresh)
    return BlockSparseAttention(sa.problem_for(wl), spec, hilbert=wl.hilbert, want_lse=True,
                                refresh_every=refresh)


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replays_equal_eager_calls(name):
    from block_sparse_attention_hilbert_amd.pipeline import GraphedCall
    wl = CASES[name].replace(name=name)
    steps = W.make_step_qkv(wl, 5, drift=0.2)
    eager = _pipe(wl, refresh=2)
    graphed_pipe = _pipe(wl, refresh=2)
    Qb, Kb, Vb = (to_dev(x) for x in steps[0])
    g = GraphedCall(graphed_pipe, Qb, Kb, Vb)
    kinds = []
    for s, (Q, K, V) in enumerate(steps):
        Qd, Kd, Vd = to_dev(Q), to_dev(K), to_dev(V)
        keep = eager.reuses_next()
        assert graphed_pipe.reuses_next() == keep
        kinds.append("keep" if keep else "form")
        O_e = eager(Qd, Kd, Vd).clone()
        lse_e = eager.lse.clone()
        torch.cuda.synchronize()
        Qb.copy_(Qd)
        Kb.copy_(Kd)
        Vb.copy_(Vd)
        O_g = g()
        torch.cuda.synchronize()
        assert torch.equal(O_g, O_e), (name, s)
        assert torch.equal(graphed_pipe.lse, lse_e), (name, s)
    log(f"[graph] {name}: {len(steps)} replays equal the eager calls ({' '.join(kinds)})")
    assert kinds == ["form", "keep", "form", "keep", "form"]
