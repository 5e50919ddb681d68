"""The allocation-free selection entry point (sparse_attn_select_noalloc),
called through the C ABI, against sparse_attn_select with a workspace on the
same inputs: keep lists, scores and compensation statistics bit for bit, on
two calls in a row (the second smaller, reusing the one scratch array)."""
import numpy as np
import pytest

import workloads as W
from parity_util import from_dev, log, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield


def _outputs(sa, prob, spec, dev):
    nb, rows = prob.nb, prob.rows
    out = sa.Selection(torch.full((rows + 1,), -7, dtype=torch.int32, device=dev),
                       torch.full((rows * nb,), -7, dtype=torch.int32, device=dev),
                       torch.full((rows * nb,), float("nan"), dtype=torch.float32, device=dev))
    if spec.want_comp:
        out.k_mean = torch.full((prob.B, prob.H, nb, prob.d), float("nan"), dtype=torch.float32,
                                device=dev)
        out.v_sum = torch.full_like(out.k_mean, float("nan"))
    return out


def _same(a, b):
    assert a.shape == b.shape
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("first,second", [(5, 2)])
def test_noalloc_select_equals_workspace_select(first, second):
    import block_sparse_attention_hilbert_amd as sa
    dev = torch.device("cuda:0")
    # the 64-token Hilbert workload at full size (sub-block scores, per-head
    # budgets, compensation statistics), then a smaller 1.3B-shaped layer
    cases = [W.WORKLOADS[first], W.WORKLOADS[second].replace(T=7, Hg=10, W=13)]
    for n, wl in enumerate(cases):
        prob, spec = sa.problem_for(wl), sa.spec_for(wl)
        Q, K, V = (to_dev(x) for x in W.make_qkv(wl))
        Vc = V if spec.want_comp else None
        ref = sa.select(prob, spec, Q, K, Vc, out=_outputs(sa, prob, spec, dev))
        got = sa.select_noalloc(prob, spec, Q, K, Vc, out=_outputs(sa, prob, spec, dev))
        torch.cuda.synchronize()
        total = int(ref.row_ptr[-1])
        log(f"[noalloc] call {n}: {wl.name} N={wl.N} nb={prob.nb} kept={total} "
            f"scratch={sa.workspace_size(prob, spec)} bytes")
        assert torch.equal(got.row_ptr, ref.row_ptr)
        assert torch.equal(got.col_idx[:total], ref.col_idx[:total])
        assert _same(got.scores, ref.scores)
        if spec.want_comp:
            assert _same(got.k_mean, ref.k_mean) and _same(got.v_sum, ref.v_sum)
