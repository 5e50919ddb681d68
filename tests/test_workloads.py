"""The seeded synthetic inputs: shapes, determinism, bf16 rounding, geometry."""
import numpy as np
import torch

import oracle
import workloads as W
from conftest import golden


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8,
                                  3.4e38, 1e-40, -1e-40], np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(W.bf16_bits_to_f32(ours),
                          torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_geometry_matches_golden():
    rows = {r[0]: r for r in golden("block_geometry.txt")}
    for wl in W.WORKLOADS.values():
        r = rows[wl.name]
        assert (wl.T, wl.Hg, wl.W, wl.block) == tuple(int(x) for x in r[1:5])
        assert wl.N == int(r[5]) and wl.nb == int(r[6])
        assert wl.N - (wl.nb - 1) * wl.block == int(r[7])
        b = oracle.block_bounds(wl.N, wl.block)
        assert b[-1] - b[-2] == int(r[7])


def test_generator_is_deterministic_and_per_head():
    wl = W.WORKLOADS[2].replace(T=3, Hg=6, W=10, H=3)
    Q1, K1, V1 = W.make_qkv(wl)
    Q2, K2, V2 = W.make_qkv(wl, heads=[2])
    assert np.array_equal(Q1[:, 2:3], Q2) and np.array_equal(V1[:, 2:3], V2)
    Q3, _, _ = W.make_qkv(wl)
    assert np.array_equal(Q1, Q3)
    assert not np.array_equal(Q1[:, 0], Q1[:, 1])


def test_smooth_field_statistics():
    wl = W.WORKLOADS[2].replace(H=1)
    Q, K, V = W.make_qkv(wl)
    q = W.bf16_bits_to_f32(Q[0, 0]).astype(np.float64)
    k = W.bf16_bits_to_f32(K[0, 0]).astype(np.float64)
    v = W.bf16_bits_to_f32(V[0, 0]).astype(np.float64)
    # Q - K is the difference of two independent N(0, 0.3^2) noises
    assert abs(np.std(q - k) - 0.3 * np.sqrt(2)) < 0.01
    assert abs(np.std(v) - 1.0) < 0.01
    # the shared field dominates: Q and K are strongly correlated
    assert np.corrcoef(q.ravel(), k.ravel())[0, 1] > 0.8


def test_smooth_field_is_the_cosine_sum():
    """The separable evaluation equals the direct sum of cosines."""
    import math
    rng = np.random.default_rng([9, 0, 0])
    T, Hg, Wd, d = 3, 4, 5, 2
    field = W._smooth_field(rng, T, Hg, Wd, d, 3, 1.0).copy()
    rng = np.random.default_rng([9, 0, 0])
    freqs = rng.integers(0, 4, size=(d, W.N_MODES, 3))
    phase = rng.uniform(0.0, 2.0 * math.pi, size=(d, W.N_MODES))
    amp = rng.standard_normal((d, W.N_MODES)) / math.sqrt(W.N_MODES)
    t, y, x = np.indices((T, Hg, Wd)).reshape(3, -1)
    for c in range(d):
        direct = sum(amp[c, m] * np.cos(2 * math.pi * (freqs[c, m, 0] * t / T +
                                                       freqs[c, m, 1] * y / Hg +
                                                       freqs[c, m, 2] * x / Wd) + phase[c, m])
                     for m in range(W.N_MODES))
        np.testing.assert_allclose(field[:, c], direct, atol=1e-5)


def test_head_density_profile_range():
    rho = W.head_density_profile(12, 5)
    assert rho.dtype == np.float32 and np.all(rho >= 0.05) and np.all(rho <= 0.5)
    assert np.array_equal(rho, W.WORKLOADS[5].densities())


def test_step_inputs_start_at_the_workload_and_drift():
    wl = W.WORKLOADS[1]
    steps = W.make_step_qkv(wl, 3, drift=0.1)
    Q, K, V = W.make_qkv(wl)
    assert all(np.array_equal(a, b) for a, b in zip(steps[0], (Q, K, V)))
    # each later step moves further from step 0, and stays bf16 of a blend
    d1 = np.abs(W.bf16_bits_to_f32(steps[1][0]) - W.bf16_bits_to_f32(Q)).mean()
    d2 = np.abs(W.bf16_bits_to_f32(steps[2][0]) - W.bf16_bits_to_f32(Q)).mean()
    assert 0 < d1 < d2
