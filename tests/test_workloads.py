"""The seeded input generators: storage formats and reproducibility."""
import numpy as np
import torch

from test_rnn_layer_amd import workloads as W


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    a = np.concatenate([g.standard_normal(100_000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 3.0e38, -1e-30, 1.00390625, 1.01171875], np.float32)])
    ours = W.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = W.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_x_ranges_regenerate_identically():
    wl = W.WORKLOADS["bidir307k"].replace(T=10_000, H=2, d=8)
    full = W.make_x(wl)
    part = W.make_x(wl, 4000, 9001)
    np.testing.assert_array_equal(full[:, 4000:9001], part)
    np.testing.assert_array_equal(W.make_x(wl, 0, 5, seq=0), full[0, :5])


def test_distributions_and_segment_shift():
    wl = W.WORKLOADS["bidir307k"].replace(T=3 * 1000, H=4, d=16, seg_len=1000)
    x = W.to_f64(W.make_x(wl)[0], wl.io_dtype)
    mu = W.segment_means(wl)
    assert mu.shape == (3, wl.D)
    for s in range(3):
        seg = x[s * 1000:(s + 1) * 1000]
        # the per-channel sample mean tracks mu_s within a few standard errors
        assert np.abs(seg.mean(0) - mu[s]).max() < 6 / np.sqrt(1000)
        assert abs((seg - mu[s]).std() - 1.0) < 0.02
    th = W.to_f64(W.make_theta(wl), wl.io_dtype)
    assert abs(th.std() * np.sqrt(wl.D) - 1.0) < 0.05
    w1, w2 = W.make_w0(wl)
    assert abs(w1.std() * np.sqrt(wl.d) - 1.0) < 0.05 and abs(w2.std() * np.sqrt(wl.m) - 1.0) < 0.05
    assert not np.array_equal(w1[0], w1[1])


def test_workload_table():
    for name in W.WORKLOAD_ORDER:
        wl = W.WORKLOADS[name]
        assert wl.m == 4 * wl.d and wl.T % wl.b == 0
    assert W.WORKLOADS["bidir307k"].T == 307_200 and W.WORKLOADS["bigstate307k"].D == 3072
