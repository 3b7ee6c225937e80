"""Synthetic workload generator: shapes, seeds, padding, budgets, bf16 rounding."""
import numpy as np
import pytest
import torch

import workloads
from workloads import synthetic


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, 1e-40], np.float32)])
    bits = workloads.bf16_bits_from_float(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = workloads.float_from_bf16_bits(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


@pytest.mark.parametrize("sparsity,nb,keep", [(0.75, 16, 4), (0.5, 88, 44), (0.75, 352, 88),
                                              (0.8, 176, 35), (0.97, 1100, 33), (0.999, 10, 1)])
def test_keep_from_sparsity(sparsity, nb, keep):
    assert workloads.keep_from_sparsity(nb, sparsity) == keep


def test_preset_shapes():
    sizes = [(1024, 16), (11264, 88), (45056, 352), (140800, 1100), (22528, 176)]
    for w, (n, nb) in zip(workloads.CONFIGS, sizes):
        assert w.layout.tokens == n and w.layout.nblocks == nb
        assert w.layout.frame_len % w.layout.block == 0


def test_tiny_preset_reproducible():
    w = workloads.config(0)
    a, b = workloads.generate(w), workloads.generate(w)
    for key in ("q", "k", "v"):
        np.testing.assert_array_equal(a[key], b[key])
        assert a[key].dtype == np.float32 and a[key].shape == (1, 1, 1024, 64)
    assert a["keep"].tolist() == [4]


def test_layer_preset_padding_and_bits():
    w = synthetic.restrict(workloads.config(1), 16)
    d = workloads.generate(w, heads=2)
    lay = w.layout
    pad = (np.arange(lay.tokens) % lay.frame_len) >= lay.frame_valid
    for key in ("q", "k", "v"):
        assert d[key].shape == (1, 2, 11264, 64)
        assert np.all(d[key][:, :, pad] == 0)
        np.testing.assert_array_equal(workloads.float_from_bf16_bits(d[key + "_bits"]), d[key])
    assert d["keep"].tolist() == [44, 44]
    # the first heads equal those of the full draw
    full = workloads.generate(workloads.config(1))
    np.testing.assert_array_equal(full["q"][:, :2], d["q"])
    np.testing.assert_array_equal(full["v"][:, :2], d["v"])


def test_cdf_preset_per_head_caps():
    """Per-head caps for 70-97 % sparsity are drawn after the values, from the seed."""
    w = workloads.config(3)
    assert w.mode == synthetic.MODE_CDF and w.cdf_tau == 0.9
    d = workloads.generate(w, heads=1)
    s_h = d["sparsity_h"]
    assert np.all((s_h >= 0.70) & (s_h <= 0.97))
    assert d["keep"].tolist() == [workloads.keep_from_sparsity(1100, s_h[0])]
    assert 33 <= d["keep"][0] <= 330
