"""Pins of the statistics harness (paper "Why Gated DeltaNet Survives 4-Bit
Quantization", section 5.1, Table 2: max/RMS, kurtosis, hot channels, 1-hot
blocks = block max/RMS > 3, i.e. one value over 9/16 of the block energy).
Closed forms on constructed tensors; runs on CPU tensors."""
import math

import numpy as np
import torch

from nvfp4_w4a4_quantized_02_amd.stats import gemm_error, tensor_stats


def test_max_over_rms_single_spike():
    x = torch.zeros(4, 64)
    x[2, 5] = -7.0
    assert math.isclose(tensor_stats(x)["max_over_rms"], math.sqrt(256), rel_tol=1e-12)


def test_kurtosis_closed_forms():
    x = torch.tensor([[1.0, -1.0] * 8] * 4)                 # two-point symmetric: kurtosis 1
    assert math.isclose(tensor_stats(x)["kurtosis"], 1.0, rel_tol=1e-12)
    g = torch.from_numpy(np.random.default_rng(0).standard_normal((512, 1024)))
    assert abs(tensor_stats(g)["kurtosis"] - 3.0) < 0.05       # Gaussian: 3
    u = torch.from_numpy(np.random.default_rng(1).uniform(-1, 1, (512, 1024)))
    assert abs(tensor_stats(u)["kurtosis"] - 1.8) < 0.02       # uniform: 9/5


def test_hot_channel_ratio():
    x = torch.ones(10, 32)
    x[:, 7] = 100.0                                            # one channel 100x the median channel
    x[:, 9] = 2.0
    assert math.isclose(tensor_stats(x)["hot_channel_ratio"], 100.0, rel_tol=1e-12)


def test_one_hot_blocks():
    x = torch.ones(2, 32)
    x[0, 3] = 10.0          # block max/RMS = 10 / sqrt(115/16) = 3.73 -> 1-hot
    x[1, 20] = 3.0          # 3 / sqrt(24/16) = 2.45 -> not
    x[1, :16] = 0.0         # an all-zero block is not counted
    s = tensor_stats(x)["one_hot_block_share"]
    assert math.isclose(s, 1.0 / 3.0, rel_tol=1e-12)


def test_one_hot_threshold_is_energy_share():
    """max/RMS > 3 over 16 values  <=>  max^2 > (9/16) * block energy."""
    g = np.random.default_rng(2)
    for _ in range(200):
        b = g.standard_normal(16) * (g.uniform(0, 1, 16) ** 6)
        b[g.integers(16)] *= g.uniform(1, 20)
        x = torch.from_numpy(b.reshape(1, 16))
        by_ratio = tensor_stats(x)["one_hot_block_share"] == 1.0
        by_energy = b.max() ** 2 > 9.0 / 16.0 * np.sum(b ** 2) if abs(b).max() == b.max() else \
            np.min(b) ** 2 > 9.0 / 16.0 * np.sum(b ** 2)
        assert by_ratio == by_energy


def test_gemm_error():
    r = torch.tensor([[3.0, 4.0]])
    assert math.isclose(gemm_error(torch.tensor([[3.0, 4.5]]), r), 0.1, rel_tol=1e-12)
    assert gemm_error(r, r) == 0.0
