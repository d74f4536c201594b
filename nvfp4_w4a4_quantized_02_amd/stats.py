"""Statistics of tensors at NVFP4 granularity and fake-quantization errors.

Paper "Why Gated DeltaNet Survives 4-Bit Quantization", section 5.1 and
Table 2 define the activation and weight statistics used to place inputs:
max/RMS, kurtosis, the hot-channel ratio, the share of "1-hot" 16-element
blocks (block max/RMS > 3, i.e. one value holds more than 9/16 of the block's
energy), and A4 / W4 = the relative error of quantizing the activation /
weight tensor alone.  Section 5.2 and Table 3 use the relative error of a
projection's output when it runs W4A4 ("gemm" column).

Readings taken where the paper gives no formula (each function repeats its
own): relative errors are Frobenius-norm ratios ||approx - exact|| / ||exact||;
kurtosis is the Pearson (non-excess) fourth standardized moment over all
elements; the hot-channel ratio is the largest per-channel RMS over the
median per-channel RMS, channels being the last (K) dimension.

The fake quantization runs through the library's own kernels
(nvfp4_quantize then nvfp4_dequantize); the reductions are plain torch
operations in float64.  Nothing here is on the serving path.
"""
from __future__ import annotations

import torch


def tensor_stats(x: torch.Tensor) -> dict:
    """max/RMS, kurtosis, hot-channel ratio and 1-hot block share of a
    [rows, K] tensor (rows = tokens or output channels, K % 16 == 0)."""
    if x.dim() != 2 or x.shape[1] % 16 != 0 or x.numel() == 0:
        raise ValueError("expected a non-empty [rows, K] tensor with K % 16 == 0")
    v = x.double()
    rms = v.square().mean().sqrt()
    amax = v.abs().max()
    mu = v.mean()
    var = (v - mu).square().mean()
    kurt = (v - mu).pow(4).mean() / var.square() if var > 0 else torch.tensor(float("nan"), dtype=torch.float64)
    ch_rms = v.square().mean(dim=0).sqrt()
    med = ch_rms.median()
    hot = ch_rms.max() / med if med > 0 else torch.tensor(float("inf"), dtype=torch.float64)
    blocks = v.reshape(v.shape[0], -1, 16)
    b_rms = blocks.square().mean(dim=2).sqrt()
    b_max = blocks.abs().amax(dim=2)
    live = b_rms > 0
    one_hot = ((b_max > 3.0 * b_rms) & live).sum().double() / live.sum().clamp(min=1).double()
    return {"max_over_rms": float(amax / rms) if rms > 0 else float("nan"),
            "kurtosis": float(kurt),
            "hot_channel_ratio": float(hot),
            "one_hot_block_share": float(one_hot)}


def fake_quant_error(x: torch.Tensor) -> dict:
    """Relative error of quantizing x alone (A4 for activations, W4 for
    weights): the whole-tensor Frobenius ratio, and the median over rows of
    the per-row ratio (per token for activations)."""
    from . import nvfp4_dequantize, nvfp4_quantize
    codes, scales, gs = nvfp4_quantize(x)
    xd = nvfp4_dequantize(codes, scales, gs, torch.float32).double()
    v = x.double()
    err = xd - v
    tot = err.norm() / v.norm() if v.norm() > 0 else torch.tensor(0.0, dtype=torch.float64)
    row_n = v.norm(dim=1)
    keep = row_n > 0
    per_row = err.norm(dim=1)[keep] / row_n[keep]
    return {"rel_error": float(tot),
            "median_row_rel_error": float(per_row.median()) if per_row.numel() else 0.0}


def gemm_error(y: torch.Tensor, y_ref: torch.Tensor) -> float:
    """Frobenius relative error of a projection output against its
    high-precision reference."""
    r = y_ref.double()
    n = r.norm()
    return float((y.double() - r).norm() / n) if n > 0 else 0.0
