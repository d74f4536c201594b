"""Helpers for the GPU parity tests: moving seeded numpy inputs to the GPU,
and the floating-point gate for GEMM outputs.

GEMM gate (the kernel accumulates exact products in FP32, the oracle sums
them exactly in int64):
  * normwise:   max|y - y*| / max|y*| <= 1e-3
  * elementwise |y - y*| <= 1e-3 * max(|y*|, rms of the row of y*)
  Both take whole output rows, so every element is judged against the rms of
  its own row.  For bf16 outputs both gates first grant 2^-8 |y*| (one bf16
  ulp: the final rounding of two fp32 sums that differ only in accumulation
  order can land one ulp apart; the paper's Appendix A puts the BF16 floor at
  about 2^-8).
"""
from __future__ import annotations

import numpy as np
import torch

REL_TOL = 1e-3


def dev():
    return torch.device("cuda:0")


def to_gpu(a: np.ndarray) -> torch.Tensor:
    """float32 -> float32 tensor; uint16 (bf16 bits) -> bfloat16 tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_np(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(y: np.ndarray) -> np.ndarray:
    if y.dtype == np.uint16:
        return (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return y.astype(np.float64)


def check_gemm(y: np.ndarray, ref: np.ndarray, out_bf16: bool, what: str = ""):
    """Gate whole rows: y and ref are [rows, N] (complete output rows)."""
    y = as_f64(y)
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert ref.ndim == 2, "%s: the gate takes whole output rows" % what
    assert np.isfinite(y).all(), "%s: non-finite outputs" % what
    d = np.abs(y - ref)
    scale = np.abs(ref).max() if ref.size else 0.0
    if scale == 0:
        assert d.size == 0 or d.max() == 0, "%s: expected all zeros" % what
        return 0.0
    # bf16 outputs: one bf16 ulp of the final rounding is not accumulation error
    dn = np.maximum(d - 2.0 ** -8 * np.abs(ref), 0.0) if out_bf16 else d
    norm_err = dn.max() / scale
    assert norm_err <= REL_TOL, "%s: normwise error %.3g > %g" % (what, norm_err, REL_TOL)
    row_rms = np.sqrt(np.mean(ref ** 2, axis=1, keepdims=True))
    allow = REL_TOL * np.maximum(np.abs(ref), row_rms)
    if out_bf16:
        allow = allow + 2.0 ** -8 * np.abs(ref)
    bad = d > allow
    assert not bad.any(), "%s: %d elements outside the elementwise gate (worst %.3g)" % (
        what, int(bad.sum()), float((d / np.maximum(allow, 1e-300)).max()))
    return float(norm_err)


def sample_rows(M: int, n: int, seed: int, must=()) -> np.ndarray:
    """n random rows of [0, M) plus the first, the last and `must`, sorted."""
    g = np.random.default_rng(seed)
    rows = g.choice(M, size=min(n, M), replace=False)
    return np.unique(np.concatenate([rows, [0, M - 1], np.asarray(must, dtype=np.int64)])).astype(np.int64)


def unpack_codes(codes: np.ndarray) -> np.ndarray:
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out
