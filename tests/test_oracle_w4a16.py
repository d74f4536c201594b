"""Pins of the oracle's W4A16 product: NVFP4 weights against bf16/fp32
activations used as given (model card "Gemma-4-31B-IT-NVFP4-FP8attn-text",
section "Limitations": without native FP4 tensor cores the weights are served
as W4A16; the weight format is the paper's, "Why Gated DeltaNet Survives
4-Bit Quantization", section 2 "NVFP4").

The weight operand is decoded independently of the oracle (a literal E2M1
table and torch's float8_e4m3fn decode of the scale bytes); the contraction
is numpy's float64 matmul, and exact rational arithmetic on a tiny problem.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads

_E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])


def _unpack(codes):
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def _deq_independent(codes, scales):
    """E2M1(code) * E4M3(scale) as float64 [N, K], without the oracle."""
    sc = torch.from_numpy(np.ascontiguousarray(scales & 0x7F)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()
    return _E2M1[_unpack(codes)] * np.repeat(sc, 16, axis=1)


def _x_f64(x):
    if x.dtype == np.uint16:
        return workloads.bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def _rel(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


@pytest.mark.parametrize("M,N,K", [(1, 64, 64), (7, 33, 160), (16, 256, 512)])
def test_matches_float64_matmul(orc, M, N, K):
    x = workloads.to_bf16_bits(workloads.student_t(11, 1, M, K, 3.0))
    w = workloads.gaussian(11, 2, N, K, 0.02)
    wc, ws, gsw = orc.quantize(w)
    got = orc.gemm_w4a16(x, wc, ws, gsw)
    ref = (_x_f64(x) @ _deq_independent(wc, ws).T) * float(gsw)
    assert _rel(got, ref) < 1e-12


def test_unit_scales_reduce_to_e2m1_matmul(orc):
    g = np.random.default_rng(4)
    M, N, K = 5, 40, 128
    codes = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = np.full((N, K // 16), 0x38, dtype=np.uint8)      # E4M3 1.0
    x = workloads.to_bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    got = orc.gemm_w4a16(x, codes, scales, 1.0)
    ref = _x_f64(x) @ _E2M1[_unpack(codes)].T
    assert _rel(got, ref) < 1e-13


def test_one_hot_rows_pick_dequantized_columns(orc):
    """x = e_k: y[:, n] is W's dequantized element (n, k) times gs_w; after
    one fp32 rounding it equals the oracle's own fp32 dequant exactly (as
    values: a -0 code dequantizes to -0.0, while the sum is +0)."""
    w = workloads.gaussian(11, 3, 48, 96, 0.05)
    wc, ws, gsw = orc.quantize(w)
    K = 96
    x = np.zeros((K, K), np.float32)
    x[np.arange(K), np.arange(K)] = 1.0
    y = orc.gemm_w4a16(x, wc, ws, gsw)                 # [K, N]: row k = column k of deq(W)
    deq = orc.dequantize(wc, ws, gsw)                  # [N, K] fp32
    assert np.array_equal(y.T.astype(np.float32), deq)


def test_exact_rational_tiny(orc):
    g = np.random.default_rng(8)
    M, N, K = 2, 3, 32
    x = (g.standard_normal((M, K)) * 2.0 ** g.integers(-20, 20, size=(M, K))).astype(np.float32)
    codes = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    scales = g.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8)
    gsw = np.float32(0.0123)
    got = orc.gemm_w4a16(x, codes, scales, gsw)
    d = _deq_independent(codes, scales)
    for m in range(M):
        for n in range(N):
            s = sum(Fraction(float(x[m, k])) * Fraction(float(d[n, k])) for k in range(K))
            exact = float(s * Fraction(float(gsw)))
            assert abs(got[m, n] - exact) <= 1e-15 * max(abs(exact), 1e-300) + 1e-300


def test_sign_power_of_two_and_dtype_invariance(orc):
    x = workloads.student_t(11, 4, 6, 256, 3.0)
    xb = workloads.to_bf16_bits(x)
    xf = workloads.bf16_bits_to_f32(xb)                # the same values as fp32
    w = workloads.gaussian(11, 5, 20, 256, 0.02)
    wc, ws, gsw = orc.quantize(w)
    y = orc.gemm_w4a16(xb, wc, ws, gsw)
    assert np.array_equal(orc.gemm_w4a16(xf, wc, ws, gsw), y)
    assert np.array_equal(orc.gemm_w4a16((-xf).astype(np.float32), wc, ws, gsw), -y)
    assert np.array_equal(orc.gemm_w4a16((xf * np.float32(8)).astype(np.float32), wc, ws, gsw), 8 * y)


def test_sampled_equals_full(orc):
    x = workloads.to_bf16_bits(workloads.student_t(11, 6, 9, 192, 3.0))
    w = workloads.gaussian(11, 7, 31, 192, 0.02)
    wc, ws, gsw = orc.quantize(w)
    full = orc.gemm_w4a16(x, wc, ws, gsw)
    mi = np.array([0, 8, 3, 5]),
    mi, ni = np.array([0, 8, 3, 5]), np.array([30, 0, 17, 17])
    assert np.array_equal(orc.gemm_w4a16_sampled(x, wc, ws, gsw, mi, ni), full[mi, ni])
