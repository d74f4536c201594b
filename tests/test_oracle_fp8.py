"""Pins of the oracle's FP8 E4M3 per-tensor quantization and its W8A16 /
W8A8 products (model card "Gemma-4-31B-IT-NVFP4-FP8attn-text", section
"What was quantized, exactly": per-tensor scale, float8_e4m3; paper "Why
Gated DeltaNet Survives 4-Bit Quantization", section 7: FP8 KV cache with
static per-tensor scales).

Independent references: torch's float32 -> float8_e4m3fn conversion (round
to nearest even) and float8_e4m3fn decode, numpy float64 matmul, and closed
forms (every grid value round-trips; ties go to the even byte; magnitudes
from 448 up saturate at 0x7E; the dynamic scale makes the largest byte 0x7E
and 448 * scale reproduce the absmax)."""
import numpy as np
import pytest
import torch

import workloads


def _e4m3_torch(b):
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


def _to_e4m3_torch(v):
    """torch's RNE conversion of float32 values (all finite, |v| <= 448)."""
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_every_grid_value_round_trips(orc):
    b = np.array([i for i in range(256) if (i & 0x7F) != 0x7F], dtype=np.uint8)
    for s in (1.0, 2.0 ** -20, 2.0 ** 30, 0.125):
        x = (_e4m3_torch(b) * s).astype(np.float32)[None, :]
        q, _ = orc.fp8_quantize(x, scale=s)
        assert np.array_equal(q[0], b), s


def test_matches_torch_conversion(orc):
    g = np.random.default_rng(0)
    x = (g.standard_normal((64, 256)) * 2.0 ** g.integers(-12, 8, size=(64, 256))).astype(np.float32)
    s = np.float32(0.37)
    r = (x / s).astype(np.float32)
    keep = np.abs(r) <= 448.0
    q, _ = orc.fp8_quantize(x, scale=s)
    assert np.array_equal(q[keep], _to_e4m3_torch(r[keep]))
    assert (q[~keep] & 0x7F == 0x7E).all()


def test_ties_to_even_and_saturation(orc):
    vals = np.array([1.0625, 1.1875, 0.5 * 2.0 ** -9, 1.5 * 2.0 ** -9, 464.0, 1e30, 448.0, 447.9,
                     -1.0625, -0.0, 0.0], dtype=np.float32)
    want = np.array([0x38, 0x3A, 0x00, 0x02, 0x7E, 0x7E, 0x7E, 0x7E, 0xB8, 0x80, 0x00], dtype=np.uint8)
    q, _ = orc.fp8_quantize(vals[None, :], scale=1.0)
    assert np.array_equal(q[0], want)


def test_dynamic_scale_identity(orc):
    x = workloads.to_bf16_bits(workloads.student_t(21, 1, 40, 512, 3.0))
    q, s = orc.fp8_quantize(x)
    amax = np.abs(workloads.bf16_bits_to_f32(x)).max()
    assert s == np.float32(amax / np.float32(448.0))
    assert (q & 0x7F).max() == 0x7E
    assert abs(448.0 * float(s) - float(amax)) <= 2.0 ** -24 * float(amax)


def test_zero_scale_keeps_signs(orc):
    x = np.array([[0.0, -0.0, 1.0, -2.0] * 4], dtype=np.float32)
    q, _ = orc.fp8_quantize(x, scale=0.0)
    assert np.array_equal(q[0], np.array([0, 0x80, 0, 0x80] * 4, dtype=np.uint8))


def test_dequantize(orc):
    b = np.arange(256, dtype=np.uint8).reshape(16, 16)
    b[(b & 0x7F) == 0x7F] = 0x11
    s = np.float32(0.0123)
    got = orc.fp8_dequantize(b, s)
    assert np.array_equal(got, (_e4m3_torch(b) * np.float64(s)).astype(np.float32))


@pytest.mark.parametrize("M,N,K", [(1, 40, 64), (9, 33, 256)])
def test_w8a16_matches_float64_matmul(orc, M, N, K):
    x = workloads.to_bf16_bits(workloads.student_t(21, 2, M, K, 3.0))
    wq, sw = orc.fp8_quantize(workloads.gaussian(21, 3, N, K, 0.02))
    got = orc.gemm_w8a16(x, wq, sw)
    ref = workloads.bf16_bits_to_f32(x).astype(np.float64) @ _e4m3_torch(wq).T * float(sw)
    assert np.max(np.abs(got - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_w8a8_exact(orc):
    g = np.random.default_rng(5)
    xq = g.integers(0, 256, size=(7, 320), dtype=np.uint8)
    wq = g.integers(0, 256, size=(11, 320), dtype=np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0
    wq[(wq & 0x7F) == 0x7F] = 0
    sx, sw = np.float32(0.5), np.float32(3.0)
    got = orc.gemm_w8a8(xq, sx, wq, sw)
    ref = (_e4m3_torch(xq) @ _e4m3_torch(wq).T) * 1.5    # integer multiples of 2^-18: exact in float64
    assert np.array_equal(got, ref)
