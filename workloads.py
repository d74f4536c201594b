"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module only draws random tensors; it holds none of the quantization or
GEMM arithmetic.  Both the oracle and the HIP library receive the same arrays
from here.

Shapes and distributions follow the NVFP4 W4A4 linear-layer workloads:
hidden size 5120 (the Qwen3.8-27B model of "Why Gated DeltaNet Survives 4-Bit
Quantization", section 2), near-Gaussian weights and heavy-tailed activations
with a few hot channels (same paper, section 5.1: median max/RMS 63.5, hot
channels about 100x the median channel).  The paper measures on captured
activations and public evaluation suites; none of those is used here, these
synthetic tensors stand in for them.

Generator: numpy ``default_rng(SeedSequence([seed, config, tensor]))``.
Values are drawn in fp32; a bf16 tensor is the round-to-nearest-even cast of
that fp32 draw, carried as uint16 bits.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

HIDDEN = 5120


def rng(config: int, tensor: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, config, tensor]))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits (uint16), round to nearest, ties to even (finite input)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def gaussian(config: int, tensor: int, rows: int, cols: int, std: float) -> np.ndarray:
    g = rng(config, tensor)
    return (g.standard_normal((rows, cols), dtype=np.float32) * np.float32(std)).astype(np.float32)


def with_hot_channels(x: np.ndarray, config: int, tensor: int, n_hot: int, factor: float) -> np.ndarray:
    """Multiply n_hot randomly chosen K-columns by factor (in place)."""
    if n_hot > 0:
        g = rng(config, 1000 + tensor)
        cols = g.choice(x.shape[1], size=n_hot, replace=False)
        x[:, cols] *= np.float32(factor)
    return x


def student_t(config: int, tensor: int, rows: int, cols: int, nu: float) -> np.ndarray:
    g = rng(config, tensor)
    out = np.empty((rows, cols), dtype=np.float32)
    step = max(1, (1 << 22) // max(cols, 1))
    for r0 in range(0, rows, step):  # chunked to bound the fp64 temporary
        r1 = min(rows, r0 + step)
        out[r0:r1] = g.standard_t(nu, size=(r1 - r0, cols)).astype(np.float32)
    return out


# ---------------------------------------------------------------- configs

@dataclass
class Linear:
    """One W4A4 linear problem: activations x [M, K] and weights w_parts
    (a list of [N_i, K] fp32 matrices, more than one for a fused group)."""
    name: str
    x: np.ndarray            # float32 or uint16 (bf16 bits)
    w_parts: list
    out_dtype: str           # "f32" or "bf16"

    @property
    def M(self):
        return self.x.shape[0]

    @property
    def K(self):
        return self.x.shape[1]

    @property
    def N(self):
        return sum(w.shape[0] for w in self.w_parts)


def tiny(M: int = 16, K: int = 256, N: int = 256) -> Linear:
    """X[16x256] fp32 N(0,1) with 2 hot channels x50; W[256x256] N(0, 0.02); fp32 out."""
    x = with_hot_channels(gaussian(1, 0, M, K, 1.0), 1, 0, 2, 50.0)
    w = gaussian(1, 1, N, K, 0.02)
    return Linear("tiny_f32", x, [w], "f32")


def decode(M: int = 1, K: int = HIDDEN, N_each: int = 17408) -> Linear:
    """X[Mx5120] bf16 N(0,1) with 0.1% of channels x100; fused gate/up
    W = 2 x [17408x5120] N(0, 0.02), each with its own tensor scale; bf16 out."""
    n_hot = int(round(0.001 * K))
    x = with_hot_channels(gaussian(2, 0, M, K, 1.0), 2, 0, n_hot, 100.0)
    gate = gaussian(2, 1, N_each, K, 0.02)
    up = gaussian(2, 2, N_each, K, 0.02)
    return Linear("decode_m%d" % M, to_bf16_bits(x), [gate, up], "bf16")


def prefill(M: int = 4096, K: int = HIDDEN, N: int = 17408) -> Linear:
    """X[4096x5120] bf16 Student-t(nu=3); W[17408x5120] N(0, 0.02); bf16 out."""
    x = student_t(3, 0, M, K, 3.0)
    w = gaussian(3, 1, N, K, 0.02)
    return Linear("prefill_m%d" % M, to_bf16_bits(x), [w], "bf16")


def fused_qkv(M: int = 2048, K: int = HIDDEN, Nq: int = 6144, Nkv: int = 1024,
              out_dtype: str = "f32") -> Linear:
    """q[6144x5120], k, v [1024x5120] N(0, 0.02), each rescaled to an absmax
    drawn from U[0.05, 0.5]; X[2048x5120] bf16 Student-t(nu=3)."""
    g = rng(4, 99)
    targets = g.uniform(0.05, 0.5, size=3).astype(np.float32)
    parts = []
    for i, n in enumerate((Nq, Nkv, Nkv)):
        w = gaussian(4, 1 + i, n, K, 0.02)
        w *= np.float32(targets[i] / np.abs(w).max())
        parts.append(w.astype(np.float32))
    x = student_t(4, 0, M, K, 3.0)
    return Linear("fused_qkv_m%d" % M, to_bf16_bits(x), parts, out_dtype)


def long_prefill_activations(M: int = 32768, K: int = HIDDEN) -> np.ndarray:
    """X[32768x5120] bf16 Student-t(nu=2.5) with 16 hot channels x200 (bf16 bits)."""
    x = with_hot_channels(student_t(5, 0, M, K, 2.5), 5, 0, 16, 200.0)
    return to_bf16_bits(x)
