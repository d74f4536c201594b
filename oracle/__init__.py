"""NVFP4 oracle: TEST INFRASTRUCTURE ONLY.

A plain CPU statement of the NVFP4 W4A4 linear layer (quantize, dequantize,
fused-module repair, exact block-scaled GEMM) and of the W4A16 form of the
same weights against 16-bit activations, plus FP8 E4M3 with one per-tensor
scale (quantize, dequantize, W8A16 and W8A8 products), written in C
(``nvfp4_oracle.c``) and wrapped here with ctypes over numpy arrays.  Only the
tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import it.  It shares nothing with the HIP library in
``nvfp4_w4a4_quantized_02_amd``; the two meet only through the seeded inputs in
``workloads.py`` and the comparisons the tests make.

Every function follows the paper "Why Gated DeltaNet Survives 4-Bit
Quantization: NVFP4 W4A4 for the Recurrent Half of a Hybrid 27B LLM",
section 2 ("NVFP4") and section 6 ("Per-module calibration vs. fused-GEMM
scaling"), and the model card "Gemma-4-31B-IT-NVFP4-FP8attn-text",
sections "Verification" and "Limitations" (W4A16); the readings where those
pages are silent are listed
at the top of ``nvfp4_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libnvfp4_oracle.so")

# -ffp-contract=off: no fused multiply-add; no -ffast-math: IEEE division,
# subnormals kept.  -O2 only; the oracle is not tuned.
_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libnvfp4_oracle.so``."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        path = build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.orc_e2m1_decode.argtypes = [ctypes.c_uint]
        L.orc_e2m1_decode.restype = ctypes.c_double
        L.orc_e4m3_decode.argtypes = [ctypes.c_uint]
        L.orc_e4m3_decode.restype = ctypes.c_double
        L.orc_e4m3_encode.argtypes = [ctypes.c_float]
        L.orc_e4m3_encode.restype = ctypes.c_uint
        L.orc_e2m1_encode_mag.argtypes = [ctypes.c_float]
        L.orc_e2m1_encode_mag.restype = ctypes.c_uint
        L.orc_e4m3_encode_many.argtypes = [P, I64, P]
        L.orc_e2m1_encode_many.argtypes = [P, I64, P]
        L.orc_tensor_scale.argtypes = [P, ctypes.c_int, I64, I64, I64]
        L.orc_tensor_scale.restype = ctypes.c_float
        L.orc_quantize_with_scale.argtypes = [P, ctypes.c_int, I64, I64, I64, ctypes.c_float, P, P]
        L.orc_quantize.argtypes = [P, ctypes.c_int, I64, I64, I64, P, P, P]
        L.orc_quantize.restype = ctypes.c_int
        L.orc_dequantize.argtypes = [P, P, ctypes.c_float, I64, I64, P]
        L.orc_dequantize_bf16.argtypes = [P, P, ctypes.c_float, I64, I64, P]
        L.orc_fuse_rescale.argtypes = [ctypes.c_int, ctypes.POINTER(P), P, I64, P, P]
        L.orc_gemm_exact.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_float, I64, I64, I64, P]
        L.orc_gemm_exact_sampled.argtypes = [P, P, ctypes.c_float, P, P, ctypes.c_float, I64, I64,
                                             P, P, P]
        L.orc_num_threads.restype = ctypes.c_int
        L.orc_gemm_w4a16.argtypes = [P, ctypes.c_int, I64, I64, I64, P, P, ctypes.c_float, I64, P]
        L.orc_gemm_w4a16_sampled.argtypes = [P, ctypes.c_int, I64, I64, P, P, ctypes.c_float, I64, P, P, P]
        L.orc_fp8_tensor_scale.argtypes = [P, ctypes.c_int, I64, I64, I64]
        L.orc_fp8_tensor_scale.restype = ctypes.c_float
        L.orc_fp8_quantize_with_scale.argtypes = [P, ctypes.c_int, I64, I64, I64, ctypes.c_float, P]
        L.orc_fp8_dequantize.argtypes = [P, ctypes.c_float, I64, I64, P]
        L.orc_gemm_w8a16.argtypes = [P, ctypes.c_int, I64, I64, I64, P, ctypes.c_float, I64, P]
        L.orc_gemm_w8a8.argtypes = [P, ctypes.c_float, P, ctypes.c_float, I64, I64, I64, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _as_input(x: np.ndarray):
    """Return (contiguous array, is_bf16).  bf16 tensors travel as uint16."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 1
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), 0
    raise TypeError("oracle input must be float32 or bf16 bits (uint16), got %s" % x.dtype)


# ---------------------------------------------------------------- codecs

def e2m1_decode(code: int) -> float:
    return lib().orc_e2m1_decode(code)


def e4m3_decode(byte: int) -> float:
    return lib().orc_e4m3_decode(byte)


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().orc_e4m3_encode_many(_ptr(v), v.size, _ptr(out))
    return out


def e2m1_encode_mag(r: np.ndarray) -> np.ndarray:
    r = np.ascontiguousarray(r, dtype=np.float32)
    out = np.empty(r.shape, dtype=np.uint8)
    lib().orc_e2m1_encode_many(_ptr(r), r.size, _ptr(out))
    return out


def e4m3_table() -> np.ndarray:
    """fp64 value of every E4M3 byte (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3_decode(b) for b in range(256)], dtype=np.float64)


def e2m1_table() -> np.ndarray:
    return np.array([e2m1_decode(c) for c in range(16)], dtype=np.float64)


# ---------------------------------------------------------------- quantize

def tensor_scale(x: np.ndarray) -> np.float32:
    xa, is_bf16 = _as_input(x)
    rows, K = xa.shape
    return np.float32(lib().orc_tensor_scale(_ptr(xa), is_bf16, rows, K, K))


def quantize(x: np.ndarray, gs: float | None = None):
    """Quantize a [rows, K] float32 / bf16-bits tensor.

    Returns (codes uint8 [rows, K/2], scales uint8 [rows, K/16], gs float32).
    With ``gs`` given, that tensor scale is used instead of amax/2688.
    """
    xa, is_bf16 = _as_input(x)
    rows, K = xa.shape
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    codes = np.zeros((rows, K // 2), dtype=np.uint8)
    scales = np.zeros((rows, K // 16), dtype=np.uint8)
    if gs is None:
        g = np.zeros(1, dtype=np.float32)
        rc = lib().orc_quantize(_ptr(xa), is_bf16, rows, K, K, _ptr(codes), _ptr(scales), _ptr(g))
        assert rc == 0
        return codes, scales, np.float32(g[0])
    lib().orc_quantize_with_scale(_ptr(xa), is_bf16, rows, K, K, float(np.float32(gs)),
                                  _ptr(codes), _ptr(scales))
    return codes, scales, np.float32(gs)


def dequantize(codes: np.ndarray, scales: np.ndarray, gs: float) -> np.ndarray:
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    rows, half = codes.shape
    K = 2 * half
    out = np.empty((rows, K), dtype=np.float32)
    lib().orc_dequantize(_ptr(codes), _ptr(scales), float(np.float32(gs)), rows, K, _ptr(out))
    return out


def dequantize_bf16(codes: np.ndarray, scales: np.ndarray, gs: float) -> np.ndarray:
    """bf16 bits (uint16) of bf16(fp32 dequant)."""
    codes = np.ascontiguousarray(codes)
    scales = np.ascontiguousarray(scales)
    rows, half = codes.shape
    K = 2 * half
    out = np.empty((rows, K), dtype=np.uint16)
    lib().orc_dequantize_bf16(_ptr(codes), _ptr(scales), float(np.float32(gs)), rows, K, _ptr(out))
    return out


def fuse_rescale(scales_list, gs_list):
    """Repair a fused group.  Returns (new scale arrays, shared gs)."""
    outs = [np.ascontiguousarray(s).copy() for s in scales_list]
    kb = outs[0].shape[1]
    for s in outs:
        assert s.shape[1] == kb
    n = len(outs)
    ptrs = (ctypes.c_void_p * n)(*[_ptr(s) for s in outs])
    rows = np.array([s.shape[0] for s in outs], dtype=np.int64)
    gs = np.array(gs_list, dtype=np.float32)
    shared = np.zeros(1, dtype=np.float32)
    lib().orc_fuse_rescale(n, ptrs, _ptr(rows), kb, _ptr(gs), _ptr(shared))
    return outs, np.float32(shared[0])


def gemm_exact(xc, xs, gsx, wc, ws, gsw) -> np.ndarray:
    """Exact y = deq(X) . deq(W)^T as fp64 [M, N]."""
    xc, xs, wc, ws = (np.ascontiguousarray(a) for a in (xc, xs, wc, ws))
    M, K = xc.shape[0], 2 * xc.shape[1]
    N = wc.shape[0]
    assert wc.shape[1] * 2 == K
    y = np.empty((M, N), dtype=np.float64)
    lib().orc_gemm_exact(_ptr(xc), _ptr(xs), float(np.float32(gsx)), _ptr(wc), _ptr(ws),
                         float(np.float32(gsw)), M, N, K, _ptr(y))
    return y


def gemm_exact_sampled(xc, xs, gsx, wc, ws, gsw, m_idx, n_idx) -> np.ndarray:
    xc, xs, wc, ws = (np.ascontiguousarray(a) for a in (xc, xs, wc, ws))
    K = 2 * xc.shape[1]
    m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
    n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
    assert m_idx.shape == n_idx.shape
    y = np.empty(m_idx.shape, dtype=np.float64)
    lib().orc_gemm_exact_sampled(_ptr(xc), _ptr(xs), float(np.float32(gsx)), _ptr(wc), _ptr(ws),
                                 float(np.float32(gsw)), K, m_idx.size, _ptr(m_idx), _ptr(n_idx),
                                 _ptr(y))
    return y


def linear(x, wc, ws, gsw):
    """The served W4A4 linear: quantize x on the fly, then the exact GEMM.

    Returns (y fp64 [M, N], (xc, xs, gsx))."""
    xc, xs, gsx = quantize(x)
    return gemm_exact(xc, xs, gsx, wc, ws, gsw), (xc, xs, gsx)


def gemm_w4a16(x, wc, ws, gsw) -> np.ndarray:
    """W4A16: y = x . deq(W)^T as fp64 [M, N], x a [M, K] float32 or
    bf16-bits tensor used as given (no activation quantization)."""
    xa, is_bf16 = _as_input(x)
    wc, ws = np.ascontiguousarray(wc), np.ascontiguousarray(ws)
    M, K = xa.shape
    N = wc.shape[0]
    assert wc.shape[1] * 2 == K and ws.shape[1] * 16 == K
    y = np.empty((M, N), dtype=np.float64)
    lib().orc_gemm_w4a16(_ptr(xa), is_bf16, M, K, K, _ptr(wc), _ptr(ws), float(np.float32(gsw)), N, _ptr(y))
    return y


def gemm_w4a16_sampled(x, wc, ws, gsw, m_idx, n_idx) -> np.ndarray:
    xa, is_bf16 = _as_input(x)
    wc, ws = np.ascontiguousarray(wc), np.ascontiguousarray(ws)
    K = xa.shape[1]
    m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
    n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
    assert m_idx.shape == n_idx.shape
    y = np.empty(m_idx.shape, dtype=np.float64)
    lib().orc_gemm_w4a16_sampled(_ptr(xa), is_bf16, K, K, _ptr(wc), _ptr(ws), float(np.float32(gsw)),
                                 m_idx.size, _ptr(m_idx), _ptr(n_idx), _ptr(y))
    return y


def fp8_tensor_scale(x) -> np.float32:
    xa, is_bf16 = _as_input(x)
    rows, K = xa.shape
    return np.float32(lib().orc_fp8_tensor_scale(_ptr(xa), is_bf16, rows, K, K))


def fp8_quantize(x, scale: float | None = None):
    """FP8 E4M3 with one per-tensor scale: returns (bytes uint8 [rows, K],
    scale float32); the scale is RN(amax / 448) unless given."""
    xa, is_bf16 = _as_input(x)
    rows, K = xa.shape
    s = fp8_tensor_scale(xa) if scale is None else np.float32(scale)
    q = np.zeros((rows, K), dtype=np.uint8)
    lib().orc_fp8_quantize_with_scale(_ptr(xa), is_bf16, rows, K, K, float(s), _ptr(q))
    return q, s


def fp8_dequantize(q, scale) -> np.ndarray:
    q = np.ascontiguousarray(q)
    rows, K = q.shape
    out = np.empty((rows, K), dtype=np.float32)
    lib().orc_fp8_dequantize(_ptr(q), float(np.float32(scale)), rows, K, _ptr(out))
    return out


def gemm_w8a16(x, wq, sw) -> np.ndarray:
    """y = x . (E4M3(wq) * sw)^T as fp64 [M, N]; x float32 or bf16 bits."""
    xa, is_bf16 = _as_input(x)
    wq = np.ascontiguousarray(wq)
    M, K = xa.shape
    N = wq.shape[0]
    assert wq.shape[1] == K
    y = np.empty((M, N), dtype=np.float64)
    lib().orc_gemm_w8a16(_ptr(xa), is_bf16, M, K, K, _ptr(wq), float(np.float32(sw)), N, _ptr(y))
    return y


def gemm_w8a8(xq, sx, wq, sw) -> np.ndarray:
    """Exact y = (E4M3(xq) * sx) . (E4M3(wq) * sw)^T as fp64 [M, N]."""
    xq, wq = np.ascontiguousarray(xq), np.ascontiguousarray(wq)
    M, K = xq.shape
    N = wq.shape[0]
    assert wq.shape[1] == K
    y = np.empty((M, N), dtype=np.float64)
    lib().orc_gemm_w8a8(_ptr(xq), float(np.float32(sx)), _ptr(wq), float(np.float32(sw)), M, N, K, _ptr(y))
    return y


def num_threads() -> int:
    return lib().orc_num_threads()
