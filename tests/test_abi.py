"""CPU tests of the C ABI: the library loads, exports every function the
header declares, and rejects invalid arguments with the documented status
before launching anything (fake device addresses are never dereferenced on
the host, and every call here fails validation)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

OK, E_NULL, E_SHAPE, E_DTYPE, E_ALIGN, E_WS, E_INVALID, E_DEVICE = range(8)
F32, BF16 = 0, 1
A = 0x10000          # a 256-byte aligned fake device address
BIG = 1 << 30


@pytest.fixture(scope="module")
def nv():
    import nvfp4_w4a4_quantized_02_amd as m
    return m


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_function(nv):
    names = _declared()
    assert len(names) >= 8
    for n in names:
        assert hasattr(nv.lib, n), "missing export %s" % n
    assert sorted(nv.EXPORTS) == names


def test_status_enum_matches_header(nv):
    src = open(HEADER).read()
    vals = dict((k, int(v)) for k, v in re.findall(r"(NVFP4_(?:OK|ERR_[A-Z]+))\s*=\s*(\d+)", src))
    assert vals == {"NVFP4_OK": 0, "NVFP4_ERR_NULL": 1, "NVFP4_ERR_SHAPE": 2, "NVFP4_ERR_DTYPE": 3,
                    "NVFP4_ERR_ALIGN": 4, "NVFP4_ERR_WORKSPACE": 5, "NVFP4_ERR_INVALID": 6,
                    "NVFP4_ERR_DEVICE": 7}
    for code in range(8):
        assert nv.status_string(code)
    assert nv.status_string(99) == "unknown status"


def test_workspace_sizes(nv):
    L = nv.lib
    assert L.nvfp4_quantize_workspace_size(32768, 5120) >= 2048 * 4
    small = L.nvfp4_gemm_workspace_size(16, 34816, 5120)
    big = L.nvfp4_gemm_workspace_size(4096, 17408, 5120)
    assert small >= 16 * 5120 * 2
    assert big >= 4096 * 5120 * 2
    # ragged M pads to the 256-row tile, ragged K to 64
    assert L.nvfp4_gemm_workspace_size(257, 0, 128) - L.nvfp4_gemm_workspace_size(0, 0, 0) == 512 * 128 * 2
    # the last partial round of 256x256 tiles is split along K: fp32 parts
    tiles = 16 * 68                                       # M=4096, N=17408
    rem = tiles % 256
    parts = 256 // rem
    extra = L.nvfp4_gemm_workspace_size(4096, 17408, 5120) - L.nvfp4_gemm_workspace_size(4096, 0, 5120)
    assert extra == rem * parts * 256 * 256 * 4


def q(nv, x=A, dt=BF16, rows=4, K=32, ld=32, codes=A, scales=A, gs=A, ws=A, nws=BIG):
    return nv.lib.nvfp4_quantize(x, dt, rows, K, ld, codes, scales, gs, ws, nws, None)


def test_quantize_rejects(nv):
    assert q(nv, dt=5) == E_DTYPE
    assert q(nv, K=24, ld=24) == E_SHAPE
    assert q(nv, rows=-1) == E_SHAPE
    assert q(nv, ld=16) == E_SHAPE
    assert q(nv, x=None) == E_NULL
    assert q(nv, gs=None) == E_NULL
    assert q(nv, codes=None) == E_NULL
    assert q(nv, x=A + 8) == E_ALIGN
    assert q(nv, dt=BF16, ld=36) == E_ALIGN          # 72-byte rows
    assert q(nv, codes=A + 4) == E_ALIGN
    assert q(nv, ws=None) == E_WS
    assert q(nv, ws=A + 64) == E_WS
    assert q(nv, nws=100) == E_WS


def g(nv, x=A, dt=BF16, M=32, K=64, ld=64, wc=A, wsc=A, wg=A, N=64, y=A, ydt=BF16, ldy=64, ws=A, nws=BIG):
    return nv.lib.nvfp4_gemm(x, dt, M, K, ld, wc, wsc, wg, N, y, ydt, ldy, ws, nws, None)


def test_gemm_rejects(nv):
    assert g(nv, dt=2) == E_DTYPE
    assert g(nv, ydt=7) == E_DTYPE
    assert g(nv, K=48, ld=48) == E_SHAPE              # K % 64
    assert g(nv, K=96, ld=96) == E_SHAPE
    assert g(nv, K=1 << 23, ld=1 << 23) == E_SHAPE    # tile rows past 32-bit offsets (M > 16)
    assert g(nv, M=16, K=1 << 23, ld=1 << 23) == E_SHAPE  # and the GEMV forms' (M <= 16)
    assert nv.lib.nvfp4_gemm_run(32, 1 << 23, A, A, A, 64, A, BF16, 64, A, BIG, None) == E_SHAPE
    assert nv.lib.nvfp4_gemm_run(4, 1 << 23, A, A, A, 64, A, BF16, 64, A, BIG, None) == E_SHAPE
    assert g(nv, N=-3) == E_SHAPE
    assert g(nv, ldy=32) == E_SHAPE
    assert g(nv, y=None) == E_NULL
    assert g(nv, wc=None) == E_NULL
    assert g(nv, wg=None) == E_NULL
    assert g(nv, y=A + 8) == E_ALIGN
    assert g(nv, wc=A + 8) == E_ALIGN
    assert g(nv, ydt=BF16, ldy=68) == E_ALIGN         # 136-byte rows
    assert g(nv, nws=10) == E_WS
    assert g(nv, ws=A + 16) == E_WS
    # empty problems are valid and launch nothing
    assert g(nv, M=0) == OK
    assert g(nv, N=0) == OK


def test_gemm_noalloc_rejects(nv):
    L = nv.lib

    def na(x=A, dt=BF16, M=32, K=64, ld=64, wc=A, wsc=A, wg=A, N=64, y=A, ydt=BF16, ldy=64):
        return L.nvfp4_gemm_noalloc(x, dt, M, K, ld, wc, wsc, wg, N, y, ydt, ldy, None)

    assert na(dt=2) == E_DTYPE
    assert na(K=48, ld=48) == E_SHAPE
    assert na(y=None) == E_NULL
    assert na(y=A + 8) == E_ALIGN
    # more scratch than the fixed array holds: refused before the device is touched
    assert L.nvfp4_gemm_workspace_size(16384, 17408, 5120) > nv.NOALLOC_SCRATCH_BYTES
    assert na(M=16384, K=5120, ld=5120, N=17408, ldy=17408) == E_WS
    assert L.nvfp4_gemm_workspace_size(4096, 17408, 5120) <= nv.NOALLOC_SCRATCH_BYTES
    assert na(M=0) == OK
    assert na(N=0) == OK


def test_dequantize_rejects(nv):
    L = nv.lib
    assert L.nvfp4_dequantize(A, A, A, 4, 32, A, 9, 32, None) == E_DTYPE
    assert L.nvfp4_dequantize(A, A, A, 4, 40, A, F32, 40, None) == E_SHAPE
    assert L.nvfp4_dequantize(None, A, A, 4, 32, A, F32, 32, None) == E_NULL
    assert L.nvfp4_dequantize(A, A, A, 4, 32, A + 4, F32, 32, None) == E_ALIGN
    assert L.nvfp4_dequantize(A, A, A, 4, 32, A, F32, 16, None) == E_SHAPE
    assert L.nvfp4_dequantize(A, A, A, 0, 32, A, F32, 32, None) == OK


def test_fuse_rescale_rejects(nv):
    L = nv.lib
    P = ctypes.c_void_p

    def call(n, scales, rows, kb, gs, shared):
        sp = (P * max(n, 1))(*scales)
        rp = (ctypes.c_int64 * max(n, 1))(*rows)
        gp = (P * max(n, 1))(*gs)
        return L.nvfp4_fuse_rescale(n, sp, rp, kb, gp, shared, None)

    assert call(0, [A], [1], 4, [A], A + 256) == E_INVALID
    assert L.nvfp4_fuse_rescale(17, None, None, 4, None, A, None) == E_INVALID
    assert call(2, [A, A + 512], [1, 1], 4, [A + 4096, A + 8192], A + 4096) == E_INVALID  # aliasing
    assert call(2, [A, None], [1, 1], 4, [A + 4096, A + 8192], A + 256) == E_NULL
    assert call(1, [A], [1], 4, [None], A + 256) == E_NULL
    assert call(1, [A], [-1], 4, [A + 4096], A + 256) == E_SHAPE
    assert L.nvfp4_fuse_rescale(1, None, None, 4, None, A, None) == E_NULL


def qs(nv, x=A, dt=BF16, rows=4, K=32, ld=32, gs=A, codes=A, scales=A):
    return nv.lib.nvfp4_quantize_static(x, dt, rows, K, ld, gs, codes, scales, None)


def test_quantize_static_rejects(nv):
    assert qs(nv, dt=5) == E_DTYPE
    assert qs(nv, K=24, ld=24) == E_SHAPE
    assert qs(nv, ld=16) == E_SHAPE
    assert qs(nv, x=None) == E_NULL
    assert qs(nv, gs=None) == E_NULL
    assert qs(nv, scales=None) == E_NULL
    assert qs(nv, x=A + 8) == E_ALIGN
    assert qs(nv, codes=A + 4) == E_ALIGN
    # nothing to write: valid, and nothing is launched (no tensor scale is produced)
    assert qs(nv, rows=0) == OK
    assert qs(nv, K=0, ld=0) == OK


def gst(nv, x=A, dt=BF16, M=32, K=64, ld=64, gx=A, wc=A, wsc=A, wg=A, N=64, y=A, ydt=BF16, ldy=64, ws=A,
        nws=BIG):
    return nv.lib.nvfp4_gemm_static(x, dt, M, K, ld, gx, wc, wsc, wg, N, y, ydt, ldy, ws, nws, None)


def test_gemm_static_rejects(nv):
    L = nv.lib
    assert gst(nv, dt=2) == E_DTYPE
    assert gst(nv, ydt=7) == E_DTYPE
    assert gst(nv, K=48, ld=48) == E_SHAPE
    assert gst(nv, gx=None) == E_NULL
    assert gst(nv, wg=None) == E_NULL
    assert gst(nv, y=A + 8) == E_ALIGN
    assert gst(nv, nws=10) == E_WS
    assert gst(nv, M=0) == OK
    assert gst(nv, N=0) == OK
    # prepare with a given scale: same checks as the absmax prepare plus the scale pointer
    assert L.nvfp4_gemm_prepare_static(A, BF16, 32, 48, 48, A, A, BIG, None) == E_SHAPE
    assert L.nvfp4_gemm_prepare_static(A, BF16, 32, 64, 64, None, A, BIG, None) == E_NULL
    assert L.nvfp4_gemm_prepare_static(A, BF16, 32, 64, 64, A, A + 16, BIG, None) == E_WS
    assert L.nvfp4_gemm_prepare_static(A, BF16, 32, 64, 64, A, A, 100, None) == E_WS
    assert L.nvfp4_gemm_prepare_static(A, BF16, 0, 64, 64, A, A, BIG, None) == OK


def w16(nv, x=A, dt=BF16, M=32, K=64, ld=64, wc=A, wsc=A, wg=A, N=64, y=A, ydt=BF16, ldy=64, ws=A, nws=BIG):
    return nv.lib.nvfp4_gemm_w4a16(x, dt, M, K, ld, wc, wsc, wg, N, y, ydt, ldy, ws, nws, None)


def test_gemm_w4a16_rejects(nv):
    L = nv.lib
    assert w16(nv, dt=F32) == E_DTYPE                  # 16-bit activations only
    assert w16(nv, dt=2) == E_DTYPE
    assert w16(nv, ydt=7) == E_DTYPE
    assert w16(nv, K=48, ld=48) == E_SHAPE
    assert w16(nv, N=-1) == E_SHAPE
    assert w16(nv, ldy=32) == E_SHAPE
    assert w16(nv, x=None) == E_NULL
    assert w16(nv, wg=None) == E_NULL
    assert w16(nv, wc=None) == E_NULL
    assert w16(nv, y=A + 8) == E_ALIGN
    assert w16(nv, x=A + 8) == E_ALIGN
    assert w16(nv, wc=A + 8) == E_ALIGN
    assert w16(nv, M=0) == OK
    assert w16(nv, N=0) == OK
    # decode sizes need no workspace; the tile GEMM needs one for its split-K tail
    assert L.nvfp4_gemm_w4a16_workspace_size(16, 34816, 5120) == 0
    need = L.nvfp4_gemm_w4a16_workspace_size(4096, 17408, 5120)
    assert need == L.nvfp4_gemm_workspace_size(4096, 17408, 5120) - L.nvfp4_gemm_workspace_size(4096, 0, 5120)
    assert w16(nv, M=4096, K=5120, ld=5120, N=17408, ldy=17408, ws=None, nws=0) == E_WS
    assert w16(nv, M=4096, K=5120, ld=5120, N=17408, ldy=17408, nws=need - 1) == E_WS


def test_fp8_rejects(nv):
    L = nv.lib
    assert L.nvfp4_fp8_quantize(A, 5, 4, 32, 32, A, A, A, BIG, None) == E_DTYPE
    assert L.nvfp4_fp8_quantize(A, BF16, 4, 24, 24, A, A, A, BIG, None) == E_SHAPE
    assert L.nvfp4_fp8_quantize(A, BF16, 4, 32, 32, None, A, A, BIG, None) == E_NULL
    assert L.nvfp4_fp8_quantize(A, BF16, 4, 32, 32, A, None, A, BIG, None) == E_NULL
    assert L.nvfp4_fp8_quantize(A, BF16, 4, 32, 32, A + 8, A, A, BIG, None) == E_ALIGN
    assert L.nvfp4_fp8_quantize(A, BF16, 4, 32, 32, A, A, None, BIG, None) == E_WS
    assert L.nvfp4_fp8_quantize(A, BF16, 4, 32, 32, A, A, A, 8, None) == E_WS
    assert L.nvfp4_fp8_quantize_static(A, BF16, 4, 32, 32, None, A, None) == E_NULL
    assert L.nvfp4_fp8_quantize_static(A, BF16, 4, 32, 32, A, A + 4, None) == E_ALIGN
    assert L.nvfp4_fp8_quantize_static(A, BF16, 0, 32, 32, A, None, None) == OK
    assert L.nvfp4_fp8_dequantize(A, A, 4, 32, A, 9, 32, None) == E_DTYPE
    assert L.nvfp4_fp8_dequantize(A, A, 4, 40, A, F32, 40, None) == E_SHAPE
    assert L.nvfp4_fp8_dequantize(None, A, 4, 32, A, F32, 32, None) == E_NULL
    assert L.nvfp4_fp8_dequantize(A, A, 4, 32, A + 4, F32, 32, None) == E_ALIGN
    assert L.nvfp4_fp8_dequantize(A, A, 0, 32, A, F32, 32, None) == OK


def test_fp8_linear_rejects(nv):
    L = nv.lib

    def w816(x=A, dt=BF16, M=32, K=64, ld=64, wq=A, wsc=A, N=64, y=A, ydt=BF16, ldy=64, ws=A, nws=BIG):
        return L.nvfp4_gemm_w8a16(x, dt, M, K, ld, wq, wsc, N, y, ydt, ldy, ws, nws, None)

    def w88(x=A, dt=BF16, M=32, K=64, ld=64, xs=None, wq=A, wsc=A, N=64, y=A, ydt=BF16, ldy=64, ws=A, nws=BIG):
        return L.nvfp4_gemm_w8a8(x, dt, M, K, ld, xs, wq, wsc, N, y, ydt, ldy, ws, nws, None)

    assert w816(dt=F32) == E_DTYPE
    assert w816(K=48, ld=48) == E_SHAPE
    assert w816(wsc=None) == E_NULL
    assert w816(wq=None) == E_NULL
    assert w816(wq=A + 8) == E_ALIGN
    assert w816(M=0) == OK
    assert L.nvfp4_gemm_w8a16_workspace_size(16, 34816, 5120) == 0
    assert w88(dt=5) == E_DTYPE
    assert w88(K=48, ld=48) == E_SHAPE
    assert w88(y=None) == E_NULL
    assert w88(y=A + 8) == E_ALIGN
    assert w88(ws=None) == E_WS
    assert w88(nws=L.nvfp4_gemm_w8a8_workspace_size(32, 64, 64) - 1) == E_WS
    assert w88(N=0) == OK
    assert w88(M=32, K=1 << 24, ld=1 << 24) == E_SHAPE    # E4M3 rows past 32-bit tile offsets
    assert w88(M=4, K=1 << 24, ld=1 << 24) == E_SHAPE
    # X in FP8 (M x K bytes) plus the split-K sums of the tile GEMM
    assert L.nvfp4_gemm_w8a8_workspace_size(4096, 17408, 5120) >= 4096 * 5120 + \
        L.nvfp4_gemm_w8a16_workspace_size(4096, 17408, 5120)
