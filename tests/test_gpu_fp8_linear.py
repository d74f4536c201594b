"""GPU parity of the FP8-weight linears with the oracle (model card
"Gemma-4-31B-IT-NVFP4-FP8attn-text", section "What was quantized, exactly":
float8_e4m3 weights with one per-tensor scale, served W8A16; W8A8 with FP8
activations).  The weights are the oracle's bytes, uploaded.  Every form is
hit: the K-split GEMV (M <= 16, K <= 5120, including a partial last slice),
the tile GEMM with and without its split-K tail, and small M with K > 5120;
full decode and prefill sizes on whole output rows.  Gate: the GEMM gate of
the W4A4 tests."""
import numpy as np
import pytest
import torch

import workloads
from parity import check_gemm, sample_rows, to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_w4a4_quantized_02_amd as m
    return m


def _sc(v):
    return torch.tensor([np.float32(v)], dtype=torch.float32, device="cuda:0")


SHAPES = [(1, 300, 512), (4, 520, 5120), (16, 129, 768), (9, 100, 320), (3, 40, 6144),
          (17, 64, 64), (100, 200, 320), (300, 257, 1088), (513, 300, 256)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w8a16_matches_oracle(nv, orc, M, N, K, out):
    x = workloads.to_bf16_bits(workloads.student_t(25, 1, M, K, 3.0))
    wq, sw = orc.fp8_quantize(workloads.gaussian(25, 2, N, K, 0.02))
    print("case: w8a16 %dx%dx%d %s" % (M, N, K, out), flush=True)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    y = to_np(nv.nvfp4_gemm_w8a16(to_gpu(x), to_gpu(wq), _sc(sw), out_dtype=od))
    torch.cuda.synchronize()
    check_gemm(y, orc.gemm_w8a16(x, wq, sw), out == "bf16", "w8a16 %dx%dx%d" % (M, N, K))


@pytest.mark.parametrize("mode", ["dynamic", "static"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w8a8_matches_oracle(nv, orc, M, N, K, mode):
    x = workloads.to_bf16_bits(workloads.student_t(25, 3, M, K, 3.0))
    wq, sw = orc.fp8_quantize(workloads.gaussian(25, 4, N, K, 0.02))
    if mode == "dynamic":
        xq, sx = orc.fp8_quantize(x)
        xs = None
    else:
        sx = np.float32(orc.fp8_tensor_scale(x) * np.float32(0.6))    # a calibrated scale: saturates the largest
        xq, _ = orc.fp8_quantize(x, scale=sx)
        xs = _sc(sx)
    print("case: w8a8 %s %dx%dx%d" % (mode, M, N, K), flush=True)
    y = to_np(nv.nvfp4_gemm_w8a8(to_gpu(x), to_gpu(wq), _sc(sw), x_scale=xs, out_dtype=torch.float32))
    torch.cuda.synchronize()
    check_gemm(y, orc.gemm_w8a8(xq, sx, wq, sw), False, "w8a8 %s %dx%dx%d" % (mode, M, N, K))


def test_w8a8_fp32_activations_and_strided_rows(nv, orc):
    M, N, K = 40, 96, 512
    x = workloads.gaussian(25, 5, M, K, 1.0)
    wq, sw = orc.fp8_quantize(workloads.gaussian(25, 6, N, K, 0.02))
    big = torch.zeros((M, K + 64), dtype=torch.float32, device="cuda:0")
    big[:, :K] = to_gpu(x)
    y = to_np(nv.nvfp4_gemm_w8a8(big[:, :K], to_gpu(wq), _sc(sw), out_dtype=torch.float32))
    xq, sx = orc.fp8_quantize(x)
    check_gemm(y, orc.gemm_w8a8(xq, sx, wq, sw), False, "w8a8 fp32 strided")


def test_fp8_linears_empty_and_k_zero(nv):
    wq = torch.zeros((8, 0), dtype=torch.uint8, device="cuda:0")
    for M in (3, 40):
        for f in (nv.nvfp4_gemm_w8a16, nv.nvfp4_gemm_w8a8):
            x = torch.zeros((M, 0), dtype=torch.bfloat16, device="cuda:0")
            y = torch.full((M, 8), 7.0, device="cuda:0")
            f(x, wq, _sc(1.0), out=y)
            torch.cuda.synchronize()
            assert torch.count_nonzero(y).item() == 0


def _rows(nv, orc, x, w, a8, rows):
    """GPU linear on FP8 weights (quantized on the GPU, byte-exact with the
    oracle by the FP8 quantize tests); the oracle recomputes whole rows."""
    sw = orc.fp8_tensor_scale(w)
    q, s = nv.nvfp4_fp8_quantize(to_gpu(w))
    torch.cuda.synchronize()
    assert np.float32(s.item()) == sw
    xg = to_gpu(x)
    if a8:
        y = to_np(nv.nvfp4_gemm_w8a8(xg, q, s, out_dtype=torch.bfloat16))
    else:
        y = to_np(nv.nvfp4_gemm_w8a16(xg, q, s, out_dtype=torch.bfloat16))
    torch.cuda.synchronize()
    del q
    wq, _ = orc.fp8_quantize(w, scale=sw)
    xs = np.ascontiguousarray(x[rows])
    if a8:
        sx = orc.fp8_tensor_scale(x)
        xq, _ = orc.fp8_quantize(xs, scale=sx)
        ref = orc.gemm_w8a8(xq, sx, wq, sw)
    else:
        ref = orc.gemm_w8a16(xs, wq, sw)
    return y[rows], ref


@pytest.mark.parametrize("a8", [False, True])
@pytest.mark.parametrize("M", [1, 16])
def test_fp8_linear_full_decode(nv, orc, M, a8):
    p = workloads.decode(M=M)
    w = np.concatenate(p.w_parts)
    print("case: %s full decode M=%d N=34816 K=5120" % ("w8a8" if a8 else "w8a16", M), flush=True)
    got, ref = _rows(nv, orc, p.x, w, a8, np.arange(M))
    check_gemm(got, ref, True, "fp8 full decode M=%d" % M)


@pytest.mark.parametrize("a8", [False, True])
def test_fp8_linear_full_prefill(nv, orc, a8):
    p = workloads.prefill()
    print("case: %s full prefill 4096x17408x5120" % ("w8a8" if a8 else "w8a16"), flush=True)
    got, ref = _rows(nv, orc, p.x, p.w_parts[0], a8, sample_rows(p.M, 10, 4, must=[3840, 4000]))
    check_gemm(got, ref, True, "fp8 full prefill")


@pytest.mark.parametrize("a8", [False, True])
def test_fp8_linear_split_tail(nv, orc, a8):
    # 2 x 129 tiles = 258 of the shared tile plan: the last 2 (tile row 1,
    # tile columns 127 and 128, both ragged) are split along K (K = 128 is 2
    # steps).  Every output.
    M, N, K = 500, 33000, 128
    p = workloads.prefill(M=M, K=K, N=N)
    print("case: %s split tail M=%d N=%d K=%d" % ("w8a8" if a8 else "w8a16", M, N, K), flush=True)
    got, ref = _rows(nv, orc, p.x, p.w_parts[0], a8, np.arange(M))
    check_gemm(got, ref, True, "fp8 split tail")
