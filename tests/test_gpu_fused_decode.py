"""One-launch decode: for up to four bf16 activation rows with K = 4096 or
5120, nvfp4_gemm quantizes the rows and runs the GEMV in a single kernel,
whose contraction runs on the FP4 MFMA over the raw codes with the block
scales applied to each (row, block) pair's exact sum.

Checks per case (paper "Why Gated DeltaNet Survives 4-Bit Quantization",
section 2 "NVFP4": activations quantized on the fly, one FP32 tensor scale,
E4M3 scale per 16 elements, the product of the two NVFP4 operands):
  * the output against the oracle's W4A4 product, under the GEMM gate, and
    the same for the two-launch path (quantize, then the fp16 GEMV) reached
    by handing the same values over as fp32; the two paths add the same
    exact block products in different orders, so only the gate binds them;
  * the workspace left as nvfp4_gemm_prepare leaves it: gs_x (byte 8192)
    with the oracle's bits, the fp16 operand E2M1 * E4M3 (from byte 8448)
    equal to the one built from the oracle's codes and scale bytes, and the
    oracle's packed codes and scale bytes after it.
Shapes cover one to four rows, a single tile (one wave of the three idle),
ragged N, an odd tile count, strided rows in and out, and the full fused
gate/up weight; inputs include rows on or next to every E2M1 and scale-byte
rounding tie, and calibrated scales."""
import numpy as np
import pytest
import torch

import workloads
from parity import check_gemm, to_gpu, to_np
from test_gpu_prepare import WS_GS, WS_X16, _expected_f16_bits, check_row_codes
from test_gpu_quantize import _scale_tie_tensor, _tie_tensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_w4a4_quantized_02_amd as m
    return m


def _weights(orc, N, K, seed):
    w = workloads.gaussian(41, seed, N, K, 0.02)
    wc, ws, gsw = orc.quantize(w)
    return (wc, ws, np.float32(gsw)), (to_gpu(wc), to_gpu(ws),
                                       torch.tensor([gsw], dtype=torch.float32, device="cuda:0"))


def _bf16_as_f32(xb: np.ndarray) -> np.ndarray:
    return (xb.astype(np.uint32) << 16).view(np.float32)


def _check_case(nv, orc, xb, w_host, w_dev, out, what, gs=None, pad=0):
    """xb: [M, K] bf16 bits; pad > 0 runs the one launch on rows pad elements
    longer than K and on output rows longer than N (strided views)."""
    print("case: fused decode", what, xb.shape, out, "given gs" if gs is not None else "", "pad %d" % pad,
          flush=True)
    M, K = xb.shape
    wc, ws, gsw = w_host
    N = wc.shape[0]
    od = torch.bfloat16 if out == "bf16" else torch.float32
    x_gs = None if gs is None else torch.tensor([float(gs)], dtype=torch.float32, device="cuda:0")
    xg = to_gpu(xb)
    if pad:
        wide = torch.zeros((M, K + pad), dtype=xg.dtype, device=xg.device)
        wide[:, :K] = xg
        xg = wide[:, :K]
        # output rows a multiple of 16 bytes apart, as the ABI requires
        yw = torch.full((M, N + (-N) % 8 + 8), float("nan"), dtype=od, device=xg.device)
        y = nv.nvfp4_gemm(xg, *w_dev, out=yw[:, :N], x_gs=x_gs)
    else:
        y = nv.nvfp4_gemm(xg, *w_dev, out_dtype=od, x_gs=x_gs)
    torch.cuda.synchronize()
    wsb = nv.workspace(0, "cuda:0").cpu().numpy()
    if pad:
        assert torch.isnan(yw[:, N:]).all(), "%s: the one launch wrote past the output rows" % what
    y = to_np(y)
    # the two-launch path on the same values
    y2 = to_np(nv.nvfp4_gemm(to_gpu(_bf16_as_f32(xb)), *w_dev, out_dtype=od, x_gs=x_gs))
    torch.cuda.synchronize()
    # oracle: workspace bytes, then the product (each path), then the two
    # paths against each other
    oc, os_, og = orc.quantize(xb, gs=gs)
    gbits = wsb[WS_GS:WS_GS + 4].view(np.uint32)[0]
    assert gbits == np.float32(og).view(np.uint32), "%s: gs_x %r vs %r" % (
        what, np.uint32(gbits).view(np.float32), og)
    x16 = wsb[WS_X16:WS_X16 + 2 * M * K].view(np.uint16).reshape(M, K)
    exp = _expected_f16_bits(orc, oc, os_)
    assert np.array_equal(x16, exp), "%s: %d fp16 operand values differ" % (what, int((x16 != exp).sum()))
    check_row_codes(wsb, oc, os_, what)
    ref = orc.gemm_exact(oc, os_, og, wc, ws, gsw)
    check_gemm(y, ref, out == "bf16", what + " (one launch)")
    check_gemm(y2, ref, out == "bf16", what + " (two launches)")


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("N", [8, 16, 300, 1000, 4097])
@pytest.mark.parametrize("K", [4096, 5120])
@pytest.mark.parametrize("M", [1, 2, 3, 4])
def test_fused_decode_shapes(nv, orc, M, K, N, out):
    xb = workloads.to_bf16_bits(workloads.student_t(41, 1, M, K, 3.0))
    w_host, w_dev = _weights(orc, N, K, 2)
    _check_case(nv, orc, xb, w_host, w_dev, out, "M=%d K=%d N=%d" % (M, K, N))


@pytest.mark.parametrize("M", [1, 3, 4])
def test_fused_decode_strided(nv, orc, M):
    """Rows of a wider activation tensor into rows of a wider output; the
    columns past N must stay untouched."""
    K, N = 5120, 300
    xb = workloads.to_bf16_bits(workloads.student_t(41, 8, M, K, 3.0))
    w_host, w_dev = _weights(orc, N, K, 9)
    _check_case(nv, orc, xb, w_host, w_dev, "bf16", "strided M=%d" % M, pad=64)


@pytest.mark.parametrize("M", [1, 4])
@pytest.mark.parametrize("factor", [0.5, 1.0, 3.0])
def test_fused_decode_static(nv, orc, factor, M):
    K, N = 5120, 300
    xb = workloads.to_bf16_bits(workloads.student_t(41, 3, M, K, 3.0))
    gs = np.float32(orc.tensor_scale(xb) * np.float32(factor))
    w_host, w_dev = _weights(orc, N, K, 4)
    _check_case(nv, orc, xb, w_host, w_dev, "bf16", "static M=%d x%g" % (M, factor), gs=gs)


def _rows(x: np.ndarray, M: int, K: int) -> np.ndarray:
    """The first M * K values of x (whole 16-element blocks) as M rows,
    padded with zeros."""
    flat = x.reshape(-1)[:M * K]
    return np.concatenate([flat, np.zeros(M * K - flat.size, np.float32)]).reshape(M, K)


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("gs0", [2.0 ** -3, 2.0 ** -100, 3.0])
def test_fused_decode_e2m1_ties(nv, orc, gs0, M):
    """126 pairs of tie blocks (4032 values) padded with zeros to M rows of
    K = 4096; the ties are exact in bf16 (at most 7 significant bits), their
    fp32 neighbours round to the tie or next to it."""
    xb = workloads.to_bf16_bits(_rows(_tie_tensor(orc, gs0), M, 4096))
    w_host, w_dev = _weights(orc, 40, 4096, 5)
    _check_case(nv, orc, xb, w_host, w_dev, "f32", "E2M1 ties M=%d gs0=%g" % (M, gs0))


@pytest.mark.parametrize("M", [1, 4])
@pytest.mark.parametrize("gs0", [1.0, 2.0 ** -9])
def test_fused_decode_scale_ties(nv, orc, gs0, M):
    """The first 320 M blocks of the scale-byte tie tensor (anchor first)."""
    xb = workloads.to_bf16_bits(_rows(_scale_tie_tensor(orc, gs0), M, 5120))
    w_host, w_dev = _weights(orc, 40, 5120, 6)
    _check_case(nv, orc, xb, w_host, w_dev, "f32", "scale ties M=%d gs0=%g" % (M, gs0))


@pytest.mark.parametrize("M", [1, 3])
def test_fused_decode_zero_row(nv, orc, M):
    xb = np.zeros((M, 4096), np.uint16)
    xb[M - 1, 5] = 0x8000                              # -0
    w_host, w_dev = _weights(orc, 64, 4096, 7)
    _check_case(nv, orc, xb, w_host, w_dev, "bf16", "zero rows M=%d" % M)


def test_fused_decode_full_weight(nv, orc):
    """The full fused gate/up weight (N = 34816) quantized member by member
    on the GPU, against the two-launch path and the oracle on every output."""
    p = workloads.decode(M=1)
    q = [nv.nvfp4_quantize(to_gpu(w)) for w in p.w_parts]
    shared = nv.nvfp4_fuse_rescale([s for _, s, _ in q], [g for _, _, g in q])
    wc = torch.cat([c for c, _, _ in q])
    ws = torch.cat([s for _, s, _ in q])
    del q
    print("case: fused decode full weight N=34816 K=5120", flush=True)
    y = to_np(nv.nvfp4_gemm(to_gpu(p.x), wc, ws, shared, out_dtype=torch.bfloat16))
    y2 = to_np(nv.nvfp4_gemm(to_gpu(_bf16_as_f32(p.x)), wc, ws, shared, out_dtype=torch.bfloat16))
    torch.cuda.synchronize()
    gss = [orc.tensor_scale(w) for w in p.w_parts]
    codes, scales = [], []
    for w, g in zip(p.w_parts, gss):
        c, s, _ = orc.quantize(w, gs=g)
        codes.append(c)
        scales.append(s)
    scales, S = orc.fuse_rescale(scales, gss)
    ref, _ = orc.linear(p.x, np.concatenate(codes), np.concatenate(scales), np.float32(S))
    check_gemm(y, ref, True, "fused decode full weight (one launch)")
    check_gemm(y2, ref, True, "fused decode full weight (two launches)")
