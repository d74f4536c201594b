"""One-launch decode: for one bf16 activation row with K = 4096 or 5120,
nvfp4_gemm quantizes the row and runs the GEMV in a single kernel, whose
contraction runs on the FP4 MFMA over the raw codes with the block scales
applied to each block's exact sum.

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
    oracle's packed codes and scale bytes from byte 0.
Shapes cover a single tile (one wave of the three idle), ragged N, an odd
tile count, and the full fused gate/up weight; inputs include rows on or
next to every E2M1 and scale-byte rounding tie, and calibrated scales."""
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


def _check_case(nv, orc, xb, w_host, w_dev, out, what, gs=None):
    """xb: [1, K] bf16 bits."""
    print("case: fused decode", what, out, "given gs" if gs is not None else "", flush=True)
    K = xb.shape[1]
    wc, ws, gsw = w_host
    od = torch.bfloat16 if out == "bf16" else torch.float32
    x_gs = None if gs is None else torch.tensor([float(gs)], dtype=torch.float32, device="cuda:0")
    y = nv.nvfp4_gemm(to_gpu(xb), *w_dev, out_dtype=od, x_gs=x_gs)
    torch.cuda.synchronize()
    wsb = nv.workspace(0, "cuda:0").cpu().numpy()
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
    x16 = wsb[WS_X16:WS_X16 + 2 * K].view(np.uint16).reshape(1, K)
    exp = _expected_f16_bits(orc, oc, os_)
    assert np.array_equal(x16, exp), "%s: %d fp16 operand values differ" % (what, int((x16 != exp).sum()))
    check_row_codes(wsb, oc, os_, what)
    ref = orc.gemm_exact(oc, os_, og, wc, ws, gsw)
    check_gemm(y, ref, out == "bf16", what + " (one launch)")
    check_gemm(y2, ref, out == "bf16", what + " (two launches)")


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("N", [8, 16, 300, 1000, 4097])
@pytest.mark.parametrize("K", [4096, 5120])
def test_fused_decode_shapes(nv, orc, K, N, out):
    xb = workloads.to_bf16_bits(workloads.student_t(41, 1, 1, K, 3.0))
    w_host, w_dev = _weights(orc, N, K, 2)
    _check_case(nv, orc, xb, w_host, w_dev, out, "K=%d N=%d" % (K, N))


@pytest.mark.parametrize("factor", [0.5, 1.0, 3.0])
def test_fused_decode_static(nv, orc, factor):
    K, N = 5120, 300
    xb = workloads.to_bf16_bits(workloads.student_t(41, 3, 1, K, 3.0))
    gs = np.float32(orc.tensor_scale(xb) * np.float32(factor))
    w_host, w_dev = _weights(orc, N, K, 4)
    _check_case(nv, orc, xb, w_host, w_dev, "bf16", "static x%g" % factor, gs=gs)


def _one_row(x: np.ndarray, K: int) -> np.ndarray:
    flat = x.reshape(-1)[:K]
    return np.concatenate([flat, np.zeros(K - flat.size, np.float32)]).reshape(1, K)


@pytest.mark.parametrize("gs0", [2.0 ** -3, 2.0 ** -100, 3.0])
def test_fused_decode_e2m1_ties(nv, orc, gs0):
    """126 pairs of tie blocks (4032 values) padded with zeros to K = 4096; the
    ties are exact in bf16 (at most 7 significant bits), their fp32
    neighbours round to the tie or next to it."""
    xb = workloads.to_bf16_bits(_one_row(_tie_tensor(orc, gs0), 4096))
    w_host, w_dev = _weights(orc, 40, 4096, 5)
    _check_case(nv, orc, xb, w_host, w_dev, "f32", "E2M1 ties gs0=%g" % gs0)


@pytest.mark.parametrize("gs0", [1.0, 2.0 ** -9])
def test_fused_decode_scale_ties(nv, orc, gs0):
    """The first 320 blocks of the scale-byte tie tensor (anchor first)."""
    xb = workloads.to_bf16_bits(_one_row(_scale_tie_tensor(orc, gs0), 5120))
    w_host, w_dev = _weights(orc, 40, 5120, 6)
    _check_case(nv, orc, xb, w_host, w_dev, "f32", "scale ties gs0=%g" % gs0)


def test_fused_decode_zero_row(nv, orc):
    xb = np.zeros((1, 4096), np.uint16)
    xb[0, 5] = 0x8000                                  # -0
    w_host, w_dev = _weights(orc, 64, 4096, 7)
    _check_case(nv, orc, xb, w_host, w_dev, "bf16", "zero row")


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
