"""Byte-level parity of the activation operand that the W4A4 contraction
actually consumes.

nvfp4_gemm_prepare (and nvfp4_gemm_prepare_static) leaves in its workspace
the activation tensor scale gs_x (one float at byte 8192) and the quantized
activations as fp16 values E2M1(code) * E4M3(scale), the tensor scale kept
apart, row-major [M, K] from byte 8448 (include/nvfp4.h documents the
layout).  Every one of those values must equal fp16(E2M1 * E4M3) built from
the oracle's codes and scale bytes, sign of zero included, and gs_x must
have the oracle's bits (paper "Why Gated DeltaNet Survives 4-Bit
Quantization", section 2 "NVFP4": activations quantized on the fly to E2M1
with an E4M3 scale per 16 and one FP32 tensor scale).

Up to four prepared rows at K = 4096 or 5120 also keep their packed codes
([M, K/2]) and then their scale bytes ([M, K/16]) right after the fp16
operand, which the FP4 GEMV contracts directly; those must equal the
oracle's bytes.

Cases cover every instantiation of the quantize kernels that writes this
form: the one-launch kernel with one workgroup (absmax from its own blocks,
M <= 3 at K = 5120) and with several, the two-pass absmax + encode kernels,
fp32 and bf16 inputs, the calibrated-scale forms of both, ragged M and K,
and inputs on or next to every rounding tie."""
import numpy as np
import pytest
import torch

import workloads
from parity import to_gpu, unpack_codes
from test_gpu_quantize import _scale_tie_tensor, _tie_tensor

pytestmark = pytest.mark.gpu

WS_GS = 8192     # byte offset of gs_x in a prepared workspace
WS_X16 = 8448    # byte offset of the fp16 activation operand


@pytest.fixture(scope="module")
def nv():
    import nvfp4_w4a4_quantized_02_amd as m
    return m


def _expected_f16_bits(orc, codes, scales):
    """fp16 bits of E2M1(code) * E4M3(scale), sign from the code (the
    product has at most 6 significant bits and lies in [2^-10, 2688], so the
    fp16 value is exact)."""
    c = unpack_codes(codes)
    mag = orc.e2m1_table()[c & 7] * orc.e4m3_table()[np.repeat(scales, 16, axis=1)]
    val = np.where((c & 8) != 0, -mag, mag)
    return val.astype(np.float16).view(np.uint16)


def keeps_codes(M, K):
    return 1 <= M <= 4 and K in (4096, 5120)


def codes_offset(M, K):
    """Byte offset of the packed codes: after the fp16 operand [M, K rounded
    up to 64], itself rounded up to 256 bytes."""
    kp = (K + 63) // 64 * 64
    return WS_X16 + (M * kp * 2 + 255) // 256 * 256


def _prepared(nv, x: np.ndarray, gs=None):
    """Run prepare on the GPU; return (gs_x bits, fp16 operand bits [M, K],
    workspace bytes)."""
    M, K = x.shape
    xg = to_gpu(x)
    x_gs = None if gs is None else torch.tensor([float(gs)], dtype=torch.float32, device=xg.device)
    prep = nv.nvfp4_gemm_prepare(xg, x_gs=x_gs)
    torch.cuda.synchronize()
    ws = prep.ws.cpu().numpy()
    gbits = ws[WS_GS:WS_GS + 4].view(np.uint32)[0]
    x16 = ws[WS_X16:WS_X16 + M * K * 2].view(np.uint16).reshape(M, K)
    return gbits, x16, ws


def check_row_codes(ws, oc, os_, what):
    """Prepared rows: packed codes [M, K/2], then scale bytes [M, K/16]."""
    M, K = oc.shape[0], oc.shape[1] * 2
    o = codes_offset(M, K)
    codes = ws[o:o + M * K // 2].reshape(M, K // 2)
    scales = ws[o + M * K // 2:o + M * K // 2 + M * K // 16].reshape(M, K // 16)
    assert np.array_equal(codes, oc), "%s: %d code bytes differ" % (what, int((codes != oc).sum()))
    assert np.array_equal(scales, os_), "%s: %d scale bytes differ" % (what, int((scales != os_).sum()))


def _check(nv, orc, x, what, gs=None):
    print("case: prepare", what, x.shape, x.dtype, "given gs" if gs is not None else "", flush=True)
    gbits, x16, ws = _prepared(nv, x, gs)
    oc, os_, og = orc.quantize(x, gs=gs)
    if keeps_codes(*x.shape):
        check_row_codes(ws, oc, os_, what)
    assert gbits == np.float32(og).view(np.uint32), "%s: gs_x %r vs %r" % (
        what, np.uint32(gbits).view(np.float32), og)
    exp = _expected_f16_bits(orc, oc, os_)
    if not np.array_equal(x16, exp):
        bad = np.argwhere(x16 != exp)
        r, k = bad[0]
        raise AssertionError("%s: %d fp16 operand values differ, first at %s (%04x vs %04x)" % (
            what, len(bad), (int(r), int(k)), x16[r, k], exp[r, k]))


def _cases():
    yield "tiny_16x256_f32", workloads.tiny().x                         # one workgroup, fp32
    for M in (1, 2, 3, 4, 16):                                          # decode rows, K = 5120
        yield "decode_m%d" % M, workloads.decode(M=M, N_each=16).x      # 1 and 3 wg bounds
    yield "ragged_m17_k320", workloads.to_bf16_bits(workloads.student_t(31, 1, 17, 320, 3.0))
    yield "ragged_m300_k1088", workloads.to_bf16_bits(workloads.student_t(31, 2, 300, 1088, 3.0))
    yield "one_launch_8192_blocks", workloads.to_bf16_bits(workloads.student_t(31, 3, 128, 1024, 3.0))
    yield "two_launches_8256_blocks", workloads.to_bf16_bits(workloads.student_t(31, 4, 129, 1024, 3.0))
    yield "fp32_m100_k256", workloads.gaussian(31, 5, 100, 256, 1.0)
    yield "fp32_m600_k512", workloads.gaussian(31, 6, 600, 512, 1.0)
    z = np.zeros((4, 64), np.float32)
    z[1, 5] = -0.0
    z[2, 7] = -1e-30
    yield "zeros_and_negative_zero", z


@pytest.mark.parametrize("name,x", list(_cases()), ids=[n for n, _ in _cases()])
def test_prepare_operand_matches_oracle(nv, orc, name, x):
    _check(nv, orc, x, name)


def test_prepare_operand_full_prefill(nv, orc):
    """The full 4096x5120 prefill activations (absmax partials + encode)."""
    _check(nv, orc, workloads.prefill(N=16).x, "full prefill 4096x5120")


@pytest.mark.parametrize("gs0", [2.0 ** -3, 2.0 ** -100, 3.0])
def test_prepare_operand_decision_points(nv, orc, gs0):
    x = _tie_tensor(orc, gs0).reshape(-1, 64)       # 16-element blocks kept whole
    _check(nv, orc, x, "E2M1 ties gs0=%g" % gs0)
    _check(nv, orc, workloads.to_bf16_bits(x), "E2M1 ties bf16 gs0=%g" % gs0)


@pytest.mark.parametrize("gs0", [1.0, 2.0 ** -9])
def test_prepare_operand_scale_byte_ties(nv, orc, gs0):
    x = _scale_tie_tensor(orc, gs0)
    _check(nv, orc, x, "scale ties gs0=%g" % gs0)


@pytest.mark.parametrize("factor", [0.5, 1.0, 3.0])
@pytest.mark.parametrize("M,K", [(1, 5120), (16, 5120), (300, 1088), (4096, 5120)])
def test_prepare_static_operand_matches_oracle(nv, orc, M, K, factor):
    """Calibrated activation scale: a factor below 1 saturates blocks at the
    largest scale byte and codes at 6, above 1 leaves headroom."""
    x = workloads.to_bf16_bits(workloads.student_t(31, 7, M, K, 3.0))
    gs = np.float32(orc.tensor_scale(x) * np.float32(factor))
    _check(nv, orc, x, "static M=%d K=%d x%g" % (M, K, factor), gs=gs)
