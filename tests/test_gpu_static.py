"""GPU parity of the calibrated (static) activation scale path with the
oracle: nvfp4_quantize_static must give the oracle's bytes for the same given
tensor scale, and nvfp4_gemm with a given activation scale the oracle's exact
GEMM of those bytes.  A scale below the absmax one saturates block scales at
448 and codes at 6; a scale above it coarsens the blocks; zero gives sign-only
codes.  Paper: "Why Gated DeltaNet Survives 4-Bit Quantization", section 2
"NVFP4" (the format) and section 3 "Checkpoints" (one FP32 scale per module
fixed by calibration)."""
import numpy as np
import pytest
import torch

import workloads
from parity import check_gemm, to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_w4a4_quantized_02_amd as m
    return m


def _gs_tensor(v):
    return torch.tensor([np.float32(v)], dtype=torch.float32, device="cuda:0")


def _compare(nv, orc, x, gs, what):
    print("case:", what, x.shape, x.dtype, "gs=%r" % float(gs), flush=True)
    c, s = nv.nvfp4_quantize_static(to_gpu(x), _gs_tensor(gs))
    torch.cuda.synchronize()
    oc, os_, _ = orc.quantize(x, gs=gs)
    sc = to_np(s)
    if not np.array_equal(sc, os_):
        bad = np.argwhere(sc != os_)[:5]
        raise AssertionError("%s: scale bytes differ at %s" % (what, bad.tolist()))
    cc = to_np(c)
    if not np.array_equal(cc, oc):
        bad = np.argwhere(cc != oc)[:5]
        raise AssertionError("%s: code bytes differ at %s (%s vs %s)" % (
            what, bad.tolist(), cc[tuple(bad[0])], oc[tuple(bad[0])]))
    return sc, cc


def _inputs():
    yield "decode_m1_bf16", workloads.decode(M=1, N_each=16).x
    yield "decode_m16_bf16", workloads.decode(M=16, N_each=16).x
    yield "ragged_f32", workloads.gaussian(9, 1, 37, 144, 1.0)
    # one launch up to 8192 blocks; above that the grid-strided kernel
    yield "8192_blocks_bf16", workloads.to_bf16_bits(workloads.student_t(9, 2, 512, 256, 3.0))
    yield "8193_blocks_bf16", workloads.to_bf16_bits(workloads.student_t(9, 3, 8193, 16, 3.0))
    hot = workloads.with_hot_channels(workloads.student_t(9, 4, 256, 5120, 2.5), 9, 5, 16, 200.0)
    yield "hot_channels_bf16", workloads.to_bf16_bits(hot)


@pytest.mark.parametrize("factor", [1.0, 0.25, 3.0, 0.0])
@pytest.mark.parametrize("name,x", list(_inputs()), ids=[n for n, _ in _inputs()])
def test_static_quantize_matches_oracle(nv, orc, name, x, factor):
    gs = np.float32(orc.tensor_scale(x) * np.float32(factor))
    sc, cc = _compare(nv, orc, x, gs, "%s x%g" % (name, factor))
    if factor == 1.0:
        # the given scale equal to the absmax one reproduces nvfp4_quantize
        c, s, g = nv.nvfp4_quantize(to_gpu(x))
        assert np.array_equal(to_np(c), cc) and np.array_equal(to_np(s), sc)
    if factor == 0.25 and x.shape[1] >= 256:
        assert int(sc.max()) == 0x7E      # the largest blocks saturate at 448


@pytest.mark.parametrize("gs", [2.0 ** -140, 2.0 ** -127, 1e-30, 7.0, 3.0e30])
def test_static_quantize_extreme_scales(nv, orc, gs):
    """Subnormal and huge scales, and products |x| / es far outside the fp32
    range (they must saturate at 6, not wrap)."""
    g = np.random.default_rng(11)
    e = g.uniform(-100, 100, size=(24, 128))
    x = (g.choice([-1, 1], size=e.shape) * 2.0 ** e).astype(np.float32)
    x[0, :16] = np.float32(3.0e38)
    x[1, :16] = np.float32(1e-45)
    _compare(nv, orc, x, np.float32(gs), "extreme gs")
    _compare(nv, orc, workloads.to_bf16_bits(x), np.float32(gs), "extreme gs bf16")


def test_static_quantize_full_size_long_prefill(nv, orc):
    """X[32768x5120] bf16 with a calibrated scale half the absmax one: every
    code and scale byte."""
    x = workloads.long_prefill_activations()
    gs = np.float32(orc.tensor_scale(x) * np.float32(0.5))
    print("case: static long prefill 32768x5120, every byte", flush=True)
    c, s = nv.nvfp4_quantize_static(to_gpu(x), _gs_tensor(gs))
    torch.cuda.synchronize()
    oc, os_, _ = orc.quantize(x, gs=gs)
    assert np.array_equal(to_np(s), os_)
    assert np.array_equal(to_np(c), oc)


def test_static_quantize_empty(nv):
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    c, s = nv.nvfp4_quantize_static(x, _gs_tensor(1.0))
    torch.cuda.synchronize()
    assert c.shape == (0, 32) and s.shape == (0, 4)


# ------------------------------------------------------------------ GEMM

def _weight(nv, orc, w):
    wc, ws, wg = nv.nvfp4_quantize(to_gpu(w))
    oc, os_, og = orc.quantize(w)
    return (wc, ws, wg), (oc, os_, og)


@pytest.mark.parametrize("M,N,K", [(1, 300, 512), (4, 520, 5120), (13, 129, 768), (16, 520, 5120),
                                   (100, 200, 320), (300, 257, 1088)])
@pytest.mark.parametrize("factor", [1.0, 0.3, 2.0])
def test_static_gemm_matches_oracle(nv, orc, M, N, K, factor):
    x = workloads.to_bf16_bits(workloads.student_t(9, 10, M, K, 3.0))
    w = workloads.gaussian(9, 11, N, K, 0.02)
    (wc, ws, wg), (oc, os_, og) = _weight(nv, orc, w)
    gx = np.float32(orc.tensor_scale(x) * np.float32(factor))
    print("case: static gemm %dx%dx%d x%g" % (M, N, K, factor), flush=True)
    y = to_np(nv.nvfp4_gemm(to_gpu(x), wc, ws, wg, out_dtype=torch.float32, x_gs=_gs_tensor(gx)))
    torch.cuda.synchronize()
    xc, xs, _ = orc.quantize(x, gs=gx)
    ref = orc.gemm_exact(xc, xs, gx, oc, os_, og)
    check_gemm(y, ref, False, "static gemm %dx%dx%d" % (M, N, K))


def test_static_prepare_then_run(nv, orc):
    """Prepare once with a calibrated scale, run against two weights."""
    M, K = 8, 1024
    x = workloads.to_bf16_bits(workloads.student_t(9, 12, M, K, 3.0))
    gx = np.float32(orc.tensor_scale(x) * np.float32(0.7))
    xc, xs, _ = orc.quantize(x, gs=gx)
    prep = nv.nvfp4_gemm_prepare(to_gpu(x), max_n=384, x_gs=_gs_tensor(gx))
    for t, N in ((13, 384), (14, 96)):
        w = workloads.gaussian(9, t, N, K, 0.05)
        (wc, ws, wg), (oc, os_, og) = _weight(nv, orc, w)
        y = to_np(nv.nvfp4_gemm_run(prep, wc, ws, wg, out_dtype=torch.bfloat16))
        torch.cuda.synchronize()
        check_gemm(y, orc.gemm_exact(xc, xs, gx, oc, os_, og), True, "prepared static N=%d" % N)


def test_static_full_decode(nv, orc):
    """Decode at the full fused gate/up size with a calibrated scale: every
    output."""
    p = workloads.decode(M=16)
    w = np.concatenate(p.w_parts)
    wc, ws, wg = nv.nvfp4_quantize(to_gpu(w))
    gx = np.float32(orc.tensor_scale(p.x) * np.float32(0.8))
    print("case: static full decode M=16 N=34816 K=5120", flush=True)
    y = to_np(nv.nvfp4_gemm(to_gpu(p.x), wc, ws, wg, out_dtype=torch.bfloat16, x_gs=_gs_tensor(gx)))
    torch.cuda.synchronize()
    del wc, ws
    oc, os_, ogw = orc.quantize(w)
    xc, xs, _ = orc.quantize(p.x, gs=gx)
    ref = orc.gemm_exact(xc, xs, gx, oc, os_, ogw)
    check_gemm(y, ref, True, "static full decode")
