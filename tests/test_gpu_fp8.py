"""GPU parity of the FP8 E4M3 per-tensor quantize / dequantize with the oracle:
bytes and scale bits identical (model card "Gemma-4-31B-IT-NVFP4-FP8attn-text",
section "What was quantized, exactly"; paper "Why Gated DeltaNet Survives
4-Bit Quantization", section 7: FP8 KV cache with static per-tensor scales).
Covers every grid value, every rounding midpoint and its neighbours, the
subnormal range, saturation, signed zeros, zero and extreme scales, both the
one-launch (small) and the two-pass (large) dynamic paths, and static
scales on KV-cache-shaped tensors."""
import numpy as np
import pytest
import torch

import workloads
from parity import to_gpu, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_w4a4_quantized_02_amd as m
    return m


def _gs(v):
    return torch.tensor([np.float32(v)], dtype=torch.float32, device="cuda:0")


def _compare(nv, orc, x, what, scale=None):
    print("case:", what, x.shape, x.dtype, flush=True)
    if scale is None:
        q, s = nv.nvfp4_fp8_quantize(to_gpu(x))
        oq, os_ = orc.fp8_quantize(x)
        assert np.float32(s.item()).view(np.uint32) == np.float32(os_).view(np.uint32), (s.item(), os_)
    else:
        q, _ = nv.nvfp4_fp8_quantize(to_gpu(x), _gs(scale))
        oq, _ = orc.fp8_quantize(x, scale=scale)
    qq = to_np(q)
    if not np.array_equal(qq, oq):
        bad = np.argwhere(qq != oq)[:5]
        raise AssertionError("%s: bytes differ at %s (%s vs %s)" % (what, bad.tolist(), qq[tuple(bad[0])],
                                                                   oq[tuple(bad[0])]))
    return oq


def _grid_values():
    b = np.array([i for i in range(128) if i != 0x7F], dtype=np.uint8)
    v = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return v


def _tie_values():
    v = _grid_values()
    mids = (v[:-1] + v[1:]) / 2.0
    out = [v, mids, np.nextafter(mids.astype(np.float32), np.float32(np.inf)),
           np.nextafter(mids.astype(np.float32), np.float32(0)),
           np.array([448.5, 449, 460, 464, 464.5, 480, 500, 1e4, 3e38, 2.0 ** -10, 2.0 ** -11, 1.0e-30, 0.0])]
    a = np.concatenate([np.asarray(o, dtype=np.float64) for o in out])
    a = np.concatenate([a, -a])
    pad = (-a.size) % 16
    return np.concatenate([a, np.zeros(pad)])


@pytest.mark.parametrize("s", [1.0, 2.0 ** -12, 2.0 ** 20, 0.37, 3.3e-30, 7.1e30])
def test_fp8_grid_and_midpoints(nv, orc, s):
    base = _tie_values()
    x = np.clip(base * s, -3.4e38, 3.4e38).astype(np.float32).reshape(-1, 16)   # inputs stay finite
    _compare(nv, orc, x, "ties s=%g" % s, scale=s)
    x[0, 0] = np.float32(-0.0)
    _compare(nv, orc, x, "ties+neg0 s=%g" % s, scale=s)


@pytest.mark.parametrize("s", [0.0, 2.0 ** -140, 1e-38, 3.0e38])
def test_fp8_degenerate_scales(nv, orc, s):
    g = np.random.default_rng(4)
    x = (g.standard_normal((8, 64)) * 2.0 ** g.integers(-60, 60, size=(8, 64))).astype(np.float32)
    x[0, :4] = [0.0, -0.0, 3e38, -3e38]
    _compare(nv, orc, x, "degenerate s=%g" % s, scale=s)


def _cases():
    yield "decode_m16_bf16", workloads.decode(M=16, N_each=16).x                        # one launch
    yield "prefill_bf16", workloads.to_bf16_bits(workloads.student_t(23, 1, 256, 5120, 3.0))  # two passes
    yield "weights_f32", workloads.gaussian(23, 2, 384, 1024, 0.02)
    yield "ragged_f32", workloads.gaussian(23, 3, 37, 144, 1.0)
    yield "8192_groups_bf16", workloads.to_bf16_bits(workloads.student_t(23, 4, 512, 256, 3.0))
    yield "8193_groups_bf16", workloads.to_bf16_bits(workloads.student_t(23, 5, 8193, 16, 3.0))
    z = np.zeros((8, 64), np.float32)
    z[3, 7] = -0.0
    yield "zeros", z


@pytest.mark.parametrize("name,x", list(_cases()), ids=[n for n, _ in _cases()])
def test_fp8_dynamic_matches_oracle(nv, orc, name, x):
    _compare(nv, orc, x, name)


@pytest.mark.parametrize("scale", [1.0, 0.0213])
def test_fp8_static_kv_cache(nv, orc, scale):
    """KV-cache-shaped tensors (tokens x heads*head_dim) with a static scale."""
    k = workloads.to_bf16_bits(workloads.student_t(23, 6, 300, 1024, 4.0))
    _compare(nv, orc, k, "kv scale=%g" % scale, scale=scale)


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_fp8_dequantize(nv, orc, out):
    x = workloads.to_bf16_bits(workloads.student_t(23, 7, 64, 512, 3.0))
    q, s = nv.nvfp4_fp8_quantize(to_gpu(x))
    d = to_np(nv.nvfp4_fp8_dequantize(q, s, out))
    oq, os_ = orc.fp8_quantize(x)
    ref = orc.fp8_dequantize(oq, os_)
    if out == torch.float32:
        assert np.array_equal(d.view(np.uint32), ref.view(np.uint32))
    else:
        assert np.array_equal(d, workloads.to_bf16_bits(ref))


def test_fp8_long_every_byte(nv, orc):
    x = workloads.long_prefill_activations()
    print("case: fp8 long prefill 32768x5120, every byte", flush=True)
    q, s = nv.nvfp4_fp8_quantize(to_gpu(x))
    torch.cuda.synchronize()
    oq, os_ = orc.fp8_quantize(x)
    assert np.float32(s.item()) == os_
    assert np.array_equal(to_np(q), oq)


def test_fp8_empty(nv):
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    q, s = nv.nvfp4_fp8_quantize(x)
    torch.cuda.synchronize()
    assert q.shape == (0, 64) and s.item() == 0.0
