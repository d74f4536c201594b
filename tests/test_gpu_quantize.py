"""GPU parity of nvfp4_quantize / nvfp4_dequantize / nvfp4_fuse_rescale with
the oracle: packed codes, scale bytes and the tensor-scale bits must be
identical (paper "Why Gated DeltaNet Survives 4-Bit Quantization", section 2
"NVFP4" and section 6 for the repair)."""
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


def _f32bits(v):
    return np.float32(v).view(np.uint32)


def _compare_quantize(nv, orc, x: np.ndarray, what: str):
    print("case:", what, x.shape, x.dtype, flush=True)
    c, s, g = nv.nvfp4_quantize(to_gpu(x))
    torch.cuda.synchronize()
    oc, os_, og = orc.quantize(x)
    assert _f32bits(g.item()) == _f32bits(og), "%s: gs %r vs %r" % (what, g.item(), og)
    gs_ok = np.array_equal(to_np(s), os_)
    if not gs_ok:
        bad = np.argwhere(to_np(s) != os_)[:5]
        raise AssertionError("%s: scale bytes differ at %s" % (what, bad.tolist()))
    cc = to_np(c)
    if not np.array_equal(cc, oc):
        bad = np.argwhere(cc != oc)[:5]
        raise AssertionError("%s: code bytes differ at %s (%s vs %s)" % (
            what, bad.tolist(), cc[tuple(bad[0])], oc[tuple(bad[0])]))
    return oc, os_, og


def _grid_tensor(orc, gs0):
    """Every non-zero E4M3 scale byte x every E2M1 code, exactly representable."""
    e2, e4 = orc.e2m1_table(), orc.e4m3_table()
    g = np.random.default_rng(3)
    blocks = []
    for S in range(1, 0x7F):
        perm = g.permutation(16)
        blocks.append(np.array([e2[c] * e4[S] * gs0 for c in perm], dtype=np.float32))
    return np.concatenate(blocks)[None, :]


def _tie_tensor(orc, gs0=2.0 ** -3):
    """Blocks whose elements sit exactly on, and one ulp around, every E2M1
    decision point, for every non-zero scale byte.  Row 0 holds the anchor
    (a +-6 code at scale 448) so that gs == gs0 exactly."""
    e4 = orc.e4m3_table()
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    rows = []
    for S in range(1, 0x7F):
        es = np.float32(e4[S] * gs0)
        vals = (mids * float(es)).astype(np.float32)           # exact multiples
        up = np.nextafter(vals, np.float32(np.inf))
        dn = np.nextafter(vals, np.float32(0))
        blk = np.concatenate([[6.0 * float(es)], vals[:5], up[:5], dn[:5]]).astype(np.float32)
        blk2 = np.concatenate([[-6.0 * float(es)], -vals[2:], up[5:], dn[5:], -up[:4], [0.0, -0.0]]).astype(np.float32)
        assert blk.size == 16 and blk2.size == 16
        rows.append(np.concatenate([blk, blk2]))
    x = np.stack(rows)
    x[0, 0] = np.float32(2688.0 * gs0)
    return x


def _cases():
    t = workloads.tiny()
    yield "tiny_x_f32", t.x
    yield "tiny_w_f32", t.w_parts[0]
    for M in (1, 4, 16):
        yield "decode_x_m%d" % M, workloads.decode(M=M, N_each=16).x
    yield "prefill_x_t3", workloads.prefill(M=64, N=16).x
    hot = workloads.with_hot_channels(workloads.student_t(5, 0, 256, 5120, 2.5), 5, 0, 16, 200.0)
    yield "long_prefill_t25", workloads.to_bf16_bits(hot)
    yield "ragged_rows_f32", workloads.gaussian(7, 1, 37, 144, 1.0)
    yield "k16_rows", workloads.to_bf16_bits(workloads.gaussian(7, 2, 1000, 16, 3.0))
    yield "tiny_magnitudes", (workloads.gaussian(7, 3, 8, 64, 1.0) * np.float32(1e-36)).astype(np.float32)
    yield "gs_underflows", (workloads.gaussian(7, 4, 4, 32, 1.0) * np.float32(1e-44)).astype(np.float32)
    yield "huge_magnitudes", (workloads.gaussian(7, 5, 8, 64, 1.0) * np.float32(1e37)).astype(np.float32)
    z = np.zeros((8, 64), np.float32)
    z[2, 3] = -0.0
    yield "zeros_with_negative_zero", z
    # around the size where one launch (absmax inside) gives way to two
    yield "one_launch_8192_blocks_bf16", workloads.to_bf16_bits(workloads.student_t(7, 6, 512, 256, 3.0))
    yield "two_launches_8193_blocks_bf16", workloads.to_bf16_bits(workloads.student_t(7, 7, 8193, 16, 3.0))
    yield "one_launch_8_workgroups_f32", workloads.gaussian(7, 8, 16, 8192, 1.0)
    # one workgroup (its own blocks give the absmax) against two, with the
    # absmax in the very last block
    for name, (r, k) in (("one_workgroup_1024_blocks", (64, 256)), ("two_workgroups_1025_blocks", (1025, 16))):
        g = workloads.gaussian(7, 9, r, k, 1.0)
        g[-1, -1] = np.float32(-50.0)
        yield name, workloads.to_bf16_bits(g)


@pytest.mark.parametrize("name,x", list(_cases()), ids=[n for n, _ in _cases()])
def test_quantize_matches_oracle(nv, orc, name, x):
    _compare_quantize(nv, orc, x, name)


@pytest.mark.parametrize("gs0", [1.0, 2.0 ** -4, 2.0 ** 10, 2.0 ** -60])
def test_quantize_all_codes_all_scales(nv, orc, gs0):
    _compare_quantize(nv, orc, _grid_tensor(orc, gs0), "grid gs0=%g" % gs0)


@pytest.mark.parametrize("gs0", [2.0 ** -3, 2.0 ** -100, 3.0])
def test_quantize_decision_points(nv, orc, gs0):
    _compare_quantize(nv, orc, _tie_tensor(orc, gs0), "ties gs0=%g" % gs0)


def _scale_tie_tensor(orc, gs0):
    """Blocks whose absmax over RN(6 gs) is exactly the midpoint between two
    consecutive E4M3 values (a scale-byte tie, settled to the even byte), and
    one ulp either side, for every pair of consecutive finite bytes.  Block 0
    is the anchor (absmax 2688 gs0, so gs == gs0 exactly; gs0 a power of two
    keeps every product exact)."""
    e4 = orc.e4m3_table().astype(np.float64)
    t = 6.0 * gs0
    g = np.random.default_rng(11)
    blocks = [np.concatenate([[2688.0 * gs0], g.uniform(-1, 1, 15) * 2688.0 * gs0])]
    for b in range(0x7E):
        mid = np.float32((e4[b] + e4[b + 1]) / 2.0 * t)
        for bmax in (mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(0))):
            rest = (g.uniform(-1, 1, 15) * float(bmax)).astype(np.float32)
            rest = np.clip(rest, -np.float32(bmax), np.float32(bmax))
            sign = -1.0 if b % 2 else 1.0
            blocks.append(np.concatenate([[sign * float(bmax)], rest]))
    x = np.concatenate(blocks).astype(np.float32)
    pad = (-x.size) % 64
    return np.concatenate([x, np.zeros(pad, np.float32)]).reshape(-1, 64)


@pytest.mark.parametrize("gs0", [1.0, 2.0 ** -9, 2.0 ** 12])
def test_quantize_scale_byte_ties(nv, orc, gs0):
    x = _scale_tie_tensor(orc, gs0)
    _compare_quantize(nv, orc, x, "scale ties gs0=%g" % gs0)
    _compare_quantize(nv, orc, workloads.to_bf16_bits(x), "scale ties bf16 gs0=%g" % gs0)


def test_quantize_random_rescales(nv, orc):
    """Random magnitudes over the whole binade range of bf16, many tensors."""
    g = np.random.default_rng(77)
    for i in range(6):
        e = g.uniform(-60, 60, size=(48, 256))
        x = (g.choice([-1, 1], size=e.shape) * 2.0 ** e).astype(np.float32)
        _compare_quantize(nv, orc, workloads.to_bf16_bits(x), "random binades %d" % i)


def test_quantize_strided_rows(nv, orc):
    x = workloads.to_bf16_bits(workloads.student_t(7, 6, 40, 512, 3.0))
    xt = to_gpu(x)
    big = torch.zeros((40, 640), dtype=torch.bfloat16, device=xt.device)
    big[:, :512] = xt
    view = big[:, :512]
    c, s, g = nv.nvfp4_quantize(view)
    oc, os_, og = orc.quantize(x)
    assert np.array_equal(to_np(c), oc) and np.array_equal(to_np(s), os_)
    assert _f32bits(g.item()) == _f32bits(og)


def test_quantize_empty(nv):
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    c, s, g = nv.nvfp4_quantize(x)
    torch.cuda.synchronize()
    assert c.shape == (0, 32) and g.item() == 0.0


def test_quantize_deterministic(nv):
    x = to_gpu(workloads.to_bf16_bits(workloads.student_t(7, 7, 512, 5120, 2.5)))
    a = [t.clone() for t in nv.nvfp4_quantize(x)]
    b = nv.nvfp4_quantize(x)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_quantize_full_size_long_prefill(nv, orc):
    """X[32768x5120] bf16 Student-t(2.5) with 16 hot channels x200: the
    tensor scale over the whole tensor and every code and scale byte."""
    x = workloads.long_prefill_activations()
    print("case: long prefill 32768x5120, every byte", flush=True)
    c, s, g = nv.nvfp4_quantize(to_gpu(x))
    torch.cuda.synchronize()
    oc, os_, og = orc.quantize(x)
    assert _f32bits(g.item()) == _f32bits(og)
    sg = to_np(s)
    assert np.array_equal(sg, os_), "scale bytes differ at %s" % np.argwhere(sg != os_)[:5].tolist()
    cg = to_np(c)
    assert np.array_equal(cg, oc), "code bytes differ at %s" % np.argwhere(cg != oc)[:5].tolist()
    # the pages' identity on the real thing: max scale * gs * 6 == absmax
    assert int(sg.max()) == 0x7E


# ------------------------------------------------------------------ dequant

@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_dequantize_matches_oracle(nv, orc, out_dtype):
    x = workloads.to_bf16_bits(workloads.student_t(7, 8, 64, 1024, 2.5))
    c, s, g = nv.nvfp4_quantize(to_gpu(x))
    d = nv.nvfp4_dequantize(c, s, g, out_dtype)
    oc, os_, og = orc.quantize(x)
    if out_dtype == torch.float32:
        ref = orc.dequantize(oc, os_, og)
        assert np.array_equal(to_np(d).view(np.uint32), ref.view(np.uint32))
    else:
        ref = orc.dequantize_bf16(oc, os_, og)
        assert np.array_equal(to_np(d), ref)


# ------------------------------------------------------------------ repair

def _members(p):
    return [np.ascontiguousarray(w) for w in p.w_parts]


@pytest.mark.parametrize("which", ["qkv_small", "gate_up_small", "qkv_full"])
def test_fuse_rescale_matches_oracle(nv, orc, which):
    if which == "qkv_small":
        parts = _members(workloads.fused_qkv(M=4, K=512, Nq=96, Nkv=32))
    elif which == "gate_up_small":
        parts = _members(workloads.decode(M=1, K=512, N_each=64))
    else:
        parts = _members(workloads.fused_qkv(M=4))
    print("case:", which, [p.shape for p in parts], flush=True)
    q = [nv.nvfp4_quantize(to_gpu(w)) for w in parts]
    oq = [orc.quantize(w) for w in parts]
    for (c, s, g), (oc, os_, og) in zip(q, oq):
        assert np.array_equal(to_np(s), os_) and _f32bits(g.item()) == _f32bits(og)
    shared = nv.nvfp4_fuse_rescale([s for _, s, _ in q], [g for _, _, g in q])
    torch.cuda.synchronize()
    new, S = orc.fuse_rescale([os_ for _, os_, _ in oq], [og for _, _, og in oq])
    assert _f32bits(shared.item()) == _f32bits(S)
    for (c, s, g), ref, (oc, _, _) in zip(q, new, oq):
        assert np.array_equal(to_np(s), ref)
        assert np.array_equal(to_np(c), oc)      # codes untouched


def test_fuse_rescale_keeps_nan_and_sign(nv, orc):
    a = np.array([[0x7E, 0x7F, 0xFF, 0xB8, 0x01, 0x09, 0x3F, 0x40]], np.uint8)
    b = np.array([[0x7E, 0x00, 0x10, 0x20, 0x30, 0x40, 0x50, 0x60]], np.uint8)
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    ga = torch.tensor([0.37], device="cuda:0")
    gb = torch.tensor([1.0], device="cuda:0")
    shared = nv.nvfp4_fuse_rescale([ta, tb], [ga, gb])
    new, S = orc.fuse_rescale([a, b], [np.float32(0.37), np.float32(1.0)])
    assert np.array_equal(to_np(ta), new[0]) and np.array_equal(to_np(tb), new[1])
    assert shared.item() == float(S)
