"""GPU parity of nvfp4_gemm (W4A4 linear with on-the-fly activation
quantization) against the oracle's exact GEMM, at small sizes element by
element and at the full workload sizes on whole sampled output rows.

Weights are quantized independently on both sides (nvfp4_quantize on the
GPU, the oracle on the CPU); the quantize tests establish that both give the
same bytes.  Paper: "Why Gated DeltaNet Survives 4-Bit Quantization",
section 2 "NVFP4" (the GEMM) and section 6 (fused groups)."""
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


def _gpu_weight(nv, parts):
    """Quantize each member on the GPU; fuse when there is more than one."""
    q = [nv.nvfp4_quantize(to_gpu(w)) for w in parts]
    if len(q) == 1:
        return q[0]
    shared = nv.nvfp4_fuse_rescale([s for _, s, _ in q], [g for _, _, g in q])
    return torch.cat([c for c, _, _ in q]), torch.cat([s for _, s, _ in q]), shared


def _oracle_weight(orc, parts, rows=None):
    """Oracle codes/scales for the fused weight (optionally only some rows)."""
    gss = [orc.tensor_scale(w) for w in parts]
    offs = np.cumsum([0] + [w.shape[0] for w in parts])
    codes, scales, member = [], [], []
    for i, w in enumerate(parts):
        if rows is None:
            sel = np.arange(w.shape[0])
        else:
            sel = rows[(rows >= offs[i]) & (rows < offs[i + 1])] - offs[i]
        c, s, _ = orc.quantize(np.ascontiguousarray(w[sel]), gs=gss[i])
        codes.append(c)
        scales.append(s)
    if len(parts) > 1:
        scales, S = orc.fuse_rescale(scales, gss)
    else:
        S = gss[0]
    return np.concatenate(codes), np.concatenate(scales), np.float32(S)


def _run(nv, p, out_dtype):
    wc, ws, wg = _gpu_weight(nv, p.w_parts)
    y = nv.nvfp4_gemm(to_gpu(p.x), wc, ws, wg, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return to_np(y)


def _full_ref(orc, p):
    wc, ws, wg = _oracle_weight(orc, p.w_parts)
    y, _ = orc.linear(p.x, wc, ws, wg)
    return y


# --------------------------------------------------------- element by element

def test_tiny_fp32(nv, orc):
    p = workloads.tiny()
    print("case: tiny 16x256x256 f32", flush=True)
    check_gemm(_run(nv, p, torch.float32), _full_ref(orc, p), False, "tiny")


@pytest.mark.parametrize("M", [1, 4, 16])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_decode_small_n(nv, orc, M, out):
    p = workloads.decode(M=M, N_each=260)          # fused gate/up, N = 520 (ragged tile)
    print("case: decode M=%d N=520 K=5120 %s" % (M, out), flush=True)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    check_gemm(_run(nv, p, od), _full_ref(orc, p), out == "bf16", "decode M=%d" % M)


@pytest.mark.parametrize("M,N,K", [(17, 300, 1088), (300, 260, 512), (256, 256, 256), (511, 129, 192),
                                   (40, 1000, 5120), (300, 257, 64), (257, 300, 128), (600, 520, 320)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_gemm_ragged(nv, orc, M, N, K, out):
    p = workloads.prefill(M=M, K=K, N=N)
    print("case: gemm M=%d N=%d K=%d %s" % (M, N, K, out), flush=True)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    check_gemm(_run(nv, p, od), _full_ref(orc, p), out == "bf16", "gemm %dx%dx%d" % (M, N, K))


# Small M (decode) shapes for every GEMV form: one-wave streaming tiles
# (M <= 4, K % 256 == 0, with 1, 2 and 4 activation rows per transfer), the
# workgroup-shared kernel (4 < M <= 16, K % 256 == 0, ragged last workgroup),
# and the general kernel for K that is not a multiple of 256.
@pytest.mark.parametrize("M,N,K", [(2, 520, 5120), (3, 520, 5120), (4, 40, 256), (5, 520, 5120),
                                   (8, 40, 256), (13, 300, 1024), (16, 520, 512), (3, 200, 320),
                                   (9, 100, 1088), (1, 7, 64), (16, 129, 768)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_gemv_shapes(nv, orc, M, N, K, out):
    p = workloads.prefill(M=M, K=K, N=N)
    print("case: gemv M=%d N=%d K=%d %s" % (M, N, K, out), flush=True)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    check_gemm(_run(nv, p, od), _full_ref(orc, p), out == "bf16", "gemv %dx%dx%d" % (M, N, K))


# More small-M shapes over the kernels that serve them: K-split (K = 1536,
# 2560, 4096, 5120: three to ten waves of 512 k), shared (K = 3840) and
# general (K = 640, 1920); ragged N and padded activation rows.
@pytest.mark.parametrize("M,N,K", [(16, 520, 640), (7, 300, 1920), (11, 33, 2560), (12, 260, 3840),
                                   (16, 1000, 5120), (6, 300, 1536), (16, 200, 4096)])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_gemv_small_m_shapes(nv, orc, M, N, K, out):
    p = workloads.prefill(M=M, K=K, N=N)
    print("case: gemv small-M M=%d N=%d K=%d %s" % (M, N, K, out), flush=True)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    check_gemm(_run(nv, p, od), _full_ref(orc, p), out == "bf16", "gemv small-M %dx%dx%d" % (M, N, K))


def test_gemm_fp32_activations(nv, orc):
    p = workloads.tiny(M=100, K=256, N=200)
    check_gemm(_run(nv, p, torch.float32), _full_ref(orc, p), False, "fp32 X, M=100")


def test_fused_qkv_small(nv, orc):
    p = workloads.fused_qkv(M=64, K=1024, Nq=192, Nkv=64)
    check_gemm(_run(nv, p, torch.float32), _full_ref(orc, p), False, "fused qkv small")


def test_k_zero_and_empty(nv):
    x = torch.zeros((20, 0), dtype=torch.bfloat16, device="cuda:0")
    wc = torch.zeros((8, 0), dtype=torch.uint8, device="cuda:0")
    ws = torch.zeros((8, 0), dtype=torch.uint8, device="cuda:0")
    wg = torch.ones(1, device="cuda:0")
    y = torch.full((20, 8), 7.0, device="cuda:0")
    nv.nvfp4_gemm(x, wc, ws, wg, out=y)
    torch.cuda.synchronize()
    assert (y == 0).all()
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    wc = torch.zeros((8, 32), dtype=torch.uint8, device="cuda:0")
    ws = torch.zeros((8, 4), dtype=torch.uint8, device="cuda:0")
    assert nv.nvfp4_gemm(x, wc, ws, wg).shape == (0, 8)


def test_gemm_deterministic(nv):
    p = workloads.prefill(M=512, K=1024, N=512)
    a = _run(nv, p, torch.float32)
    b = _run(nv, p, torch.float32)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_unrepaired_fusion_is_misscaled(nv, orc):
    """Serving a fused group with the largest tensor scale but the members'
    own block scales (no repair) scales member i by S / gs_i: the GPU shows
    the same error the oracle predicts, and the repair removes it."""
    p = workloads.fused_qkv(M=32, K=512, Nq=64, Nkv=32)
    q = [nv.nvfp4_quantize(to_gpu(w)) for w in p.w_parts]
    gss = [g.item() for _, _, g in q]
    S = max(gss)
    wc = torch.cat([c for c, _, _ in q])
    ws = torch.cat([s for _, s, _ in q])
    bad = nv.nvfp4_gemm(to_gpu(p.x), wc, ws, torch.tensor([S], device="cuda:0"), out_dtype=torch.float32)
    ref = _full_ref(orc, p)                       # repaired oracle
    offs = np.cumsum([0] + [w.shape[0] for w in p.w_parts])
    badn = to_np(bad).astype(np.float64)
    for i in range(3):
        sl = slice(offs[i], offs[i + 1])
        ratio = np.linalg.norm(badn[:, sl]) / np.linalg.norm(ref[:, sl])
        assert abs(ratio - S / gss[i]) < 0.07 * S / gss[i]
    check_gemm(_run(nv, p, torch.float32), ref, False, "repaired")


# --------------------------------------------------------- full sizes, whole rows
# At the full workload sizes the oracle recomputes whole output rows (the
# complete weight against a sample of activation rows, the tensor scale taken
# over the whole activation tensor), so every element is gated against the
# rms of its own row.

def _rows(nv, orc, p, out_dtype, rows):
    wc, ws, wg = _gpu_weight(nv, p.w_parts)
    y = to_np(nv.nvfp4_gemm(to_gpu(p.x), wc, ws, wg, out_dtype=out_dtype))
    torch.cuda.synchronize()
    del wc, ws
    owc, ows, owg = _oracle_weight(orc, p.w_parts)
    gx = orc.tensor_scale(p.x)
    oxc, oxs, _ = orc.quantize(np.ascontiguousarray(p.x[rows]), gs=gx)
    return y[rows], orc.gemm_exact(oxc, oxs, gx, owc, ows, owg)


# Split-K tail: when the tiles do not fill whole rounds of the 256 compute
# units, the remaining tiles (the last ones in row-major order) are split
# along K and a second kernel adds the parts.
def test_split_tail_every_output(nv, orc):
    # 2 x 129 tiles = 258: the last 2 (tile row 1, tile columns 127 and 128,
    # both ragged) are split in 2 (K = 128 is 2 steps).  Every output.
    M, N, K = 500, 33000, 128
    p = workloads.prefill(M=M, K=K, N=N)
    print("case: split tail gemm M=%d N=%d K=%d" % (M, N, K), flush=True)
    got, ref = _rows(nv, orc, p, torch.float32, np.arange(M))
    check_gemm(got, ref, False, "split tail %dx%dx%d" % (M, N, K))


def test_split_tail_16_parts(nv, orc):
    # 2 x 257 tiles = 514: the last 2 (tile row 1, tile columns 255 and 256)
    # are split in 16 (K = 1024 is 16 steps): every row of the split tiles
    # (256..299) and a sample of the others, whole
    M, N, K = 300, 65600, 1024
    p = workloads.prefill(M=M, K=K, N=N)
    print("case: split tail 16 parts M=%d N=%d K=%d" % (M, N, K), flush=True)
    rows = sample_rows(M, 8, 5, must=np.arange(256, M))
    got, ref = _rows(nv, orc, p, torch.float32, rows)
    check_gemm(got, ref, False, "split tail 16 parts")


@pytest.mark.parametrize("M", [1, 4, 16])
def test_full_decode(nv, orc, M):
    p = workloads.decode(M=M)
    print("case: full decode M=%d N=34816 K=5120, every output" % M, flush=True)
    got, ref = _rows(nv, orc, p, torch.bfloat16, np.arange(M))
    check_gemm(got, ref, True, "full decode M=%d" % M)


def test_full_prefill(nv, orc):
    p = workloads.prefill()
    print("case: full prefill 4096x17408x5120, whole rows", flush=True)
    # rows of the first and last tile rows and of the split tail (tile row 15)
    rows = sample_rows(p.M, 10, 0, must=[255, 256, 3840, 4000])
    got, ref = _rows(nv, orc, p, torch.bfloat16, rows)
    check_gemm(got, ref, True, "full prefill")


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_full_fused_qkv(nv, orc, out):
    p = workloads.fused_qkv()
    print("case: full fused qkv 2048x8192x5120 %s, whole rows" % out, flush=True)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    got, ref = _rows(nv, orc, p, od, sample_rows(p.M, 12, 1 if out == "f32" else 2))
    check_gemm(got, ref, out == "bf16", "full fused qkv")
