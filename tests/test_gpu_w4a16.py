"""GPU parity of nvfp4_gemm_w4a16 (NVFP4 weights against bf16 activations
used as given) with the oracle's W4A16 product: model card
"Gemma-4-31B-IT-NVFP4-FP8attn-text", section "Limitations" (W4A16 serving of
NVFP4 weights); weight format from the paper "Why Gated DeltaNet Survives
4-Bit Quantization", section 2 "NVFP4".

The weights are the oracle's bytes, uploaded; every GEMV form (streaming,
K-split, shared, general) and the tile GEMM with its split-K tail are hit at
ragged shapes, and the full decode and prefill shapes on whole output rows.
Gate: the GEMM gate of the W4A4 tests (accumulation order is free)."""
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


def _weight(orc, w):
    wc, ws, gsw = orc.quantize(w)
    return (wc, ws, gsw), (to_gpu(wc), to_gpu(ws), torch.tensor([gsw], dtype=torch.float32, device="cuda:0"))


# (M, N, K): streaming (M <= 4, K % 256 == 0), K-split (4 < M <= 16,
# K % 512 == 0, K <= 5120), shared (4 < M <= 16, K % 256 == 0), general
# (other K),
# tile GEMM (M > 16) with and without a split-K tail
SHAPES = [(1, 300, 512), (2, 520, 5120), (4, 40, 256), (3, 200, 320), (1, 7, 64),
          (5, 520, 5120), (16, 520, 512), (13, 129, 768), (9, 100, 1088), (16, 129, 768),
          (16, 520, 640), (7, 300, 1920), (16, 200, 4096),
          (17, 64, 64), (100, 200, 320), (300, 257, 1088), (513, 300, 256)]


@pytest.mark.parametrize("out", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_w4a16_matches_oracle(nv, orc, M, N, K, out):
    x = workloads.to_bf16_bits(workloads.student_t(13, 1, M, K, 3.0))
    w = workloads.gaussian(13, 2, N, K, 0.02)
    (wc, ws, gsw), (gwc, gws, ggs) = _weight(orc, w)
    print("case: w4a16 %dx%dx%d %s" % (M, N, K, out), flush=True)
    od = torch.bfloat16 if out == "bf16" else torch.float32
    y = to_np(nv.nvfp4_gemm_w4a16(to_gpu(x), gwc, gws, ggs, out_dtype=od))
    torch.cuda.synchronize()
    check_gemm(y, orc.gemm_w4a16(x, wc, ws, gsw), out == "bf16", "w4a16 %dx%dx%d" % (M, N, K))


def test_w4a16_strided_rows(nv, orc):
    M, N, K = 20, 70, 512
    x = workloads.to_bf16_bits(workloads.student_t(13, 3, M, K, 3.0))
    w = workloads.gaussian(13, 4, N, K, 0.02)
    (wc, ws, gsw), (gwc, gws, ggs) = _weight(orc, w)
    big = torch.zeros((M, K + 64), dtype=torch.bfloat16, device="cuda:0")
    big[:, :K] = to_gpu(x)
    for view in (big[:, :K], big[:3, :K]):
        y = to_np(nv.nvfp4_gemm_w4a16(view, gwc, gws, ggs, out_dtype=torch.float32))
        m = view.shape[0]
        check_gemm(y, orc.gemm_w4a16(np.ascontiguousarray(x[:m]), wc, ws, gsw), False, "strided %d" % m)


def test_w4a16_empty_and_k_zero(nv):
    wc = torch.zeros((8, 0), dtype=torch.uint8, device="cuda:0")
    ws = torch.zeros((8, 0), dtype=torch.uint8, device="cuda:0")
    wg = torch.ones(1, device="cuda:0")
    for M in (3, 40):
        x = torch.zeros((M, 0), dtype=torch.bfloat16, device="cuda:0")
        y = torch.full((M, 8), 7.0, device="cuda:0")
        nv.nvfp4_gemm_w4a16(x, wc, ws, wg, out=y)
        torch.cuda.synchronize()
        assert torch.count_nonzero(y).item() == 0
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda:0")
    y = nv.nvfp4_gemm_w4a16(x, torch.zeros((8, 32), dtype=torch.uint8, device="cuda:0"),
                            torch.zeros((8, 4), dtype=torch.uint8, device="cuda:0"), wg)
    assert y.shape == (0, 8)


def test_w4a16_rejects_fp32_activations(nv):
    x = torch.zeros((4, 64), dtype=torch.float32, device="cuda:0")
    wc = torch.zeros((8, 32), dtype=torch.uint8, device="cuda:0")
    ws = torch.zeros((8, 4), dtype=torch.uint8, device="cuda:0")
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_gemm_w4a16(x, wc, ws, torch.ones(1, device="cuda:0"))


def _rows(nv, orc, x, w_parts, rows):
    """Fused weight quantized member by member and repaired on the GPU; the
    oracle recomputes whole output rows from the same member scales."""
    q = [nv.nvfp4_quantize(to_gpu(w)) for w in w_parts]
    if len(q) > 1:
        shared = nv.nvfp4_fuse_rescale([s for _, s, _ in q], [g for _, _, g in q])
        wc = torch.cat([c for c, _, _ in q])
        ws = torch.cat([s for _, s, _ in q])
    else:
        wc, ws, shared = q[0]
    y = to_np(nv.nvfp4_gemm_w4a16(to_gpu(x), wc, ws, shared, out_dtype=torch.bfloat16))
    torch.cuda.synchronize()
    del q, wc, ws
    gss = [orc.tensor_scale(w) for w in w_parts]
    codes, scales = [], []
    for w, g in zip(w_parts, gss):
        c, s, _ = orc.quantize(w, gs=g)
        codes.append(c)
        scales.append(s)
    if len(w_parts) > 1:
        scales, S = orc.fuse_rescale(scales, gss)
    else:
        S = gss[0]
    ref = orc.gemm_w4a16(np.ascontiguousarray(x[rows]), np.concatenate(codes), np.concatenate(scales), S)
    return y[rows], ref


@pytest.mark.parametrize("M", [1, 4, 16])
def test_w4a16_full_decode(nv, orc, M):
    p = workloads.decode(M=M)
    print("case: w4a16 full decode M=%d N=34816 K=5120" % M, flush=True)
    got, ref = _rows(nv, orc, p.x, p.w_parts, np.arange(M))
    check_gemm(got, ref, True, "w4a16 full decode M=%d" % M)


def test_w4a16_full_prefill(nv, orc):
    p = workloads.prefill()
    print("case: w4a16 full prefill 4096x17408x5120", flush=True)
    got, ref = _rows(nv, orc, p.x, p.w_parts, sample_rows(p.M, 10, 2, must=[3840, 4000]))
    check_gemm(got, ref, True, "w4a16 full prefill")


def test_w4a16_split_tail(nv, orc):
    # 2 x 129 tiles = 258: the last 2 (tile row 1, tile columns 127 and 128,
    # both ragged) are split along K (K = 128 is 2 steps).  Every output.
    M, N, K = 500, 33000, 128
    p = workloads.prefill(M=M, K=K, N=N)
    print("case: w4a16 split tail M=%d N=%d K=%d" % (M, N, K), flush=True)
    got, ref = _rows(nv, orc, p.x, p.w_parts, np.arange(M))
    check_gemm(got, ref, True, "w4a16 split tail")
