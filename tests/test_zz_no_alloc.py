"""GPU test of nvfp4_gemm_noalloc, the W4A4 linear whose scratch lives in the
library's fixed device array instead of a caller workspace (for callers that
cannot allocate).  Called through the C ABI, it must give exactly what
nvfp4_gemm gives on the same inputs (same kernels, deterministic), on calls in
a row that reuse the array, the second one smaller than the first; the first
is also gated against the oracle."""
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


def _noalloc_abi(nv, x, wc, ws, wg, y):
    M, K = x.shape
    N = wc.shape[0]
    return nv.lib.nvfp4_gemm_noalloc(x.data_ptr(), 1 if x.dtype == torch.bfloat16 else 0, M, K, x.stride(0),
                                     wc.data_ptr(), ws.data_ptr(), wg.data_ptr(), N, y.data_ptr(),
                                     1 if y.dtype == torch.bfloat16 else 0, y.stride(0),
                                     torch.cuda.current_stream().cuda_stream)


# (M, N, K, seed): a tile GEMM with a split-K tail, then smaller shapes that
# reuse the same array (a decode GEMV, the one-launch decode of one bf16 row,
# then a one-tile GEMM).
CASES = [(300, 520, 1024, 1), (4, 264, 512, 2), (1, 304, 4096, 4), (40, 136, 256, 3)]


@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
def test_noalloc_matches_gemm_on_calls_in_a_row(nv, orc, out):
    for i, (M, N, K, seed) in enumerate(CASES):
        print("case: noalloc call %d M=%d N=%d K=%d %s" % (i, M, N, K, out), flush=True)
        x = to_gpu(workloads.to_bf16_bits(workloads.student_t(33, seed, M, K, 3.0)))
        w = workloads.gaussian(33, 100 + seed, N, K, 0.02)
        wc, ws, wg = nv.nvfp4_quantize(to_gpu(w))
        y = torch.full((M, N), float("nan"), dtype=out, device=x.device)
        assert _noalloc_abi(nv, x, wc, ws, wg, y) == 0
        ref = nv.nvfp4_gemm(x, wc, ws, wg, out_dtype=out)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), "call %d differs from nvfp4_gemm" % i
        if i == 0:
            owc, ows, owg = orc.quantize(w)
            xr = to_np(x)
            yo, _ = orc.linear(xr, owc, ows, owg)
            check_gemm(to_np(y), yo, out == torch.bfloat16, "noalloc vs oracle")


def test_noalloc_binding_and_limit(nv):
    M, N, K = 16, 128, 256
    x = to_gpu(workloads.to_bf16_bits(workloads.student_t(33, 9, M, K, 3.0)))
    wc, ws, wg = nv.nvfp4_quantize(to_gpu(workloads.gaussian(33, 109, N, K, 0.02)))
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    nv.nvfp4_gemm_noalloc(x, wc, ws, wg, y)
    torch.cuda.synchronize()
    assert torch.equal(y, nv.nvfp4_gemm(x, wc, ws, wg))
    # a shape whose workspace passes the fixed array is refused before any launch
    big = torch.empty((16384, 5120), dtype=torch.bfloat16, device=x.device)
    need = nv.lib.nvfp4_gemm_workspace_size(16384, N, 5120)
    assert need > nv.NOALLOC_SCRATCH_BYTES
    wcb = torch.zeros((N, 2560), dtype=torch.uint8, device=x.device)
    wsb = torch.zeros((N, 320), dtype=torch.uint8, device=x.device)
    yb = torch.empty((16384, N), dtype=torch.bfloat16, device=x.device)
    with pytest.raises(nv.Nvfp4Error):
        nv.nvfp4_gemm_noalloc(big, wcb, wsb, wg, yb)
