"""The library's calls can be captured into a HIP graph (they allocate
nothing and record no memset): each form is captured once, replayed several
times with eager work and synchronizations in between, and every replay must
reproduce the eager result bit for bit (the kernels are deterministic)."""
import numpy as np
import pytest
import torch

import workloads
from parity import to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_w4a4_quantized_02_amd as m
    return m


def _check_replays(fn, out, n=3):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for r in range(n):
        out.zero_()
        scratch = torch.randn(1 << 20, device="cuda:0")          # unrelated eager work between replays
        scratch.mul_(2.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs" % r


def _weight(nv, N, K, seed):
    return nv.nvfp4_quantize(to_gpu(workloads.gaussian(29, seed, N, K, 0.02)))


@pytest.mark.parametrize("M", [1, 16, 300])
def test_w4a4_linear_in_graph(nv, M):
    N, K = 520, 1024
    wc, ws, wg = _weight(nv, N, K, 1)
    x = to_gpu(workloads.to_bf16_bits(workloads.student_t(29, 2, M, K, 3.0)))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda:0")
    wsb = torch.empty(nv.lib.nvfp4_gemm_workspace_size(M, N, K), dtype=torch.uint8, device="cuda:0")
    print("case: graph w4a4 M=%d" % M, flush=True)
    _check_replays(lambda: nv.nvfp4_gemm_run(nv.nvfp4_gemm_prepare(x, ws=wsb), wc, ws, wg, out=y), y)


@pytest.mark.parametrize("M", [4, 300])
def test_w4a16_and_fp8_in_graph(nv, M):
    N, K = 520, 1024
    wc, ws, wg = _weight(nv, N, K, 3)
    x = to_gpu(workloads.to_bf16_bits(workloads.student_t(29, 4, M, K, 3.0)))
    y = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
    print("case: graph w4a16 M=%d" % M, flush=True)
    _check_replays(lambda: nv.nvfp4_gemm_w4a16(x, wc, ws, wg, out=y), y)
    wq, sw = nv.nvfp4_fp8_quantize(to_gpu(workloads.gaussian(29, 5, N, K, 0.02)))
    print("case: graph w8a16 / w8a8 M=%d" % M, flush=True)
    _check_replays(lambda: nv.nvfp4_gemm_w8a16(x, wq, sw, out=y), y)
    _check_replays(lambda: nv.nvfp4_gemm_w8a8(x, wq, sw, out=y), y)


def test_quantize_in_graph(nv):
    x = to_gpu(workloads.to_bf16_bits(workloads.student_t(29, 6, 2048, 1024, 3.0)))
    q = torch.empty((2048, 1024), dtype=torch.uint8, device="cuda:0")
    s = torch.empty(1, device="cuda:0")
    ws = nv.workspace(nv.lib.nvfp4_fp8_quantize_workspace_size(2048, 1024), x.device)

    def fp8():
        assert nv.lib.nvfp4_fp8_quantize(x.data_ptr(), 1, 2048, 1024, 1024, q.data_ptr(), s.data_ptr(),
                                         ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream) == 0
    print("case: graph fp8 quantize", flush=True)
    _check_replays(fp8, q)
    codes = torch.empty((2048, 512), dtype=torch.uint8, device="cuda:0")
    scales = torch.empty((2048, 64), dtype=torch.uint8, device="cuda:0")
    gs = torch.empty(1, device="cuda:0")
    qws = nv.workspace(nv.lib.nvfp4_quantize_workspace_size(2048, 1024), x.device)

    def nvfp4():
        assert nv.lib.nvfp4_quantize(x.data_ptr(), 1, 2048, 1024, 1024, codes.data_ptr(), scales.data_ptr(),
                                     gs.data_ptr(), qws.data_ptr(), qws.numel(),
                                     torch.cuda.current_stream().cuda_stream) == 0
    print("case: graph nvfp4 quantize", flush=True)
    _check_replays(nvfp4, codes)
