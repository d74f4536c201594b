"""CPU tests of the Python binding's argument checks: tensors that the C ABI
cannot validate itself (their device, shape, dtype and strides) are refused
with ValueError / TypeError before any pointer reaches the library."""
import pytest
import torch


@pytest.fixture(scope="module")
def nv():
    import nvfp4_w4a4_quantized_02_amd as m
    return m


CPU = torch.device("cpu")


def test_host_tensors_are_refused(nv):
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    wc = torch.zeros((8, 32), dtype=torch.uint8)
    ws = torch.zeros((8, 4), dtype=torch.uint8)
    g = torch.ones(1)
    with pytest.raises(ValueError):
        nv.nvfp4_quantize(x)
    with pytest.raises(ValueError):
        nv.nvfp4_gemm(x, wc, ws, g)
    with pytest.raises(ValueError):
        nv.nvfp4_gemm_w4a16(x, wc, ws, g)
    with pytest.raises(ValueError):
        nv.nvfp4_gemm_w8a16(x, torch.zeros((8, 64), dtype=torch.uint8), g)
    with pytest.raises(ValueError):
        nv.nvfp4_dequantize(wc, ws, g)
    with pytest.raises(ValueError):
        nv.nvfp4_fp8_dequantize(torch.zeros((8, 64), dtype=torch.uint8), g)
    with pytest.raises(ValueError):
        nv.nvfp4_fuse_rescale([ws], [g])
    with pytest.raises(ValueError):
        nv.workspace(1024, "cpu")


def test_check_out(nv):
    ok = torch.empty((5, 24), dtype=torch.bfloat16)
    assert nv._check_out(ok, 5, 24, CPU) is ok
    assert nv._check_out(torch.empty((5, 32), dtype=torch.float32)[:, :24], 5, 24, CPU) is not None
    with pytest.raises(ValueError):
        nv._check_out(torch.empty((4, 24), dtype=torch.bfloat16), 5, 24, CPU)     # one row short
    with pytest.raises(ValueError):
        nv._check_out(torch.empty((5, 25), dtype=torch.bfloat16), 5, 24, CPU)
    with pytest.raises(TypeError):
        nv._check_out(torch.empty((5, 24), dtype=torch.float16), 5, 24, CPU)
    with pytest.raises(ValueError):
        nv._check_out(torch.empty((24, 5), dtype=torch.float32).t(), 5, 24, CPU)  # strided rows
    with pytest.raises(ValueError):
        nv._check_out(torch.empty((1, 24), dtype=torch.float32).expand(5, 24), 5, 24, CPU)  # rows overlap
    with pytest.raises(ValueError):
        nv._check_out(ok, 5, 24, torch.device("meta"))


def test_check_weight(nv):
    wc = torch.zeros((8, 32), dtype=torch.uint8)
    ws = torch.zeros((8, 4), dtype=torch.uint8)
    g = torch.ones(1)
    assert nv._check_weight(wc, ws, g, 64, CPU) == 8
    with pytest.raises(ValueError):
        nv._check_weight(wc, ws, g, 128, CPU)                               # K mismatch
    with pytest.raises(ValueError):
        nv._check_weight(torch.zeros((32, 8), dtype=torch.uint8).t(), ws, g, 64, CPU)   # not contiguous
    with pytest.raises(ValueError):
        nv._check_weight(wc.to(torch.int16), ws, g, 64, CPU)
    with pytest.raises(ValueError):
        nv._check_weight(wc, torch.zeros((8, 5), dtype=torch.uint8), g, 64, CPU)
    with pytest.raises(ValueError):
        nv._check_weight(wc, ws, torch.ones(1, dtype=torch.float64), 64, CPU)
    with pytest.raises(ValueError):
        nv._check_weight(wc, ws, torch.ones(0), 64, CPU)
    with pytest.raises(ValueError):
        nv._check_fp8_weight(torch.zeros((8, 60), dtype=torch.uint8), g, 64, CPU)


def test_ld_out(nv):
    assert nv._ld_out(torch.empty((3, 8))[:, :5], 3, 5) == 8
    assert nv._ld_out(torch.empty((1, 8))[:, :5], 1, 5) == 8
    assert nv._ld_out(torch.empty((1, 5)), 1, 5) == 5
