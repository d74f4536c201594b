"""GPU check of the fake-quantization error of the statistics harness
against the oracle's quantize/dequantize (paper "Why Gated DeltaNet Survives
4-Bit Quantization", section 5.1, Table 2: A4/W4 = relative error of
quantizing a tensor alone), and of the weight-error band the model card
"Gemma-4-31B-IT-NVFP4-FP8attn-text" reports for Gaussian-like weights."""
import numpy as np
import pytest
import torch

import workloads
from parity import to_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def st():
    from nvfp4_w4a4_quantized_02_amd import stats
    return stats


def _oracle_rel(orc, x):
    c, s, g = orc.quantize(x)
    xd = orc.dequantize(c, s, g).astype(np.float64)
    v = workloads.bf16_bits_to_f32(x).astype(np.float64) if x.dtype == np.uint16 else x.astype(np.float64)
    return np.linalg.norm(xd - v) / np.linalg.norm(v)


@pytest.mark.parametrize("name", ["decode_x", "prefill_x", "weight"])
def test_fake_quant_error_matches_oracle(st, orc, name):
    if name == "decode_x":
        x = workloads.decode(M=16, N_each=16).x
    elif name == "prefill_x":
        x = workloads.to_bf16_bits(workloads.student_t(3, 0, 256, 5120, 3.0))
    else:
        x = workloads.gaussian(3, 1, 512, 5120, 0.02)
    got = st.fake_quant_error(to_gpu(x))["rel_error"]
    ref = _oracle_rel(orc, x)
    assert abs(got - ref) <= 1e-9 * ref
    if name == "weight":
        assert 0.04 <= got <= 0.10


def test_tensor_stats_on_device_match_host(st):
    x = workloads.to_bf16_bits(workloads.student_t(3, 2, 64, 512, 2.5))
    a = st.tensor_stats(to_gpu(x))
    b = st.tensor_stats(torch.from_numpy(workloads.bf16_bits_to_f32(x)))
    for k in a:
        assert abs(a[k] - b[k]) <= 1e-9 * abs(b[k])
