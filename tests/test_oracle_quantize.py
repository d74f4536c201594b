"""Pins of the oracle's quantize / dequantize against facts fixed by the
pages and by the arithmetic, not by the oracle itself.

* Model card "Gemma-4-31B-IT-NVFP4-FP8attn-text", section "Verification":
  max(block scale) x tensor scale x 6 reproduces the absmax of the tensor
  (two-level scale), and NVFP4 relative weight error is 4-10%.
* Paper "Why Gated DeltaNet Survives 4-Bit Quantization", section 2
  ("NVFP4"): a block's largest value fixes its scale, so an outlier only
  affects its own block.
* Exhaustive round trip over all 16 E2M1 codes x all non-zero finite E4M3
  scales (an exactly representable tensor must come back unchanged).
* An independent re-derivation with library codecs (torch float8_e4m3fn and
  Python round-half-even) on random data.
"""
import math

import numpy as np
import pytest
import torch

import workloads

import json, os
FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def _unpack(codes):
    lo = codes & 0x0F
    hi = codes >> 4
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


# ------------------------------------------------------------ round trip

def _grid_tensor(orc, gs0):
    """One row: for every scale byte S in 1..0x7E a block holding the 16 E2M1
    codes (in a scrambled order) times dec(S) * gs0.  The S = 0x7E block
    holds +-6 * 448 * gs0 = 2688 * gs0, so amax / 2688 == gs0 exactly."""
    e2 = orc.e2m1_table()
    e4 = orc.e4m3_table()
    g = np.random.default_rng(3)
    blocks, codes, scales = [], [], []
    for S in range(1, 0x7F):
        perm = g.permutation(16)
        vals = np.array([e2[c] * e4[S] * gs0 for c in perm])
        assert (vals.astype(np.float32).astype(np.float64) == vals).all()
        blocks.append(vals.astype(np.float32))
        codes.append(perm.astype(np.uint8))
        scales.append(S)
    x = np.concatenate(blocks)[None, :]
    return x, np.concatenate(codes)[None, :], np.array(scales, dtype=np.uint8)[None, :]


@pytest.mark.parametrize("gs0", [1.0, 2.0 ** -4, 2.0 ** 10])
def test_round_trip_all_codes_all_scales(orc, gs0):
    x, codes_ref, scales_ref = _grid_tensor(orc, gs0)
    codes, scales, gs = orc.quantize(x)
    assert gs == np.float32(gs0)
    np.testing.assert_array_equal(scales, scales_ref)
    np.testing.assert_array_equal(_unpack(codes), codes_ref)
    # dequant of the exact tensor is exact
    np.testing.assert_array_equal(orc.dequantize(codes, scales, gs), x)


def test_packed_shape_halves_the_input_dim(orc):
    f = FACTS["packed_shape"]
    x = np.zeros((4, f["unpacked"][1]), np.float32)
    codes, scales, gs = orc.quantize(x)
    assert codes.shape[1] == f["packed_cols"]
    assert scales.shape[1] == f["unpacked"][1] // FACTS["block_size"]["value"]


def test_packing_low_nibble_first(orc):
    # element 0 = 0.5 (code 1), element 1 = -6 (code 0xF) -> byte 0xF1
    x = np.zeros((1, 16), np.float32)
    x[0, 0] = 0.5
    x[0, 1] = -6.0
    codes, scales, gs = orc.quantize(x)
    assert codes[0, 0] == 0xF1
    assert scales[0, 0] == 0x7E


# ---------------------------------------------------- two-level identity

@pytest.mark.parametrize("maker", ["tiny_x", "tiny_w", "t25", "gauss_big"])
def test_absmax_identity(orc, maker):
    if maker == "tiny_x":
        x = workloads.tiny().x
    elif maker == "tiny_w":
        x = workloads.tiny().w_parts[0]
    elif maker == "t25":
        x = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(workloads.student_t(9, 0, 64, 512, 2.5)))
    else:
        x = workloads.gaussian(9, 1, 512, 1024, 0.02)
    codes, scales, gs = orc.quantize(x)
    amax = np.abs(x).max()
    # the block that holds the absmax gets the largest scale, 448 = byte 0x7E
    assert scales.max() == 0x7E
    recon = orc.e4m3_decode(int(scales.max())) * float(gs) * 6.0
    assert abs(recon - float(amax)) <= 2.0 ** -22 * float(amax)


def test_gaussian_weight_error_band(orc):
    # model card: NVFP4 weight relative error 4-10% ("correct for e2m1")
    for shape in [(256, 256), (1024, 5120)]:
        w = workloads.gaussian(9, 2, shape[0], shape[1], 0.02)
        codes, scales, gs = orc.quantize(w)
        wh = orc.dequantize(codes, scales, gs)
        rel = np.linalg.norm((wh - w).astype(np.float64)) / np.linalg.norm(w.astype(np.float64))
        lo, hi = FACTS["weight_rel_error_band"]["value"]
        assert lo <= rel <= hi, rel


# ---------------------------------------------------------- invariants

def test_block_locality(orc):
    x = workloads.gaussian(9, 3, 8, 256, 1.0)
    x[0, 0] = 40.0                                   # holds the absmax
    c0, s0, g0 = orc.quantize(x)
    y = x.copy()
    y[3, 32:48] = workloads.gaussian(9, 4, 1, 16, 3.0)   # rewrite one block
    assert np.abs(y).max() == np.abs(x).max()
    c1, s1, g1 = orc.quantize(y)
    assert g1 == g0
    ds = np.argwhere(s0 != s1)
    assert all((r, b) == (3, 2) for r, b in ds)
    dc = np.argwhere(c0 != c1)
    assert all(r == 3 and 16 <= c < 24 for r, c in dc)


@pytest.mark.parametrize("j", [-20, -3, 1, 7])
def test_power_of_two_scaling(orc, j):
    x = workloads.gaussian(9, 5, 16, 512, 1.0)
    c0, s0, g0 = orc.quantize(x)
    c1, s1, g1 = orc.quantize((x * np.float32(2.0 ** j)).astype(np.float32))
    np.testing.assert_array_equal(c0, c1)
    np.testing.assert_array_equal(s0, s1)
    assert g1 == np.float32(g0 * np.float32(2.0 ** j))


def test_negation_flips_only_signs(orc):
    x = workloads.gaussian(9, 6, 16, 512, 1.0)
    x[x == 0] = 1.0
    c0, s0, g0 = orc.quantize(x)
    c1, s1, g1 = orc.quantize(-x)
    np.testing.assert_array_equal(s0, s1)
    assert g0 == g1
    np.testing.assert_array_equal(c1, c0 ^ 0x88)


def test_zero_tensor(orc):
    x = np.zeros((4, 64), np.float32)
    x[1, 5] = -0.0
    codes, scales, gs = orc.quantize(x)
    assert gs == 0.0
    assert (scales == 0).all()
    u = _unpack(codes)
    assert u[1, 5] == 8 and (np.delete(u.ravel(), 1 * 64 + 5) == 0).all()


def test_signed_zero_keeps_sign_bit(orc):
    x = np.array([[1.0, -0.0, -1e-30] + [0.0] * 13], np.float32)
    codes, scales, gs = orc.quantize(x)
    u = _unpack(codes)[0]
    assert u[0] == 7 and u[1] == 8 and u[2] == 8


def test_bf16_input_equals_widened_fp32(orc):
    xb = workloads.to_bf16_bits(workloads.student_t(9, 7, 32, 256, 3.0))
    a = orc.quantize(xb)
    b = orc.quantize(workloads.bf16_bits_to_f32(xb))
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


# --------------------------------------- independent library re-derivation

def _e2m1_rne_sat_torch(r):
    """E2M1 magnitude codes via torch rounding of a value scaled to keep one
    fractional significand bit (torch.round is round-half-even)."""
    r = r.to(torch.float64)
    sub = torch.round(r * 2) / 2                               # grid below 1
    e = torch.floor(torch.log2(torch.clamp(r, min=1.0)))
    nor = torch.round(r / 2 ** e * 2) / 2 * 2 ** e
    q = torch.where(r < 1.0, sub, nor)
    q = torch.clamp(q, max=6.0)
    lut = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    return torch.tensor([lut[float(v)] for v in q.flatten()], dtype=torch.uint8).reshape(q.shape)


def test_quantize_matches_torch_rederivation(orc):
    x = workloads.bf16_bits_to_f32(workloads.to_bf16_bits(
        workloads.with_hot_channels(workloads.student_t(9, 8, 24, 128, 2.5), 9, 8, 3, 200.0)))
    codes, scales, gs = orc.quantize(x)
    t = torch.from_numpy(x)
    amax = t.abs().max()
    gs_t = amax / torch.tensor(2688.0, dtype=torch.float32)
    assert gs_t.item() == float(gs)
    blocks = t.reshape(24, 8, 16)
    bmax = blocks.abs().amax(dim=2)
    sbf = bmax / (torch.tensor(6.0) * gs_t)                  # fp32 ops
    sb = torch.clamp(sbf, max=448.0).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(sb.view(torch.uint8).numpy(), scales)
    es = sb.to(torch.float32) * gs_t
    r = blocks.abs() / es[:, :, None]
    mag = _e2m1_rne_sat_torch(r)
    sign = torch.signbit(blocks).to(torch.uint8) << 3
    ref_codes = (mag | sign).reshape(24, 128).numpy()
    np.testing.assert_array_equal(_unpack(codes), ref_codes)


def test_dequant_bf16_is_rounded_fp32(orc):
    w = workloads.gaussian(9, 9, 8, 64, 0.02)
    codes, scales, gs = orc.quantize(w)
    f = orc.dequantize(codes, scales, gs)
    b = orc.dequantize_bf16(codes, scales, gs)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)
    # dequant equals code * scale * gs, with code*scale exact
    e2, e4 = orc.e2m1_table(), orc.e4m3_table()
    u = _unpack(codes)
    exact = e2[u] * np.repeat(e4[scales], 16, axis=1) * float(gs)
    np.testing.assert_array_equal(f, exact.astype(np.float32))
