"""Pins of the oracle's exact block-scaled GEMM and fused-module repair.

GEMM: numpy float64 matmul of independently decoded operands (torch's
float8_e4m3fn decode for scales), unit-scale and one-hot special cases, and
exact rational arithmetic (``fractions.Fraction``) on a tiny problem.

Repair: paper "Why Gated DeltaNet Survives 4-Bit Quantization", section 6,
paragraph "Per-module calibration vs. fused-GEMM scaling": serving a fused
group with the largest member scale and untouched local scales mis-scales the
other members; the repair rewrites every member onto the shared scale and
folds the ratio into the E4M3 block scales, with re-rounding error at most
6.2% per affected scale (the E4M3 half-ulp 2^-4 = 6.25%) and the ratios the
paper reports (1.82x, 2.75x, worst 2.81x).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads

import json, os
FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def _unpack(codes):
    out = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = codes & 0x0F
    out[:, 1::2] = codes >> 4
    return out


def _e4m3_torch(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn) \
        .to(torch.float64).numpy()


_E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0.0, -.5, -1, -1.5, -2, -3, -4, -6])


def _deq64(codes, scales):
    """fp64 code * scale (no tensor scale) with library / table decoders."""
    return _E2M1[_unpack(codes)] * np.repeat(_e4m3_torch(scales), 16, axis=1)


def test_gemm_matches_float64_matmul(orc):
    p = workloads.tiny()
    xc, xs, gx = orc.quantize(p.x)
    wc, ws, gw = orc.quantize(p.w_parts[0])
    y = orc.gemm_exact(xc, xs, gx, wc, ws, gw)
    ref = (_deq64(xc, xs) @ _deq64(wc, ws).T) * float(gx) * float(gw)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_gemm_unit_scales_is_e2m1_matmul(orc):
    g = np.random.default_rng(11)
    M, N, K = 5, 7, 64
    xc = g.integers(0, 256, (M, K // 2), dtype=np.uint8)
    wc = g.integers(0, 256, (N, K // 2), dtype=np.uint8)
    ones_x = np.full((M, K // 16), 0x38, np.uint8)   # E4M3 0x38 == 1.0
    ones_w = np.full((N, K // 16), 0x38, np.uint8)
    assert orc.e4m3_decode(0x38) == 1.0
    y = orc.gemm_exact(xc, ones_x, 1.0, wc, ones_w, 1.0)
    ref = _E2M1[_unpack(xc)] @ _E2M1[_unpack(wc)].T
    np.testing.assert_array_equal(y, ref)


def test_gemm_one_hot_selects_weight_column(orc):
    p = workloads.tiny()
    wc, ws, gw = orc.quantize(p.w_parts[0])
    K = p.K
    for k in (0, 17, 255):
        x = np.zeros((1, K), np.float32)
        x[0, k] = 3.0
        xc, xs, gx = orc.quantize(x)
        y = orc.gemm_exact(xc, xs, gx, wc, ws, gw)[0]
        # the lone non-zero quantizes to +6 at scale 448 (it fixes amax)
        assert _unpack(xc)[0, k] == 7 and xs[0, k // 16] == 0x7E
        ref = 6.0 * 448.0 * _deq64(wc, ws)[:, k] * float(gx) * float(gw)
        np.testing.assert_allclose(y, ref, rtol=1e-14)


def test_gemm_fraction_brute_force(orc):
    g = np.random.default_rng(5)
    x = g.standard_normal((3, 32)).astype(np.float32)
    w = g.standard_normal((4, 32)).astype(np.float32)
    xc, xs, gx = orc.quantize(x)
    wc, ws, gw = orc.quantize(w)
    y = orc.gemm_exact(xc, xs, gx, wc, ws, gw)
    xu, wu = _unpack(xc), _unpack(wc)
    e4 = orc.e4m3_table()
    for m in range(3):
        for n in range(4):
            acc = Fraction(0)
            for k in range(32):
                a = Fraction(_E2M1[xu[m, k]]) * Fraction(e4[xs[m, k // 16]])
                b = Fraction(_E2M1[wu[n, k]]) * Fraction(e4[ws[n, k // 16]])
                acc += a * b
            exact = acc * Fraction(float(gx)) * Fraction(float(gw))
            assert abs(Fraction(y[m, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_gemm_sampled_equals_full(orc):
    p = workloads.tiny()
    xc, xs, gx = orc.quantize(p.x)
    wc, ws, gw = orc.quantize(p.w_parts[0])
    y = orc.gemm_exact(xc, xs, gx, wc, ws, gw)
    g = np.random.default_rng(1)
    mi = g.integers(0, p.M, 50)
    ni = g.integers(0, p.N, 50)
    np.testing.assert_array_equal(orc.gemm_exact_sampled(xc, xs, gx, wc, ws, gw, mi, ni), y[mi, ni])


# ------------------------------------------------------------- repair

def _quantize_members(orc, parts):
    q = [orc.quantize(w) for w in parts]
    return [a for a, _, _ in q], [b for _, b, _ in q], [g for _, _, g in q]


def test_repair_keeps_largest_member_and_bounds_rerounding(orc):
    p = workloads.fused_qkv(M=8, K=256, Nq=96, Nkv=32)
    codes, scales, gss = _quantize_members(orc, p.w_parts)
    new, S = orc.fuse_rescale(scales, gss)
    assert S == max(gss)
    e4 = orc.e4m3_table()
    for i, (old, nw, g) in enumerate(zip(scales, new, gss)):
        rho = np.float32(g / S)
        if g == S:
            np.testing.assert_array_equal(old, nw)   # ratio 1: byte-identical
            continue
        target = e4[old].astype(np.float32) * rho      # fp32 product
        got = e4[nw]
        normal = target >= 2.0 ** -6
        rel = np.abs(got[normal] - target[normal]) / target[normal]
        assert rel.max() <= 2.0 ** -4 + 1e-12          # E4M3 half ulp
        assert rel.max() <= FACTS["rerounding_bound"]["value"] + 5e-4   # paper: <= 6.2%
        assert (np.abs(got[~normal] - target[~normal]) <= 2.0 ** -10 + 1e-18).all()
        assert (nw <= old).all()                       # rho <= 1: nothing grows


@pytest.mark.parametrize("ratio", FACTS["fused_scale_ratios"]["value"] + [FACTS["fused_scale_ratios"]["worst"]])
def test_unrepaired_fusion_misscales_by_the_ratio(orc, ratio):
    """Serving member b with the larger member's tensor scale and b's own
    block scales multiplies b's outputs by exactly S / gs_b."""
    g = np.random.default_rng(int(ratio * 100))
    K = 128
    a = g.standard_normal((24, K)).astype(np.float32) * np.float32(0.02)
    b = g.standard_normal((16, K)).astype(np.float32) * np.float32(0.02)
    ca, sa, ga = orc.quantize(a)
    cb, sb, _ = orc.quantize(b)
    gb = np.float32(ga / np.float32(ratio))
    cb, sb, gb = orc.quantize(b, gs=gb)       # member b calibrated with its own smaller scale
    x = workloads.tiny(M=4, K=K).x
    xc, xs, gx = orc.quantize(x)
    y_b = orc.gemm_exact(xc, xs, gx, cb, sb, gb)
    S = max(ga, gb)
    y_bad = orc.gemm_exact(xc, xs, gx, cb, sb, S)            # max gs, local scales untouched
    np.testing.assert_allclose(y_bad, y_b * (float(S) / float(gb)), rtol=1e-12)
    assert abs(float(S) / float(gb) - ratio) < 1e-5
    # repaired: the shared scale with rescaled block scales reproduces y_b
    new, S2 = orc.fuse_rescale([sa, sb], [ga, gb])
    y_fix = orc.gemm_exact(xc, xs, gx, cb, new[1], S2)
    err = np.linalg.norm(y_fix - y_b) / np.linalg.norm(y_b)
    bad = np.linalg.norm(y_bad - y_b) / np.linalg.norm(y_b)
    assert err < 0.07 and bad > ratio - 1.001


def test_repair_zero_group(orc):
    s = [np.zeros((2, 4), np.uint8), np.zeros((3, 4), np.uint8)]
    new, S = orc.fuse_rescale(s, [0.0, 0.0])
    assert S == 0.0
    for a, b in zip(s, new):
        np.testing.assert_array_equal(a, b)


def test_repair_keeps_nan_and_sign_bytes(orc):
    s = [np.array([[0x7E, 0x7F, 0xFF, 0xB8]], np.uint8), np.array([[0x7E, 0, 0, 0]], np.uint8)]
    new, S = orc.fuse_rescale(s, [0.5, 1.0])
    assert new[0][0, 1] == 0x7F and new[0][0, 2] == 0xFF
    assert new[0][0, 0] == 0x76                      # 448 * 0.5 = 224 = 0x76
    assert new[0][0, 3] == 0xB0                      # -1.0 * 0.5 = -0.5
