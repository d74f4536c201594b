"""Pins of the oracle's E2M1 / E4M3 codecs against sources other than itself.

E4M3: torch's float8_e4m3fn dtype (an independent library implementation of
the OCP 8-bit format) for decoding all 256 bytes and for round-to-nearest-even
encoding below its overflow threshold.  E2M1: the largest magnitude 6.0 stated
by the model card "Gemma-4-31B-IT-NVFP4-FP8attn-text" (section "Verification"),
and Python's round-half-even ``round()`` applied to a value scaled to one
fractional significand bit.
"""
import math

import numpy as np
import pytest
import torch

import json, os
FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))


def _torch_e4m3_decode_all():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    return b.to(torch.float64).numpy()


def _torch_e4m3_encode(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_e4m3_decode_matches_torch(orc):
    ours = orc.e4m3_table()
    ref = _torch_e4m3_decode_all()
    nan_o, nan_r = np.isnan(ours), np.isnan(ref)
    assert (nan_o == nan_r).all()
    assert sorted(np.flatnonzero(nan_o).tolist()) == [0x7F, 0xFF]
    np.testing.assert_array_equal(ours[~nan_o], ref[~nan_r])
    # signed zero: 0x80 decodes to -0.0
    assert math.copysign(1.0, ours[0x80]) == -1.0


def test_e4m3_extremes(orc):
    t = orc.e4m3_table()
    finite = t[:0x7F]
    assert finite.max() == 448.0 and finite.argmax() == 0x7E
    assert t[1] == 2.0 ** -9            # smallest subnormal
    assert t[8] == 2.0 ** -6            # smallest normal
    assert 6.0 * 448.0 == 2688.0        # the tensor-scale divisor


def _e4m3_probe_values(orc):
    t = orc.e4m3_table()[:0x7F]
    mids = (t[:-1] + t[1:]) / 2.0
    vals = [t.astype(np.float32), mids.astype(np.float32)]
    m32 = mids.astype(np.float32)
    assert (m32.astype(np.float64) == mids).all()  # midpoints are exact in fp32
    vals.append(np.nextafter(m32, np.float32(0)))
    vals.append(np.nextafter(m32, np.float32(np.inf)))
    g = np.random.default_rng(12345)
    vals.append((2.0 ** g.uniform(-14, math.log2(448.0), 200_000)).astype(np.float32))
    vals.append(g.uniform(0, 2.0 ** -6, 50_000).astype(np.float32))
    vals.append(np.array([0.0, 1e-45, 1e-30, 2.0 ** -10, 447.99997, 448.0, 455.0, 463.99997],
                         dtype=np.float32))
    return np.concatenate(vals)


def test_e4m3_encode_matches_torch_below_overflow(orc):
    v = _e4m3_probe_values(orc)
    v = v[v < 464.0]          # torch turns values at/after the overflow midpoint into NaN
    np.testing.assert_array_equal(orc.e4m3_encode(v), _torch_e4m3_encode(v))


def test_e4m3_encode_saturates(orc):
    v = np.array([448.0, 464.0, 480.0, 1e6, 3.0e38, np.inf], dtype=np.float32)
    assert (orc.e4m3_encode(v) == 0x7E).all()


def test_e4m3_subnormal_ties_go_to_even(orc):
    # 0.5 * 2^-9 lies between 0x00 and 0x01 -> 0x00; 1.5 * 2^-9 -> 0x02; 7.5*2^-9 -> 0x08
    v = np.array([0.5, 1.5, 2.5, 7.5], dtype=np.float32) * np.float32(2.0 ** -9)
    assert orc.e4m3_encode(v).tolist() == [0x00, 0x02, 0x02, 0x08]


# ------------------------------------------------------------------ E2M1

def test_e2m1_value_set(orc):
    t = orc.e2m1_table()
    mags = t[:8]
    # 6.0 is the largest E2M1 magnitude (model card, "Verification")
    assert mags.max() == FACTS["e2m1_max"]["value"] and mags.argmax() == 7
    assert (np.diff(mags) > 0).all()               # codes increase with magnitude
    assert mags[0] == 0.0 and mags[1] == 0.5       # one subnormal step of 0.5
    # 1 mantissa bit: every non-zero magnitude has at most 2 significant bits
    for v in mags[1:]:
        m, e = math.frexp(v)
        assert (m * 4) == int(m * 4)
    # sign bit is bit 3, magnitudes mirror
    np.testing.assert_array_equal(t[8:], -t[:8])
    assert math.copysign(1.0, t[8]) == -1.0


def _round_e2m1_library(r: float) -> int:
    """Reference for E2M1 RNE via Python's round-half-even: keep one
    fractional significand bit (subnormal step 0.5 below 1)."""
    if r >= 6.0:
        return 7
    if r < 1.0:
        q = round(r * 2.0) / 2.0          # grid 0, 0.5, 1.0
    else:
        m, e = math.frexp(r)              # r = m * 2^e, m in [0.5, 1)
        q = math.ldexp(round(m * 4.0) / 4.0, e)
        q = min(q, 6.0)                   # 7 would round to 8 -> saturate; 5..6 stays
    table = {0.0: 0, 0.5: 1, 1.0: 2, 1.5: 3, 2.0: 4, 3.0: 5, 4.0: 6, 6.0: 7}
    if q == 8.0:
        return 7
    return table[q]


def test_e2m1_encode_matches_round_half_even(orc):
    mags = orc.e2m1_table()[:8]
    mids = ((mags[:-1] + mags[1:]) / 2.0).astype(np.float32)
    g = np.random.default_rng(7)
    r = np.concatenate([
        mags.astype(np.float32), mids,
        np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
        g.uniform(0, 8, 100_000).astype(np.float32),
        (2.0 ** g.uniform(-40, 3, 20_000)).astype(np.float32),
        np.array([0.0, 1e-45, 5.999999, 6.0, 7.0, 1e30, np.inf], dtype=np.float32),
    ])
    ours = orc.e2m1_encode_mag(r)
    ref = np.array([_round_e2m1_library(float(v)) for v in r], dtype=np.uint8)
    np.testing.assert_array_equal(ours, ref)


@pytest.mark.parametrize("r,code", [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4),
                                    (2.5, 4), (3.5, 6), (5.0, 6), (6.4, 7)])
def test_e2m1_ties(orc, r, code):
    assert orc.e2m1_encode_mag(np.array([r], np.float32))[0] == code
