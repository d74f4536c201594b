"""Exhaustive pins of the oracle's two element encoders over every
non-negative binary32 value (0 .. +inf, 2^31 + 1 bit patterns; the encoders
are only ever called with magnitudes and non-negative quotients).

* E4M3 (block scales): against torch's own fp32 -> float8_e4m3fn conversion
  (round to nearest even) wherever that conversion is in range, and against
  saturation to 448 (byte 0x7E) at and above 448 (model card
  "Gemma-4-31B-IT-NVFP4-FP8attn-text", section "Verification": 448 is the
  largest E4M3 scale).
* E2M1 (element codes): against a piecewise round-half-even on the grid's
  three spacings (0.5 below 2, 1 from 2 to 4, 2 from 4 to 6) and saturation
  at 6 (paper "Why Gated DeltaNet Survives 4-Bit Quantization", section 2
  "NVFP4"; 6.0 is the largest E2M1 magnitude per the model card).

Several minutes of CPU work (the oracle's E4M3 encoder searches all 127
candidates per value), so these run only with NVFP4_SLOW=1."""
import numpy as np
import pytest
import torch

CHUNK = 1 << 24
LAST = 0x7F800000          # +inf


def _chunks():
    for start in range(0, LAST + 1, CHUNK):
        stop = min(LAST + 1, start + CHUNK)
        yield np.arange(start, stop, dtype=np.uint32).view(np.float32)


@pytest.mark.slow
def test_e4m3_encode_every_nonnegative_fp32(orc):
    for v in _chunks():
        got = orc.e4m3_encode(v)
        ref = np.full(v.shape, 0x7E, dtype=np.uint8)            # saturation at and above 448
        below = v < np.float32(448.0)
        ref[below] = torch.from_numpy(v[below]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        if not np.array_equal(got, ref):
            i = int(np.argmax(got != ref))
            raise AssertionError("E4M3 encode of %r (0x%08x): oracle 0x%02x, reference 0x%02x" % (
                float(v[i]), int(v[i:i + 1].view(np.uint32)[0]), got[i], ref[i]))


def _e2m1_reference(v: np.ndarray) -> np.ndarray:
    r = v.astype(np.float64)                  # exact; the scalings below are exact too
    code = np.full(r.shape, 7, dtype=np.int64)
    lo = r < 2.0
    code[lo] = np.rint(2.0 * r[lo]).astype(np.int64)                    # 0, .5, 1, 1.5, 2 -> codes 0..4
    mid = (r >= 2.0) & (r < 4.0)
    code[mid] = np.rint(r[mid]).astype(np.int64) + 2                    # 2, 3, 4 -> codes 4..6
    hi = (r >= 4.0) & (r < 6.0)
    code[hi] = np.rint(0.5 * r[hi]).astype(np.int64) + 4                # 4, 6 -> codes 6, 7
    return code.astype(np.uint8)


@pytest.mark.slow
def test_e2m1_encode_every_nonnegative_fp32(orc):
    for v in _chunks():
        got = orc.e2m1_encode_mag(v)
        ref = _e2m1_reference(v)
        if not np.array_equal(got, ref):
            i = int(np.argmax(got != ref))
            raise AssertionError("E2M1 encode of %r: oracle %d, reference %d" % (float(v[i]), got[i], ref[i]))


def test_e2m1_reference_ties():
    """The reference itself at the tie points the rule fixes."""
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 1e30, np.inf], dtype=np.float32)
    assert _e2m1_reference(ties).tolist() == [0, 2, 2, 4, 4, 6, 6, 7, 7, 7]
