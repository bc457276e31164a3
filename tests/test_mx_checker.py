"""The tie-tolerant E4M3 image check (tests/mx_layout.py) that the MXFP8 GPU
tests apply to dG | dU, whose codes the device decides on its own fp32
values: it accepts the oracle's encoding and a neighbouring code or scale
exactly where fp32 rounding of the value could have moved the decision, and
rejects any other difference. CPU only."""
import numpy as np
import pytest

from oracle import moe_oracle as O
import mx_layout as ML


def _vals(seed=0, R=64, C=128):
    return np.random.default_rng(seed).standard_normal((R, C))


def test_exact_encoding_passes():
    v = _vals()
    q, s = O.mx_quantize(v, "cols")
    ML.assert_codes_near(q, s, v, "exact")


def test_fp32_rounded_values_pass():
    v = _vals(1)
    q, s = O.mx_quantize(v.astype(np.float32).astype(np.float64) * (1 + 1e-7), "cols")
    ML.assert_codes_near(q, s, v, "fp32 rounding")


def test_neighbour_code_at_a_tie_passes_and_elsewhere_fails():
    v = _vals(2)
    q, s = O.mx_quantize(v, "cols")
    # Put element (0, 5) on the midpoint of two codes under its block's scale,
    # a hair below: the oracle rounds down, the neighbouring code is allowed.
    scale = 2.0 ** (int(s[0, 0]) - 127)
    y = v[0, 5] / scale
    lo = O.e4m3_decode(O.e4m3_encode(np.array([abs(y)])))[0]
    codes = np.arange(127, dtype=np.uint8)
    vals = O.e4m3_decode(codes)
    hi = vals[vals > lo].min()
    mid = 0.5 * (lo + hi)
    v2 = v.copy()
    v2[0, 5] = np.sign(y) * (mid - 1e-9 * mid) * scale
    q2, s2 = O.mx_quantize(v2, "cols")
    flipped = q2.copy()
    flipped[0, 5] = O.e4m3_encode(np.array([np.sign(y) * hi]))[0]
    ML.assert_codes_near(flipped, s2, v2, "near tie")
    # The same flip on a value far from the midpoint is rejected.
    far = q.copy()
    far[3, 7] = O.e4m3_encode(np.array([O.e4m3_decode(q[3:4, 7])[0] * 1.25]))[0]
    if far[3, 7] == q[3, 7]:
        far[3, 7] ^= 1
    with pytest.raises(AssertionError):
        ML.assert_codes_near(far, s, v, "far flip")


def test_scale_step_only_at_a_power_of_two():
    v = _vals(3)
    v[2, :32] *= 0.5
    v[2, 0] = 4.0 * (1 - 1e-9)  # block maximum a hair below 4
    q, s = O.mx_quantize(v, "cols")
    s_up = s.copy()
    s_up[2, 0] += 1  # the device saw the maximum as 4.0
    y = v[2, :32] / 2.0 ** (int(s_up[2, 0]) - 127)
    q_up = q.copy()
    q_up[2, :32] = O.e4m3_encode(y)
    ML.assert_codes_near(q_up, s_up, v, "scale at a power of two")
    s_bad = s.copy()
    s_bad[5, 1] += 1
    with pytest.raises(AssertionError):
        ML.assert_codes_near(q, s_bad, v, "scale elsewhere")
