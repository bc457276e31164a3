"""Pins for the oracle's MXFP8 (E4M3 + per-32 E8M0) encoding.

References: the OCP format tables (tests/golden/e4m3_ocp_table.json), an
exhaustive nearest-of-all-codes search, and torch's float8_e4m3fn cast.
"""
import json
import os

import numpy as np
import pytest
import torch

from moe_inputs import bf16_bits_to_f32
from oracle import moe_oracle as O

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_table.json")))


def _val(v):
    return float("nan") if v == "nan" else float(v)


def test_decode_matches_spec_table():
    for row in GOLDEN["e4m3"]:
        got = O.e4m3_decode([int(row["code"], 16)])[0]
        want = _val(row["value"])
        if np.isnan(want):
            assert np.isnan(got), row
        else:
            assert got == want and np.signbit(got) == np.signbit(want), row
    for row in GOLDEN["e8m0"]:
        got = O.e8m0_decode([int(row["code"], 16)])[0]
        want = _val(row["value"])
        assert (np.isnan(got) and np.isnan(want)) or got == want, row
    assert O.E4M3_EMAX == GOLDEN["e4m3_emax"]


def _brute_encode(y):
    """Nearest non-negative finite E4M3 magnitude by exhaustive search; on a
    tie the code with an even mantissa (even code) wins; then the sign bit."""
    mags = O.e4m3_decode(np.arange(0x7F))          # codes 0x00..0x7E, increasing
    a = np.abs(y)[:, None]
    dist = np.abs(a - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    codes = np.arange(0x7F)[None, :]
    # Prefer even codes among the tied candidates.
    pick = np.where(cand & (codes % 2 == 0), codes, 1000).min(axis=1)
    pick = np.where(pick == 1000, np.where(cand, codes, 1000).min(axis=1), pick)
    return (pick | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def _all_bf16_values():
    with np.errstate(invalid="ignore"):
        v = bf16_bits_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16)).astype(np.float64)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("shift", [0, -4, -9, 3])
def test_encode_exhaustive_over_bf16(shift):
    v = _all_bf16_values() * 2.0 ** shift
    v = v[np.abs(v) < 1024]
    for chunk in np.array_split(v, 8):
        np.testing.assert_array_equal(O.e4m3_encode(chunk), _brute_encode(chunk))


def test_encode_matches_torch_cast_in_range():
    v = _all_bf16_values()
    v = v[np.abs(v) <= 448]
    ours = O.e4m3_encode(v)
    ref = torch.tensor(v, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_saturation_and_signed_zero():
    assert O.e4m3_encode([1e6])[0] == 0x7E and O.e4m3_encode([-500.0])[0] == 0xFE
    assert O.e4m3_encode([464.0])[0] == 0x7E          # midpoint to the (absent) 480
    assert O.e4m3_encode([-1e-9])[0] == 0x80 and O.e4m3_encode([-0.0])[0] == 0x80
    assert O.e4m3_encode([2.0 ** -10])[0] == 0x00      # tie between 0 and 2^-9 -> even (0)
    assert O.e4m3_encode([3 * 2.0 ** -10])[0] == 0x02  # tie between codes 1 and 2 -> 2


def test_scale_code_closed_form():
    for p in range(-120, 128, 7):
        for m in (1.0, 1.5, 1.9999):
            assert O.mx_block_scale_code([m * 2.0 ** p])[0] == min(max(p - 8 + 127, 0), 254)
    assert O.mx_block_scale_code([0.0])[0] == 0
    assert O.mx_block_scale_code([2.0 ** -133])[0] == 0  # clamped at the bottom code


def test_quantize_blocks_and_bound():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((6, 96)) * np.exp(rng.uniform(-8, 8, size=(6, 1)))
    a[2, 32:64] = 0.0
    q, s = O.mx_quantize(a, "cols")
    assert q.shape == (6, 96) and s.shape == (6, 3)
    assert s[2, 1] == 0 and (q[2, 32:64] == 0).all()
    deq = O.mx_dequantize(q, s, "cols")
    blocks = a.reshape(6, 3, 32)
    scale = O.e8m0_decode(s)
    y = blocks / scale[:, :, None]
    # Unsaturated elements: relative error <= 2^-4 (3 mantissa bits) or the
    # subnormal half-spacing 2^-10 in scaled units.
    err = np.abs(deq.reshape(6, 3, 32) - blocks) / scale[:, :, None]
    ok = np.abs(y) <= 448
    assert (err[ok] <= np.maximum(np.abs(y[ok]) * 2.0 ** -4, 2.0 ** -10) + 1e-300).all()
    # Saturated elements lose at most 64 scaled units (amax / scale < 512).
    assert (err[~ok] < 64).all()
    # The blocked element of largest magnitude lands in [256, 512) before saturation.
    amax = np.abs(y).max(axis=2)
    assert ((amax >= 256) & (amax < 512) | (amax == 0)).all()


def test_rows_axis_is_transpose_of_cols():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((64, 40))
    q, s = O.mx_quantize(a, "rows")
    qt, st = O.mx_quantize(a.T, "cols")
    np.testing.assert_array_equal(q, qt.T)
    np.testing.assert_array_equal(s, st.T)
    np.testing.assert_array_equal(O.mx_dequantize(q, s, "rows"), O.mx_dequantize(qt, st, "cols").T)
