"""Pins of the MX decision checker (tests/mx_check.py) on hand-made codes:
the oracle's own codes are admissible, a code one step off is admissible
only when the value lies within delta of the rounding boundary, and a scale
one step off only when the block maximum lies within delta of the power of
two where the scale changes."""
import numpy as np

import oracle as orc
from mx_check import check_block_decisions, dequantize, segment_columns


def test_oracle_codes_are_admissible_and_far_flips_are_not():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((6, 96))
    c, s = orc.mx_quantize_rows(v)
    assert check_block_decisions(v, np.zeros_like(v), c, s) == (0, 0, 0)
    np.testing.assert_array_equal(dequantize(c, s), orc.mx_roundtrip_rows(v))
    c2 = c.copy()
    c2[2, 5] ^= 0x04                         # a different mantissa, far away
    bs, bc, differ = check_block_decisions(v, np.full_like(v, 1e-6), c2, s)
    assert (bs, bc, differ) == (0, 1, 1)


def test_e5m2_codes_are_checked_in_their_own_format():
    rng = np.random.default_rng(4)
    v = rng.standard_normal((6, 96)) * np.exp(2 * rng.standard_normal((6, 96)))
    c, s = orc.mx_quantize_rows(v, "e5m2")
    assert check_block_decisions(v, np.zeros_like(v), c, s, "e5m2") == (0, 0, 0)
    np.testing.assert_array_equal(dequantize(c, s, "e5m2"), orc.mx_roundtrip_rows(v, "e5m2"))
    # the same bytes read as E4M3 are inadmissible (scales and codes differ)
    bs, bc, _ = check_block_decisions(v, np.zeros_like(v), c, s, "e4m3")
    assert bs > 0 and bc > 0
    c2 = c.copy()
    c2[1, 7] ^= 0x08                         # another exponent, far away
    assert check_block_decisions(v, np.full_like(v, 1e-9), c2, s, "e5m2")[1] == 1


def test_neighbouring_code_near_a_tie_needs_delta():
    # one block: 448 fixes the scale (X = 0 for amax in [256, 512)), and
    # 9.5 + eps lies just above the tie between codes for 9 and 10
    v = np.zeros((1, 32))
    v[0, 0] = 448.0
    v[0, 1] = 9.5 + 1e-9
    c, s = orc.mx_quantize_rows(v)
    assert orc.e4m3_value(int(c[0, 1])) == 10.0
    alt = c.copy()
    alt[0, 1] = orc.e4m3_encode(9.0)
    assert check_block_decisions(v, np.zeros_like(v), alt, s)[1] == 1
    d = np.zeros_like(v); d[0, 1] = 1e-6
    assert check_block_decisions(v, d, alt, s)[:2] == (0, 0)


def test_neighbouring_scale_near_a_power_of_two_needs_delta():
    v = np.zeros((1, 32))
    v[0, 0] = 512.0 - 1e-7                   # X = 0; 512 would give X = 1
    v[0, 1] = 3.0
    c, s = orc.mx_quantize_rows(v)
    assert s[0, 0] == 127
    c1, s1 = orc.mx_quantize_rows(np.where(v == v[0, 0], 512.0, v))
    assert s1[0, 0] == 128
    assert check_block_decisions(v, np.zeros_like(v), c1, s1)[0] == 1
    assert check_block_decisions(v, np.full_like(v, 1e-6), c1, s1)[:2] == (0, 0)


def test_segment_columns_layout():
    v = np.arange(12, dtype=np.float64).reshape(6, 2)
    out = segment_columns(v, [0, 2, 2, 6], [0, 32, 32, 64], 64)
    assert out.shape == (2, 64)
    np.testing.assert_array_equal(out[:, :2], v[:2].T)
    np.testing.assert_array_equal(out[:, 32:36], v[2:6].T)
    assert not out[:, 2:32].any() and not out[:, 36:].any()
