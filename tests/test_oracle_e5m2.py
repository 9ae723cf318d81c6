"""Pins of the oracle's E5M2 gradient option (CPU only).

The element format is the OCP FP8 E5M2 (bias 15, two mantissa bits,
infinities and NaNs in exponent field 31, largest finite 57344); the MX
shared exponent for it is X = floor(log2 amax) - 15.  Pinned here against
torch's float8_e5m2 (decode of all 256 codes, round-to-nearest-even encode in
range), hand values, the scale rule, exact round trips on the grid, and, for
every backward GEMM of the MXFP8 step, operands on the E5M2 grid along that
GEMM's K: with grad_fmt="e5m2" the quantised result equals the unquantised
one, with "e4m3" (the wrong format for those operands) it does not, and the
non-gradient operand keeps E4M3 (a weight on the E5M2 grid but not on the
E4M3 grid is still changed).
"""
import numpy as np
import torch

import oracle as orc

rng = np.random.default_rng(2024)


def test_e5m2_decode_matches_torch_float8_e5m2():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e5m2).to(torch.float64).numpy()
    ours = np.array([orc.e5m2_value(c) for c in range(256)])
    nan = np.isnan(lib)
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], lib[~nan])


def test_e5m2_encode_matches_torch_rne_in_range():
    v = np.concatenate([rng.standard_normal(4000) * 3000,
                        rng.standard_normal(2000) * 1e-3,
                        rng.standard_normal(2000) * 1e-5,
                        np.linspace(-57344, 57344, 3001)])
    v = v[np.abs(v) <= 57344].astype(np.float32)
    lib = torch.from_numpy(v).to(torch.float8_e5m2).view(torch.uint8).numpy()
    ours = orc.e5m2_encode_array(v.astype(np.float64))
    np.testing.assert_array_equal(ours, lib)


def test_e5m2_hand_values_and_saturation():
    assert orc.e5m2_encode(1.0) == 0x3C
    assert orc.e5m2_encode(57344.0) == 0x7B
    assert orc.e5m2_encode(1e9) == 0x7B and orc.e5m2_encode(-1e9) == 0xFB
    assert orc.e5m2_encode(2.0 ** -16) == 0x01        # smallest subnormal
    assert orc.e5m2_encode(2.0 ** -17) == 0x00        # tie -> even (0)
    assert orc.e5m2_encode(1.125) == 0x3C             # tie -> even (1.0)
    assert orc.e5m2_encode(1.375) == 0x3E             # tie -> even (1.5)
    assert orc.e5m2_encode(-0.0) == 0x80
    assert orc.e5m2_value(0x7C) == np.inf and np.isnan(orc.e5m2_value(0x7D))


def test_mx_scale_rule_e5m2():
    assert orc.mx_scale_byte(0.0, "e5m2") == 0
    assert orc.mx_scale_byte(1.0, "e5m2") == 127 - 15
    assert orc.mx_scale_byte(57344.0, "e5m2") == 127
    assert orc.mx_scale_byte(65535.0, "e5m2") == 127
    assert orc.mx_scale_byte(65536.0, "e5m2") == 128
    assert orc.mx_scale_byte(2.0 ** -120, "e5m2") == 0     # clamped at -127
    # the two formats differ by their largest normal exponents (15 - 8)
    for a in (0.3, 1.0, 7.5, 1000.0):
        assert orc.mx_scale_byte(a, "e4m3") - orc.mx_scale_byte(a, "e5m2") == 7


def test_mx_quantize_e5m2_nearest_and_range():
    v = rng.standard_normal((5, 70)) * np.exp(3 * rng.standard_normal((5, 70)))
    c, s = orc.mx_quantize_rows(v, "e5m2")
    table = np.array([orc.e5m2_value(q) for q in range(0x7C)])
    for r in range(5):
        for j in range(70):
            sc = 2.0 ** (int(s[r, j // 32]) - 127)
            a = abs(v[r, j]) / sc
            best = np.min(np.abs(table - a))
            assert abs(orc.e5m2_value(c[r, j] & 0x7F) - a) == best
        for b in range(3):
            blk = np.abs(v[r, 32 * b:32 * b + 32]).max()
            assert 2.0 ** 15 <= blk / 2.0 ** (int(s[r, b]) - 127) < 2.0 ** 16
    deq = orc.mx_dequantize_rows(c, s, "e5m2")
    np.testing.assert_array_equal(deq, orc.mx_roundtrip_rows(v, "e5m2"))


# Matrices on the E5M2 grid along each row: values sign * m * 2^j with
# m in {4, 5, 6, 7} and j spanning 29 binades below each block's maximum
# 7 * 2^jmax (set in the block's first column).  Block scale X = jmax - 13,
# so the scaled values are m * 2^(j - jmax + 13) in [2^-13, 57344], all on
# the E5M2 grid.  E4M3 (range 2^-9 .. 448 after its own scale) flushes or
# rounds the small ones, so the two formats give different results.


def _grid5_rows(M, K, g):
    jmax = g.integers(-6, 7, M)[:, None]
    j = jmax - g.integers(0, 29, (M, K))
    m = g.integers(4, 8, (M, K)).astype(np.float64)
    sgn = g.choice([-1.0, 1.0], (M, K))
    v = sgn * m * 2.0 ** j
    for b in range(0, K, 32):
        v[:, b] = g.choice([-1.0, 1.0], M) * 7.0 * 2.0 ** jmax[:, 0]
    return v


def _grid5_segment_rows(offs, N, g):
    out = np.zeros((int(offs[-1]), N))
    for e in range(len(offs) - 1):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        if r1 > r0:
            out[r0:r1] = _grid5_rows(N, r1 - r0, g).T
    return out


def _grid4_rows(M, K, g):
    """On the E4M3 grid along each row (integers up to 14 times a per-row
    power of two, one 8..14 per block)."""
    ints = g.integers(-14, 15, (M, K)).astype(np.float64)
    for b in range(0, K, 32):
        ints[:, b] = g.choice([-1.0, 1.0], M) * g.integers(8, 15, M)
    return ints * (2.0 ** g.integers(-6, 7, M))[:, None]


def test_grid5_is_exact_in_e5m2_and_not_in_e4m3():
    g = np.random.default_rng(50)
    A = _grid5_rows(8, 96, g)
    np.testing.assert_array_equal(orc.mx_roundtrip_rows(A, "e5m2"), A)
    assert not np.array_equal(orc.mx_roundtrip_rows(A, "e4m3"), A)


OFFS = np.array([0, 40, 40, 100])


def test_backward_down_da_uses_grad_format_for_dy_only():
    g = np.random.default_rng(51)
    n, H, I = 3, 64, 96
    R = OFFS[-1]
    dy = _grid5_rows(R, H, g)                                   # along H
    wd = np.stack([_grid4_rows(I, H, g).T for _ in range(n)])   # [n, H, I], along H
    gg = g.standard_normal((R, I)); uu = g.standard_normal((R, I)); s = g.random(R)
    p = orc.mxfp8_backward_down(dy, gg, uu, s, OFFS, wd, quantize=False)
    q5 = orc.mxfp8_backward_down(dy, gg, uu, s, OFFS, wd, grad_fmt="e5m2")
    q4 = orc.mxfp8_backward_down(dy, gg, uu, s, OFFS, wd, grad_fmt="e4m3")
    for k in ("da", "dg", "du", "ds"):
        np.testing.assert_array_equal(q5[k], p[k])
    assert not np.allclose(q4["da"], p["da"], rtol=1e-6, atol=0)
    # W_d on the E5M2 grid but not on E4M3's: it is quantised as E4M3
    wd5 = np.stack([_grid5_rows(I, H, g).T for _ in range(n)])
    p2 = orc.mxfp8_backward_down(dy, gg, uu, s, OFFS, wd5, quantize=False)
    q2 = orc.mxfp8_backward_down(dy, gg, uu, s, OFFS, wd5, grad_fmt="e5m2")
    assert not np.allclose(q2["da"], p2["da"], rtol=1e-6, atol=0)


def test_backward_down_dw_down_uses_grad_format_for_dy_only():
    g = np.random.default_rng(52)
    n, H, I = 3, 64, 96
    R = OFFS[-1]
    dy = _grid5_segment_rows(OFFS, H, g)                        # down segments
    uu = np.zeros((R, I))
    for e in range(n):                                          # a = 32 u on E4M3's grid
        r0, r1 = OFFS[e], OFFS[e + 1]
        if r1 > r0:
            uu[r0:r1] = _grid4_rows(I, r1 - r0, g).T
    gg = np.full((R, I), 64.0); s = np.full(R, 0.5)
    wd = g.standard_normal((n, H, I))
    p = orc.mxfp8_backward_down(dy, gg, uu, s, OFFS, wd, quantize=False)
    q5 = orc.mxfp8_backward_down(dy, gg, uu, s, OFFS, wd, grad_fmt="e5m2")
    q4 = orc.mxfp8_backward_down(dy, gg, uu, s, OFFS, wd, grad_fmt="e4m3")
    np.testing.assert_array_equal(q5["dw_down"], p["dw_down"])
    assert not np.allclose(q4["dw_down"], p["dw_down"], rtol=1e-6, atol=0)


def test_backward_gate_up_uses_grad_format_for_dg_du_only():
    g = np.random.default_rng(53)
    n, H, I = 3, 64, 96
    R = OFFS[-1]
    dg, du = _grid5_rows(R, I, g), _grid5_rows(R, I, g)         # along I
    wg = np.stack([_grid4_rows(H, I, g).T for _ in range(n)])   # [n, I, H], along I
    wu = np.stack([_grid4_rows(H, I, g).T for _ in range(n)])
    x = g.standard_normal((R, H))
    p = orc.mxfp8_backward_gate_up(dg, du, x, OFFS, wg, wu, quantize=False)
    q5 = orc.mxfp8_backward_gate_up(dg, du, x, OFFS, wg, wu, grad_fmt="e5m2")
    q4 = orc.mxfp8_backward_gate_up(dg, du, x, OFFS, wg, wu, grad_fmt="e4m3")
    np.testing.assert_array_equal(q5["dx"], p["dx"])
    assert not np.allclose(q4["dx"], p["dx"], rtol=1e-6, atol=0)
    # weight gradients: dg, du on the E5M2 grid and x on E4M3's, down segments
    dg, du = _grid5_segment_rows(OFFS, I, g), _grid5_segment_rows(OFFS, I, g)
    x = np.zeros((R, H))
    for e in range(n):
        r0, r1 = OFFS[e], OFFS[e + 1]
        if r1 > r0:
            x[r0:r1] = _grid4_rows(H, r1 - r0, g).T
    p = orc.mxfp8_backward_gate_up(dg, du, x, OFFS, wg, wu, quantize=False)
    q5 = orc.mxfp8_backward_gate_up(dg, du, x, OFFS, wg, wu, grad_fmt="e5m2")
    q4 = orc.mxfp8_backward_gate_up(dg, du, x, OFFS, wg, wu, grad_fmt="e4m3")
    for k in ("dw_gate", "dw_up"):
        np.testing.assert_array_equal(q5[k], p[k])
        assert not np.allclose(q4[k], p[k], rtol=1e-6, atol=0)
    # x on the E5M2 grid only: it stays E4M3, so dW_g changes
    x5 = _grid5_segment_rows(OFFS, H, g)
    p3 = orc.mxfp8_backward_gate_up(dg, du, x5, OFFS, wg, wu, quantize=False)
    q3 = orc.mxfp8_backward_gate_up(dg, du, x5, OFFS, wg, wu, grad_fmt="e5m2")
    assert not np.allclose(q3["dw_gate"], p3["dw_gate"], rtol=1e-6, atol=0)


def test_step_grad_format_leaves_the_forward_alone():
    g = np.random.default_rng(54)
    R, H, I, n = 70, 64, 96, 3
    x = g.standard_normal((R, H)); dy = g.standard_normal((R, H))
    wg = g.standard_normal((n, I, H)) * 0.2; wu = g.standard_normal((n, I, H)) * 0.2
    wd = g.standard_normal((n, H, I)) * 0.2; s = g.random(R)
    offs = np.array([0, 30, 30, R])
    a = orc.mxfp8_mlp_step(x, offs, s, wg, wu, wd, dy)
    b = orc.mxfp8_mlp_step(x, offs, s, wg, wu, wd, dy, grad_fmt="e5m2")
    for k in ("g", "u", "a", "y"):
        np.testing.assert_array_equal(a[k], b[k])
    assert not np.array_equal(a["dx"], b["dx"])
    # both are the same chain rule: near the unquantised gradients (a sanity
    # bound on the whole tensor, about 9-11% here for both formats)
    p = orc.mxfp8_mlp_step(x, offs, s, wg, wu, wd, dy, quantize=False)
    for k in ("dx", "dw_gate", "dw_up", "dw_down"):
        for q in (a, b):
            rel = np.linalg.norm(q[k] - p[k]) / np.linalg.norm(p[k])
            assert rel < 0.15, (k, rel)
