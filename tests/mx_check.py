"""Checks of MX quantisation decisions taken on computed values.

When the device and the oracle compute the same value (fp32 against fp64)
and then MX-quantise it, a value lying within their difference of an E4M3
rounding boundary, or a block maximum lying that close to a power of two,
can get neighbouring codes or scales on the two sides; both are correct
roundings of values the two sides may legitimately hold.  The rule applied
here: the computed values themselves are compared directly (they are
unique), every code the device chose must be the rounding (the same OCP
rule, through the oracle's own encoder) of some value within `delta` of the
oracle's value, and every GEMM that consumes the codes must equal the
oracle's exact product of those codes (see the tests).
"""
import numpy as np

import oracle as orc

_LUT = {"e4m3": np.array([orc.e4m3_value(c) for c in range(256)]),
        "e5m2": np.array([orc.e5m2_value(c) for c in range(256)])}
_ENCODE = {"e4m3": orc.e4m3_encode_array, "e5m2": orc.e5m2_encode_array}


def _scale_bytes(amax, fmt):
    return np.vectorize(lambda a: orc.mx_scale_byte(a, fmt), otypes=[np.uint8])(amax)


def check_block_decisions(v, delta, codes, scales, fmt="e4m3"):
    """v [rows, cols] fp64 (blocks of 32 along each row, a shorter last
    block padded with zeros), delta [rows, cols] >= 0, codes [rows, cols] u8
    and scales [rows, ceil(cols/32)] u8 from the device, elements of format
    fmt.  Returns (number of inadmissible scales, number of inadmissible
    codes, number of codes that differ from the oracle's own quantisation of
    v)."""
    v = np.asarray(v, dtype=np.float64)
    rows, cols = v.shape
    nb = -(-cols // 32)
    padc = nb * 32 - cols
    vb = np.pad(v, ((0, 0), (0, padc))).reshape(rows, nb, 32)
    db = np.pad(delta, ((0, 0), (0, padc))).reshape(rows, nb, 32)
    amax = np.abs(vb).max(axis=2)
    dmax = db.max(axis=2)
    lo = _scale_bytes(np.maximum(amax - dmax, 0.0), fmt)
    hi = _scale_bytes(amax + dmax, fmt)
    sc = np.asarray(scales, dtype=np.int64)[:, :nb]
    bad_s = int(((sc < lo) | (sc > hi)).sum())
    # codes at the scale the device chose: between the roundings of v - d
    # and v + d at that scale (rounding is monotone in the value)
    X = np.repeat(sc - 127, 32, axis=1)[:, :cols].astype(np.float64)
    inv = 2.0 ** (-X)
    lut = _LUT[fmt]
    c_lo = _ENCODE[fmt]((v - delta) * inv)
    c_hi = _ENCODE[fmt]((v + delta) * inv)
    got = lut[np.asarray(codes)[:, :cols]]
    bad_c = int(((got < lut[c_lo]) | (got > lut[c_hi])).sum())
    rc, _ = orc.mx_quantize_rows(v, fmt)
    differ = int((np.asarray(codes)[:, :cols] != rc).sum())
    return bad_s, bad_c, differ


def segment_columns(v, offsets, pad, width):
    """The column-wise layout of per-segment MX copies: out[c, pad[e] + j] =
    v[offsets[e] + j, c] for j < n_e, zeros elsewhere ([cols, width])."""
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros((v.shape[1], width))
    for e in range(len(offsets) - 1):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        out[:, int(pad[e]):int(pad[e]) + (r1 - r0)] = v[r0:r1].T
    return out


def dequantize(codes, scales, fmt="e4m3"):
    """Exact fp64 values of device codes and scales (blocks along rows)."""
    c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    return orc.mx_dequantize_rows(c, np.ascontiguousarray(scales[:, :-(-c.shape[1] // 32)]),
                                  fmt)
