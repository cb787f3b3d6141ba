"""Pins of the oracle's MXFP4 storage (OCP Microscaling Formats v1.0, MXFP4:
FP4 E2M1 elements, one E8M0 power-of-two scale per 32 consecutive elements of
a row): the code table against the format's closed forms, the quantiser
against an independent threshold evaluation at every rounding boundary and on
random rows, the block exponent rule, exact round trips and the packing."""
import numpy as np
import pytest

import oracle
import workloads as W

MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_code_table_closed_forms():
    v = oracle.e2m1_values()
    assert v[:8].tolist() == MAGS                      # e = 0: m/2; else 2^(e-1)(1 + m/2)
    assert np.array_equal(v[8:], -v[:8]) and np.signbit(v[8])  # sign bit 3; code 8 is -0
    assert v[0b0010] == 1.0 and v[0b0111] == 6.0 and v[0b0001] == 0.5


def threshold_code(y):
    """Independent rounding of a magnitude to its E2M1 code: count the
    decision boundaries at or below y (ties go to the even code)."""
    y = np.asarray(y, np.float64)
    return ((y > 0.25).astype(int) + (y >= 0.75) + (y > 1.25) + (y >= 1.75) + (y > 2.5) + (y >= 3.5) + (y > 5.0))


def unpack(q):
    lo, hi = q & 15, q >> 4
    return np.stack([lo, hi], axis=-1).reshape(q.shape[:-1] + (q.shape[-1] * 2,))


def block_exponent(a):
    """floor(log2 a) - 2, clamped to [-127, 127]; -127 for a < 2^-126."""
    a = np.asarray(a, np.float64)
    out = np.full(a.shape, -127, np.int64)
    ok = a >= 2.0 ** -126
    out[ok] = np.clip(np.floor(np.log2(a[ok])).astype(np.int64) - 2, -127, 127)
    return out


def check_against_thresholds(x_f32):
    w = W.f32_to_bf16_bits(x_f32)
    q, s = oracle.quantize_mxfp4_rows(w)
    xv = W.bf16_bits_to_f32(w).astype(np.float64)
    blocks = xv.reshape(xv.shape[0], -1, 32)
    xexp = block_exponent(np.abs(blocks).max(axis=2))
    assert np.array_equal(s.astype(np.int64), xexp + 127)
    y = np.abs(blocks) / np.exp2(xexp)[..., None]
    codes = threshold_code(y) | np.where(np.signbit(blocks), 8, 0)
    assert np.array_equal(unpack(q).reshape(codes.shape), codes)
    return q, s


def test_every_boundary_and_one_ulp_around_it():
    # a block fixed to scale 2^0 by a 4.0 element; the rest walk the boundaries
    pts = []
    for b in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0) + tuple(MAGS[1:]):
        bits = W.f32_to_bf16_bits(np.array([b], np.float32))[0]
        for d in (-1, 0, 1):
            pts.append(W.bf16_bits_to_f32(np.array([int(bits) + d], np.uint16))[0])
    pts = np.array(pts, np.float32)
    rows = []
    for chunk in range(0, len(pts), 31):
        part = pts[chunk:chunk + 31]
        row = np.zeros(32, np.float32)
        row[0] = 4.0
        row[1:1 + len(part)] = part
        rows.append(row)
        rows.append(-row)
    check_against_thresholds(np.stack(rows))


@pytest.mark.parametrize("std", [1e-30, 0.02, 1.0, 300.0, 1e30])
def test_random_rows_match_thresholds(std):
    rng = np.random.default_rng(int(np.log10(std) + 40))
    x = (rng.standard_normal((64, 256)) * std).astype(np.float32)
    x[rng.integers(0, 64, 30), rng.integers(0, 256, 30)] *= 20.0
    x[3, :32] = 0.0                 # an all-zero block: scale byte 0, codes 0
    x[4, 32:64] = -0.0              # negative zeros keep their sign
    q, s = check_against_thresholds(x)
    assert s[3, 0] == 0 and np.all(q[3, :16] == 0)
    assert np.all(unpack(q[4:5])[0, 32:64] == 8)


def test_exact_round_trip_of_representable_blocks():
    rng = np.random.default_rng(3)
    v = oracle.e2m1_values()
    rows = []
    for x in (-127, -60, -2, 0, 5, 100):
        codes = rng.integers(0, 16, 32)
        codes[rng.integers(0, 32)] = 7  # a 6.0 in the block fixes its exponent at x
        rows.append((v[codes] * 2.0 ** x).astype(np.float32))
    w = W.f32_to_bf16_bits(np.stack(rows))
    q, s = oracle.quantize_mxfp4_rows(w)
    assert s.ravel().tolist() == [0, 67, 125, 127, 132, 227]
    assert np.array_equal(oracle.dequantize_mxfp4_rows(q, s), w)


def test_error_bound_and_saturation():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((32, 320)) * 0.02).astype(np.float32)
    w = W.f32_to_bf16_bits(x)
    q, s = oracle.quantize_mxfp4_rows(w)
    d = W.bf16_bits_to_f32(oracle.dequantize_mxfp4_rows(q, s)).astype(np.float64)
    xv = W.bf16_bits_to_f32(w).astype(np.float64)
    scale = np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=1)
    y = np.abs(xv) / scale
    inside = y <= 6.0
    # within half of the local spacing (0.25 below 2, 0.5 below 4, 1 below 6) times the scale
    half = np.where(y < 2, 0.25, np.where(y < 4, 0.5, 1.0)) * scale
    assert np.all(np.abs(d - xv)[inside] <= half[inside] + 1e-300)
    # past 6 (a block maximum in [6, 8) times the scale) the value saturates to 6
    assert np.all(np.abs(d[~inside]) == 6.0 * scale[~inside])
