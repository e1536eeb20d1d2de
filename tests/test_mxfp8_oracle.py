"""Pins of the MXFP8 quantisation oracle against what the OCP formats fix.

The element format is OCP 8-bit float E4M3 (OFP8 specification: bias 7, no
infinities, S.1111.111 NaN) and the block format is MXFP8 of the OCP
Microscaling (MX) specification v1.0 (32 elements, one E8M0 scale whose
exponent is floor(log2 amax) - 8).  Each test checks the oracle against a
value or property those definitions fix, computed another way: the
specification's table of special values, a brute-force nearest-value search,
exact round trips, tie cases, error bounds and the power-of-two invariance.
"""
import math

import numpy as np
import pytest

from oracle import mxfp8 as MX


def test_e4m3_special_values():
    # OFP8 E4M3 table: max normal S.1111.110 = 448, min normal S.0001.000 =
    # 2^-6, max subnormal S.0000.111 = 0.875 * 2^-6, min subnormal
    # S.0000.001 = 2^-9, S.1111.111 NaN, 1.0 = S.0111.000
    assert MX.e4m3_value(0x7E) == 448.0
    assert MX.e4m3_value(0xFE) == -448.0
    assert MX.e4m3_value(0x08) == 2.0 ** -6
    assert MX.e4m3_value(0x07) == 0.875 * 2.0 ** -6
    assert MX.e4m3_value(0x01) == 2.0 ** -9
    assert MX.e4m3_value(0x38) == 1.0
    assert MX.e4m3_value(0xB8) == -1.0
    assert math.isnan(MX.e4m3_value(0x7F)) and math.isnan(MX.e4m3_value(0xFF))
    assert MX.e4m3_value(0x00) == 0.0 and MX.e4m3_value(0x80) == 0.0
    # 0x78 = 2^8, 0x77 = 1.875 * 2^7: every exponent field 1..15 is normal
    assert MX.e4m3_value(0x78) == 256.0 and MX.e4m3_value(0x77) == 240.0


def _brute_nearest(y):
    """Nearest finite E4M3 code by scanning all 256 codes (ties: even code),
    saturating at 448."""
    best = None
    for c in range(256):
        v = MX.e4m3_value(c)
        if math.isnan(v) or (c & 0x80) != (0x80 if y < 0 else 0):
            continue
        key = (abs(v - y), c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    code = best[1]
    if abs(y) >= 448.0:
        code = 0x7E | (0x80 if y < 0 else 0)
    return code


def test_encode_matches_brute_force():
    g = np.random.default_rng(5)
    ys = np.concatenate([g.normal(0, 50, 400), g.normal(0, 0.01, 200), g.uniform(-520, 520, 200),
                         np.ldexp(g.uniform(-1, 1, 100), g.integers(-12, 9, 100))])
    got = MX.e4m3_encode(ys)
    want = np.array([_brute_nearest(float(y)) for y in ys], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_representable_values_round_trip():
    # blocks of 448 (which fixes the shared exponent at 0) and representable values
    vals = np.array([MX.e4m3_value(c) for c in range(1, 0x7F)])
    vals = np.concatenate([vals, -vals])
    g = np.random.default_rng(6)
    g.shuffle(vals)
    n = len(vals) // 31
    blocks = np.concatenate([np.full((n, 1), 448.0), vals[: n * 31].reshape(n, 31)], axis=1)
    codes, scales = MX.quantize(blocks)
    assert np.all(scales == 127)
    assert np.array_equal(MX.dequantize(codes, scales), blocks)


def test_ties_go_to_even_code():
    block = np.zeros(32)
    # 1.0625 is halfway between 1.0 (0x38) and 1.125 (0x39); 1.1875 between
    # 0x39 and 1.25 (0x3A); 2^-10 between 0 and 2^-9 (0x01); 1.5 * 2^-9
    # between 0x01 and 0x02
    block[:6] = [448.0, 1.0625, 1.1875, 2.0 ** -10, 1.5 * 2.0 ** -9, -1.0625]
    codes, scales = MX.quantize(block[None])
    assert scales[0, 0] == 127
    assert list(codes[0, :6]) == [0x7E, 0x38, 0x3A, 0x00, 0x02, 0xB8]


def test_shared_scale_codes():
    def scale_of(amax):
        b = np.zeros((1, 32))
        b[0, 3] = amax
        return int(MX.quantize(b)[1][0, 0])
    assert scale_of(1.0) == 127 - 8            # floor(log2 1) - 8 = -8
    assert scale_of(3.0) == 127 - 7            # floor(log2 3) = 1
    assert scale_of(448.0) == 127              # 448 = 1.75 * 2^8
    assert scale_of(-0.75) == 127 - 9          # sign does not matter
    assert scale_of(1.5 * 2.0 ** 127) == 127 + 119
    assert scale_of(2.0 ** -130) == 0          # clamped to 2^-127
    codes, scales = MX.quantize(np.zeros((2, 64)))
    assert np.all(scales == 0) and np.all(codes == 0)


def test_saturation():
    # amax = 1.99 * 2^8: shared exponent 0, the element 509.4 is above 448
    block = np.zeros((1, 32))
    block[0, 0] = 1.99 * 256
    block[0, 1] = -1.99 * 256
    codes, scales = MX.quantize(block)
    assert scales[0, 0] == 127
    assert codes[0, 0] == 0x7E and codes[0, 1] == 0xFE


def test_error_bound():
    g = np.random.default_rng(7)
    x = g.normal(0, 1, (64, 128)) * np.exp(g.normal(0, 2, (64, 1)))
    codes, scales = MX.quantize(x)
    deq = MX.dequantize(codes, scales)
    X = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=1)
    y = np.abs(x) / X
    err = np.abs(deq - x)
    normal = (y >= 2.0 ** -6) & (y < 448)
    # half an ulp: 2^-4 relative in the normal range, 2^-10 X below it
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-12))
    assert np.all(err[y < 2.0 ** -6] <= 2.0 ** -10 * X[y < 2.0 ** -6] * (1 + 1e-12))
    assert np.all(np.abs(deq[y >= 448]) == 448 * X[y >= 448])


def test_power_of_two_invariance():
    g = np.random.default_rng(8)
    x = g.normal(0, 1, (16, 64))
    c0, s0 = MX.quantize(x)
    for k in (-20, -3, 5, 40):
        ck, sk = MX.quantize(np.ldexp(x, k))
        assert np.array_equal(ck, c0)
        assert np.array_equal(sk.astype(int), s0.astype(int) + k)


@pytest.mark.parametrize("d", [32, 128])
def test_quantize_layout(d):
    # block b of a row covers columns 32 b .. 32 b + 31: scaling one block
    # changes that block's scale only
    g = np.random.default_rng(9)
    x = g.normal(0, 1, (3, d))
    c0, s0 = MX.quantize(x)
    x2 = x.copy()
    x2[1, 32 * (d // 32 - 1):] *= 16.0
    c2, s2 = MX.quantize(x2)
    assert np.array_equal(c2, c0)
    diff = s2.astype(int) - s0.astype(int)
    assert diff[1, -1] == 4 and np.count_nonzero(diff) == 1
