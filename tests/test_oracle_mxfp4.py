"""Pins of the MXFP4 oracle (OCP Microscaling v1.0 definitions; reading R30)
against things other than itself: torch's decoders of two other formats built
from the same bit-field definitions, worked round-to-nearest-even cases,
brute-force nearest-value search, exact round trips and the error bound."""

import math

import numpy as np
import torch

from oracle.mxfp4 import (e2m1_decode, e8m0_decode, quantize_block, quantize_mxfp4,
                          dequantize_mxfp4, BLOCK)


def _e2m1_as_e4m3_byte(c):
    """The OCP e4m3fn byte with the value of E2M1 code c: a normal E2M1
    (exponent e >= 1, bias 1) has e4m3 exponent e - 1 + 7 and mantissa m << 2;
    the subnormal 0.5 is 2^-1 (exponent 6), zero is zero."""
    s, e, m = (c >> 3) & 1, (c >> 1) & 3, c & 1
    if e == 0:
        body = 0 if m == 0 else (6 << 3)
    else:
        body = ((e + 6) << 3) | (m << 2)
    return (s << 7) | body


def test_e2m1_decode_matches_torch_e4m3_decoder():
    codes = np.arange(16)
    as_e4m3 = torch.tensor([_e2m1_as_e4m3_byte(int(c)) for c in codes], dtype=torch.uint8)
    lib = as_e4m3.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(e2m1_decode(codes), lib)
    mags = e2m1_decode(np.arange(8))
    assert np.all(np.diff(mags) > 0)                      # codes 0..7 increase
    assert np.array_equal(e2m1_decode(np.arange(8, 16)), -mags)


def test_e8m0_decode_matches_torch():
    e = np.arange(1, 255)
    lib = torch.from_numpy(e.astype(np.uint8)).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    assert np.array_equal(e8m0_decode(e), lib)


def test_quantize_worked_ties_and_saturation():
    # amax 7 -> floor(log2 7) - 2 = 0: scale 1, so each value is its own
    # element; expected codes from round-to-nearest-even on the E2M1 grid
    vals = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0, -0.2, 0.3, -3.0, 6.0, 0.0, -0.0,
            1.0, 0.5]
    want = [0x0, 0x2, 0x2, 0x4, 0x4, 0x6, 0x6, 0x7, 0x8, 0x1, 0xD, 0x7, 0x0, 0x8, 0x2, 0x1]
    v = np.zeros(BLOCK)
    v[:len(vals)] = vals
    codes, scale = quantize_block(v)
    assert int(scale) == 127
    assert list(codes[:len(vals)]) == want
    assert np.all(codes[len(vals):] == 0)


def test_quantize_scale_exponent_and_clamp():
    rng = np.random.default_rng(3)
    for amax_exp in (-30, -7, -1, 0, 3, 40):
        v = rng.uniform(-1, 1, BLOCK) * 2.0 ** amax_exp
        _, scale = quantize_block(v)
        amax = np.abs(v).max()
        assert int(scale) - 127 == math.floor(math.log2(amax)) - 2
    _, scale = quantize_block(np.zeros(BLOCK))
    assert int(scale) == 2                                # 2^-125
    _, scale = quantize_block(np.full(BLOCK, 2.0 ** -140))
    assert int(scale) == 2


def test_quantize_is_nearest_by_brute_force():
    rng = np.random.default_rng(11)
    w = rng.standard_normal((40, 4 * BLOCK)) * np.exp2(rng.integers(-12, 4, (40, 1)))
    packed, scales = quantize_mxfp4(w)
    dq = dequantize_mxfp4(packed, scales)
    grid = e2m1_decode(np.arange(16))
    for r in range(w.shape[0]):
        for b in range(w.shape[1] // BLOCK):
            x = e8m0_decode(scales[r, b])
            for i in range(b * BLOCK, (b + 1) * BLOCK):
                best = np.abs(grid * x - w[r, i]).min()
                assert abs(dq[r, i] - w[r, i]) == best


def test_quantize_error_bound():
    rng = np.random.default_rng(5)
    w = rng.standard_normal((64, 8 * BLOCK)) * 0.02
    packed, scales = quantize_mxfp4(w)
    err = np.abs(dequantize_mxfp4(packed, scales) - w)
    x = np.repeat(e8m0_decode(scales), BLOCK, axis=-1)
    a = np.abs(w) / x
    assert np.all(a < 8)                                  # amax / scale in [4, 8)
    assert np.all(err[a < 2] <= 0.25 * x[a < 2])          # half the 0.5 spacing
    assert np.all(err[(a >= 2) & (a < 4)] <= 0.5 * x[(a >= 2) & (a < 4)])
    assert np.all(err[a >= 4] <= 2.0 * x[a >= 4])         # spacing 2, then saturation


def test_quantize_round_trip_is_identity():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 16, (50, BLOCK)).astype(np.uint8)
    codes[:, 0] = rng.choice([6, 7, 14, 15], 50)          # the block max is 4 or 6
    scales = rng.integers(10, 240, (50, 1)).astype(np.uint8)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    v = dequantize_mxfp4(packed, scales)
    p2, s2 = quantize_mxfp4(v)
    assert np.array_equal(s2, scales)
    # negative zero survives only through its sign: compare values and signs
    assert np.array_equal(dequantize_mxfp4(p2, s2), v)
    assert np.array_equal(p2, packed)


def test_nibble_order_and_vectorized_form():
    v = np.zeros(BLOCK)
    v[0], v[1] = 1.0, -6.0                                # scale 1 after amax 6
    packed, scales = quantize_mxfp4(v[None])
    assert packed[0, 0] == (0x2 | (0xF << 4))             # element 0 in the low nibble
    rng = np.random.default_rng(2)
    w = rng.standard_normal((12, 3 * BLOCK)) * 0.05
    packed, scales = quantize_mxfp4(w)
    for r in range(12):
        for b in range(3):
            c, s = quantize_block(w[r, b * BLOCK:(b + 1) * BLOCK])
            assert s == scales[r, b]
            assert np.array_equal(c[0::2] | (c[1::2] << 4), packed[r, b * 16:(b + 1) * 16])
