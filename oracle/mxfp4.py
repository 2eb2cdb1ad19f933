"""Oracle of MXFP4 expert weights (float64).

Test infrastructure (see ``oracle/__init__.py``).

What the pages fix: the quantized deployments run the model with 4-bit
floating-point weights on hardware that supports them natively, through
NVFP4 kernels ([GN] "최적화와 실행 환경").  NVFP4 is a block-scaled E2M1 format; its gfx950 counterpart
is MXFP4 from the OCP Microscaling Formats (MX) v1.0 specification, whose
definitions this module follows:

  * an element is FP4 E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa
    bit; exponent 0 is subnormal (value m / 2); no infinities or NaN, so the
    magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6;
  * a block of 32 consecutive elements along the reduction axis shares one
    E8M0 scale: an unsigned 8-bit exponent e meaning 2^(e - 127) (255 is NaN);
  * a block's value i is scale * element_i.

Readings (R30):
  * quantization follows the specification's conversion: the shared exponent
    is floor(log2(amax)) - 2 (2 = the largest E2M1 exponent), each element is
    v / 2^shared rounded to the nearest E2M1 value, ties to the even mantissa,
    magnitudes beyond 6 saturate to 6; the sign of v is kept (so a negative
    value that rounds to zero is the code 0x8, negative zero);
  * the shared exponent is clamped to [-125, 127]: an all-zero block (or one
    whose amax is below 2^-123) uses 2^-125, so that every decoded value is a
    normal bfloat16 number or zero;
  * two elements per byte, element 2j in the low nibble of byte j;
  * the product multiplies the bf16 activations by the exact decoded weights
    (W4A16); the oracle uses exactly decode(code) * 2^(e - 127).
"""

import numpy as np

BLOCK = 32
E2M1_MAX = 6.0
SCALE_EXP_MIN = -125
SCALE_EXP_MAX = 127


def e2m1_decode(code):
    """Value of 4-bit E2M1 codes from the bit fields: sign bit 3, exponent
    bits 2..1 (bias 1), mantissa bit 0; exponent 0 is subnormal."""
    c = np.asarray(code).astype(np.int64) & 0xF
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    normal = (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)
    sub = m * 0.5
    return sign * np.where(e == 0, sub, normal)


def e8m0_decode(e):
    """2^(e - 127) for E8M0 scale bytes (255, NaN, is not used here)."""
    return np.exp2(np.asarray(e).astype(np.float64) - 127.0)


# the 8 magnitudes in code order (codes 0..7) and their mantissa bits
_MAGS = e2m1_decode(np.arange(8))


def _nearest_code(a):
    """Magnitude code (0..7) of the E2M1 value nearest to a >= 0, ties to the
    even mantissa (code bit 0 clear); beyond 6 saturates to code 7."""
    if a >= E2M1_MAX:
        return 7
    d = np.abs(_MAGS - a)
    best = d.min()
    cands = [i for i in range(8) if d[i] == best]
    if len(cands) == 1:
        return cands[0]
    even = [i for i in cands if i % 2 == 0]
    return even[0]


def quantize_block(v):
    """One block of 32 values -> (codes [32] uint8 in 0..15, scale byte)."""
    v = np.asarray(v, np.float64)
    assert v.shape == (BLOCK,)
    amax = np.abs(v).max()
    if amax > 0:
        _, ex = np.frexp(amax)                 # amax = f * 2^ex, f in [0.5, 1)
        shared = int(ex) - 1 - 2               # floor(log2 amax) - emax(E2M1)
    else:
        shared = SCALE_EXP_MIN
    shared = min(max(shared, SCALE_EXP_MIN), SCALE_EXP_MAX)
    x = np.ldexp(1.0, shared)
    codes = np.zeros(BLOCK, np.uint8)
    for i in range(BLOCK):
        mag = _nearest_code(abs(v[i]) / x)
        codes[i] = mag | (8 if np.signbit(v[i]) else 0)
    return codes, np.uint8(shared + 127)


def quantize_mxfp4(w):
    """Row-major OCP MXFP4 of w [..., K] (K % 32 == 0): returns packed codes
    [..., K / 2] uint8 (element 2j in the low nibble of byte j) and scales
    [..., K / 32] uint8 (E8M0).  The steps of ``quantize_block`` over all
    blocks at once (nearest of the 8 magnitudes by brute force)."""
    w = np.asarray(w, np.float64)
    K = w.shape[-1]
    assert K % BLOCK == 0
    blocks = w.reshape(-1, BLOCK)
    amax = np.abs(blocks).max(axis=1)
    _, ex = np.frexp(amax)
    shared = np.where(amax > 0, ex.astype(np.int64) - 1 - 2, SCALE_EXP_MIN)
    shared = np.clip(shared, SCALE_EXP_MIN, SCALE_EXP_MAX)
    a = np.abs(blocks) / np.ldexp(1.0, shared)[:, None]
    d = np.abs(a[..., None] - _MAGS)                      # [blocks, 32, 8]
    cand = d == d.min(axis=-1, keepdims=True)
    even = cand & (np.arange(8) % 2 == 0)
    mag = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    mag = np.where(a >= E2M1_MAX, 7, mag)
    codes = (mag | np.where(np.signbit(blocks), 8, 0)).astype(np.uint8).reshape(-1, K)
    packed = codes[:, 0::2] | (codes[:, 1::2] << 4)
    scales = (shared + 127).astype(np.uint8)
    return (packed.reshape(w.shape[:-1] + (K // 2,)),
            scales.reshape(w.shape[:-1] + (K // BLOCK,)))


def dequantize_mxfp4(packed, scales):
    """Exact float64 values of row-major MXFP4 codes [..., K / 2] with scales
    [..., K / 32]."""
    p = np.asarray(packed, np.uint8)
    lo = p & 0xF
    hi = p >> 4
    codes = np.stack([lo, hi], axis=-1).reshape(p.shape[:-1] + (2 * p.shape[-1],))
    vals = e2m1_decode(codes)
    sc = np.repeat(e8m0_decode(scales), BLOCK, axis=-1)
    return vals * sc
