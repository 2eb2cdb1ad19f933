"""Philox4x32-10 counter-based generator and the draws the sampler takes from it.

Test infrastructure (see ``oracle/__init__.py``): used only by tests, smoke and
the bench's CPU-baseline leg.

The pages fix neither a generator nor a seeding scheme; they only say that the
canvas starts from random placeholder tokens ([GN] "텍스트 확산의 작동 방식";
[GUIDE] "Uniform State Diffusion") and that unconfident tokens are
re-randomized ([GUIDE] "Uniform State Diffusion").  Reading R11: every random
number is one 32-bit word of Philox4x32-10 as published by Salmon, Moraes,
Dror and Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11):

  * one round maps the counter (c0, c1, c2, c3) under key (k0, k1) to
        (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))
    with M0 = 0xD2511F53, M1 = 0xCD9E8D57;
  * ten rounds; between rounds the key advances by the Weyl constants
    (0x9E3779B9, 0xBB67AE85);
  * key = (seed mod 2^32, seed >> 32).

Counter layout (R11): (word, absolute position, step, (stream << 24) | row).
Streams: 0 = Gumbel noise (word = v >> 2, output lane v & 3),
1 = re-noise id (word 0, lane 0), 2 = initial canvas id (word 0, lane 0,
step field 0).

Derived draws:
  * uniform24(w) = ((w >> 8) + 1/2) * 2^-24, exact in float32 and float64;
  * Gumbel g = -ln(-ln u);
  * uniform id (R12) = floor(w * V / 2^32) by a 64-bit product.
"""

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

STREAM_GUMBEL = 0
STREAM_RENOISE = 1
STREAM_CANVAS = 2


def philox4x32_10(c0, c1, c2, c3, seed):
    """Return the four 32-bit output words (uint32 arrays) for the given
    counters (broadcastable integer arrays) under key derived from ``seed``."""
    c0, c1, c2, c3 = np.broadcast_arrays(
        *[np.asarray(c, dtype=np.uint64) & _MASK for c in (c0, c1, c2, c3)])
    seed = int(seed)
    k0 = seed & 0xFFFFFFFF
    k1 = (seed >> 32) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + W0) & 0xFFFFFFFF
            k1 = (k1 + W1) & 0xFFFFFFFF
        p0 = M0 * c0            # < 2^64: exact in uint64
        p1 = M1 * c2
        hi0, lo0 = p0 >> _S32, p0 & _MASK
        hi1, lo1 = p1 >> _S32, p1 & _MASK
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(k0), lo1,
                          hi0 ^ c3 ^ np.uint64(k1), lo0)
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))


def stream_word(stream, row):
    """The fourth counter word: (stream << 24) | row."""
    return (int(stream) << 24) | int(row)


def uniform24(w):
    """u = ((w >> 8) + 0.5) * 2^-24 in (0, 1); exact in float64."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w >> np.uint64(8)).astype(np.float64) + 0.5) * (2.0 ** -24)


def gumbel_from_word(w):
    """Standard Gumbel draw from one 32-bit word: g = -ln(-ln u)."""
    u = uniform24(w)
    return -np.log(-np.log(u))


def uniform_id(w, V):
    """Uniform integer in [0, V): floor(w * V / 2^32) (R12)."""
    w = np.asarray(w, dtype=np.uint64)
    return ((w * np.uint64(V)) >> _S32).astype(np.int64)


def gumbel_row(seed, pos, step, row, V):
    """Gumbel noise g[v], v in [0, V), for one canvas position (stream 0)."""
    words = np.arange((V + 3) // 4, dtype=np.uint64)
    out = philox4x32_10(words, pos, step, stream_word(STREAM_GUMBEL, row), seed)
    w = np.stack(out, axis=-1).reshape(-1)[:V]   # lane v & 3 of word v >> 2
    return gumbel_from_word(w)


def renoise_id(seed, pos, step, row, V):
    """Re-noise token id for one position at one step (stream 1)."""
    w = philox4x32_10(0, pos, step, stream_word(STREAM_RENOISE, row), seed)[0]
    return int(uniform_id(w, V))


def canvas_id(seed, pos, row, V):
    """Initial canvas token id at absolute position ``pos`` (stream 2)."""
    w = philox4x32_10(0, pos, 0, stream_word(STREAM_CANVAS, row), seed)[0]
    return int(uniform_id(w, V))
