"""Second, independent implementation of the seeded Gaussian sketch generator.
TEST INFRASTRUCTURE ONLY (imported by ``tests/`` and ``__graft_entry__.smoke()``).

The QJL sign sketch draws an m x d matrix S of iid N(0, 1) entries, rounded
to bfloat16 (D'Alberto summary, "Problem statement" and "Contribution 1": a
1-bit sketch with a Gaussian matrix; the bf16 rounding and the generator are
this implementation's reading).  The generator is a counter-based stream
written here from its published definitions, in plain Python integers and
the platform's libm (``math``), sharing nothing with the product library:

  * SplitMix64 (G. Steele, D. Lea, C. Flood, "Fast splittable pseudorandom
    number generators", OOPSLA 2014; the 64-bit finaliser with the
    multipliers 0xBF58476D1CE4E5B9 and 0x94D049BB133111EB and shifts 30, 27,
    31): the state advances by the golden-ratio increment 0x9E3779B97F4A7C15
    and each output is the finaliser of the new state.
  * a uniform in (0, 1]: the top 53 bits of an output, plus one, times 2^-53.
  * Box and Muller (1958): from uniforms u1, u2 the pair
    sqrt(-2 ln u1) cos(2 pi u2), sqrt(-2 ln u1) sin(2 pi u2) in fp64,
    consumed in row-major order (the sine of the last pair is dropped when
    m*d is odd).
  * each value rounded to fp32 (nearest even), then to bfloat16 (nearest
    even on the fp32 bit pattern).
"""
from __future__ import annotations

import math
import struct

import numpy as np

_MASK = (1 << 64) - 1
_GAMMA = 0x9E3779B97F4A7C15


def splitmix64_stream(seed: int):
    """Infinite SplitMix64 output stream from a 64-bit seed."""
    state = seed & _MASK
    while True:
        state = (state + _GAMMA) & _MASK
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
        yield z ^ (z >> 31)


def _bf16_bits_of_f32(x: float) -> int:
    """fp64 -> fp32 (nearest even) -> bfloat16 bits (nearest even)."""
    u = struct.unpack("<I", struct.pack("<f", x))[0]
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16) & 0xFFFF


def sketch_bf16_bits(seed: int, m: int, d: int) -> np.ndarray:
    """S as uint16 bfloat16 bit patterns, shape [m][d], row-major."""
    n = m * d
    out = np.zeros(n, np.uint16)
    gen = splitmix64_stream(seed)
    two_pi = 2.0 * math.pi
    i = 0
    while i < n:
        u1 = ((next(gen) >> 11) + 1) * 2.0 ** -53
        u2 = ((next(gen) >> 11) + 1) * 2.0 ** -53
        r = math.sqrt(-2.0 * math.log(u1))
        out[i] = _bf16_bits_of_f32(r * math.cos(two_pi * u2))
        if i + 1 < n:
            out[i + 1] = _bf16_bits_of_f32(r * math.sin(two_pi * u2))
        i += 2
    return out.reshape(m, d)
