"""OCP 8-bit floating point E4M3 ("E4M3FN") decoder, from the format definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The long-context page ("[Perf] Ship the qualified SM70 long-context layout...",
What and Measurement) stores the target K/V cache as E4M3 and decodes it through
a lookup table because its hardware has no FP8 unit.  The format itself is the
OCP 8-bit floating point specification (E4M3 variant): one sign bit, four
exponent bits with bias 7, three mantissa bits, no infinities, and the two
all-ones codes S.1111.111 are NaN.

    exponent field e, mantissa field f (0..7), sign s:
      e == 15 and f == 7  -> NaN
      e == 0              -> (-1)^s * f * 2^-9             (subnormal)
      otherwise           -> (-1)^s * (1 + f/8) * 2^(e-7)
"""

from __future__ import annotations

import math

import numpy as np


def _decode_one(byte: int) -> float:
    s = (byte >> 7) & 1
    e = (byte >> 3) & 0xF
    f = byte & 0x7
    if e == 0xF and f == 0x7:
        return math.nan
    if e == 0:
        mag = f * 2.0 ** -9
    else:
        mag = (1.0 + f / 8.0) * 2.0 ** (e - 7)
    return -mag if s else mag


def e4m3_table() -> np.ndarray:
    """float64 value of each of the 256 codes, indexed by the code."""
    return np.array([_decode_one(b) for b in range(256)], dtype=np.float64)


_TABLE = e4m3_table()


def e4m3_decode(codes) -> np.ndarray:
    """Decode an array of uint8 E4M3 codes to float64 (exact)."""
    c = np.asarray(codes)
    if c.dtype != np.uint8:
        raise TypeError("E4M3 codes must be uint8")
    return _TABLE[c]
