"""bfloat16 <-> float32, written from the definitions (oracle; test infrastructure only).

bfloat16 here is the upper half of an IEEE binary32: 1 sign bit, 8 exponent
bits, 7 stored mantissa bits.  Values travel as ``numpy.uint16`` bit patterns.

* ``widen``: a bf16 value is exactly the binary32 whose upper 16 bits are the
  bf16 pattern and whose lower 16 bits are zero.
* ``rne``: the bf16 *nearest* to the binary32 value, ties going to the
  candidate whose last stored mantissa bit is 0 (round-to-nearest-even).
  Overflow follows IEEE 754: a magnitude at or beyond the midpoint between
  the largest finite bf16 and 2**128 rounds to infinity.  Subnormals are kept,
  -0 stays -0.  Any NaN becomes the canonical quiet NaN 0x7FC0 (a reading:
  the pages fix no NaN rule; finite inputs never produce one).

The reduce in the pages' Atom layer (Purlin: Separating Orchestration from the
Datapath of Collectives, "The Purlin PDF describes a three-layer design")
produces one bf16 result per element; the decode workload fixes fp32
accumulation with a single round-to-nearest-even at the end.

Parity pinned by: torch's CPU float->bfloat16 conversion (a library
round-to-nearest-even), hand tie cases in ``tests/golden/bf16_rne_cases.txt``.
"""

import numpy as np

CANONICAL_NAN = np.uint16(0x7FC0)


def widen(b):
    """bf16 bit patterns (uint16) -> float32 values, exactly."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _bf16_value_f64(pattern_mag):
    """Magnitude of a non-negative bf16 pattern as float64; 0x7F80 -> 2**128.

    Treating the infinity pattern as 2**128 makes "nearest" reproduce the IEEE
    overflow rule: values from the midpoint (2**128 - 2**119) up round to it.
    """
    p = np.asarray(pattern_mag, dtype=np.uint32)
    v = (p << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.where(p == 0x7F80, np.float64(2.0) ** 128, v)


def rne(x):
    """float32 values -> bf16 bit patterns, round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    sign = (u >> np.uint32(16)) & np.uint32(0x8000)
    mag_bits = u & np.uint32(0x7FFFFFFF)
    is_nan = mag_bits > np.uint32(0x7F800000)
    is_inf = mag_bits == np.uint32(0x7F800000)

    # Candidates: the bf16 just below-or-equal in magnitude (drop the low 16
    # bits) and the next one up.
    lo = mag_bits >> np.uint32(16)
    hi = lo + np.uint32(1)
    with np.errstate(invalid="ignore"):  # signalling NaNs; replaced below
        xv = np.abs(x.astype(np.float64))
        d_lo = xv - _bf16_value_f64(np.minimum(lo, 0x7F80))  # exact in float64
        d_hi = _bf16_value_f64(np.minimum(hi, 0x7F80)) - xv
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & np.uint32(1)) == 1))
    mag = np.where(pick_hi, hi, lo)
    mag = np.where(is_inf, np.uint32(0x7F80), mag)
    out = (sign | mag).astype(np.uint16)
    out = np.where(is_nan, CANONICAL_NAN, out)
    return out.astype(np.uint16)


def from_f32_values(values):
    """Convenience: any float array -> float32 -> bf16 patterns via ``rne``."""
    return rne(np.asarray(values, dtype=np.float32))
