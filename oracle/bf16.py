"""bfloat16 <-> float64 conversions for the oracle (test infrastructure only).

bfloat16 is the IEEE-754 binary32 format with the low 16 bits of the
significand dropped: 1 sign bit, 8 exponent bits, 7 stored significand bits
(8 significant bits for normal numbers).  The Cosmos3-H-Dreams model card
("Software Integration") states BF16 mixed precision for inference; the pages
say nothing about rounding, so the oracle uses IEEE round-to-nearest,
ties-to-even, applied once, directly from the exact fp64 value.
"""

import numpy as np


def bits_to_f64(bits):
    """Value of bf16 bit patterns (uint16) as float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bits(x):
    """Round float64 values to bf16 (round-to-nearest-even), return uint16 bits.

    The rounding is done in the fp64 domain on |x| = m * 2**e (0.5 <= m < 1):
    the bf16 quantum is 2**(e-8) for normal results and 2**-133 below
    2**-126 (bf16 subnormals).  Scaling by a power of two is exact, so
    ``rint`` (ties to even) performs exactly one rounding.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    finite = np.isfinite(ax)
    axf = np.where(finite, ax, 0.0)
    _, e = np.frexp(axf)
    qexp = np.maximum(e - 8, -133)
    n = np.rint(np.ldexp(axf, -qexp))
    y = np.ldexp(n, qexp)
    y = np.where(y >= 2.0 ** 128, np.inf, y)
    y = np.where(np.isinf(ax), np.inf, y)
    # y now holds at most 8 significant bits (or is inf): exact in binary32.
    with np.errstate(over="ignore"):
        y32 = y.astype(np.float32)
    bits = (y32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits = bits | np.where(np.signbit(x), np.uint16(0x8000), np.uint16(0)).astype(np.uint16)
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits).astype(np.uint16)
    return bits
