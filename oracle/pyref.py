"""Second, pure-Python statement of the reduction result, for small cases only.

TEST INFRASTRUCTURE ONLY (see the package docstring).  It pins the C oracle
with a different method: elements are decoded through Python's ``struct``
half/single formats, summed as Python floats (IEEE binary64) in rank order,
and rounded to the output type by exact rational comparison of the two
neighbouring representable values (ties to the even bit pattern), instead of
the bit-shifting in ``oracle.c``.

Definition followed: "Every Microsecond Matters" (agihunt.info summary) --
the AllReduce adds the tensor-parallel shard outputs (paragraph "Two-shot
LL128": addition only; FP32/FP16/BF16).  Order, precision and rounding are the
readings stated in ``oracle.c``.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

F32, F16, BF16 = 0, 1, 2

# (exponent bits, stored fraction bits) of each format
_FMT = {F32: (8, 23), F16: (5, 10), BF16: (8, 7)}


def decode(bits: int, dtype: int) -> float:
    """Exact value of one element via the struct module's own formats."""
    if dtype == F32:
        return struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]
    if dtype == F16:
        return struct.unpack("<e", struct.pack("<H", bits & 0xFFFF))[0]
    # bfloat16 is the upper half of a binary32 pattern
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def _layout(dtype: int):
    eb, mb = _FMT[dtype]
    inf_bits = ((1 << eb) - 1) << mb
    sign_bit = 1 << (eb + mb)
    return eb, mb, inf_bits, sign_bit


def round_to_bits(x: float, dtype: int) -> int:
    """Nearest representable element to x, ties to even, by exact comparison."""
    eb, mb, inf_bits, sign_bit = _layout(dtype)
    if math.isnan(x):
        return inf_bits | (1 << (mb - 1))
    neg = math.copysign(1.0, x) < 0
    sgn = sign_bit if neg else 0
    ax = abs(x)
    if math.isinf(ax):
        return sgn | inf_bits
    target = Fraction(ax)
    max_bits = inf_bits - 1
    # bit patterns of non-negative finite values are ordered like their values:
    # binary search the largest pattern whose value is <= |x|
    lo, hi = 0, max_bits
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if Fraction(decode(mid, dtype)) <= target:
            lo = mid
        else:
            hi = mid - 1
    below = lo
    v_below = Fraction(decode(below, dtype))
    if v_below == target:
        return sgn | below
    above = below + 1
    if above > max_bits:
        # beyond the largest finite value: the next step up is Inf, one ulp away
        ulp = Fraction(decode(max_bits, dtype)) - Fraction(decode(max_bits - 1, dtype))
        v_above = Fraction(decode(max_bits, dtype)) + ulp
    else:
        v_above = Fraction(decode(above, dtype))
    d_lo = target - v_below
    d_hi = v_above - target
    if d_lo < d_hi:
        pick = below
    elif d_hi < d_lo:
        pick = above
    else:
        pick = below if (below & 1) == 0 else above
    return sgn | pick


def allreduce(partials, dtype: int):
    """partials: list of N lists of element bit patterns.  Returns output bits."""
    n_ranks = len(partials)
    n = len(partials[0])
    out = []
    for i in range(n):
        s = decode(partials[0][i], dtype)
        for r in range(1, n_ranks):
            s = s + decode(partials[r][i], dtype)
        out.append(round_to_bits(s, dtype))
    return out
