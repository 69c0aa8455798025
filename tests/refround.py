"""Rounding and decoding references that do not use the oracle's code.

fp16 goes through Python's ``struct`` 'e' format (IEEE binary16, correctly
rounded, ties to even; values that round past the largest finite raise
OverflowError, which stands for inf).  bf16 is decoded as the top half of a
binary32 via ``struct`` and rounded by brute force: nearest of all finite
bfloat16 values, ties to the even pattern.
"""
import math
import struct
from fractions import Fraction

import numpy as np

F16 = 0
BF16 = 1


def f16_value(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", int(bits)))[0]


def bf16_value(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def value(dtype: int, bits: int) -> float:
    return f16_value(bits) if dtype == F16 else bf16_value(bits)


def f16_round_bits(x: float) -> int:
    if math.isnan(x):
        return 0x7E00
    try:
        return struct.unpack("<H", struct.pack("<e", x))[0]
    except OverflowError:
        return 0xFC00 if x < 0 else 0x7C00


# non-negative finite bf16 patterns 0x0000..0x7F7F are monotone in value
_BF16_POS_BITS = np.arange(0x7F80, dtype=np.int64)
_BF16_POS_VALS = np.array([bf16_value(b) for b in range(0x7F80)], dtype=np.float64)
_BF16_INF_AT = 2.0 ** 128  # the value the next pattern (0x7F80) would have


def bf16_round_bits(x: float) -> int:
    if math.isnan(x):
        return 0x7FC0
    sign = 0x8000 if math.copysign(1.0, x) < 0 else 0
    ax = abs(x)
    vals = _BF16_POS_VALS
    idx = int(np.searchsorted(vals, ax))
    if idx < len(vals) and vals[idx] == ax:
        return sign | idx
    lo = idx - 1
    lo_v = vals[lo]
    if idx < len(vals):
        hi, hi_v = idx, vals[idx]
    else:
        hi, hi_v = 0x7F80, _BF16_INF_AT
    dlo, dhi = ax - lo_v, hi_v - ax
    if dlo < dhi:
        pick = lo
    elif dhi < dlo:
        pick = hi
    else:
        pick = lo if lo % 2 == 0 else hi
    return sign | pick


def round_bits(dtype: int, x: float) -> int:
    return f16_round_bits(x) if dtype == F16 else bf16_round_bits(x)


def _all_finite_fracs(dtype: int):
    if dtype == F16:
        pos = [(b, Fraction(f16_value(b))) for b in range(0x7C00)]
        top = Fraction(2 ** 16)
        inf_bits = 0x7C00
    else:
        pos = [(b, Fraction(bf16_value(b))) for b in range(0x7F80)]
        top = Fraction(2 ** 128)
        inf_bits = 0x7F80
    return pos, top, inf_bits


_FRACS = {}


def round_fraction_bits(dtype: int, q: Fraction) -> int:
    """Nearest `dtype` pattern to an exact rational, ties to even (brute force)."""
    if dtype not in _FRACS:
        _FRACS[dtype] = _all_finite_fracs(dtype)
    pos, top, inf_bits = _FRACS[dtype]
    sign = 0x8000 if q < 0 else 0
    aq = abs(q)
    cands = pos + [(inf_bits, top)]
    # binary search on the monotone list
    lo, hi = 0, len(cands) - 1
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if cands[mid][1] <= aq:
            lo = mid
        else:
            hi = mid
    (bl, vl), (bh, vh) = cands[lo], cands[hi]
    if aq >= vh:
        return sign | bh
    dl, dh = aq - vl, vh - aq
    if dl < dh:
        return sign | bl
    if dh < dl:
        return sign | bh
    return sign | (bl if bl % 2 == 0 else bh)
