"""Exact-rational mini-oracle for tiny inputs (TEST INFRASTRUCTURE ONLY).

An independent re-derivation of the coding rules with ``fractions.Fraction``:
every binary32/binary16 rounding is done by an explicit rational rounding
routine, and every code is chosen by brute force over all 16 levels (nearest
level, ties to the lower NF4 index / to the even integer level), instead of the
C oracle's closed forms (binary64 distances, rint + clamp).  Agreement of the
two on small inputs pins the C oracle's divisions, roundings and tie rules.

Sources: "What is 4-bit quantization and why does it matter?" ("How 4-bit
quantization works": INT4-sym levels and scale, the NF4 table), "INT4" ("How it
works", "Components": asymmetric levels and integer zero-point), "Loading a
model in 4-bit" ("Block-wise quantisation, stated exactly": nearest of 16
codebook entries after dividing by the block absmax).
"""

from __future__ import annotations

from fractions import Fraction as Fr

# The printed table, as decimal strings; each entry is taken as the nearest
# binary32 value (rounded exactly below).
NF4_DECIMALS = ["-1.0", "-0.696", "-0.525", "-0.395", "-0.284", "-0.185", "-0.091", "0.0",
                "0.079", "0.161", "0.246", "0.338", "0.441", "0.562", "0.720", "1.0"]


def round_binary(v: Fr, p: int, emin: int) -> Fr:
    """Round rational v to the nearest value with a p-bit significand and
    smallest normal exponent emin (gradual underflow), ties to even."""
    if v == 0:
        return Fr(0)
    sgn = -1 if v < 0 else 1
    a = abs(v)
    # exponent of the leading bit: 2^E <= a < 2^(E+1)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fr(2) ** E > a:
        E -= 1
    elif Fr(2) ** (E + 1) <= a:
        E += 1
    E = max(E, emin)
    quantum = Fr(2) ** (E - (p - 1))
    t = a / quantum
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fr(1, 2) or (rem == Fr(1, 2) and n % 2 == 1):
        n += 1
    return sgn * n * quantum


def rn32(v: Fr) -> Fr:
    return round_binary(v, 24, -126)


def rn16(v: Fr) -> Fr:
    """binary16 rounding (no overflow handling: callers stay below 65504)."""
    r = round_binary(v, 11, -14)
    assert abs(r) <= 65504
    return r


def f16_value(bits: int) -> Fr:
    sign = -1 if bits & 0x8000 else 1
    ex = (bits >> 10) & 0x1F
    man = bits & 0x3FF
    assert ex != 31, "finite values only"
    if ex == 0:
        return sign * Fr(man, 1 << 24)
    return sign * Fr(1024 + man, 1 << 10) * Fr(2) ** (ex - 15)


NF4_TABLE = [rn32(Fr(d)) for d in NF4_DECIMALS]


def nf4_nearest(x: Fr) -> int:
    """Brute force over the 16 entries; a tie keeps the lower index."""
    dists = [abs(x - q) for q in NF4_TABLE]
    best = min(dists)
    return dists.index(best)


def e2m1_value(code: int) -> Fr:
    """The E2M1 element value of a 4-bit code: bit 3 the sign, bits 2..1 the
    exponent e, bit 0 the mantissa m; m/2 for e = 0, else 2^(e-1) (1 + m/2)."""
    sign = -1 if code & 8 else 1
    e, m = (code >> 1) & 3, code & 1
    mag = Fr(m, 2) if e == 0 else Fr(2) ** (e - 1) * (1 + Fr(m, 2))
    return sign * mag


# FP4 codebook (a reading; the pages name the format without a table): the
# E2M1 values divided by 6, each the nearest binary32.  The sign of zero is
# not a Fraction property: code 8 is -0 (checked by the tests separately).
FP4_TABLE = [rn32(e2m1_value(c) / 6) for c in range(16)]


def fp4_nearest(x: Fr) -> int:
    """Brute force over the 16 entries; a tie keeps the lower index."""
    dists = [abs(x - q) for q in FP4_TABLE]
    best = min(dists)
    return dists.index(best)


def nearest_int_level(x: Fr, lo: int, hi: int) -> int:
    """Brute force over the integer levels lo..hi: nearest to x, ties to the
    even level."""
    best = None
    for t in range(lo, hi + 1):
        d = abs(x - t)
        if best is None or d < best[0] or (d == best[0] and t % 2 == 0):
            best = (d, t)
    return best[1]


def quantize_group(fmt: int, w_bits: list[int]):
    """Exact codes of one group (list of fp16 bit patterns).

    fmt: 0 NF4, 1 INT4-sym, 2 INT4-asym, 4 FP4.  Returns (nibbles, scale, zero) where
    scale is an exact Fraction (the stored binary32 absmax or binary16 scale)
    and zero is the asym zero-point (None otherwise)."""
    w = [f16_value(b) for b in w_bits]
    if fmt == 4:
        c = max(abs(v) for v in w)
        if c == 0:
            return [0] * len(w), c, None
        return [fp4_nearest(rn32(v / c)) for v in w], c, None
    if fmt == 0:
        c = max(abs(v) for v in w)
        if c == 0:
            return [7] * len(w), c, None
        return [nf4_nearest(rn32(v / c)) for v in w], c, None
    if fmt == 1:
        a = max(abs(v) for v in w)
        s = rn16(rn32(a / 7))
        if s == 0:
            return [8] * len(w), s, None
        return [nearest_int_level(rn32(v / s), -8, 7) + 8 for v in w], s, None
    lo = min(min(w), Fr(0))
    hi = max(max(w), Fr(0))
    s = rn16(rn32(rn32(hi - lo) / 15))
    if s == 0:
        return [0] * len(w), s, 0
    z = nearest_int_level(rn32(-lo / s), 0, 15)
    return [nearest_int_level(rn32(v / s), -z, 15 - z) + z for v in w], s, z
