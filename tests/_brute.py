"""Exact brute-force references used to pin the oracle (tests only).

Nearest-grid-point search with Python Fractions: no midpoints, no thresholds, no
vectorisation -- every candidate distance is computed exactly and the smallest wins, ties
going to the even code.  Independent of the oracle's midpoint-counting formulation.
"""
from fractions import Fraction


def e2m1_codes_table():
    """(code, value) for the 16 E2M1 codes, written out by hand from the format."""
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
            Fraction(4), Fraction(6)]
    out = []
    for c in range(16):
        v = mags[c & 7]
        out.append((c, -v if c & 8 else v))
    return out


def e4m3_nonneg_table():
    """(code, value) for E4M3FN codes 0..126 enumerated by exponent/mantissa fields."""
    out = []
    for c in range(127):
        e, m = c >> 3, c & 7
        if e == 0:
            v = Fraction(m, 8) * Fraction(1, 64)
        else:
            v = (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))
        out.append((c, v))
    return out


def nearest_code(q: Fraction, table):
    """Code whose value is nearest to q; ties -> even code; beyond range -> nearest end."""
    best = None
    for c, v in table:
        d = abs(q - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0 and best[1] % 2 == 1):
            best = (d, c)
    return best[1]


def e2m1_encode_brute(x: Fraction, unit: Fraction) -> int:
    """Signed E2M1 nibble for x/unit: nearest among the 15 distinct signed values, ties to the
    even code, zero always stored as code 0."""
    q = x / unit
    table = [(c, v) for c, v in e2m1_codes_table() if c != 8]   # drop the -0 code
    best = None
    for c, v in table:
        d = abs(q - v)
        if best is None or d < best[0]:
            best = (d, c, v)
        elif d == best[0]:
            # tie: prefer the even magnitude code (sign does not enter the parity)
            if (c & 7) % 2 == 0 and (best[1] & 7) % 2 == 1:
                best = (d, c, v)
    return best[1]


def fraction_to_f32(x: Fraction):
    """Round-to-nearest-even of an exact rational to fp32 (zero and the normal range)."""
    import numpy as np
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = a / Fraction(2) ** (e - 23)                  # in [2^23, 2^24)
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return np.float32(sign * float(Fraction(n) * Fraction(2) ** (e - 23)))
