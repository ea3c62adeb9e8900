"""IEEE 754 binary32 arithmetic from first principles, on exact rationals.

A test helper, independent of the oracle and of numpy's float arithmetic:
values are bit patterns (Python ints); a finite value is decoded into an
exact Fraction, the operation is carried out exactly, and the result is
rounded once to binary32 with round-to-nearest, ties to even, with gradual
underflow (subnormals kept) and overflow to infinity.  Signed zeros follow
the IEEE rules for round-to-nearest: an exact zero sum is +0 unless both
addends are -0; a product's zero takes the sign xor; a non-zero result that
rounds to zero keeps its sign.

Used to pin the oracle's per-term arithmetic on small random cases: one
rounding per product and per sum in exact mode, one rounding per fused
multiply-add in fast mode.
"""
from __future__ import annotations

from fractions import Fraction

QNAN = 0x7FC00000
PINF = 0x7F800000
NINF = 0xFF800000


def is_nan(b: int) -> bool:
    return (b & 0x7F800000) == 0x7F800000 and (b & 0x007FFFFF) != 0


def is_inf(b: int) -> bool:
    return (b & 0x7FFFFFFF) == 0x7F800000


def sign(b: int) -> int:
    return (b >> 31) & 1


def is_zero(b: int) -> bool:
    return (b & 0x7FFFFFFF) == 0


def value(b: int) -> Fraction:
    """Exact value of a finite binary32 bit pattern."""
    e = (b >> 23) & 0xFF
    f = b & 0x7FFFFF
    assert e != 0xFF
    if e == 0:
        mag = Fraction(f, 1 << 149)          # f * 2^-149
    else:
        mag = Fraction((1 << 23) | f) * (Fraction(2) ** (e - 150))
    return -mag if sign(b) else mag


def _floor_log2(a: Fraction) -> int:
    """The e with 2^e <= a < 2^(e+1), for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_to_f32(q: Fraction, sign_if_zero: int = 0) -> int:
    """Round an exact rational once to binary32 (RNE); an exact zero takes `sign_if_zero`."""
    if q == 0:
        return sign_if_zero << 31
    s = 1 if q < 0 else 0
    a = -q if s else q
    e = _floor_log2(a)
    if e > 127:
        return (s << 31) | 0x7F800000
    e = max(e, -126)                          # below the normal range the spacing stays 2^-149
    quantum = Fraction(2) ** (e - 23)
    t = a / quantum
    n = t.numerator // t.denominator
    r = t - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and (n & 1)):
        n += 1
    if n == (1 << 24):                        # carried into the next binade
        n = 1 << 23
        e += 1
        if e > 127:
            return (s << 31) | 0x7F800000
    if n == 0:
        return s << 31
    if n < (1 << 23):                         # subnormal (only when e == -126)
        return (s << 31) | n
    return (s << 31) | ((e + 127) << 23) | (n - (1 << 23))


def mul(x: int, y: int) -> int:
    if is_nan(x) or is_nan(y):
        return QNAN
    s = sign(x) ^ sign(y)
    if is_inf(x) or is_inf(y):
        if is_zero(x) or is_zero(y):
            return QNAN
        return (s << 31) | 0x7F800000
    return round_to_f32(value(x) * value(y), s)


def add(x: int, y: int) -> int:
    if is_nan(x) or is_nan(y):
        return QNAN
    if is_inf(x) and is_inf(y):
        return x if sign(x) == sign(y) else QNAN
    if is_inf(x):
        return x
    if is_inf(y):
        return y
    q = value(x) + value(y)
    zero_sign = 1 if (is_zero(x) and is_zero(y) and sign(x) and sign(y)) else 0
    return round_to_f32(q, zero_sign)


def fma(a: int, b: int, c: int) -> int:
    """a*b + c with one rounding."""
    if is_nan(a) or is_nan(b) or is_nan(c):
        return QNAN
    ps = sign(a) ^ sign(b)
    if is_inf(a) or is_inf(b):
        if is_zero(a) or is_zero(b):
            return QNAN
        if is_inf(c) and sign(c) != ps:
            return QNAN
        return (ps << 31) | 0x7F800000
    if is_inf(c):
        return c
    prod = value(a) * value(b)
    q = prod + value(c)
    if q == 0:
        # exact zero: -0 only when the product is a zero of sign - and c is -0
        zero_sign = 1 if (prod == 0 and ps == 1 and is_zero(c) and sign(c) == 1) else 0
        return round_to_f32(q, zero_sign)
    return round_to_f32(q)


def canonical(b: int) -> int:
    return QNAN if is_nan(b) else b


def dot_exact_mode(a_bits, b_bits) -> int:
    acc = 0
    for x, y in zip(a_bits, b_bits):
        acc = add(acc, mul(x, y))
    return canonical(acc)


def dot_fast_mode(a_bits, b_bits) -> int:
    acc = 0
    for x, y in zip(a_bits, b_bits):
        acc = fma(x, y, acc)
    return canonical(acc)
