"""Exact IEEE round-to-nearest-even on rationals (integer arithmetic only).

Used by the oracle's pins as an implementation of the codec's rounding steps
that is independent of numpy's float32 division, float16 cast and rint.
"""

from fractions import Fraction
import math

INF = float("inf")


def _floor_log2(a: Fraction) -> int:
    """e with 2**e <= a < 2**(e+1), for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    return e


def round_half_even_int(n: Fraction) -> int:
    fl = math.floor(n)
    d = n - fl
    if d > Fraction(1, 2):
        return fl + 1
    if d < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def round_to_format(f: Fraction, p: int, emin: int, emax: int):
    """Round rational f to the binary format with p significand bits
    (implicit bit included), minimum normal exponent emin and maximum
    exponent emax.  Returns a Fraction, or +-inf on overflow."""
    if f == 0:
        return Fraction(0)
    sign = -1 if f < 0 else 1
    a = abs(f)
    e = _floor_log2(a)
    q = max(e, emin) - (p - 1)
    n = round_half_even_int(a / Fraction(2) ** q)
    r = n * Fraction(2) ** q
    if r >= Fraction(2) ** (emax + 1):
        return sign * INF
    return sign * r


def rne_f32(f: Fraction):
    return round_to_format(f, 24, -126, 127)


def rne_f16(f: Fraction):
    return round_to_format(f, 11, -14, 15)


def codec_scale(absmax: float, qmax: int) -> Fraction:
    """fp16 scale of the codec: RNE32(a / qmax) then RNE16, overflow -> 65504."""
    s32 = rne_f32(Fraction(absmax) / qmax)
    s16 = rne_f16(s32)
    if s16 == INF:
        return Fraction(65504)
    return s16


def codec_code(x: float, s: Fraction, qmax: int) -> int:
    if s == 0:
        return 0
    r = rne_f32(Fraction(x) / s)
    if r in (INF, -INF):
        return qmax if r > 0 else -qmax
    c = round_half_even_int(r)
    return max(-qmax, min(qmax, c))


def affine_scale(lo: float, hi: float, qmax: int) -> Fraction:
    """fp16 scale of the affine codec: RNE32(RNE32(hi - lo) / qmax) then RNE16,
    overflow -> 65504 (lo <= 0 <= hi already widened)."""
    rng = rne_f32(Fraction(hi) - Fraction(lo))
    if rng == INF:
        return Fraction(65504)
    s16 = rne_f16(rne_f32(rng / qmax))
    if s16 == INF:
        return Fraction(65504)
    return s16


def affine_zero(lo: float, s: Fraction, qmax: int) -> int:
    if s == 0:
        return 0
    return max(0, min(qmax, round_half_even_int(rne_f32(-Fraction(lo) / s))))


def affine_code(x: float, s: Fraction, z: int, qmax: int) -> int:
    if s == 0:
        return 0
    r = rne_f32(Fraction(x) / s)
    if r in (INF, -INF):
        return qmax if r > 0 else 0
    return max(0, min(qmax, round_half_even_int(r) + z))
