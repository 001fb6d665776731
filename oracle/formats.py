"""Tier 0: binary floating-point formats in exact rational arithmetic.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

A value is a ``Val``: a kind ('num', 'inf' or 'nan'), a sign bit and an exact
magnitude.  The sign bit is carried on zero too: [Drift, "First, catching
myself"] reports an exact reference that lost the sign of zero, and the 8-bit
formats spend a code on negative zero.

Formats [MP-card, items (1)-(3)]:

* FP16: a sign bit, five exponent bits and ten mantissa bits; largest finite value
  2^15 * (2 - 2^-10) = 65504, smallest normal 2^-14, smallest subnormal 2^-24.
* BF16 = 1 + 8 + 7 bits, the exponent range of fp32 (about +-3.4e38).
* E4M3 = 4 exponent + 3 mantissa bits with largest value about 448; E5M2 =
  5 + 2 bits with largest value about 57344.

The pages give no bias or special-value encoding for the FP8 formats.  The
reading adopted (and pinned by the tests from the printed maxima): E4M3 has
bias 7, no infinity, and only the all-ones exponent-and-mantissa pattern (per
sign) is NaN -- the only layout with 4+3 bits whose largest finite value is
448 while keeping a negative zero.  E5M2 is IEEE-style with bias 15 (largest
finite 57344 = 1.75 * 2^15, all-ones exponent reserved for Inf and NaN).
"""

from dataclasses import dataclass
from fractions import Fraction

ZERO = Fraction(0)
HALF = Fraction(1, 2)


def pow2(n: int) -> Fraction:
    """2**n as an exact rational (n may be negative)."""
    return Fraction(1 << n) if n >= 0 else Fraction(1, 1 << (-n))


def floor_log2(x: Fraction) -> int:
    """The integer e with 2**e <= x < 2**(e+1), for a rational x > 0."""
    if x <= 0:
        raise ValueError("floor_log2 needs a positive value")
    n, d = x.numerator, x.denominator
    e = n.bit_length() - d.bit_length()
    # n/d < 2**e  <=>  n * 2**-e < d  (e < 0)  or  n < d * 2**e  (e >= 0)
    below = (n << -e) < d if e < 0 else n < (d << e)
    return e - 1 if below else e


def round_half_even(t: Fraction) -> int:
    """Round a non-negative rational to the nearest integer, ties to even."""
    f = t.numerator // t.denominator
    rem = t - f
    if rem > HALF or (rem == HALF and f % 2 == 1):
        f += 1
    return f


@dataclass(frozen=True)
class Val:
    kind: str        # 'num', 'inf' or 'nan'
    neg: bool        # the sign bit (meaningful on zero as well)
    mag: Fraction    # exact magnitude for 'num'; 0 otherwise

    @staticmethod
    def num(neg: bool, mag) -> "Val":
        mag = Fraction(mag)
        if mag < 0:
            raise ValueError("magnitude must be non-negative")
        return Val("num", bool(neg), mag)

    @staticmethod
    def of(x) -> "Val":
        """A signed rational (or float) as a value; -0.0 keeps its sign."""
        if isinstance(x, float):
            import math
            if math.isnan(x):
                return Val("nan", False, ZERO)
            if math.isinf(x):
                return Val("inf", x < 0, ZERO)
            return Val("num", math.copysign(1.0, x) < 0, abs(Fraction(x)))
        x = Fraction(x)
        return Val("num", x < 0, abs(x))

    @property
    def finite(self) -> bool:
        return self.kind == "num"

    @property
    def signed(self) -> Fraction:
        """The real number (sign applied); only for finite values."""
        assert self.kind == "num"
        return -self.mag if self.neg else self.mag


@dataclass(frozen=True)
class Fmt:
    """A binary floating-point format with 1 sign bit.

    specials = 'ieee': the all-ones exponent field holds Inf (mantissa 0) and
    NaN (mantissa != 0).  specials = 'fn': there is no Inf; the all-ones
    exponent field is finite except for the all-ones mantissa, which is NaN.
    """
    name: str
    ebits: int
    mbits: int
    bias: int
    specials: str
    qnan: int        # the canonical NaN code this format's encoder emits

    @property
    def nbits(self) -> int:
        return 1 + self.ebits + self.mbits

    @property
    def sign_bit(self) -> int:
        return 1 << (self.nbits - 1)

    @property
    def emin(self) -> int:
        """Exponent of the smallest normal value."""
        return 1 - self.bias

    @property
    def emax(self) -> int:
        """Exponent of the largest finite value."""
        top = (1 << self.ebits) - 1
        return (top - 1 - self.bias) if self.specials == "ieee" else (top - self.bias)

    @property
    def maxval(self) -> Fraction:
        """Largest finite magnitude."""
        if self.specials == "ieee":
            sig = 2 - pow2(-self.mbits)
        else:
            sig = 2 - pow2(1 - self.mbits)
        return sig * pow2(self.emax)

    @property
    def min_subnormal(self) -> Fraction:
        return pow2(self.emin - self.mbits)

    # -- decoding ---------------------------------------------------------

    def decode(self, code: int) -> Val:
        if not 0 <= code < (1 << self.nbits):
            raise ValueError("code out of range")
        neg = bool(code & self.sign_bit)
        e_field = (code >> self.mbits) & ((1 << self.ebits) - 1)
        m_field = code & ((1 << self.mbits) - 1)
        top = (1 << self.ebits) - 1
        if self.specials == "ieee" and e_field == top:
            return Val("inf", neg, ZERO) if m_field == 0 else Val("nan", neg, ZERO)
        if self.specials == "fn" and e_field == top and m_field == (1 << self.mbits) - 1:
            return Val("nan", neg, ZERO)
        frac = Fraction(m_field, 1 << self.mbits)
        if e_field == 0:
            mag = frac * pow2(self.emin)
        else:
            mag = (1 + frac) * pow2(e_field - self.bias)
        return Val.num(neg, mag)

    # -- rounding and encoding -------------------------------------------

    def round_mag(self, mag: Fraction) -> Fraction:
        """Round-to-nearest-even of a magnitude onto this format's grid, with
        an unbounded exponent above (no overflow handling here).

        The spacing of the grid at a value v is 2^(e(v) - mbits) for v at or
        above the smallest normal and 2^(emin - mbits) below it.
        """
        if mag == 0:
            return ZERO
        e = floor_log2(mag)
        quantum = pow2(max(e, self.emin) - self.mbits)
        return round_half_even(mag / quantum) * quantum

    def code_of(self, neg: bool, mag: Fraction) -> int:
        """The code of a magnitude that lies exactly on the finite grid."""
        sign = self.sign_bit if neg else 0
        if mag == 0:
            return sign
        if mag > self.maxval:
            raise ValueError("magnitude above the largest finite value")
        e = floor_log2(mag)
        if e >= self.emin:
            e_field = e + self.bias
            m = (mag / pow2(e) - 1) * (1 << self.mbits)
        else:
            e_field = 0
            m = mag / pow2(self.emin - self.mbits)
        if m.denominator != 1:
            raise ValueError("magnitude not on the grid")
        return sign | (e_field << self.mbits) | int(m)

    def max_code(self, neg: bool = False) -> int:
        return self.code_of(neg, self.maxval)

    def inf_code(self, neg: bool = False) -> int:
        assert self.specials == "ieee"
        top = (1 << self.ebits) - 1
        return (self.sign_bit if neg else 0) | (top << self.mbits)

    def encode(self, v: Val, saturate: bool) -> int:
        """Round-to-nearest-even of a value into this format.

        saturate=True: a magnitude that rounds above the largest finite value,
        and +-Inf, become the largest finite value of the same sign; NaN
        becomes the canonical NaN code.  saturate=False: IEEE overflow, i.e.
        such magnitudes become +-Inf ('ieee' formats) or NaN ('fn').
        """
        if v.kind == "nan":
            return self.qnan
        if v.kind == "inf":
            if saturate:
                return self.max_code(v.neg)
            return self.inf_code(v.neg) if self.specials == "ieee" else self.qnan
        r = self.round_mag(v.mag)
        if r > self.maxval:
            if saturate:
                return self.max_code(v.neg)
            return self.inf_code(v.neg) if self.specials == "ieee" else self.qnan
        return self.code_of(v.neg, r)


E4M3 = Fmt("e4m3", 4, 3, 7, "fn", qnan=0x7F)
E5M2 = Fmt("e5m2", 5, 2, 15, "ieee", qnan=0x7F)
FP16 = Fmt("fp16", 5, 10, 15, "ieee", qnan=0x7E00)
BF16 = Fmt("bf16", 8, 7, 127, "ieee", qnan=0x7FC0)
FP32 = Fmt("fp32", 8, 23, 127, "ieee", qnan=0x7FC00000)

FORMATS = {"e4m3": E4M3, "e5m2": E5M2}


def fp32_value(bits: int) -> Val:
    """The value of a 32-bit IEEE binary32 pattern."""
    return FP32.decode(bits & 0xFFFFFFFF)


def bf16_value(bits: int) -> Val:
    """The value of a 16-bit bfloat16 pattern."""
    return BF16.decode(bits & 0xFFFF)
