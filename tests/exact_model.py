"""Exact-arithmetic model of the fixed-order sum all-reduce, used to pin the oracle.

This is independent of ``oracle/oracle.c``: values are exact rationals
(``fractions.Fraction``), every binary32 add is the exact sum rounded by an
explicit round-to-nearest-even routine written from the IEEE-754 definition
(roundTiesToEven, gradual underflow, overflow to infinity), and the final
narrowing rounds the exact value of the binary32 accumulator straight to the
target format.  No hardware float add, no bit-shuffling narrowing and no
library float conversion is involved, so a mistake shared by the two would have
to be made twice in unrelated forms.

A value is one of
  ("nan",)              any NaN
  ("inf", s)            s = 0 for +inf, 1 for -inf
  ("fin", s, q)         finite; q >= 0 a Fraction, s the sign bit (kept for zeros)
"""
from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction


@dataclass(frozen=True)
class Fmt:
    name: str
    ebits: int      # exponent field width
    mbits: int      # stored mantissa bits

    @property
    def bias(self) -> int:
        return (1 << (self.ebits - 1)) - 1

    @property
    def p(self) -> int:         # significand precision incl. the hidden bit
        return self.mbits + 1

    @property
    def emin(self) -> int:
        return 1 - self.bias

    @property
    def emax(self) -> int:
        return self.bias


BF16 = Fmt("bf16", 8, 7)
FP16 = Fmt("fp16", 5, 10)
FP32 = Fmt("fp32", 8, 23)
FORMATS = {"bf16": BF16, "fp16": FP16, "fp32": FP32}


def decode(bits: int, fmt: Fmt):
    """Exact value of an encoding."""
    s = (bits >> (fmt.ebits + fmt.mbits)) & 1
    e = (bits >> fmt.mbits) & ((1 << fmt.ebits) - 1)
    m = bits & ((1 << fmt.mbits) - 1)
    if e == (1 << fmt.ebits) - 1:
        return ("nan",) if m else ("inf", s)
    if e == 0:
        q = Fraction(m, 1) * Fraction(2) ** (fmt.emin - fmt.mbits)
    else:
        q = Fraction(m + (1 << fmt.mbits), 1) * Fraction(2) ** (e - fmt.bias - fmt.mbits)
    return ("fin", s, q)


def _floor_log2(q: Fraction) -> int:
    """floor(log2(q)) for q > 0, exactly."""
    n, d = q.numerator, q.denominator
    e = n.bit_length() - d.bit_length()
    # now 2^(e-1) < n/d < 2^(e+1); settle which side of 2^e
    if e >= 0:
        if n < d << e:
            e -= 1
    else:
        if n << (-e) < d:
            e -= 1
    return e


def round_to(v, fmt: Fmt):
    """Round an exact value to ``fmt`` with roundTiesToEven."""
    if v[0] != "fin":
        return v
    s, q = v[1], v[2]
    if q == 0:
        return v
    e = max(_floor_log2(q), fmt.emin)
    quantum = Fraction(2) ** (e - fmt.mbits)
    units = q / quantum
    n = units.numerator // units.denominator
    rem = units - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    if r >= Fraction(2) ** (fmt.emax + 1):
        return ("inf", s)
    return ("fin", s, r)


def encode(v, fmt: Fmt) -> int:
    """Bits of a value already representable in ``fmt`` (NaN -> canonical quiet)."""
    top = fmt.ebits + fmt.mbits
    emask = (1 << fmt.ebits) - 1
    if v[0] == "nan":
        return (emask << fmt.mbits) | (1 << (fmt.mbits - 1))
    if v[0] == "inf":
        return (v[1] << top) | (emask << fmt.mbits)
    s, q = v[1], v[2]
    if q == 0:
        return s << top
    e = _floor_log2(q)
    if e < fmt.emin:
        m = q / Fraction(2) ** (fmt.emin - fmt.mbits)
        assert m.denominator == 1, "value not representable"
        return (s << top) | int(m)
    m = q / Fraction(2) ** (e - fmt.mbits)
    assert m.denominator == 1, "value not representable"
    return (s << top) | ((e + fmt.bias) << fmt.mbits) | (int(m) - (1 << fmt.mbits))


def add_exact_then_round(a, b, fmt: Fmt = FP32):
    """IEEE addition a + b in ``fmt`` under roundTiesToEven."""
    if a[0] == "nan" or b[0] == "nan":
        return ("nan",)
    if a[0] == "inf" and b[0] == "inf":
        return a if a[1] == b[1] else ("nan",)
    if a[0] == "inf":
        return a
    if b[0] == "inf":
        return b
    sa, qa = a[1], a[2]
    sb, qb = b[1], b[2]
    exact = (-qa if sa else qa) + (-qb if sb else qb)
    if exact == 0:
        # exact zero sum: -0 only when both operands are -0 (IEEE 754 sec. 6.3)
        if qa == 0 and qb == 0:
            return ("fin", sa & sb, Fraction(0))
        return ("fin", 0, Fraction(0))
    return round_to(("fin", 1 if exact < 0 else 0, abs(exact)), fmt)


def allreduce_column(bits: list[int], dtype: str) -> int:
    """Output bits for one element given the R input bit patterns, rank order 0..R-1."""
    fmt = FORMATS[dtype]
    acc = decode(bits[0], fmt)          # widening to binary32 is exact
    for b in bits[1:]:
        acc = add_exact_then_round(acc, decode(b, fmt), FP32)
    return encode(round_to(acc, fmt), fmt)


def exact_sum(bits: list[int], dtype: str):
    """The exact rational sum of finite inputs (None when a NaN/inf is present)."""
    fmt = FORMATS[dtype]
    total = Fraction(0)
    mags = Fraction(0)
    for b in bits:
        v = decode(b, fmt)
        if v[0] != "fin":
            return None
        total += -v[2] if v[1] else v[2]
        mags += v[2]
    return total, mags


def value_of(bits: int, dtype: str):
    """Signed exact value of finite bits as a Fraction (None for NaN/inf)."""
    v = decode(bits, FORMATS[dtype])
    if v[0] != "fin":
        return None
    return -v[2] if v[1] else v[2]


def is_nan_bits(bits: int, dtype: str) -> bool:
    return decode(bits, FORMATS[dtype])[0] == "nan"


def allreduce_column_grouped(bits: list[int], dtype: str, group: int) -> int:
    """Hierarchical order: binary32 partial per group of ``group`` consecutive
    ranks (in rank order), then the partials summed in group order; one final
    rounding to the format."""
    fmt = FORMATS[dtype]
    total = None
    for g in range(len(bits) // group):
        part = decode(bits[g * group], fmt)
        for b in bits[g * group + 1:(g + 1) * group]:
            part = add_exact_then_round(part, decode(b, fmt), FP32)
        total = part if total is None else add_exact_then_round(total, part, FP32)
    return encode(round_to(total, fmt), fmt)
