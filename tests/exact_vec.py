"""A vectorised exact model of the fixed-order sum all-reduce, for pins over
millions of columns.

Independent of ``oracle/oracle.c`` (which adds with the host's binary32
hardware) and of ``exact_model.py`` (exact rationals): every binary32 addition
here is done in 64-bit integers from the IEEE-754 definition, the way a
software floating-point adder does it, and rounded with roundTiesToEven:

* an operand is (sign, integer significand M, exponent E) with value
  (-1)^sign * M * 2^E -- an exact decoding of its bits;
* the two operands are aligned on the smaller exponent while the exponent
  difference d is at most 37 (then 2 * (M_a * 2^d + M_b) < 2^63 is exact);
  for a larger d the smaller operand is shifted right into 37 spare low bits
  and what falls off is kept as a sticky bit, which makes the doubled sum
  odd, so it can never look like a tie (at least 2 bits are discarded);
* the exact (or sticky-marked) sum is rounded to 24 significant bits with
  gradual underflow at 2^-149 and overflow to infinity at 2^128;
* an exact zero sum is +0 unless both operands are -0.
The final narrowing rounds the binary32 accumulator straight to bfloat16 or
float16 the same way (p = 8 or 11, gradual underflow, overflow to infinity).

Finite inputs only (NaN and infinity are covered by the rational model); an
accumulator that overflows stays infinite.  ``tests/test_oracle_pins.py``
checks this model against the rational one before using it.
"""
from __future__ import annotations

import numpy as np

# (exponent bits, stored mantissa bits) per format
_FMT = {"bf16": (8, 7), "fp16": (5, 10), "fp32": (8, 23)}


def _params(dtype):
    ebits, mbits = _FMT[dtype]
    bias = (1 << (ebits - 1)) - 1
    p = mbits + 1
    emin = 1 - bias
    return ebits, mbits, bias, p, emin, bias  # emax = bias


def _bitlen(v: np.ndarray) -> np.ndarray:
    """Bit length of non-negative int64 values (0 for 0)."""
    v = v.astype(np.uint64)
    n = np.zeros(v.shape, dtype=np.int64)
    for k in (32, 16, 8, 4, 2, 1):
        big = (v >> np.uint64(k)) != 0
        n += np.where(big, k, 0)
        v = np.where(big, v >> np.uint64(k), v)
    return n + (v != 0)


def decode(bits: np.ndarray, dtype: str):
    """(sign, M, E) of finite encodings."""
    ebits, mbits, bias, p, emin, emax = _params(dtype)
    b = bits.astype(np.int64)
    s = (b >> (ebits + mbits)) & 1
    e = (b >> mbits) & ((1 << ebits) - 1)
    m = b & ((1 << mbits) - 1)
    assert not (e == (1 << ebits) - 1).any(), "finite inputs only"
    sub = e == 0
    M = np.where(sub, m, m | (1 << mbits))
    E = np.where(sub, emin - mbits, e - bias - mbits)
    return s, M, E


def _round(M: np.ndarray, U: np.ndarray, p: int, emin: int):
    """Round M * 2^U (M > 0, int64) to p significant bits with roundTiesToEven
    and gradual underflow below 2^emin.  Returns (m, q): value m * 2^q."""
    L = _bitlen(M) - 1 + U                      # floor(log2(value))
    q = np.maximum(L - (p - 1), emin - (p - 1))
    shift = q - U
    left = np.maximum(-shift, 0)                # exact: more room than bits
    right = np.clip(shift, 0, 63)
    Mu = M.astype(np.uint64)
    m_exact = (Mu << left.astype(np.uint64)).astype(np.int64)
    m0 = (Mu >> right.astype(np.uint64)).astype(np.int64)
    mask = (np.uint64(1) << right.astype(np.uint64)) - np.uint64(1)
    rem = (Mu & mask).astype(np.int64)
    half = np.where(right > 0, (np.uint64(1) << np.maximum(right - 1, 0).astype(np.uint64))
                    .astype(np.int64), 0)
    up = (right > 0) & ((rem > half) | ((rem == half) & ((m0 & 1) == 1)))
    m = np.where(shift > 0, m0 + up, m_exact)
    carry = m == (1 << p)
    m = np.where(carry, m >> 1, m)
    q = np.where(carry, q + 1, q)
    return m, q


def add32(a, b):
    """IEEE binary32 a + b under roundTiesToEven on (sign, M, E, inf) arrays."""
    sa, Ma, Ea, ia = a
    sb, Mb, Eb, ib = b
    # order so that the first operand has the larger exponent (or b is zero)
    swap = ((Eb > Ea) & (Mb != 0)) | (Ma == 0)
    s1, M1, E1 = np.where(swap, sb, sa), np.where(swap, Mb, Ma), np.where(swap, Eb, Ea)
    s2, M2, E2 = np.where(swap, sa, sb), np.where(swap, Ma, Mb), np.where(swap, Ea, Eb)
    d = np.where(M2 == 0, 0, E1 - E2)
    same = s1 == s2
    near = d <= 37
    # d <= 37: exact on the smaller exponent
    Sn = (M1 << np.minimum(d, 37)) + np.where(same, M2, -M2)
    Tn = 2 * Sn                                  # LSB weight 2^(E2 - 1)
    Un = np.where(M2 == 0, E1, E2)               # a zero operand has no say in the unit
    # d > 37: the smaller operand falls into 37 spare bits and a sticky bit
    k = np.clip(d - 37, 0, 63)
    bs = (M2.astype(np.uint64) >> k.astype(np.uint64)).astype(np.int64)
    sticky = (M2.astype(np.uint64) & ((np.uint64(1) << k.astype(np.uint64)) - np.uint64(1))) != 0
    sticky = np.where(d - 37 >= 64, M2 != 0, sticky)
    bs = np.where(d - 37 >= 64, 0, bs)
    base = M1 << 37
    Tf = np.where(same, 2 * (base + bs) + sticky,
                  np.where(sticky, 2 * (base - bs - 1) + 1, 2 * (base - bs)))
    Uf = E1 - 37
    T = np.where(near, Tn, Tf)
    U = np.where(near, Un, Uf)
    # T is signed relative to operand 1's sign
    neg = T < 0
    s = np.where(neg, 1 - s1, s1)
    mag = np.abs(T)
    zero = mag == 0
    both_neg_zero = (Ma == 0) & (Mb == 0) & (sa == 1) & (sb == 1)
    m, q = _round(np.where(zero, 1, mag), U - 1, 24, -126)
    inf = ia | ib | (~zero & (q + _bitlen(m) - 1 > 127))
    s = np.where(zero, np.where(both_neg_zero, 1, 0), s)
    m = np.where(zero | inf, 0, m)
    q = np.where(zero | inf, 0, q)
    # infinite operands: the sign of the infinite one (finite inputs cannot
    # give inf + -inf before overflow, which the callers check)
    s = np.where(ia, sa, np.where(ib, sb, s))
    return s, m, q, inf


def narrow(acc, dtype: str) -> np.ndarray:
    """Bits of the binary32 accumulator rounded to ``dtype``."""
    ebits, mbits, bias, p, emin, emax = _params(dtype)
    s, M, E, inf = acc
    zero = M == 0
    if dtype == "fp32":
        m, q = M, E
    else:
        m, q = _round(np.where(zero, 1, M), E, p, emin)
    inf = inf | (~zero & (q + _bitlen(m) - 1 > emax))
    m = np.where(zero | inf, 0, m)
    bl = _bitlen(m)
    normal = bl == p
    efield = np.where(normal, q + (p - 1) + bias, 0)
    mfield = np.where(normal, m - (1 << mbits), m)
    efield = np.where(inf, (1 << ebits) - 1, efield)
    mfield = np.where(inf, 0, mfield)
    return (s << (ebits + mbits)) | (efield << mbits) | mfield


def _sum32(bits: np.ndarray, dtype: str):
    """binary32 sum of the columns of ``bits`` in column order, from the first
    one's value (not from +0)."""
    cols, R = bits.shape
    s, M, E = decode(bits[:, 0], dtype)
    acc = (s, M, E, np.zeros(cols, dtype=bool))
    for j in range(1, R):
        s, M, E = decode(bits[:, j], dtype)
        acc = add32(acc, (s, M, E, np.zeros(cols, dtype=bool)))
    return acc


def allreduce_columns(bits: np.ndarray, dtype: str, group: int | None = None) -> np.ndarray:
    """Output bits for each column of ``bits`` (ncols, R).

    Flat order (``group`` None): binary32 sum in rank order from rank 0's
    value, rounded once to ``dtype``.  Grouped order: a binary32 partial per
    run of ``group`` consecutive ranks (each from its first rank's value),
    the partials summed in group order from the first partial, one rounding."""
    if group is None or group == bits.shape[1]:
        return narrow(_sum32(bits, dtype), dtype)
    cols, R = bits.shape
    assert group >= 1 and R % group == 0
    parts = [_sum32(bits[:, g * group:(g + 1) * group], dtype) for g in range(R // group)]
    total = parts[0]
    for part in parts[1:]:
        total = add32(total, part)
    return narrow(total, dtype)


def allreduce_columns_chunked(bits: np.ndarray, dtype: str, group: int | None = None,
                              workers: int = 4, chunk: int = 1 << 17) -> np.ndarray:
    """``allreduce_columns`` over slices of columns on a few threads (numpy
    releases the interpreter lock inside its array operations)."""
    from concurrent.futures import ThreadPoolExecutor
    starts = range(0, bits.shape[0], chunk)
    with ThreadPoolExecutor(max_workers=workers) as pool:
        parts = pool.map(lambda a: allreduce_columns(bits[a:a + chunk], dtype, group), starts)
        return np.concatenate(list(parts)) if bits.shape[0] else np.zeros(0, dtype=np.int64)
