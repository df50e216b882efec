"""Pins for the CPU oracle: checks against things other than the oracle itself.

Every function takes an ``oracle.Oracle`` and raises ``AssertionError`` when a
pin fails.  ``tests/test_oracle_pins.py`` runs them on the real oracle at full
size; ``tests/test_oracle_mutants.py`` runs the quick forms on copies of
``oracle.c`` with a planted mistake and requires that at least one fails.

What pins what (the pages print no worked example, so the pins come from the
IEEE-754 definitions and from mathematics):

* brute force   -- ``exact_model`` (exact rationals + an explicit RNE routine)
                   over every 3-rank column of a hand-picked value set, and
                   random columns at R = 8, 16, 32;
* wide brute    -- ``exact_vec`` (an integer IEEE binary32 adder, itself
                   checked against ``exact_model``) over 10^6 columns at
                   R = 8, 16, 32 in five value regimes, flat, and grouped in
                   nodes of 2, 4 and 8;
* hand cases    -- ``tests/golden/hand_cases.txt``, derived by hand;
* closed form   -- integer-valued inputs sum exactly;
* textbook case -- when every partial sum is exact, the result is the
                   correctly rounded exact sum;
* invariants    -- identical outputs, one-hot columns, 2^k scaling, negation,
                   rank permutation of integer data, R = 1, signed zeros;
* error bound   -- recursive summation bound gamma_{R-1} * sum|x_j| (Higham,
                   Accuracy and Stability of Numerical Algorithms, sec. 4.2)
                   plus half an ulp of the output format;
* converters    -- fp32 -> bf16/fp16 against torch's CPU ``.to()`` and numpy's
                   ``astype(float16)``, all 2^32 patterns (or a sample).
"""
from __future__ import annotations

import functools
import itertools
from fractions import Fraction
from pathlib import Path

import numpy as np
import torch

import exact_model as em

GOLDEN = Path(__file__).resolve().parent / "golden" / "hand_cases.txt"

# ---------------------------------------------------------------------------
# value sets for the exhaustive 3-rank brute force
# ---------------------------------------------------------------------------
# bf16: signed zeros, powers of two spread over the range (1, 2^-8 and 2^-30
# together expose an accumulator wider than binary32), all-ones mantissas,
# odd mantissas next to ties, subnormals, the largest finite value, inf, NaN.
V_BF16 = [
    0x0000, 0x8000, 0x3F80, 0xBF80, 0x3B80, 0xBB80, 0x3C00, 0x3B00,
    0x3080, 0xB080, 0x3380, 0x3780, 0x3F81, 0xBF81, 0x3FC0, 0xBFC0,
    0x3FFF, 0xBFFF, 0x4380, 0xC380, 0x437F, 0x4400, 0x4780, 0x4B80,
    0xCB80, 0x4E80, 0xCE80, 0x3F00, 0x4040, 0x4049, 0x3DCD, 0xBDCD,
    0x7F7F, 0xFF7F, 0x7F00, 0x7F80, 0xFF80, 0x7FC0, 0x0001, 0x007F,
    0x0080, 0x8001, 0x3F82, 0x4B81, 0x3F7F, 0xBF7F, 0x4C00, 0x2F80,
]
# fp16: the same roles; 1, 2^-11 and 2^-24 together expose a wide accumulator.
V_FP16 = [
    0x0000, 0x8000, 0x3C00, 0xBC00, 0x1000, 0x9000, 0x1400, 0x0001,
    0x8001, 0x0400, 0x03FF, 0x0C00, 0x3C01, 0xBC01, 0x3E00, 0xBE00,
    0x3FFF, 0xBFFF, 0x6800, 0x67FF, 0xE800, 0x7BFF, 0xFBFF, 0x7800,
    0x4C00, 0x4800, 0x2E66, 0xAE66, 0x4200, 0x7C00, 0xFC00, 0x7E00,
    0x3800, 0x6400, 0x6401, 0x0200, 0x8200, 0x3C02, 0x7BFE, 0x5BFF,
    0x0800, 0x1800, 0x0002, 0x83FF, 0x3BFF, 0xBBFF, 0x7A00, 0x2000,
]
# fp32: the accumulator itself; 1 with 2^-24 and 2^-25 exercise ties.
V_FP32 = [
    0x00000000, 0x80000000, 0x3F800000, 0xBF800000, 0x33800000, 0xB3800000,
    0x33000000, 0x34000000, 0x3F800001, 0xBF800001, 0x3FC00000, 0xBFC00000,
    0x3FFFFFFF, 0xBFFFFFFF, 0x4B800000, 0xCB800000, 0x4B7FFFFF, 0x4E800000,
    0xCE800000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F000000, 0x7F800000, 0xFF800000,
    0x7FC00000, 0x00000001, 0x007FFFFF, 0x00800000, 0x80000001, 0x3DCCCCCD,
    0xBDCCCCCD, 0x40490FDB, 0x3F000000, 0x4B800001, 0x3F7FFFFF, 0xBF7FFFFF,
    0x2F800000, 0x30000000, 0x4F000000, 0xCF000000, 0x34800000, 0x3F800002,
    0x00000002, 0x00400000, 0x80400000, 0x3E000000, 0x42C80000, 0xC2C80000,
]
VALUE_SETS = {"bf16": V_BF16, "fp16": V_FP16, "fp32": V_FP32}


def np_dtype(dtype: str):
    return np.float32 if dtype == "fp32" else np.uint16


def to_array(cols: list[list[int]], dtype: str) -> np.ndarray:
    """(ncols, R) list of bit patterns -> (R, ncols) oracle input array."""
    a = np.array(cols, dtype=np.uint32 if dtype == "fp32" else np.uint16).T.copy()
    if dtype == "fp32":
        a = a.view(np.float32)
    return a


def bits_of(a: np.ndarray, dtype: str) -> np.ndarray:
    return a.view(np.uint32) if dtype == "fp32" else a.view(np.uint16)


def nan_mask(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return (bits & 0x7FFFFFFF) > 0x7F800000
    if dtype == "bf16":
        return (bits & 0x7FFF) > 0x7F80
    return (bits & 0x7FFF) > 0x7C00


def assert_same_bits(got: np.ndarray, want: np.ndarray, dtype: str, what: str):
    """Bitwise equality, NaNs compared by class only."""
    g = bits_of(np.ascontiguousarray(got), dtype).astype(np.int64)
    w = np.asarray(want).astype(np.int64)
    gn, wn = nan_mask(g, dtype), nan_mask(w, dtype)
    bad = (gn != wn) | (~gn & ~wn & (g != w))
    if bad.any():
        idx = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} mismatches, first at {idx.tolist()}: "
                             f"got {[hex(int(x)) for x in g.ravel()[idx]]} "
                             f"want {[hex(int(x)) for x in w.ravel()[idx]]}")


# ---------------------------------------------------------------------------
# brute force against the exact model
# ---------------------------------------------------------------------------
@functools.lru_cache(maxsize=None)
@functools.lru_cache(maxsize=None)
def _exhaustive_cols(dtype: str, R: int):
    vals = VALUE_SETS[dtype]
    cols = [list(c) for c in itertools.product(vals, repeat=R)]
    want = np.array([em.allreduce_column(c, dtype) for c in cols], dtype=np.int64)
    return cols, want


def pin_bruteforce_exhaustive(orc, dtype: str, R: int = 3):
    """Every R-rank column over the value set, against the exact model."""
    cols, want = _exhaustive_cols(dtype, R)
    x = to_array(cols, dtype)
    out = orc.allreduce(x, dtype, nthreads=2)
    for r in range(R):
        assert_same_bits(out[r], want, dtype, f"exhaustive {dtype} R={R} rank {r}")


def random_bits(rng: np.random.Generator, dtype: str, shape, emin=-12, emax=12) -> np.ndarray:
    """Finite encodings with exponents spread over [emin, emax] and random mantissas."""
    fmt = em.FORMATS[dtype]
    s = rng.integers(0, 2, shape, dtype=np.int64)
    e = rng.integers(emin, emax + 1, shape, dtype=np.int64) + fmt.bias
    m = rng.integers(0, 1 << fmt.mbits, shape, dtype=np.int64)
    bits = (s << (fmt.ebits + fmt.mbits)) | (e << fmt.mbits) | m
    return bits.astype(np.uint32 if dtype == "fp32" else np.uint16)


@functools.lru_cache(maxsize=None)
def _random_cols(dtype: str, R: int, ncols: int, seed: int):
    rng = np.random.default_rng(seed)
    bits = random_bits(rng, dtype, (ncols, R))
    want = np.array([em.allreduce_column([int(b) for b in row], dtype) for row in bits],
                    dtype=np.int64)
    return bits, want


def pin_bruteforce_random(orc, dtype: str, R: int, ncols: int, seed: int = 1):
    bits, want = _random_cols(dtype, R, ncols, seed)
    x = bits.T.copy()
    if dtype == "fp32":
        x = x.view(np.float32)
    out = orc.allreduce(x, dtype, nthreads=2)
    for r in range(R):
        assert_same_bits(out[r], want, dtype, f"random {dtype} R={R} rank {r}")


def mixed_bits(rng: np.random.Generator, dtype: str, ncols: int, R: int) -> np.ndarray:
    """Finite columns (ncols, R) in five regimes, a fifth each: exponents in
    [-12, 12]; exponent fields uniform below a per-column cap that is itself
    uniform over the finite range (subnormal inputs and sums, and overflow of
    the accumulator for bfloat16); exponents in [-1, 1] with random signs
    (heavy cancellation, exact zeros); the first regime with a third of the
    entries replaced by signed zeros; and only signed zeros, nine in ten
    negative (so that all-negative-zero columns, whose sum is -0, occur)."""
    fmt = em.FORMATS[dtype]
    top = (1 << fmt.ebits) - 2
    s = rng.integers(0, 2, (ncols, R), dtype=np.int64)
    m = rng.integers(0, 1 << fmt.mbits, (ncols, R), dtype=np.int64)
    regime = rng.integers(0, 5, (ncols, 1))
    s = np.where(regime == 4, (rng.random((ncols, R)) < 0.9).astype(np.int64), s)
    cap = rng.integers(0, top + 1, (ncols, 1))     # full range: a per-column top exponent
    e = np.where(regime == 1, rng.integers(0, cap + 1, (ncols, R)),
                 np.where(regime == 2, rng.integers(-1, 2, (ncols, R)) + fmt.bias,
                          rng.integers(-12, 13, (ncols, R)) + fmt.bias))
    bits = (s << (fmt.ebits + fmt.mbits)) | (e << fmt.mbits) | m
    zero = ((regime == 3) & (rng.random((ncols, R)) < 1 / 3)) | (regime == 4)
    bits = np.where(zero, s << (fmt.ebits + fmt.mbits), bits)
    return bits.astype(np.uint32 if dtype == "fp32" else np.uint16)


def pin_vector_model(dtype: str, seed: int = 21):
    """``exact_vec`` (integer IEEE adder, used for the wide pin below) against
    ``exact_model`` (exact rationals): every finite 3-rank column of the value
    set, then mixed-regime random columns in the flat and grouped orders."""
    import exact_vec as ev
    fin = [v for v in VALUE_SETS[dtype] if not em.is_nan_bits(v, dtype)
           and em.decode(v, em.FORMATS[dtype])[0] == "fin"]
    cols, want = _exhaustive_cols(dtype, 3)
    keep = np.array([all(v in fin for v in c) for c in cols])
    got = ev.allreduce_columns(np.array(cols, dtype=np.int64)[keep], dtype)
    assert np.array_equal(got, want[keep]), f"vector model, exhaustive {dtype}"
    rng = np.random.default_rng(seed)
    for R, ncols, group in ((2, 3000, None), (3, 2000, None), (8, 1000, None), (32, 300, None),
                            (16, 400, 8), (8, 600, 2)):
        bits = mixed_bits(rng, dtype, ncols, R)
        got = ev.allreduce_columns(bits, dtype, group)
        if group is None:
            want = [em.allreduce_column([int(b) for b in row], dtype) for row in bits]
        else:
            want = [em.allreduce_column_grouped([int(b) for b in row], dtype, group)
                    for row in bits]
        bad = np.flatnonzero(got != np.array(want, dtype=np.int64))
        assert bad.size == 0, (f"vector model {dtype} R={R} group={group}: "
                               f"{[hex(int(b)) for b in bits[bad[0]]]}")


def pin_bruteforce_wide(orc, dtype: str, R: int, ncols: int = 10**6, group: int | None = None,
                        seed: int = 31):
    """The oracle against ``exact_vec`` on ``ncols`` mixed-regime columns."""
    import exact_vec as ev
    bits = mixed_bits(np.random.default_rng(seed + R), dtype, ncols, R)
    want = ev.allreduce_columns_chunked(bits, dtype, group)
    x = bits.T.copy()
    if dtype == "fp32":
        x = x.view(np.float32)
    if group is None:
        out = orc.allreduce(x, dtype, nthreads=4)
    else:
        out = orc.allreduce_grouped(x, dtype, group, nthreads=4)
    for r in range(R):
        assert_same_bits(out[r], want, dtype, f"wide {dtype} R={R} group={group} rank {r}")


# ---------------------------------------------------------------------------
# hand-derived cases
# ---------------------------------------------------------------------------
def load_hand_cases():
    cases = []
    for line in GOLDEN.read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        dtype, ins, out = line.split("|")
        cases.append((dtype.strip(), [int(t, 16) for t in ins.split()], int(out.strip(), 16)))
    return cases


def pin_hand_cases(orc):
    cases = load_hand_cases()
    assert len(cases) >= 20, "hand-case fixture went missing"
    for dtype, ins, want in cases:
        x = to_array([ins], dtype)
        out = orc.allreduce(x, dtype)
        for r in range(len(ins)):
            assert_same_bits(out[r], np.array([want]), dtype,
                             f"hand case {dtype} {[hex(v) for v in ins]}")


# ---------------------------------------------------------------------------
# closed form: integer data sums exactly
# ---------------------------------------------------------------------------
def _exact_int_bits(total: np.ndarray, dtype: str) -> np.ndarray:
    fmt = em.FORMATS[dtype]
    return np.array([em.encode(("fin", 1 if t < 0 else 0, Fraction(abs(int(t)))), fmt)
                     for t in total], dtype=np.int64)


def pin_integer_closed_form(orc, dtype: str, R: int, n: int = 4096, seed: int = 5):
    """Integer values in [-4, 4]: |sum| <= 4R is exact in every format here."""
    rng = np.random.default_rng(seed + R)
    ints = rng.integers(-4, 5, (R, n), dtype=np.int64)
    fmt = em.FORMATS[dtype]
    enc = {v: em.encode(("fin", 1 if v < 0 else 0, Fraction(abs(v))), fmt) for v in range(-4, 5)}
    bits = np.vectorize(enc.get)(ints)
    x = bits.astype(np.uint32 if dtype == "fp32" else np.uint16)
    if dtype == "fp32":
        x = x.view(np.float32)
    out = orc.allreduce(x, dtype)
    want = _exact_int_bits(ints.sum(axis=0), dtype)
    for r in range(R):
        assert_same_bits(out[r], want, dtype, f"integer closed form {dtype} R={R}")
    # rank permutation leaves integer sums unchanged
    perm = rng.permutation(R)
    out_p = orc.allreduce(x[perm].copy(), dtype)
    assert_same_bits(out_p[0], want, dtype, f"permuted integer data {dtype} R={R}")


# ---------------------------------------------------------------------------
# textbook special case: exact partial sums -> correctly rounded sum
# ---------------------------------------------------------------------------
def pin_exact_partials(orc, dtype: str, R: int = 8, n: int = 2000, seed: int = 7):
    rng = np.random.default_rng(seed)
    bits = random_bits(rng, dtype, (n, R), emin=-3, emax=3)
    fmt = em.FORMATS[dtype]
    want = []
    for row in bits:
        vals = [em.value_of(int(b), dtype) for b in row]
        partial = Fraction(0)
        for v in vals:
            partial += v
            if partial != 0:
                r = em.round_to(("fin", 0, abs(partial)), em.FP32)
                assert r[2] == abs(partial), "partial sum not exact; widen the generator"
        total = sum(vals, Fraction(0))
        want.append(em.encode(em.round_to(("fin", 1 if total < 0 else 0, abs(total)), fmt), fmt))
    x = bits.T.copy()
    if dtype == "fp32":
        x = x.view(np.float32)
    out = orc.allreduce(x, dtype)
    # an exact zero total with mixed signs is +0 under RNE
    assert_same_bits(out[0], np.array(want, dtype=np.int64), dtype, f"exact partials {dtype}")


# ---------------------------------------------------------------------------
# invariants
# ---------------------------------------------------------------------------
def pin_invariants(orc, dtype: str, R: int = 8, n: int = 4096, seed: int = 11):
    rng = np.random.default_rng(seed)
    fmt = em.FORMATS[dtype]
    top = fmt.ebits + fmt.mbits
    # exponent span that stays normal in the format, also after 2^k scaling
    span, ks = ((-6, 6), (-4, 4)) if dtype == "fp16" else ((-20, 20), (-6, 6))
    x = random_bits(rng, dtype, (R, n), emin=span[0], emax=span[1])
    xv = x.view(np.float32) if dtype == "fp32" else x
    out = orc.allreduce(xv, dtype)
    ob = bits_of(out, dtype)
    # 1. every rank receives the same vector
    for r in range(1, R):
        assert np.array_equal(ob[0], ob[r]), "outputs differ between ranks"
    # 2. 2^k scaling: add k to every exponent field
    for k in ks:
        xs = (x.astype(np.int64) + (k << fmt.mbits)).astype(x.dtype)
        os_ = bits_of(orc.allreduce(xs.view(np.float32) if dtype == "fp32" else xs, dtype), dtype)
        ob64 = ob[0].astype(np.int64)
        nz = (ob64 & ((1 << top) - 1)) != 0
        # finite nonzero outputs with room in the exponent field
        exp = (ob64 >> fmt.mbits) & ((1 << fmt.ebits) - 1)
        ok = nz & (exp + k > 0) & (exp + k < (1 << fmt.ebits) - 1) & (exp > 0)
        want = ob64 + (k << fmt.mbits)
        assert np.array_equal(os_[0].astype(np.int64)[ok], want[ok]), f"2^{k} scaling broken"
        assert ok.mean() > 0.9, "scaling check covered too few elements"
    # 3. negation: flip every sign bit; zeros compare equal regardless of sign
    xn = (x.astype(np.int64) ^ (1 << top)).astype(x.dtype)
    on = bits_of(orc.allreduce(xn.view(np.float32) if dtype == "fp32" else xn, dtype), dtype)
    a, b = ob[0].astype(np.int64), on[0].astype(np.int64)
    mag = (1 << top) - 1
    zero = (a & mag) == 0
    assert np.array_equal((a ^ (1 << top))[~zero], b[~zero]), "negation not symmetric"
    assert np.all((b[zero] & mag) == 0), "negation of a zero sum is not zero"
    # 4. one-hot columns: the single nonzero value passes through unchanged
    hot = rng.integers(0, R, n)
    xo = np.zeros_like(x)
    xo[hot, np.arange(n)] = x[hot, np.arange(n)]
    oo = bits_of(orc.allreduce(xo.view(np.float32) if dtype == "fp32" else xo, dtype), dtype)
    assert np.array_equal(oo[0], x[hot, np.arange(n)]), "one-hot column altered"
    # 5. R = 1 is the identity (finite data)
    o1 = bits_of(orc.allreduce(xv[:1].copy(), dtype), dtype)
    assert np.array_equal(o1[0], x[0]), "R=1 is not the identity"
    # 6. signed zeros: all +0 -> +0, all -0 -> -0, mixed -> +0
    for fill, want in ((0, 0), (1 << top, 1 << top)):
        z = np.full((R, 64), fill, dtype=x.dtype)
        oz = bits_of(orc.allreduce(z.view(np.float32) if dtype == "fp32" else z, dtype), dtype)
        assert np.all(oz.astype(np.int64) == want), f"all-{hex(fill)} zeros gave {hex(int(oz[0][0]))}"
    z = np.full((R, 64), 1 << top, dtype=x.dtype)
    z[R // 2] = 0
    oz = bits_of(orc.allreduce(z.view(np.float32) if dtype == "fp32" else z, dtype), dtype)
    assert np.all(oz == 0), "mixed-sign zeros must sum to +0"


# ---------------------------------------------------------------------------
# error bound
# ---------------------------------------------------------------------------
def pin_error_bound(orc, dtype: str, R: int, n: int = 1500, seed: int = 13):
    rng = np.random.default_rng(seed + R)
    fmt = em.FORMATS[dtype]
    hi = 8 if dtype == "fp16" else 10          # keep fp16 sums below 65504
    bits = random_bits(rng, dtype, (R, n), emin=-10, emax=hi)
    out = bits_of(orc.allreduce(bits.view(np.float32) if dtype == "fp32" else bits, dtype), dtype)
    u = Fraction(1, 1 << 24)
    gamma = (R - 1) * u / (1 - (R - 1) * u)
    for i in range(n):
        col = [int(b) for b in bits[:, i]]
        total, mags = em.exact_sum(col, dtype)
        y = em.value_of(int(out[0][i]), dtype)
        assert y is not None, "finite inputs gave a non-finite sum"
        # half an ulp of the output format at the larger of |y| and |total|
        big = max(abs(y), abs(total))
        e = max(em._floor_log2(big), fmt.emin) if big else fmt.emin
        half_ulp = Fraction(2) ** (e - fmt.mbits) / 2
        assert abs(y - total) <= gamma * mags + half_ulp, f"error bound broken at column {i}"


# ---------------------------------------------------------------------------
# converters against library routines
# ---------------------------------------------------------------------------
def _torch_bits(f32: np.ndarray, dtype: str) -> np.ndarray:
    t = torch.from_numpy(f32)
    tgt = torch.bfloat16 if dtype == "bf16" else torch.float16
    return t.to(tgt).view(torch.int16).numpy().view(np.uint16)


def converter_patterns_sample(seed: int = 17, n: int = 1 << 20) -> np.ndarray:
    """Random fp32 patterns plus every exponent with edge mantissas and ties."""
    rng = np.random.default_rng(seed)
    rand = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    exps = np.arange(256, dtype=np.uint32) << 23
    mants = np.array([0, 1, 2, 0x7FFF, 0x8000, 0x8001, 0x18000, 0xFFFF, 0x10000,
                      0xFFF, 0x1000, 0x1001, 0x3000, 0x7FFFFF, 0x7FFFFE, 0x400000,
                      0x7F8000, 0x7FE000, 0x7FF000], dtype=np.uint32)
    edge = (exps[:, None] | mants[None, :]).ravel()
    edge = np.concatenate([edge, edge | 0x80000000])
    return np.concatenate([rand, edge])


def pin_converters(orc, patterns: np.ndarray, nthreads: int = 8, with_numpy: bool = True):
    f = patterns.view(np.float32)
    for dtype, conv in (("bf16", orc.rne_bf16), ("fp16", orc.rne_fp16)):
        got = conv(f, nthreads=nthreads)
        assert_same_bits(got, _torch_bits(f, dtype), dtype, f"rne_{dtype} vs torch .to()")
    if with_numpy:
        # numpy's float16 cast is a second, independent library rounding
        with np.errstate(over="ignore", invalid="ignore"):
            npf16 = f.astype(np.float16).view(np.uint16)
        assert_same_bits(orc.rne_fp16(f, nthreads=nthreads), npf16, "fp16", "rne_fp16 vs numpy")


def pin_converters_slice(orc, start: int, count: int, nthreads: int = 8):
    """Patterns start .. start+count-1 (one sign half at a time), compared in torch."""
    assert count <= 1 << 31 and (start >> 31) == ((start + count - 1) >> 31)
    base = start - (1 << 32) if start >= 1 << 31 else start
    pats = torch.arange(count, dtype=torch.int32).add_(base)
    f = pats.view(torch.float32)
    fn = f.numpy()
    for dtype, conv, tgt, inf in (("bf16", orc.rne_bf16, torch.bfloat16, 0x7F80),
                                  ("fp16", orc.rne_fp16, torch.float16, 0x7C00)):
        got = torch.from_numpy(conv(fn, nthreads=nthreads).view(np.int16))
        want = f.to(tgt).view(torch.int16)
        gn = (got & 0x7FFF) > inf
        wn = (want & 0x7FFF) > inf
        bad = (gn != wn) | (~gn & ~wn & (got != want))
        nbad = int(bad.sum())
        if nbad:
            i = int(bad.nonzero()[0])
            raise AssertionError(f"rne_{dtype} vs torch: {nbad} mismatches in slice at {start:#x}, "
                                 f"first pattern {int(pats[i]) & 0xFFFFFFFF:#010x}: "
                                 f"got {int(got[i]) & 0xFFFF:#06x} want {int(want[i]) & 0xFFFF:#06x}")


def pin_widen_fp16(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.widen_fp16(h)
    want = h.view(np.float16).astype(np.float32)
    assert_same_bits(got, want.view(np.uint32), "fp32", "widen_fp16 vs numpy")


# ---------------------------------------------------------------------------
# hierarchical (grouped) order
# ---------------------------------------------------------------------------
GOLDEN_GROUPED = Path(__file__).resolve().parent / "golden" / "hand_cases_grouped.txt"


def load_grouped_hand_cases():
    """(dtype, group, [rank input bits], output bits) from the grouped fixture."""
    cases = []
    for line in GOLDEN_GROUPED.read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        dtype, group, ins, out = [t.strip() for t in line.split("|")]
        cases.append((dtype, int(group), [int(t, 16) for t in ins.split()], int(out, 16)))
    return cases


def pin_grouped_hand_cases(orc):
    cases = load_grouped_hand_cases()
    for dtype, group, ins, out in cases:
        got = orc.allreduce_grouped(to_array([ins], dtype), dtype, group)
        for r in range(len(ins)):
            assert_same_bits(got[r], np.array([out]), dtype,
                             f"grouped hand case {dtype} g={group} {[hex(v) for v in ins]}")
    assert len(cases) >= 5, "grouped hand-case fixture went missing"


@functools.lru_cache(maxsize=None)
def _grouped_cols(dtype: str, R: int, group: int, ncols: int, seed: int):
    rng = np.random.default_rng(seed)
    bits = random_bits(rng, dtype, (ncols, R))
    want = np.array([em.allreduce_column_grouped([int(b) for b in row], dtype, group)
                     for row in bits], dtype=np.int64)
    return bits, want


def pin_grouped_random(orc, dtype: str, R: int, group: int, ncols: int, seed: int = 3):
    bits, want = _grouped_cols(dtype, R, group, ncols, seed)
    x = bits.T.copy()
    if dtype == "fp32":
        x = x.view(np.float32)
    out = orc.allreduce_grouped(x, dtype, group, nthreads=2)
    for r in range(R):
        assert_same_bits(out[r], want, dtype, f"grouped {dtype} R={R} g={group} rank {r}")


@functools.lru_cache(maxsize=None)
def _grouped_exhaustive(dtype: str):
    vals = VALUE_SETS[dtype][:16]
    cols = [list(c) for c in itertools.product(vals, repeat=4)]
    want = np.array([em.allreduce_column_grouped(c, dtype, 2) for c in cols], dtype=np.int64)
    return cols, want


def pin_grouped_exhaustive(orc, dtype: str):
    """Every 4-rank column over 16 values, groups of 2, against the exact model."""
    cols, want = _grouped_exhaustive(dtype)
    out = orc.allreduce_grouped(to_array(cols, dtype), dtype, 2, nthreads=2)
    for r in range(4):
        assert_same_bits(out[r], want, dtype, f"grouped exhaustive {dtype} rank {r}")


def pin_grouped_integer(orc, dtype: str, R: int, group: int, n: int = 4096, seed: int = 9):
    rng = np.random.default_rng(seed + R)
    ints = rng.integers(-4, 5, (R, n), dtype=np.int64)
    fmt = em.FORMATS[dtype]
    enc = {v: em.encode(("fin", 1 if v < 0 else 0, Fraction(abs(v))), fmt) for v in range(-4, 5)}
    x = np.vectorize(enc.get)(ints).astype(np.uint32 if dtype == "fp32" else np.uint16)
    if dtype == "fp32":
        x = x.view(np.float32)
    out = orc.allreduce_grouped(x, dtype, group)
    assert_same_bits(out[0], _exact_int_bits(ints.sum(axis=0), dtype), dtype,
                     f"grouped integer {dtype} R={R} g={group}")


def check_order_tolerance(x_bits: np.ndarray, y1: np.ndarray, y2: np.ndarray, dtype: str):
    """Two summation orders of the same inputs agree to the rounding-error bound.

    Each binary32 order is within gamma_{R-1} * sum|x_j| of the exact sum
    (Higham, Accuracy and Stability of Numerical Algorithms, sec. 4.2), so two
    orders differ by at most twice that plus one unit in the last place of the
    output format.  Where the column does not cancel (|sum x| >= sum|x| / 2)
    that is at most one unit in the last place for bf16/fp16.  Returns the
    number of elements where the two differ."""
    R = x_bits.shape[0]
    fmt = em.FORMATS[dtype]
    if dtype == "fp32":
        xv = x_bits.view(np.float32).astype(np.float64)
        a, b = y1.view(np.float32).astype(np.float64), y2.view(np.float32).astype(np.float64)
    else:
        tdt = torch.bfloat16 if dtype == "bf16" else torch.float16
        conv = lambda u: torch.from_numpy(np.ascontiguousarray(u).view(np.int16)).view(tdt).double().numpy()
        xv, a, b = conv(x_bits), conv(y1), conv(y2)
    mags = np.abs(xv).sum(axis=0)
    total = xv.sum(axis=0)
    u = 2.0 ** -24
    gamma = (R - 1) * u / (1 - (R - 1) * u)
    big = np.maximum(np.abs(a), np.abs(b))
    e = np.maximum(np.floor(np.log2(np.where(big > 0, big, 1.0))), fmt.emin)
    ulp = np.exp2(e - fmt.mbits)
    diff = np.abs(a - b)
    bad = diff > 2 * gamma * mags + ulp
    assert not bad.any(), f"{int(bad.sum())} elements outside the two-order bound"
    if dtype != "fp32":
        well = np.abs(total) >= mags / 2
        assert np.all(diff[well] <= ulp[well]), "a well-conditioned column differs by > 1 ulp"
    else:
        # normwise relative difference against the exact sums
        rel = np.linalg.norm(a - b) / np.linalg.norm(total)
        assert rel <= 1e-6, f"fp32 normwise relative difference {rel:.3g} > 1e-6"
    return int((diff > 0).sum())
