"""The CPU oracle against its pins (see ``tests/pins.py`` for what each pins)."""
import numpy as np
import pytest

import exact_model as em
import pins

DTYPES = ["bf16", "fp16", "fp32"]


def test_hand_cases_agree_with_exact_model():
    # the hand derivations and the exact model are two independent routes
    for dtype, ins, want in pins.load_hand_cases():
        got = em.allreduce_column(ins, dtype)
        if em.is_nan_bits(want, dtype):
            assert em.is_nan_bits(got, dtype)
        else:
            assert got == want, (dtype, [hex(v) for v in ins])


def test_hand_cases(orc):
    pins.pin_hand_cases(orc)


@pytest.mark.parametrize("dtype", DTYPES)
def test_bruteforce_exhaustive_R3(orc, dtype):
    pins.pin_bruteforce_exhaustive(orc, dtype, R=3)


@pytest.mark.parametrize("dtype", DTYPES)
def test_bruteforce_exhaustive_R2(orc, dtype):
    pins.pin_bruteforce_exhaustive(orc, dtype, R=2)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,ncols", [(8, 3000), (16, 1500), (32, 800)])
def test_bruteforce_random(orc, dtype, R, ncols):
    pins.pin_bruteforce_random(orc, dtype, R, ncols)


@pytest.mark.parametrize("dtype", DTYPES)
def test_vector_model_agrees_with_exact_model(dtype):
    pins.pin_vector_model(dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R", [8, 16, 32])
def test_bruteforce_million_columns(orc, dtype, R):
    pins.pin_bruteforce_wide(orc, dtype, R)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,group", [(16, 8), (32, 8), (32, 4), (8, 2)])
def test_grouped_bruteforce_wide(orc, dtype, R, group):
    pins.pin_bruteforce_wide(orc, dtype, R, ncols=200_000, group=group)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R", [2, 3, 8, 16, 32])
def test_integer_closed_form(orc, dtype, R):
    pins.pin_integer_closed_form(orc, dtype, R)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_exact_partial_sums_give_correctly_rounded_sum(orc, dtype):
    pins.pin_exact_partials(orc, dtype)


@pytest.mark.parametrize("dtype", DTYPES)
def test_invariants(orc, dtype):
    pins.pin_invariants(orc, dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R", [2, 8, 32])
def test_error_bound(orc, dtype, R):
    pins.pin_error_bound(orc, dtype, R)


def test_converters_sample(orc):
    pins.pin_converters(orc, pins.converter_patterns_sample())


def test_widen_fp16_exhaustive(orc):
    pins.pin_widen_fp16(orc)


def test_converters_exhaustive(orc):
    """All 2^32 binary32 patterns, in slices, against torch and numpy."""
    step = 1 << 27
    for start in range(0, 1 << 32, step):
        pins.pin_converters_slice(orc, start, step)


def test_thread_count_does_not_change_bits(orc):
    rng = np.random.default_rng(3)
    x = pins.random_bits(rng, "bf16", (8, 100_003), emin=-20, emax=20)
    a = orc.allreduce(x, "bf16", nthreads=1)
    b = orc.allreduce(x, "bf16", nthreads=7)
    assert np.array_equal(a, b)


def test_in_place_equals_out_of_place(orc):
    rng = np.random.default_rng(4)
    x = pins.random_bits(rng, "bf16", (8, 5000), emin=-20, emax=20)
    want = orc.allreduce(x, "bf16")
    y = x.copy()
    orc.allreduce_into(list(y), list(y), "bf16")
    assert np.array_equal(y, want)


# ---- the hierarchical (grouped) order ----------------------------------------
def test_grouped_hand_cases(orc):
    pins.pin_grouped_hand_cases(orc)


@pytest.mark.parametrize("dtype", DTYPES)
def test_grouped_exhaustive_R4_groups_of_2(orc, dtype):
    pins.pin_grouped_exhaustive(orc, dtype)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,group,ncols", [(16, 8, 1500), (32, 8, 800), (8, 2, 2000), (8, 4, 2000)])
def test_grouped_random(orc, dtype, R, group, ncols):
    pins.pin_grouped_random(orc, dtype, R, group, ncols)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("R,group", [(16, 8), (32, 8), (32, 4)])
def test_grouped_integer_closed_form(orc, dtype, R, group):
    pins.pin_grouped_integer(orc, dtype, R, group)


def test_grouped_rejects_bad_groups(orc):
    x = np.zeros((6, 4), dtype=np.uint16)
    for g in (0, 4, 7):
        with pytest.raises(ValueError):
            orc.allreduce_grouped(x, "bf16", g)


def test_grouped_orders_really_differ(orc):
    # the pins above would pass for the flat order too if the two never differed
    rng = np.random.default_rng(12)
    x = pins.random_bits(rng, "fp32", (16, 20000), emin=-20, emax=20).view(np.float32)
    flat = orc.allreduce(x, "fp32")
    grouped = orc.allreduce_grouped(x, "fp32", 8)
    assert int((flat[0].view(np.uint32) != grouped[0].view(np.uint32)).sum()) > 100


@pytest.mark.parametrize("dtype", DTYPES)
def test_flat_and_grouped_orders_agree_to_the_rounding_bound(orc, dtype):
    rng = np.random.default_rng(5)
    lo, hi = (-12, 12) if dtype != "fp16" else (-12, 10)
    xb = pins.random_bits(rng, dtype, (32, 100_000), emin=lo, emax=hi)
    x = xb.view(np.float32) if dtype == "fp32" else xb
    flat = pins.bits_of(orc.allreduce(x, dtype, nthreads=4), dtype)[0]
    grouped = pins.bits_of(orc.allreduce_grouped(x, dtype, 8, nthreads=4), dtype)[0]
    assert pins.check_order_tolerance(xb, flat, grouped, dtype) > 0


@pytest.mark.parametrize("dtype", DTYPES)
def test_grouped_degenerate_groups_are_the_flat_order(orc, dtype):
    # nodes of one rank, or one node of every rank, add in the flat order 0..R-1
    rng = np.random.default_rng(21)
    xb = pins.random_bits(rng, dtype, (12, 5000), emin=-12, emax=12)
    x = xb.view(np.float32) if dtype == "fp32" else xb
    flat = pins.bits_of(orc.allreduce(x, dtype), dtype)
    for g in (1, 12):
        same = pins.bits_of(orc.allreduce_grouped(x, dtype, g), dtype)
        pins.assert_same_bits(same[0], flat[0], dtype, f"group {g}")


def test_timed_entry_point_computes_the_same(orc):
    # the CPU-baseline timing wrapper runs the pinned all-reduce unchanged
    rng = np.random.default_rng(22)
    xb = pins.random_bits(rng, "bf16", (8, 3001), emin=-8, emax=8)
    want = orc.allreduce(xb, "bf16")
    out = np.empty_like(xb)
    t = orc.allreduce_into(list(xb), list(out), "bf16", nthreads=2, timed=True)
    assert t >= 0.0
    pins.assert_same_bits(out[0], want[0], "bf16", "timed entry point")
    assert np.array_equal(out, want)
