"""The hierarchical (two-level) order, arOptNodeRanks, on the GPU.

R ranks form nodes of `group` consecutive ranks; the result is each node's
binary32 partial (rank order), summed over nodes in order, rounded once.  The
HB and LL kernels must match the grouped oracle bit for bit; against the flat order it
may differ only as two binary32 summation orders may (twice the recursive
summation bound plus one unit in the last place; one unit where the column
does not cancel).
"""
import numpy as np
import pytest
import torch

import all_reduce_amd as ar
import pins
from all_reduce_amd import inputs
from gpu_util import bits, dtype_name, from_bits, note, oracle_view, run_allreduce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def comm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = ar.Comm(device="cuda:0", max_ranks=32, max_ll_bytes_per_rank=1 << 20)
    yield c
    c.close()


def grouped(comm, group):
    class _Ctx:
        def __enter__(self):
            comm.set_option(ar.arOption.arOptNodeRanks, group)

        def __exit__(self, *exc):
            comm.set_option(ar.arOption.arOptNodeRanks, 0)
    return _Ctx()


def expect_grouped(orc, x, group):
    dt = dtype_name(x)
    out = orc.allreduce_grouped(oracle_view(x), dt, group, nthreads=16)
    return out.view(np.uint32) if dt == "fp32" else out.view(np.uint16)


def check(got, want, dt, what):
    g = bits(got)
    for r in range(g.shape[0]):
        pins.assert_same_bits(g[r], want[r], dt, f"{what} rank {r}")


@pytest.mark.parametrize("protocol", ["hb", "ll"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("R,group", [(16, 8), (32, 8), (32, 4), (32, 16), (32, 2), (16, 4),
                                     (16, 2), (8, 4), (8, 2), (4, 2), (24, 8), (12, 4), (12, 3)])
@pytest.mark.parametrize("N", [1, 7, 1029, 131072 + 13])
def test_grouped_matches_grouped_oracle(comm, orc, protocol, dtype, R, group, N):
    x = inputs.make(R, N, dtype, "outliers" if N > 1000 else "normal", seed=90 + R + group + N)
    with grouped(comm, group):
        got = run_allreduce(comm, x, protocol)
    check(got, expect_grouped(orc, x, group), dtype, f"grouped {protocol} R={R} g={group} N={N}")


@pytest.mark.parametrize("width", [8, 16])
@pytest.mark.parametrize("R,group", [(16, 8), (32, 4), (8, 2), (24, 8)])
def test_grouped_ll_packet_widths_in_place(comm, orc, width, R, group):
    """LL in the hierarchical order with each packet width, in place and out of
    place, at a size with several slices and a ragged last packet."""
    x = inputs.make(R, 100_003, "bf16", "outliers", seed=290 + R + group + width)
    want = expect_grouped(orc, x, group)
    comm.set_option(ar.arOption.arOptLLPacketBytes, width)
    try:
        with grouped(comm, group):
            check(run_allreduce(comm, x, "ll"), want, "bf16", f"grouped ll{width} R={R}")
            check(run_allreduce(comm, x, "ll", inplace=True), want, "bf16",
                  f"grouped ll{width} in place R={R}")
    finally:
        comm.set_option(ar.arOption.arOptLLPacketBytes, 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("R,group", [(16, 8), (32, 4), (32, 16), (8, 2), (24, 8)])
def test_grouped_with_cached_accesses(comm, orc, dtype, R, group):
    """The hierarchical kernels with ordinary (cached) loads and stores, the
    policy the tuner can pick: compile-time and run-time node sizes."""
    x = inputs.make(R, 70_001, dtype, "outliers", seed=190 + R + group)
    try:
        comm.set_option(ar.arOption.arOptHBNonTemporal, 0)
        with grouped(comm, group):
            got = run_allreduce(comm, x, "hb")
    finally:
        comm.set_option(ar.arOption.arOptHBNonTemporal, -1)
    check(got, expect_grouped(orc, x, group), dtype, f"grouped cached R={R} g={group}")


def test_grouped_in_place_and_auto(comm, orc):
    x = inputs.make(16, 100_003, "bf16", "outliers", seed=95)
    want = expect_grouped(orc, x, 8)
    with grouped(comm, 8):
        check(run_allreduce(comm, x, "hb", inplace=True), want, "bf16", "grouped in place")
        check(run_allreduce(comm, x, "auto"), want, "bf16", "grouped auto")


@pytest.mark.parametrize("R", [16, 32])
def test_c5_shapes_hierarchical(comm, orc, R):
    """2^18 fp16 integers per rank, nodes of 8: exact integer sums, grouped oracle."""
    x = inputs.make(**inputs.integer_case(R, "fp16"))
    with grouped(comm, 8):
        got = run_allreduce(comm, x, "hb")
    check(got, expect_grouped(orc, x, 8), "fp16", f"C5 fp16 R={R} nodes of 8")
    assert torch.equal(got[0].to(torch.int64), x.to(torch.int64).sum(0))


def test_c5_fp32_full_size_hierarchical(comm, orc):
    x = inputs.make(**inputs.integer_case(32, "fp32"))
    with grouped(comm, 8):
        got = run_allreduce(comm, x, "hb")
    exact = x.to(torch.int64).sum(0)
    assert torch.equal(got[31].to(torch.int64), exact)
    g = torch.Generator().manual_seed(98)
    idx = torch.randint(0, x.shape[1], (1 << 20,), generator=g)
    check(got[:, idx].contiguous(), expect_grouped(orc, x[:, idx].contiguous(), 8), "fp32",
          "C5 fp32 R=32 nodes of 8 sampled")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_flat_and_hierarchical_agree_to_the_rounding_bound(comm, dtype):
    """The two HB orders differ only as two binary32 summation orders may
    (an error bound, one ulp where the column does not cancel); inputs with
    24 binades of spread so that the orders really do round differently."""
    rng = np.random.default_rng(5)
    lo, hi = (-12, 12) if dtype != "fp16" else (-12, 10)
    xb = pins.random_bits(rng, dtype, (32, 100_000), emin=lo, emax=hi)
    x = from_bits(xb, dtype)
    flat = bits(run_allreduce(comm, x, "hb"))[0]
    with grouped(comm, 8):
        hier = bits(run_allreduce(comm, x, "hb"))[0]
    assert pins.check_order_tolerance(xb, flat, hier, dtype) > 0


def test_grouping_rules(comm):
    x = torch.zeros((12, 64), dtype=torch.bfloat16, device="cuda")
    p = [t.data_ptr() for t in x]
    s = torch.cuda.current_stream().cuda_stream
    note("grouping rules")
    with grouped(comm, 8):  # 12 ranks are not nodes of 8
        assert ar.arAllReduce(p, p, 64, 0, 0, 12, 1, comm.handle, s) == ar.arResult.arInvalidUsage
    y = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    q = [t.data_ptr() for t in y]
    with grouped(comm, 8):  # both protocols and auto run the hierarchical order
        for proto in (0, 1, 2):
            assert ar.arAllReduce(q, q, 64, 0, 0, 16, proto, comm.handle, s) == ar.arResult.arSuccess
    # the sequenced LL ablation keeps the flat order
    comm.set_option(ar.arOption.arOptLLFlagScheme, 1)
    try:
        with grouped(comm, 8):
            assert ar.arAllReduce(q, q, 64, 0, 0, 16, 0, comm.handle, s) == \
                ar.arResult.arUnsupported
    finally:
        comm.set_option(ar.arOption.arOptLLFlagScheme, 0)
    # the staged HB form becomes the two-level form, which needs a workspace
    comm.set_option(ar.arOption.arOptHBStaged, 1)
    try:
        with grouped(comm, 8):
            assert ar.arAllReduce(q, q, 64, 0, 0, 16, 1, comm.handle, s) == \
                ar.arResult.arInvalidUsage
    finally:
        comm.set_option(ar.arOption.arOptHBStaged, 0)
    comm.set_option(ar.arOption.arOptLLFlagScheme, 1)
    try:
        with grouped(comm, 8):  # auto avoids the sequenced LL scheme under a hierarchy
            assert ar.arAllReduce(q, q, 64, 0, 0, 16, 2, comm.handle, s) == ar.arResult.arSuccess
    finally:
        comm.set_option(ar.arOption.arOptLLFlagScheme, 0)
    with grouped(comm, 16):  # a group of all ranks is the flat order; LL allowed
        assert ar.arAllReduce(q, q, 64, 0, 0, 16, 0, comm.handle, s) == ar.arResult.arSuccess
    torch.cuda.synchronize()
    with pytest.raises(ar.ArError):
        comm.set_option(ar.arOption.arOptNodeRanks, 33)


def test_grouped_hand_cases(comm):
    """The hand-derived grouped cases, through the C ABI on the HB kernel."""
    for dtype, group, ins, out in pins.load_grouped_hand_cases():
        x = from_bits(pins.to_array([ins], dtype).view(
            np.uint32 if dtype == "fp32" else np.uint16), dtype)
        with grouped(comm, group):
            got = bits(run_allreduce(comm, x, "hb"))
        for r in range(len(ins)):
            pins.assert_same_bits(got[r], np.array([out]), dtype,
                                  f"grouped hand case {dtype} g={group} {[hex(v) for v in ins]}")
