"""LL with the sequenced flag scheme (arOptLLFlagScheme = 1), on the GPU.

The sequenced scheme is an ablation of the default, in which the reader
clears every packet it consumes.  Here nothing consumed is cleared: every
512-byte group of a rank's packet region has a sequence number, producers
flag packets with the group's next number and the group's single consumer
wave advances it.  What
can go wrong is a stale packet taken for a new one, so besides parity with the
oracle at every tail, rank count, dtype and packet width, these tests run long
mixed sequences of calls -- sizes that end inside a group after larger ones,
rank counts up and down, both schemes and both widths interleaved -- check every
call, replay graphs, and start the numbers just below their 32-bit wrap.
"""
import random

import numpy as np
import pytest
import torch

import all_reduce_amd as ar
import pins
from all_reduce_amd import inputs
from gpu_util import CODES, PROTO, assert_parity, bits, expect, from_bits, note, run_allreduce

pytestmark = pytest.mark.gpu

SCHEME = ar.arOption.arOptLLFlagScheme
WIDTH = ar.arOption.arOptLLPacketBytes


@pytest.fixture(scope="module")
def comm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = ar.Comm(device="cuda:0", max_ranks=32, max_ll_bytes_per_rank=1 << 20)
    c.set_option(SCHEME, 1)
    yield c
    c.close()


@pytest.fixture(params=[8, 16], ids=["pkt8", "pkt16"])
def width(comm, request):
    comm.set_option(WIDTH, request.param)
    yield request.param
    comm.set_option(WIDTH, 0)


def check(comm, orc, x, inplace=False, what=""):
    got = run_allreduce(comm, x, "ll", inplace=inplace)
    assert_parity(got, expect(orc, x), what or f"llseq {tuple(x.shape)} {x.dtype}")
    return got


def test_c1(comm, orc, width):
    check(comm, orc, inputs.make(**inputs.WORKLOADS["C1"]))


@pytest.mark.parametrize("k", range(10, 20))
def test_c2_sweep(comm, orc, width, k):
    check(comm, orc, inputs.make(**inputs.sweep(k)))


def test_c3_decode(comm, orc, width):
    check(comm, orc, inputs.make(**inputs.WORKLOADS["C3"]))


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8, 13, 16, 24, 32])
@pytest.mark.parametrize("N", [1, 3, 7, 9, 255, 257, 1023, 1025, 65536 + 5])
def test_tails_and_rank_counts(comm, orc, width, dtype, R, N):
    x = inputs.make(R, N, dtype, "normal", seed=5000 + R * 31 + N)
    check(comm, orc, x)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_largest_message_32_ranks(comm, orc, width, dtype):
    es = 2 if dtype == "bf16" else 4
    x = inputs.make(32, (1 << 20) // es, dtype, "outliers", seed=5100)
    check(comm, orc, x)


def test_in_place(comm, orc, width):
    x = inputs.make(8, 100_003, "bf16", "normal", seed=5101)
    a = run_allreduce(comm, x, "ll")
    b = run_allreduce(comm, x, "ll", inplace=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert_parity(b, expect(orc, x), "llseq in place")


def test_mixed_sequence_of_calls(comm, orc):
    """Seeded plan of calls that leaves stale packets behind on purpose: each
    call is checked, whatever scheme, width, rank count and size came before."""
    rng = random.Random(5102)
    sizes = [1, 2, 5, 63, 64, 65, 127, 129, 255, 256, 257, 1000, 4099, 40_000, 70_001,
             1 << 18, (1 << 19) - 1, 1 << 19]
    try:
        for i in range(80):
            scheme = rng.choice([0, 1, 1])
            width = rng.choice([8, 16])
            R = rng.choice([1, 2, 3, 4, 7, 8, 8, 16, 32])
            dtype = rng.choice(["bf16", "fp16", "fp32"])
            n = rng.choice(sizes)
            if dtype == "fp32":
                n = max(1, n // 2)
            comm.set_option(SCHEME, scheme)
            comm.set_option(WIDTH, width)
            x = inputs.make(R, n, dtype, "uniform", seed=5200 + i)
            check(comm, orc, x, what=f"call {i}: scheme {scheme} width {width} R={R} N={n} {dtype}")
    finally:
        comm.set_option(SCHEME, 1)
        comm.set_option(WIDTH, 0)
    assert comm.async_error() == ar.arResult.arSuccess


def test_shrinking_messages_end_inside_a_group(comm, orc, width):
    """Each call ends a few packets earlier than the last, inside the same
    512-byte group, so the previous call's packets sit just past the end."""
    R = 8
    for i, n in enumerate([1 << 16, (1 << 16) - 2, (1 << 16) - 3, (1 << 16) - 17, (1 << 16) - 130,
                           (1 << 16) - 255, 300, 257, 256, 255, 2, 1, 513, 1 << 16]):
        x = inputs.make(R, n, "bf16", "uniform", seed=5300 + i)
        check(comm, orc, x, what=f"shrinking call {i} N={n}")


@pytest.mark.parametrize("opt,values", [
    (ar.arOption.arOptLLThreads, [64, 128, 512, 1024]),
    (ar.arOption.arOptLLBlocksPerRank, [1, 3, 16, 64]),
])
def test_launch_shapes_keep_bits(comm, orc, width, opt, values):
    x = inputs.make(8, 200_003, "bf16", "outliers", seed=5103)
    want = expect(orc, x)
    try:
        for v in values:
            comm.set_option(opt, v)
            assert_parity(run_allreduce(comm, x, "ll"), want, f"llseq {opt.name}={v}")
    finally:
        comm.set_option(opt, 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_exhaustive_value_set_three_ranks(comm, dtype):
    cols, want = pins._exhaustive_cols(dtype, 3)
    x = from_bits(pins.to_array(cols, dtype).view(np.uint32 if dtype == "fp32" else np.uint16),
                  dtype)
    got = run_allreduce(comm, x, "ll")
    for r in range(3):
        pins.assert_same_bits(bits(got[r]), want, dtype, f"llseq value set {dtype} rank {r}")


def _call(comm, sv, rv, n):
    rc = ar.arAllReduce([t.data_ptr() for t in sv], [t.data_ptr() for t in rv], n,
                        CODES["bf16"], ar.arRedOp.arSum, len(sv), PROTO["ll"], comm.handle,
                        torch.cuda.current_stream().cuda_stream)
    assert rc == ar.arResult.arSuccess, ar.arGetErrorString(rc)


def test_graph_replays_of_mixed_sizes(comm, orc, width):
    """One graph of 10 calls, alternating a message that ends inside a group
    with a larger one; replayed with the outputs poisoned in between."""
    R = 8
    na, nb = 1027, 1 << 19
    xa = inputs.make(R, na, "bf16", "uniform", seed=5104)
    xb = inputs.make(R, nb, "bf16", "uniform", seed=5105)
    want_a, want_b = expect(orc, xa), expect(orc, xb)
    _, sa = ar.rank_buffers(R, na, torch.bfloat16, "cuda")
    _, sb = ar.rank_buffers(R, nb, torch.bfloat16, "cuda")
    pa, da = ar.rank_buffers(R, na, torch.bfloat16, "cuda")
    pb, db = ar.rank_buffers(R, nb, torch.bfloat16, "cuda")
    for r in range(R):
        sa[r].copy_(xa[r])
        sb[r].copy_(xb[r])
    note(f"llseq graph width {width}: warm-up and capture of 10 calls")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(comm, sa, da, na)
        _call(comm, sb, db, nb)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(10):
            if i % 2 == 0:
                _call(comm, sa, da, na)
            else:
                _call(comm, sb, db, nb)
    torch.cuda.synchronize()
    x_small = inputs.make(R, 777, "bf16", "normal", seed=5106)
    for rep in range(4):
        note(f"llseq graph width {width}: replay {rep}")
        pa.view(torch.uint8).fill_(0xA5)
        pb.view(torch.uint8).fill_(0x5A)
        g.replay()
        torch.cuda.synchronize()
        assert_parity(torch.stack([t.cpu() for t in da]), want_a, f"replay {rep} A")
        assert_parity(torch.stack([t.cpu() for t in db]), want_b, f"replay {rep} B")
        assert_parity(run_allreduce(comm, x_small, "ll"), expect(orc, x_small), "eager")
    assert comm.async_error() == ar.arResult.arSuccess


@pytest.mark.parametrize("start", [0xFFFFFFFC, 0xFFFFFFFE, 0xFFFFFFFF])
def test_sequence_numbers_wrap(comm, orc, start):
    """Table entries set just below the wrap by arCommReset: the numbers pass
    0xFFFFFFFE, skip 0 and 0xFFFFFFFF, and every call stays correct."""
    try:
        comm.set_option(ar.arOption.arOptDebugSeqStart, start)
        comm.reset()
        torch.cuda.synchronize()
        for i, n in enumerate([4099, 4099, 300, 4099, 1 << 16, 257, 4099, 1 << 16]):
            x = inputs.make(8, n, "bf16", "uniform", seed=5400 + i)
            check(comm, orc, x, what=f"start {start:#x} call {i} N={n}")
    finally:
        comm.set_option(ar.arOption.arOptDebugSeqStart, 0)
        comm.reset()
    assert comm.async_error() == ar.arResult.arSuccess


def test_forced_timeout_then_reset(comm, orc, width):
    x = inputs.make(8, 4096, "bf16", "uniform", seed=5107)
    assert comm.async_error() == ar.arResult.arSuccess
    try:
        comm.set_option(ar.arOption.arOptPollTimeoutUs, 2000)
        comm.set_option(ar.arOption.arOptDebugFlagSkew, 1)
        note(f"llseq width {width} with a flag no producer writes (2 ms bound)")
        run_allreduce(comm, x, "ll")
        assert comm.async_error() == ar.arResult.arTimeout
    finally:
        comm.set_option(ar.arOption.arOptDebugFlagSkew, 0)
        comm.set_option(ar.arOption.arOptPollTimeoutUs, 2_000_000)
    comm.reset()
    assert comm.async_error() == ar.arResult.arSuccess
    check(comm, orc, x, what="llseq after reset")
    check(comm, orc, x, what="llseq after reset, second call")


def test_option_values(comm):
    for bad in (2, -1, 16):
        with pytest.raises(ar.ArError):
            comm.set_option(SCHEME, bad)
    for good in (0, 1):
        comm.set_option(SCHEME, good)
        assert comm.get_option(SCHEME) == good
    comm.set_option(SCHEME, 1)
    for bad in (-1, 1 << 32):
        with pytest.raises(ar.ArError):
            comm.set_option(ar.arOption.arOptDebugSeqStart, bad)
    comm.set_option(ar.arOption.arOptDebugSeqStart, 0xFFFFFFFF)
    assert comm.get_option(ar.arOption.arOptDebugSeqStart) == 0xFFFFFFFF
    comm.set_option(ar.arOption.arOptDebugSeqStart, 0)


@pytest.mark.parametrize("scheme", [0, 1])
@pytest.mark.parametrize("width", [8, 16])
def test_odd_ll_limit_uses_the_whole_region(orc, scheme, width):
    """A communicator whose LL limit (1000 bytes per rank) is no whole number of
    512-byte packet groups: calls up to the limit, including one that ends a
    few packets before the end of the rounded region, stay exact in either
    scheme and width, and one element more is refused."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with ar.Comm(device="cuda:0", max_ranks=8, max_ll_bytes_per_rank=1000) as small:
        small.set_option(SCHEME, scheme)
        small.set_option(WIDTH, width)
        for i, n in enumerate([500, 499, 1, 257, 500, 64, 500]):
            x = inputs.make(8, n, "bf16", "uniform", seed=5500 + i)
            got = run_allreduce(small, x, "ll")
            assert_parity(got, expect(orc, x), f"limit 1000 B, N={n}, scheme {scheme}")
        _, bufs = ar.rank_buffers(8, 501, torch.bfloat16, "cuda")
        with pytest.raises(ar.ArError) as err:
            small.all_reduce(bufs, protocol="ll")
        assert err.value.code == ar.arResult.arInvalidUsage
        assert small.async_error() == ar.arResult.arSuccess
