"""LL with 16-byte packets (arOptLLPacketBytes = 16), on the GPU.

A 16-byte packet carries two 4-byte payload words, each next to its own flag,
and is written and read as one 128-bit access.  The result must be the same
bits as with 8-byte packets and as the oracle, for every tail length (a
message can end 2, 4 or 6 bytes into its last packet), rank count, dtype, in
place, inside graphs, and when calls switch packet width (packet memory is
clean after every call, whichever width wrote it).
"""
import numpy as np
import pytest
import torch

import all_reduce_amd as ar
import pins
from all_reduce_amd import inputs
from gpu_util import CODES, PROTO, assert_parity, bits, expect, from_bits, note, run_allreduce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def comm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = ar.Comm(device="cuda:0", max_ranks=32, max_ll_bytes_per_rank=1 << 20)
    c.set_option(ar.arOption.arOptLLPacketBytes, 16)
    yield c
    c.close()


def check(comm, orc, x, inplace=False, what=""):
    got = run_allreduce(comm, x, "ll", inplace=inplace)
    assert_parity(got, expect(orc, x), what or f"ll16 {tuple(x.shape)} {x.dtype}")
    return got


def test_c1(comm, orc):
    check(comm, orc, inputs.make(**inputs.WORKLOADS["C1"]))


@pytest.mark.parametrize("k", range(10, 20))
def test_c2_sweep(comm, orc, k):
    check(comm, orc, inputs.make(**inputs.sweep(k)))


def test_c3_decode(comm, orc):
    check(comm, orc, inputs.make(**inputs.WORKLOADS["C3"]))


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8, 13, 16, 24, 32])
@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 6, 7, 9, 1023, 1025, 1026, 65536 + 5])
def test_tails_and_rank_counts(comm, orc, dtype, R, N):
    x = inputs.make(R, N, dtype, "normal", seed=3000 + R * 31 + N)
    check(comm, orc, x)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_largest_message_32_ranks(comm, orc, dtype):
    es = 2 if dtype == "bf16" else 4
    x = inputs.make(32, (1 << 20) // es, dtype, "outliers", seed=3100)
    check(comm, orc, x)


def test_in_place(comm, orc):
    x = inputs.make(8, 100_003, "bf16", "normal", seed=3101)
    a = run_allreduce(comm, x, "ll")
    b = run_allreduce(comm, x, "ll", inplace=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert_parity(b, expect(orc, x), "ll16 in place")


def test_switching_packet_width_between_calls(comm, orc):
    xs = [inputs.make(8, n, "bf16", "uniform", seed=3102 + n) for n in (4099, 70001, 1 << 19)]
    try:
        for width in (8, 16, 8, 16, 16, 8):
            comm.set_option(ar.arOption.arOptLLPacketBytes, width)
            for x in xs:
                check(comm, orc, x, what=f"width {width} N={x.shape[1]}")
    finally:
        comm.set_option(ar.arOption.arOptLLPacketBytes, 16)
    assert comm.async_error() == ar.arResult.arSuccess


@pytest.mark.parametrize("opt,values", [
    (ar.arOption.arOptLLThreads, [64, 128, 512, 1024]),
    (ar.arOption.arOptLLBlocksPerRank, [1, 3, 16, 64]),
])
def test_launch_shapes_keep_bits(comm, orc, opt, values):
    x = inputs.make(8, 200_003, "bf16", "outliers", seed=3103)
    want = expect(orc, x)
    try:
        for v in values:
            comm.set_option(opt, v)
            assert_parity(run_allreduce(comm, x, "ll"), want, f"ll16 {opt.name}={v}")
    finally:
        comm.set_option(opt, 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_exhaustive_value_set_three_ranks(comm, dtype):
    cols, want = pins._exhaustive_cols(dtype, 3)
    x = from_bits(pins.to_array(cols, dtype).view(np.uint32 if dtype == "fp32" else np.uint16),
                  dtype)
    got = run_allreduce(comm, x, "ll")
    for r in range(3):
        pins.assert_same_bits(bits(got[r]), want, dtype, f"ll16 value set {dtype} rank {r}")


def _call(comm, sv, rv, n):
    rc = ar.arAllReduce([t.data_ptr() for t in sv], [t.data_ptr() for t in rv], n,
                        CODES["bf16"], ar.arRedOp.arSum, len(sv), PROTO["ll"], comm.handle,
                        torch.cuda.current_stream().cuda_stream)
    assert rc == ar.arResult.arSuccess, ar.arGetErrorString(rc)


@pytest.mark.parametrize("N", [1024 + 3, 1 << 19])
def test_graph_replays(comm, orc, N):
    R = 8
    xa = inputs.make(R, N, "bf16", "uniform", seed=3104)
    xb = inputs.make(R, N, "bf16", "uniform", seed=3105)
    want_a, want_b = expect(orc, xa), expect(orc, xb)
    _, sa = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    _, sb = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    pa, da = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    pb, db = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    for r in range(R):
        sa[r].copy_(xa[r])
        sb[r].copy_(xb[r])
    note(f"ll16 graph N={N}: warm-up and capture of 10 calls")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _call(comm, sa, da, N)
        _call(comm, sb, db, N)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(10):
            _call(comm, sa if i % 2 == 0 else sb, da if i % 2 == 0 else db, N)
    torch.cuda.synchronize()
    x_small = inputs.make(R, 777, "bf16", "normal", seed=3106)
    for rep in range(3):
        note(f"ll16 graph N={N}: replay {rep}")
        pa.view(torch.uint8).fill_(0xA5)
        pb.view(torch.uint8).fill_(0x5A)
        g.replay()
        torch.cuda.synchronize()
        assert_parity(torch.stack([t.cpu() for t in da]), want_a, f"replay {rep} A")
        assert_parity(torch.stack([t.cpu() for t in db]), want_b, f"replay {rep} B")
        assert_parity(run_allreduce(comm, x_small, "ll"), expect(orc, x_small), "eager")
    assert comm.async_error() == ar.arResult.arSuccess


def test_forced_timeout_then_reset(comm, orc):
    x = inputs.make(8, 4096, "bf16", "uniform", seed=3107)
    assert comm.async_error() == ar.arResult.arSuccess
    try:
        comm.set_option(ar.arOption.arOptPollTimeoutUs, 2000)
        comm.set_option(ar.arOption.arOptDebugFlagSkew, 1)
        note("ll16 with a flag no producer writes (2 ms bound)")
        run_allreduce(comm, x, "ll")
        assert comm.async_error() == ar.arResult.arTimeout
    finally:
        comm.set_option(ar.arOption.arOptDebugFlagSkew, 0)
        comm.set_option(ar.arOption.arOptPollTimeoutUs, 2_000_000)
    comm.reset()
    assert comm.async_error() == ar.arResult.arSuccess
    check(comm, orc, x, what="ll16 after reset")


def test_option_values(comm):
    for bad in (4, 12, 32, -8):
        with pytest.raises(ar.ArError):
            comm.set_option(ar.arOption.arOptLLPacketBytes, bad)
    for good in (0, 8, 16):
        comm.set_option(ar.arOption.arOptLLPacketBytes, good)
        assert comm.get_option(ar.arOption.arOptLLPacketBytes) == good


def test_large_packet_region():
    """A communicator whose packet memory reaches 4 GiB (32 ranks x 64 MiB of LL
    message per rank): 16-byte packets are refused (their buffer offsets are
    32-bit), and an LL call with 8-byte packets whose last ranks' packets lie
    past the 4 GiB mark is exact (integer data, so the sum is known)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R, N = 32, (64 << 20) // 2
    with ar.Comm(device="cuda:0", max_ranks=R, max_ll_bytes_per_rank=64 << 20) as big:
        with pytest.raises(ar.ArError) as err:
            big.set_option(ar.arOption.arOptLLPacketBytes, 16)
        assert err.value.code == ar.arResult.arUnsupported
        big.set_option(ar.arOption.arOptLLPacketBytes, 8)
        g = torch.Generator(device="cuda").manual_seed(3200)
        plane, sv = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
        plane.copy_(torch.randint(-4, 5, plane.shape, generator=g, device="cuda").to(torch.bfloat16))
        want = torch.stack(sv).float().sum(0).to(torch.bfloat16)   # exact: |sum| <= 128
        _, rv = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
        note("LL, 32 ranks x 64 MiB, packets past 4 GiB")
        big.all_reduce(sv, rv, protocol="ll")
        torch.cuda.synchronize()
        assert big.async_error() == ar.arResult.arSuccess
        for r in range(R):
            assert torch.equal(rv[r].view(torch.int16), want.view(torch.int16)), f"rank {r}"
