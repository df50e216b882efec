"""LL with three-element packets (arOptLLDense), on the GPU.

Each 8-byte packet carries three bfloat16 / float16 elements and a 16-bit
flag; the kernel stages its data through LDS to keep its accesses coalesced.
It must give the oracle's bits for every message length (a message can end
one or two elements into its last packet, anywhere in a 512-packet put round
or a 16-byte output vector), rank count, launch shape, in place, in graphs,
interleaved with word-packet calls on the same communicator (packet memory is
zero between calls in both formats), and it must report and recover from a
forced timeout like the word-packet kernel.
"""
import pytest
import torch

import all_reduce_amd as ar
from all_reduce_amd import inputs
from gpu_util import assert_parity, expect, note, run_allreduce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def comm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = ar.Comm(device="cuda:0", max_ranks=32, max_ll_bytes_per_rank=1 << 20)
    yield c
    c.close()


class dense:
    def __init__(self, comm, value=1, threads=0, blocks=0):
        self.comm, self.value, self.threads, self.blocks = comm, value, threads, blocks

    def __enter__(self):
        self.comm.set_option(ar.arOption.arOptLLDense, self.value)
        self.comm.set_option(ar.arOption.arOptLLThreads, self.threads)
        self.comm.set_option(ar.arOption.arOptLLBlocksPerRank, self.blocks)

    def __exit__(self, *exc):
        self.comm.set_option(ar.arOption.arOptLLDense, -1)
        self.comm.set_option(ar.arOption.arOptLLThreads, 0)
        self.comm.set_option(ar.arOption.arOptLLBlocksPerRank, 0)


def check(comm, orc, x, inplace=False, what=""):
    got = run_allreduce(comm, x, "ll", inplace=inplace)
    rec = comm.last_launch()
    assert rec["packetPayloadBytes"] == 6 and rec["packetBytes"] == 8, rec
    assert_parity(got, expect(orc, x), what or f"dense {tuple(x.shape)} {x.dtype}")
    return got


LENGTHS = [1, 2, 3, 4, 5, 7, 8, 9, 23, 24, 25, 47, 48, 191, 192, 193, 1535, 1536, 1537,
           3 * 4096 + 1, 65536 + 5, 131072 + 13, 1 << 18, (1 << 19) - 1, 1 << 19]


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("R", [1, 2, 3, 8, 13, 16, 32])
@pytest.mark.parametrize("N", LENGTHS)
def test_lengths_and_rank_counts(comm, orc, dtype, R, N):
    x = inputs.make(R, N, dtype, "normal", seed=800 + R * 37 + N)
    with dense(comm):
        check(comm, orc, x, what=f"dense R={R} N={N} {dtype}")


@pytest.mark.parametrize("R", [8, 32])
@pytest.mark.parametrize("threads", [64, 128, 256, 512])
@pytest.mark.parametrize("blocks", [1, 3, 8, 64])
def test_launch_shapes(comm, orc, R, threads, blocks):
    x = inputs.make(R, 100_003, "bf16", "outliers", seed=900 + R + threads + blocks)
    with dense(comm, threads=threads, blocks=blocks):
        check(comm, orc, x, what=f"dense R={R} {threads}x{blocks}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("R,N", [(8, 1 << 19), (8, 70_001), (16, 1 << 18), (32, 33_335), (5, 4099)])
def test_in_place(comm, orc, dtype, R, N):
    x = inputs.make(R, N, dtype, "outliers", seed=950 + R + N)
    with dense(comm):
        check(comm, orc, x, inplace=True, what=f"dense in place R={R} N={N}")


def test_default_picks_the_format_by_size(comm, orc):
    """By default bfloat16 / float16 take three-element packets above 512 KiB
    per rank at 1, 2 and 4 ranks, from 256 KiB at 3 and 5 to 8 ranks, above
    128 KiB from 9 to 16 ranks and from 128 KiB above 16, word packets below;
    float32 always word packets."""
    for R, n, dtype, payload in ((8, (256 << 10) // 2, "bf16", 6), (8, (192 << 10) // 2, "bf16", 4),
                                 (2, (512 << 10) // 2, "bf16", 4), (2, (640 << 10) // 2, "bf16", 6),
                                 (4, (512 << 10) // 2, "fp16", 4), (4, (1 << 20) // 2, "fp16", 6),
                                 (3, (256 << 10) // 2, "bf16", 6), (6, (256 << 10) // 2, "bf16", 6),
                                 (16, (256 << 10) // 2, "fp16", 6), (16, (128 << 10) // 2, "fp16", 4),
                                 (16, (128 << 10) // 2 + 1, "fp16", 6), (12, (136 << 10) // 2, "bf16", 6),
                                 (12, (128 << 10) // 2, "bf16", 4),
                                 (32, (128 << 10) // 2, "bf16", 6), (32, (64 << 10) // 2, "bf16", 4),
                                 (8, 1 << 18, "fp32", 4)):
        x = inputs.make(R, n, dtype, "normal", seed=960 + R + n)
        assert_parity(run_allreduce(comm, x, "ll"), expect(orc, x), f"default R={R} n={n}")
        assert comm.last_launch()["packetPayloadBytes"] == payload, (R, n, dtype)


def test_mixed_with_word_packets(comm, orc):
    """A seeded sequence of calls that switch packet format, width, rank count
    and size on one communicator: each is bit-exact (every format leaves the
    packet memory zero)."""
    g = torch.Generator().manual_seed(970)
    for i in range(60):
        R = [2, 5, 8, 16, 32][int(torch.randint(0, 5, (1,), generator=g))]
        N = int(torch.randint(1, 200_000, (1,), generator=g))
        fmt = int(torch.randint(0, 3, (1,), generator=g))  # 0 word 8 B, 1 word 16 B, 2 dense
        dtype = "bf16" if i % 2 else "fp16"
        x = inputs.make(R, N, dtype, "normal", seed=980 + i)
        comm.set_option(ar.arOption.arOptLLDense, 1 if fmt == 2 else 0)
        comm.set_option(ar.arOption.arOptLLPacketBytes, 16 if fmt == 1 else 8)
        try:
            assert_parity(run_allreduce(comm, x, "ll"), expect(orc, x),
                          f"mixed call {i} R={R} N={N} fmt={fmt}")
        finally:
            comm.set_option(ar.arOption.arOptLLDense, -1)
            comm.set_option(ar.arOption.arOptLLPacketBytes, 0)
    assert comm.async_error() == ar.arResult.arSuccess


def test_graph_replays_with_new_inputs(comm, orc):
    R, N = 8, 300_001
    _, sv = ar.rank_buffers(R, N, torch.bfloat16, comm.device)
    plane, rv = ar.rank_buffers(R, N, torch.bfloat16, comm.device)
    g = torch.cuda.CUDAGraph()
    with dense(comm):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            comm.prepare(sv, rv, "ll")()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            call = comm.prepare(sv, rv, "ll")
            for _ in range(3):
                call()
    for rep, seed in enumerate((990, 991, 992)):
        x = inputs.make(R, N, "bf16", "outliers", seed=seed)
        for r in range(R):
            sv[r].copy_(x[r])
        plane.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        note(f"dense graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        assert_parity(torch.stack([t.cpu() for t in rv]), expect(orc, x), f"dense replay {rep}")
    assert comm.async_error() == ar.arResult.arSuccess


def test_forced_timeout_then_reset(orc):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with ar.Comm(device="cuda:0", max_ranks=8, max_ll_bytes_per_rank=1 << 18) as c:
        x = inputs.make(8, 40_000, "bf16", "uniform", seed=995)
        c.set_option(ar.arOption.arOptLLDense, 1)
        c.set_option(ar.arOption.arOptPollTimeoutUs, 2000)
        c.set_option(ar.arOption.arOptDebugFlagSkew, 1)
        note("dense LL with a flag no producer writes (2 ms bound)")
        run_allreduce(c, x, "ll")
        assert c.async_error() == ar.arResult.arTimeout
        c.set_option(ar.arOption.arOptDebugFlagSkew, 0)
        c.reset()
        assert c.async_error() == ar.arResult.arSuccess
        note("dense LL after reset")
        assert_parity(run_allreduce(c, x, "ll"), expect(orc, x), "dense after reset")
        assert c.async_error() == ar.arResult.arSuccess
