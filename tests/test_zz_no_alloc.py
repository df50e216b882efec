"""arAllReduceNoAlloc, on the GPU: the HB all-reduce without a communicator,
whose staged two-level form keeps its node partials in the library's static
device scratch.

Through the C ABI, each call must give the same bits as arAllReduce on a
communicator in the same mode (the two-level form with a caller workspace, or
the fused flat kernel), which is itself held bit-exact against the oracle; two
calls in a row, the second smaller, so the second reads nothing the first
left behind.  Also: inside a graph, and the size and argument rules.
"""
import numpy as np
import pytest
import torch

import all_reduce_amd as ar
import pins
from all_reduce_amd import inputs
from gpu_util import CODES, bits, dtype_name, note, oracle_view

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def comm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = ar.Comm(device="cuda:0", max_ranks=32, max_ll_bytes_per_rank=1 << 12)
    c.set_workspace(torch.empty(64 << 20, dtype=torch.uint8, device=c.device))
    yield c
    c.close()


def planes(x, inplace=False):
    R, N = x.shape
    _, sv = ar.rank_buffers(R, N, x.dtype, "cuda:0")
    for r in range(R):
        sv[r].copy_(x[r])
    if inplace:
        return sv, sv
    plane, rv = ar.rank_buffers(R, N, x.dtype, "cuda:0")
    plane.view(torch.uint8).fill_(0xA5)
    return sv, rv


def no_alloc(x, node_ranks, inplace=False):
    R, N = x.shape
    sv, rv = planes(x, inplace)
    note(f"arAllReduceNoAlloc R={R} N={N} {dtype_name(x)} nodeRanks={node_ranks} "
         f"inplace={inplace}")
    rc = ar.arAllReduceNoAlloc([t.data_ptr() for t in sv], [t.data_ptr() for t in rv], N,
                               CODES[dtype_name(x)], ar.arRedOp.arSum, R, node_ranks,
                               torch.cuda.current_stream().cuda_stream)
    assert rc == ar.arResult.arSuccess, ar.arGetErrorString(rc)
    torch.cuda.synchronize()
    return torch.stack([t.cpu() for t in rv])


def with_comm(comm, x, node_ranks, inplace=False):
    R, N = x.shape
    sv, rv = planes(x, inplace)
    two_level = 1 < node_ranks < R
    comm.set_option(ar.arOption.arOptNodeRanks, node_ranks if two_level else 0)
    comm.set_option(ar.arOption.arOptHBStaged, 1 if two_level else 0)
    try:
        note(f"arAllReduce R={R} N={N} {dtype_name(x)} nodeRanks={node_ranks}")
        rc = ar.arAllReduce([t.data_ptr() for t in sv], [t.data_ptr() for t in rv], N,
                            CODES[dtype_name(x)], ar.arRedOp.arSum, R, ar.arProtocol.arProtoHB,
                            comm.handle, torch.cuda.current_stream().cuda_stream)
        assert rc == ar.arResult.arSuccess, ar.arGetErrorString(rc)
        torch.cuda.synchronize()
    finally:
        comm.set_option(ar.arOption.arOptNodeRanks, 0)
        comm.set_option(ar.arOption.arOptHBStaged, 0)
    return torch.stack([t.cpu() for t in rv])


def same(a, b, what):
    ga, gb = bits(a), bits(b)
    for r in range(ga.shape[0]):
        pins.assert_same_bits(ga[r], gb[r], dtype_name(a), f"{what} rank {r}")


@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
@pytest.mark.parametrize("dtype,R,node", [("fp16", 16, 8), ("bf16", 32, 8), ("fp32", 32, 4),
                                          ("bf16", 24, 8), ("fp32", 12, 3), ("bf16", 8, 0),
                                          ("fp32", 16, 16)])
def test_two_calls_match_arallreduce(comm, orc, dtype, R, node, inplace):
    """Two calls in a row, the second with a smaller input; each against
    arAllReduce in the same mode, and the two-level ones against the
    grouped oracle too."""
    for seed, N in ((700, 300_007), (701, 40_001)):
        x = inputs.make(R, N, dtype, "outliers", seed=seed + R + node)
        got = no_alloc(x, node, inplace)
        want = with_comm(comm, x, node, inplace)
        same(got, want, f"no-alloc vs arAllReduce R={R} node={node} N={N}")
        if 1 < node < R:
            ref = orc.allreduce_grouped(oracle_view(x), dtype, node, nthreads=16)
            ref = ref.view(np.uint32) if dtype == "fp32" else ref.view(np.uint16)
            g = bits(got)
            for r in range(R):
                pins.assert_same_bits(g[r], ref[r], dtype, f"no-alloc vs grouped oracle r{r}")


def test_largest_two_level_message(comm):
    """A message whose node partials fill the scratch exactly, then one that
    needs one more byte: the second is refused before anything runs."""
    R, node = 16, 8
    N = (ar.AR_NOALLOC_SCRATCH_BYTES // 2) // 4  # 2 nodes x N floats = the whole scratch
    x = inputs.make(R, N, "bf16", "int4", seed=702)
    got = no_alloc(x, node)
    exact = torch.zeros(N, dtype=torch.int32)
    for r in range(R):
        exact += x[r].to(torch.int32)
    for r in range(R):
        assert torch.equal(got[r].to(torch.int32), exact), f"rank {r}"
    # 16-byte aligned, non-overlapping addresses that are never dereferenced:
    # the size rule is checked before anything touches the device
    base, span = 0x7F0000000000, 1 << 26
    send = [base + r * span for r in range(R)]
    recv = [base + (R + r) * span for r in range(R)]
    rc = ar.arAllReduceNoAlloc(send, recv, N + 64, CODES["bf16"], ar.arRedOp.arSum, R, node,
                               torch.cuda.current_stream().cuda_stream)
    assert rc == ar.arResult.arInvalidUsage


def test_argument_rules():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    y = torch.zeros((12, 64), dtype=torch.bfloat16, device="cuda:0")
    p = [t.data_ptr() for t in y]
    s = torch.cuda.current_stream().cuda_stream
    assert ar.arAllReduceNoAlloc(p, p, 64, 0, 0, 12, 33, s) == ar.arResult.arInvalidArgument
    assert ar.arAllReduceNoAlloc(p, p, 64, 0, 0, 12, -1, s) == ar.arResult.arInvalidArgument
    assert ar.arAllReduceNoAlloc(p, p, 64, 0, 0, 12, 8, s) == ar.arResult.arInvalidUsage
    assert ar.arAllReduceNoAlloc(p, p, 64, 0, 1, 12, 4, s) == ar.arResult.arUnsupported
    assert ar.arAllReduceNoAlloc(p, p, 0, 0, 0, 12, 4, s) == ar.arResult.arSuccess
    assert ar.arAllReduceNoAlloc(p, p, 64, 0, 0, 12, 4, s) == ar.arResult.arSuccess
    torch.cuda.synchronize()


def test_in_graph_replays(orc):
    """Captured no-alloc calls replay with new inputs: every replay equals
    the grouped oracle."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R, N, node = 16, 100_003, 4
    _, sv = ar.rank_buffers(R, N, torch.float16, "cuda:0")
    plane, rv = ar.rank_buffers(R, N, torch.float16, "cuda:0")
    sp, rp = [t.data_ptr() for t in sv], [t.data_ptr() for t in rv]

    def call(stream):
        rc = ar.arAllReduceNoAlloc(sp, rp, N, CODES["fp16"], ar.arRedOp.arSum, R, node,
                                   stream.cuda_stream)
        assert rc == ar.arResult.arSuccess

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(torch.cuda.current_stream())
        call(torch.cuda.current_stream())
    for rep, seed in enumerate((710, 711)):
        x = inputs.make(R, N, "fp16", "outliers", seed=seed)
        for r in range(R):
            sv[r].copy_(x[r])
        plane.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        note(f"no-alloc graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        ref = orc.allreduce_grouped(oracle_view(x), "fp16", node, nthreads=16).view(np.uint16)
        got = bits(torch.stack([t.cpu() for t in rv]))
        for r in range(R):
            pins.assert_same_bits(got[r], ref[r], "fp16", f"no-alloc replay {rep} rank {r}")
