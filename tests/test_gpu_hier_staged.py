"""The staged two-level HB form (arOptHBStaged with arOptNodeRanks), on the GPU.

R = G * L ranks in G nodes of L: stage 1 writes each node's binary32 partial
(rank order inside the node) to the communicator's workspace, a kernel
boundary separates the levels, stage 2 folds the G partials in node order and
rounds once.  The result must equal the grouped oracle bit for bit, and the
fused HB kernel in the same order, for every shape, dtype, access policy, in
place and out of place, at the C5 shapes in full and inside graph replays.
"""
import functools

import numpy as np
import pytest
import torch

import all_reduce_amd as ar
import pins
from all_reduce_amd import inputs
from gpu_util import bits, dtype_name, note, oracle_view, run_allreduce

pytestmark = pytest.mark.gpu

WS_BYTES = 512 << 20  # node partials of the largest case: 4 nodes x 112 MiB


@pytest.fixture(scope="module")
def comm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = ar.Comm(device="cuda:0", max_ranks=32, max_ll_bytes_per_rank=1 << 16)
    c.set_workspace(torch.empty(WS_BYTES, dtype=torch.uint8, device=c.device))
    yield c
    c.close()


class two_level:
    """Staged two-level form in nodes of `group` for the duration of a block."""

    def __init__(self, comm, group, staged=True):
        self.comm, self.group, self.staged = comm, group, staged

    def __enter__(self):
        self.comm.set_option(ar.arOption.arOptNodeRanks, self.group)
        self.comm.set_option(ar.arOption.arOptHBStaged, 1 if self.staged else 0)

    def __exit__(self, *exc):
        self.comm.set_option(ar.arOption.arOptNodeRanks, 0)
        self.comm.set_option(ar.arOption.arOptHBStaged, 0)


def expect_grouped(orc, x, group):
    dt = dtype_name(x)
    out = orc.allreduce_grouped(oracle_view(x), dt, group, nthreads=16)
    return out.view(np.uint32) if dt == "fp32" else out.view(np.uint16)


def check(got, want, dt, what):
    g = bits(got)
    for r in range(g.shape[0]):
        pins.assert_same_bits(g[r], want[r], dt, f"{what} rank {r}")


@pytest.mark.parametrize("nt", [1, 0])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("R,group", [(16, 8), (32, 8), (32, 4), (32, 16), (32, 2), (16, 4),
                                     (8, 4), (8, 2), (4, 2), (24, 8), (12, 4), (12, 3),
                                     (30, 6), (32, 1)])
@pytest.mark.parametrize("N", [1, 7, 9, 1029, 131072 + 13])
def test_two_level_matches_grouped_oracle(comm, orc, nt, dtype, R, group, N):
    """Every compiled node size (2, 4, 8, 16) and node count (2, 4, 8, 16),
    run-time ones (3, 6 ranks per node; 3, 5 nodes), tails of every length
    and a multi-tile size; group 1 is the flat order (the fused kernel)."""
    x = inputs.make(R, N, dtype, "outliers" if N > 1000 else "normal",
                    seed=400 + R * 3 + group + N)
    want = expect_grouped(orc, x, group) if group > 1 else None
    comm.set_option(ar.arOption.arOptHBNonTemporal, nt)
    try:
        with two_level(comm, group):
            got = run_allreduce(comm, x, "hb")
            rec = comm.last_launch()
    finally:
        comm.set_option(ar.arOption.arOptHBNonTemporal, -1)
    if group > 1:
        assert rec["kernels"] == 2 and rec["staged"] == 1 and rec["nodeRanks"] == group
        check(got, want, dtype, f"two-level R={R} L={group} N={N} nt={nt}")
    else:
        from gpu_util import expect
        check(got, expect(orc, x), dtype, f"R={R} group 1 N={N}")


@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
@pytest.mark.parametrize("R,group", [(16, 8), (32, 8), (32, 4)])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_two_level_equals_fused_hierarchical(comm, R, group, dtype, inplace):
    """Same bits as the fused kernel in the same hierarchical order, on data
    where the order matters (0.1 % of entries x1000), in place and out."""
    N = 300_001
    x = inputs.make(R, N, dtype, "outliers", seed=500 + R + group)
    with two_level(comm, group, staged=False):
        fused = run_allreduce(comm, x, "hb", inplace=inplace)
    with two_level(comm, group):
        staged = run_allreduce(comm, x, "hb", inplace=inplace)
    assert torch.equal(bits_t(fused), bits_t(staged))


def bits_t(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


@functools.lru_cache(maxsize=1)
def _c5(R, dtype):
    x = inputs.make(**inputs.integer_case(R, dtype))
    exact = torch.zeros(x.shape[1], dtype=torch.int32)
    for r in range(R):
        exact += x[r].to(torch.int32)
    return x, exact


@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
@pytest.mark.parametrize("R", [16, 32])
def test_c5a_two_level(comm, orc, R, inplace):
    """C5a (R x 2^18 fp16 integers) in nodes of 8: the grouped oracle on every
    element, and the exact integer sums."""
    x, exact = _c5(R, "fp16")
    with two_level(comm, 8):
        got = run_allreduce(comm, x, "hb", inplace=inplace)
    check(got, expect_grouped(orc, x, 8), "fp16", f"C5a two-level R={R}")
    for r in range(R):
        assert torch.equal(got[r].to(torch.int32), exact), f"rank {r}"


@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
@pytest.mark.parametrize("R", [16, 32])
def test_c5b_two_level_full_size(comm, orc, R, inplace):
    """C5b (R x 4096*7168 fp32 integers, 112 MiB per rank) in nodes of 8: the
    exact integer sums on every element of every rank, the grouped oracle on
    2^20 sampled columns."""
    x, exact = _c5(R, "fp32")
    with two_level(comm, 8):
        got = run_allreduce(comm, x, "hb", inplace=inplace)
    exact_f = exact.to(torch.float32)
    for r in range(R):
        assert torch.equal(got[r], exact_f), f"rank {r}"
    idx = torch.randint(0, x.shape[1], (1 << 20,), generator=torch.Generator().manual_seed(99))
    want = expect_grouped(orc, x[:, idx].contiguous(), 8)
    check(got[:, idx].contiguous(), want, "fp32", f"C5b two-level R={R} sampled")


def test_two_level_in_graph_replays(comm, orc):
    """Captured calls replay correctly with new inputs between replays (the
    workspace is reused by every call).  The prepared call is made inside the
    capture, so it is bound to the capturing stream."""
    R, N, group = 16, 50_003, 4
    _, sv = ar.rank_buffers(R, N, torch.bfloat16, comm.device)
    plane, rv = ar.rank_buffers(R, N, torch.bfloat16, comm.device)
    g = torch.cuda.CUDAGraph()
    with two_level(comm, group):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            comm.prepare(sv, rv, "hb")()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            call = comm.prepare(sv, rv, "hb")
            call()
            call()
    for rep, seed in enumerate((601, 602, 603)):
        x = inputs.make(R, N, "bf16", "outliers", seed=seed)
        for r in range(R):
            sv[r].copy_(x[r])
        plane.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        note(f"two-level graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        check(torch.stack([t.cpu() for t in rv]), expect_grouped(orc, x, group), "bf16",
              f"two-level replay {rep}")
