"""Calls captured in a HIP graph and replayed (through torch.cuda.CUDAGraph).

Replays freeze the kernel arguments, so nothing in an LL call may depend on a
per-call value from the host: packet memory must be clean after every call,
or two inputs alternating in one graph would read each other's stale packets.
Every replay is checked against the oracle, with eager calls and
synchronisations between replays.
"""
import pytest
import torch

import all_reduce_amd as ar
from all_reduce_amd import inputs
from gpu_util import CODES, PROTO, assert_parity, expect, note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def comm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = ar.Comm(device="cuda:0", max_ranks=32, max_ll_bytes_per_rank=1 << 20)
    yield c
    c.close()


def call(comm, sv, rv, n, dtype, protocol):
    rc = ar.arAllReduce([t.data_ptr() for t in sv], [t.data_ptr() for t in rv], n,
                        CODES[dtype], ar.arRedOp.arSum, len(sv), PROTO[protocol], comm.handle,
                        torch.cuda.current_stream().cuda_stream)
    assert rc == ar.arResult.arSuccess, ar.arGetErrorString(rc)


@pytest.mark.parametrize("protocol", ["ll", "hb"])
@pytest.mark.parametrize("N", [1024, 65536 + 3, 1 << 19])
def test_graph_alternating_inputs(comm, orc, protocol, N):
    R, dt = 8, "bf16"
    xa = inputs.make(R, N, dt, "uniform", seed=41)
    xb = inputs.make(R, N, dt, "uniform", seed=42)
    want_a, want_b = expect(orc, xa), expect(orc, xb)
    _, sa = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    _, sb = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    pa, da = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    pb, db = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    for r in range(R):
        sa[r].copy_(xa[r])
        sb[r].copy_(xb[r])
    note(f"graph {protocol} N={N}: warm-up")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            call(comm, sa, da, N, dt, protocol)
            call(comm, sb, db, N, dt, protocol)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    note(f"graph {protocol} N={N}: capture 10 calls")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(10):
            if i % 2 == 0:
                call(comm, sa, da, N, dt, protocol)
            else:
                call(comm, sb, db, N, dt, protocol)
    torch.cuda.synchronize()

    x_small = inputs.make(R, 777, dt, "normal", seed=43)
    for rep in range(4):
        note(f"graph {protocol} N={N}: replay {rep}")
        pa.view(torch.uint8).fill_(0xA5)
        pb.view(torch.uint8).fill_(0x5A)
        g.replay()
        torch.cuda.synchronize()
        assert_parity(torch.stack([t.cpu() for t in da]), want_a, f"replay {rep} A")
        assert_parity(torch.stack([t.cpu() for t in db]), want_b, f"replay {rep} B")
        # eager work of another size between replays uses the same packet memory
        from gpu_util import run_allreduce
        assert_parity(run_allreduce(comm, x_small, protocol), expect(orc, x_small), "eager")
    assert comm.async_error() == ar.arResult.arSuccess


@pytest.mark.parametrize("protocol,pkt", [("ll", 8), ("ll", 16), ("hb", 0)])
@pytest.mark.parametrize("N", [1024 + 3, 65536 + 5, 1 << 19])
def test_stress_thousands_of_replayed_calls(comm, orc, protocol, pkt, N):
    """50 calls alternating two inputs in one graph, replayed 40 times (2000
    calls): every replay's outputs and the error word are checked, so a packet
    left stale by any call would show up in the next one."""
    R, dt = 8, "bf16"
    xa = inputs.make(R, N, dt, "uniform", seed=141)
    xb = inputs.make(R, N, dt, "normal", seed=142)
    want_a, want_b = expect(orc, xa), expect(orc, xb)
    _, sa = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    _, sb = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    _, da = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    _, db = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    for r in range(R):
        sa[r].copy_(xa[r])
        sb[r].copy_(xb[r])
    old = comm.get_option(ar.arOption.arOptLLPacketBytes)
    comm.set_option(ar.arOption.arOptLLPacketBytes, pkt)
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(comm, sa, da, N, dt, protocol)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(50):
                call(comm, sa if i % 2 == 0 else sb, da if i % 2 == 0 else db, N, dt, protocol)
        torch.cuda.synchronize()
        note(f"stress {protocol}/{pkt} N={N}: 40 replays of 50 calls")
        for rep in range(40):
            g.replay()
            if rep % 10 == 9:
                torch.cuda.synchronize()
                assert comm.async_error() == ar.arResult.arSuccess, f"replay {rep}"
                assert_parity(torch.stack([t.cpu() for t in da]), want_a, f"A after {rep}")
                assert_parity(torch.stack([t.cpu() for t in db]), want_b, f"B after {rep}")
        torch.cuda.synchronize()
        del g
    finally:
        comm.set_option(ar.arOption.arOptLLPacketBytes, old)
    assert comm.async_error() == ar.arResult.arSuccess


@pytest.mark.parametrize("scheme", [0, 1])
def test_reset_captured_in_a_graph(comm, orc, scheme):
    """arCommReset enqueues a kernel and records no memset, so it may sit inside
    a captured graph: a reset followed by LL calls of two inputs, replayed with
    the outputs poisoned in between, in either LL flag scheme."""
    R, N, dt = 8, 70_001, "bf16"
    xa = inputs.make(R, N, dt, "uniform", seed=45)
    xb = inputs.make(R, N, dt, "uniform", seed=46)
    want_a, want_b = expect(orc, xa), expect(orc, xb)
    _, sa = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    _, sb = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    pa, da = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    pb, db = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    for r in range(R):
        sa[r].copy_(xa[r])
        sb[r].copy_(xb[r])
    comm.set_option(ar.arOption.arOptLLFlagScheme, scheme)
    try:
        note(f"graph with arCommReset, scheme {scheme}: warm-up")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            comm.reset()
            call(comm, sa, da, N, dt, "ll")
            call(comm, sb, db, N, dt, "ll")
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            comm.reset()
            call(comm, sa, da, N, dt, "ll")
            call(comm, sb, db, N, dt, "ll")
        torch.cuda.synchronize()
        for rep in range(4):
            note(f"graph with arCommReset, scheme {scheme}: replay {rep}")
            pa.view(torch.uint8).fill_(0xA5)
            pb.view(torch.uint8).fill_(0x5A)
            g.replay()
            torch.cuda.synchronize()
            assert_parity(torch.stack([t.cpu() for t in da]), want_a, f"replay {rep} A")
            assert_parity(torch.stack([t.cpu() for t in db]), want_b, f"replay {rep} B")
            # an eager call between replays, on the state the graph left
            call(comm, sb, da, N, dt, "ll")
            torch.cuda.synchronize()
            assert_parity(torch.stack([t.cpu() for t in da]), want_b, f"eager after {rep}")
        assert comm.async_error() == ar.arResult.arSuccess
    finally:
        comm.set_option(ar.arOption.arOptLLFlagScheme, 0)


@pytest.mark.parametrize("protocol", ["ll", "hb"])
def test_prepared_calls_captured(comm, orc, protocol):
    """Calls made with Comm.prepare inside the capture (so they are bound to the
    capturing stream) replay like direct calls: each replay, with new inputs
    copied in between, matches the oracle."""
    R, N, dt = 8, 40_003, "bf16"
    plane, sv = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    _, rv = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    x0 = inputs.make(R, N, dt, "normal", seed=4300)
    for r in range(R):
        sv[r].copy_(x0[r])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        warm = comm.prepare(sv, rv, protocol)
        warm()
        warm()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    note(f"prepared {protocol}: capture 3 calls")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step = comm.prepare(sv, rv, protocol)
        for _ in range(3):
            step()
    for i in range(3):
        x = inputs.make(R, N, dt, "normal", seed=4301 + i)
        for r in range(R):
            sv[r].copy_(x[r])
        rv[0].zero_()
        torch.cuda.synchronize()
        note(f"prepared {protocol}: replay {i}")
        g.replay()
        torch.cuda.synchronize()
        assert_parity(torch.stack([t.cpu() for t in rv]), expect(orc, x),
                      f"prepared {protocol} replay {i}")
    assert comm.async_error() == ar.arResult.arSuccess
