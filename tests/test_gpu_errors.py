"""Error paths on the GPU, forced from the host so every kernel still exits.

An LL wait is bounded; a communicator option makes the consumers wait for a
flag value no producer writes, with a 2 ms bound, so each wait runs out,
records arTimeout and the kernel finishes.  arCommReset then clears the state
and the next call is correct again.
"""
import pytest
import torch

import all_reduce_amd as ar
from all_reduce_amd import inputs
from gpu_util import assert_parity, expect, note, run_allreduce

pytestmark = pytest.mark.gpu


@pytest.fixture()
def comm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = ar.Comm(device="cuda:0", max_ranks=8, max_ll_bytes_per_rank=1 << 16)
    yield c
    c.close()


def test_forced_timeout_is_reported_then_reset_recovers(comm, orc):
    x = inputs.make(8, 4096, "bf16", "uniform", seed=51)
    assert comm.async_error() == ar.arResult.arSuccess
    comm.set_option(ar.arOption.arOptPollTimeoutUs, 2000)
    comm.set_option(ar.arOption.arOptDebugFlagSkew, 1)
    note("LL with a flag no producer writes (2 ms bound)")
    run_allreduce(comm, x, "ll")
    assert comm.async_error() == ar.arResult.arTimeout
    comm.set_option(ar.arOption.arOptDebugFlagSkew, 0)
    # the error is sticky until reset
    run_allreduce(comm, x, "hb")
    assert comm.async_error() == ar.arResult.arTimeout
    comm.reset()
    assert comm.async_error() == ar.arResult.arSuccess
    note("LL after reset")
    assert_parity(run_allreduce(comm, x, "ll"), expect(orc, x), "after reset")
    assert comm.async_error() == ar.arResult.arSuccess


def test_limits_of_the_communicator(comm):
    x = torch.zeros((8, (1 << 16) // 2 + 8), dtype=torch.bfloat16, device="cuda")
    ptrs = [t.data_ptr() for t in x]
    s = torch.cuda.current_stream().cuda_stream
    # LL above maxLLBytesPerRank, and more ranks than the communicator holds
    assert ar.arAllReduce(ptrs, ptrs, x.shape[1], 0, 0, 8, 0, comm.handle, s) == \
        ar.arResult.arInvalidUsage
    y = torch.zeros((16, 64), dtype=torch.bfloat16, device="cuda")
    p16 = [t.data_ptr() for t in y]
    assert ar.arAllReduce(p16, p16, 64, 0, 0, 16, 0, comm.handle, s) == ar.arResult.arInvalidUsage
    # HB has no such limits
    assert ar.arAllReduce(p16, p16, 64, 0, 0, 16, 1, comm.handle, s) == ar.arResult.arSuccess
    torch.cuda.synchronize()


def test_option_ranges(comm):
    with pytest.raises(ar.ArError):
        comm.set_option(ar.arOption.arOptHBUnroll, 3)
    with pytest.raises(ar.ArError):
        comm.set_option(ar.arOption.arOptLLThreads, 96)
    comm.set_option(ar.arOption.arOptHBUnroll, 4)
    assert comm.get_option(ar.arOption.arOptHBUnroll) == 4
    # HB access policy: -1 (tuned, the default), 0 or 1
    with ar.Comm(device="cuda:0", max_ranks=2, max_ll_bytes_per_rank=0) as fresh:
        assert fresh.get_option(ar.arOption.arOptHBNonTemporal) == -1
    for bad in (-2, 2):
        with pytest.raises(ar.ArError):
            comm.set_option(ar.arOption.arOptHBNonTemporal, bad)
    # tuning method: 0 (unchanged inputs, the default) or 1 (fresh inputs)
    with ar.Comm(device="cuda:0", max_ranks=2, max_ll_bytes_per_rank=0) as fresh:
        assert fresh.get_option(ar.arOption.arOptTuneFreshInputs) == 0
    for bad in (-1, 2):
        with pytest.raises(ar.ArError):
            comm.set_option(ar.arOption.arOptTuneFreshInputs, bad)


def test_two_communicators_on_two_streams_at_once(orc):
    """Each communicator has its own packet memory, so LL calls of two of them
    may overlap in time on two streams."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from gpu_util import CODES, PROTO, assert_parity, expect
    comms = [ar.Comm(device="cuda:0", max_ranks=8, max_ll_bytes_per_rank=1 << 20)
             for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    R, N = 8, 100_003
    xs = [inputs.make(R, N, "bf16", "uniform", seed=60 + i) for i in range(2)]
    planes = []
    for x in xs:
        _, sv = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
        _, rv = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
        for r in range(R):
            sv[r].copy_(x[r])
        planes.append((sv, rv))
    torch.cuda.synchronize()
    note("two communicators, LL on two streams, 20 calls each")
    for _ in range(20):
        for c, st, (sv, rv) in zip(comms, streams, planes):
            rc = ar.arAllReduce([t.data_ptr() for t in sv], [t.data_ptr() for t in rv], N,
                                CODES["bf16"], ar.arRedOp.arSum, R, PROTO["ll"], c.handle,
                                st.cuda_stream)
            assert rc == ar.arResult.arSuccess
    torch.cuda.synchronize()
    for c, x, (sv, rv) in zip(comms, xs, planes):
        assert c.async_error() == ar.arResult.arSuccess
        assert_parity(torch.stack([t.cpu() for t in rv]), expect(orc, x), "concurrent LL")
        c.close()
