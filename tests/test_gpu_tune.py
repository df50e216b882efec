"""Size-bucketed tuning (arCommTune) and arProtoAuto, on the GPU.

Tuning only changes launch shapes, so every result must stay bit-exact with
the oracle; the tuned table must cover every power-of-two size it was asked
for, in place and out of place, for each protocol the communicator can run
there.
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
    c = ar.Comm(device="cuda:0", max_ranks=16, max_ll_bytes_per_rank=1 << 20)
    note("arCommTune bf16 R=8 up to 4 MiB, fp32 R=16 up to 256 KiB")
    c.tune(torch.bfloat16, 8, 4 << 20)
    c.tune(torch.float32, 16, 256 << 10)
    yield c
    c.close()


@pytest.mark.parametrize("in_place", [False, True])
def test_table_covers_the_tuned_sizes(comm, in_place):
    for b in range(9, 23):
        hb = comm.tuned_shape(torch.bfloat16, 8, "hb", 1 << b, in_place)
        assert hb is not None and hb[0] in (0, 128, 256, 512) and hb[2] > 0
        assert hb[3] == 0 and hb[4] in (0, 1)
        ll = comm.tuned_shape(torch.bfloat16, 8, "ll", 1 << b, in_place)
        if (1 << b) <= comm.max_ll_bytes_per_rank:
            assert ll is not None and ll[0] in (0, 128, 256, 512, 1024) and ll[2] > 0
            assert ll[3] == 8 and ll[4] == 0  # the tuner times 8-byte packets only
        else:
            assert ll is None, "LL cannot run above maxLLBytesPerRank"
    # sizes round up to their bucket; untuned dtype / rank counts stay untuned
    assert comm.tuned_shape(torch.bfloat16, 8, "hb", 3000) == comm.tuned_shape(
        torch.bfloat16, 8, "hb", 4096)
    assert comm.tuned_shape(torch.float16, 8, "hb", 4096) is None
    assert comm.tuned_shape(torch.bfloat16, 8, "hb", 1 << 23) is None
    assert comm.tuned_shape(torch.float32, 16, "ll", 1 << 18) is not None


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("protocol", ["ll", "hb", "auto"])
@pytest.mark.parametrize("k", [10, 13, 16, 19, 21])
def test_tuned_shapes_keep_bits(comm, orc, protocol, k, in_place):
    if protocol == "ll" and ((1 << k) + 3) * 2 > comm.max_ll_bytes_per_rank:
        pytest.skip("above the communicator's LL limit")
    x = inputs.make(8, (1 << k) + 3, "bf16", "outliers", seed=60 + k)
    assert_parity(run_allreduce(comm, x, protocol, inplace=in_place), expect(orc, x),
                  f"tuned {protocol} 2^{k} in_place={in_place}")


def test_mode_argument_is_checked(comm):
    r = ar.arCommGetTunedShape(comm.handle, 0, 8, 1, 4096, 2)[0]
    assert r == ar.arResult.arInvalidArgument


def test_auto_on_untuned_sizes_and_fp32(comm, orc):
    x = inputs.make(16, 50_001, "fp32", "normal", seed=70)
    assert_parity(run_allreduce(comm, x, "auto"), expect(orc, x), "auto fp32 R=16")
    y = inputs.make(3, 10_007, "fp16", "normal", seed=71)
    assert_parity(run_allreduce(comm, y, "auto"), expect(orc, y), "auto fp16 R=3 untuned")
    assert comm.async_error() == ar.arResult.arSuccess


def test_options_override_the_table(comm, orc):
    x = inputs.make(8, 1 << 16, "bf16", "normal", seed=72)
    want = expect(orc, x)
    try:
        comm.set_option(ar.arOption.arOptLLThreads, 64)
        comm.set_option(ar.arOption.arOptHBThreads, 64)
        for proto in ("ll", "hb", "auto"):
            assert_parity(run_allreduce(comm, x, proto), want, f"override {proto}")
    finally:
        comm.set_option(ar.arOption.arOptLLThreads, 0)
        comm.set_option(ar.arOption.arOptHBThreads, 0)


def test_tuning_up_to_a_size_that_is_no_power_of_two(orc):
    """The last bucket is timed at the limit itself (5000 bytes here, bucket
    2^13); sizes in it use that entry, larger buckets stay untuned, and the
    tuned calls keep their bits."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with ar.Comm(device="cuda:0", max_ranks=4, max_ll_bytes_per_rank=1 << 16) as c:
        note("arCommTune fp16 R=4 up to 5000 bytes")
        c.tune(torch.float16, 4, 5000)
        for proto in ("ll", "hb"):
            for b in range(9, 14):
                assert c.tuned_shape(torch.float16, 4, proto, 1 << b) is not None
            assert c.tuned_shape(torch.float16, 4, proto, 5000) == c.tuned_shape(
                torch.float16, 4, proto, 8192)
            assert c.tuned_shape(torch.float16, 4, proto, 8193) is None
        for n in (2500, 2049, 17):
            x = inputs.make(4, n, "fp16", "normal", seed=80 + n)
            for proto in ("ll", "hb", "auto"):
                assert_parity(run_allreduce(c, x, proto), expect(orc, x), f"{proto} N={n}")


def test_tuning_on_fresh_inputs(orc):
    """arOptTuneFreshInputs = 1: each candidate is timed after a rewrite of its
    inputs, the rewrites' time subtracted.  The table covers every size and
    mode with positive times, calls keep their bits, and the tuner leaves the
    caller's buffers alone (it rewrites only its own scratch planes)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    with ar.Comm(device="cuda:0", max_ranks=8, max_ll_bytes_per_rank=1 << 18) as c:
        x = inputs.make(8, 70_001, "bf16", "normal", seed=91)
        want = expect(orc, x)
        _, sv = ar.rank_buffers(8, x.shape[1], torch.bfloat16, c.device)
        for r in range(8):
            sv[r].copy_(x[r])
        c.set_option(ar.arOption.arOptTuneFreshInputs, 1)
        note("arCommTune bf16 R=8 up to 4 MiB, fresh inputs")
        c.tune(torch.bfloat16, 8, 4 << 20)
        assert torch.equal(torch.stack([t.cpu() for t in sv]), x), "tuning touched caller data"
        for in_place in (False, True):
            for b in range(9, 23):
                hb = c.tuned_shape(torch.bfloat16, 8, "hb", 1 << b, in_place)
                assert hb is not None and hb[2] > 0 and hb[4] in (0, 1)
                ll = c.tuned_shape(torch.bfloat16, 8, "ll", 1 << b, in_place)
                assert (ll is not None and ll[2] > 0) == ((1 << b) <= (1 << 18))
        for proto in ("ll", "hb", "auto"):
            for in_place in (False, True):
                assert_parity(run_allreduce(c, x, proto, inplace=in_place), want,
                              f"fresh-tuned {proto} in_place={in_place}")
        assert c.async_error() == ar.arResult.arSuccess
