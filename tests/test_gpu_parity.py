"""GPU parity: the HIP all-reduce, called through the C ABI, against the oracle.

The bar is bit-exact equality (NaNs by class): the kernels sum in the same
rank order 0..R-1 in binary32 and round once with RNE, like the oracle.
Inputs come from ``all_reduce_amd.inputs`` (seeded), never from the GPU path.
"""
import functools

import numpy as np
import pytest
import torch

import all_reduce_amd as ar
import exact_model as em
import pins
from all_reduce_amd import inputs
from gpu_util import assert_parity, bits, expect, from_bits, note, run_allreduce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def comm():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = ar.Comm(device="cuda:0", max_ranks=32, max_ll_bytes_per_rank=1 << 20)
    yield c
    c.close()


def check(comm, orc, x, protocol, inplace=False, what=""):
    got = run_allreduce(comm, x, protocol, inplace=inplace)
    assert_parity(got, expect(orc, x), what or f"{protocol} {tuple(x.shape)} {x.dtype}")
    return got


# ---- the named workloads ----------------------------------------------------
@pytest.mark.parametrize("protocol", ["ll", "hb"])
def test_c1_small_bf16(comm, orc, protocol):
    x = inputs.make(**inputs.WORKLOADS["C1"])
    check(comm, orc, x, protocol)


@pytest.mark.parametrize("k", range(10, 20))
@pytest.mark.parametrize("protocol", ["ll", "hb"])
def test_c2_message_sweep(comm, orc, k, protocol):
    x = inputs.make(**inputs.sweep(k))
    check(comm, orc, x, protocol)


def test_c3_decode_ll_and_hb_agree(comm, orc):
    x = inputs.make(**inputs.WORKLOADS["C3"])
    a = check(comm, orc, x, "ll")
    b = check(comm, orc, x, "hb")
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_c4_prefill_in_place_full_size(comm, orc):
    """8 x 64M bf16 with 0.1% outliers, in place, checked element by element."""
    x = inputs.make(**inputs.WORKLOADS["C4"])
    want = expect(orc, x)
    got = run_allreduce(comm, x, "hb", inplace=True)
    assert_parity(got, want, "C4 in place")
    # the outliers make the result order-sensitive, so this parity checks the order
    rev = orc.allreduce(bits(x.flip(0)), "bf16", nthreads=16)
    assert int((rev[0] != want[0]).sum()) > 0


@functools.lru_cache(maxsize=2)
def _c5_case(R, dtype):
    """C5 inputs (integers -4..4) and their exact sums, computed once per shape."""
    x = inputs.make(**inputs.integer_case(R, dtype))
    exact = torch.zeros(x.shape[1], dtype=torch.int32)
    for r in range(R):
        exact += x[r].to(torch.int32)
    return x, exact


@pytest.fixture
def chunk_layout(comm, request):
    """HB chunk layout for one test (0: contiguous N/R chunks, 1: interleaved
    tiles), restored to the default afterwards."""
    comm.set_option(ar.arOption.arOptHBChunkLayout, request.param)
    yield request.param
    comm.set_option(ar.arOption.arOptHBChunkLayout, 1)


@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
@pytest.mark.parametrize("chunk_layout", [0, 1], ids=["chunk_N_over_R", "interleaved"],
                         indirect=True)
@pytest.mark.parametrize("R", [16, 32])
def test_c5_fp16_integer_sums(comm, orc, R, chunk_layout, inplace):
    """R x 2^18 fp16 integers, HB with chunk = N/R (the configured layout) and
    with interleaved tiles: oracle on every element, exact integer sums."""
    x, exact = _c5_case(R, "fp16")
    got = check(comm, orc, x, "hb", inplace=inplace,
                what=f"C5 fp16 R={R} layout={chunk_layout} inplace={inplace}")
    for r in range(R):
        assert torch.equal(got[r].to(torch.int32), exact), f"rank {r}"


@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
@pytest.mark.parametrize("chunk_layout", [0, 1], ids=["chunk_N_over_R", "interleaved"],
                         indirect=True)
@pytest.mark.parametrize("R", [16, 32])
def test_c5_fp32_integer_sums_full_size(comm, orc, R, chunk_layout, inplace):
    """R x 4096*7168 fp32, HB with chunk = N/R (the configured layout) and with
    interleaved tiles: exact integer sums on every element of every rank, the
    oracle on 2^20 sampled columns."""
    x, exact = _c5_case(R, "fp32")
    got = run_allreduce(comm, x, "hb", inplace=inplace)
    exact_f = exact.to(torch.float32)
    for r in range(R):
        assert torch.equal(got[r], exact_f), f"rank {r}"
    g = torch.Generator().manual_seed(99)
    idx = torch.randint(0, x.shape[1], (1 << 20,), generator=g)
    want = expect(orc, x[:, idx].contiguous())
    assert_parity(got[:, idx].contiguous(), want,
                  f"C5 fp32 R={R} layout={chunk_layout} inplace={inplace} sampled")


# ---- the prepared call ---------------------------------------------------------
@pytest.mark.parametrize("protocol", ["ll", "hb", "auto"])
def test_prepared_call(comm, orc, protocol):
    """Comm.prepare marshals the arguments once; every call of the result is a
    full all-reduce: new inputs give new sums, out of place and in place."""
    R, N = 8, 10_007
    _, sv = ar.rank_buffers(R, N, torch.bfloat16, comm.device)
    plane, rv = ar.rank_buffers(R, N, torch.bfloat16, comm.device)
    out_of_place = comm.prepare(sv, rv, protocol)
    in_place = comm.prepare(sv, None, protocol)
    for seed in (51, 52):
        x = inputs.make(R, N, "bf16", "normal", seed=seed)
        want = expect(orc, x)
        for r in range(R):
            sv[r].copy_(x[r])
        plane.view(torch.uint8).fill_(0xA5)
        note(f"prepared {protocol} out of place, seed {seed}")
        out_of_place()
        torch.cuda.synchronize()
        assert_parity(torch.stack([t.cpu() for t in rv]), want, f"prepared {protocol} seed {seed}")
        note(f"prepared {protocol} in place, seed {seed}")
        in_place()
        torch.cuda.synchronize()
        assert_parity(torch.stack([t.cpu() for t in sv]), want,
                      f"prepared {protocol} in place seed {seed}")


def test_prepared_call_reports_errors(comm):
    """A prepared call raises the library's error like all_reduce does (here:
    LL above the communicator's LL size limit)."""
    R, N = 2, (2 << 20) // 2
    _, sv = ar.rank_buffers(R, N, torch.bfloat16, comm.device)
    call = comm.prepare(sv, None, "ll")
    with pytest.raises(ar.ArError) as err:
        call()
    assert err.value.code == ar.arResult.arInvalidUsage
    with pytest.raises(ValueError):
        comm.prepare(sv, sv[:1], "hb")


def test_prepared_call_after_close_raises(orc):
    """A prepared call reads the communicator's handle at each call: after the
    communicator is closed it raises instead of passing a freed handle on."""
    R, N = 4, 1000
    x = inputs.make(R, N, "fp16", "normal", seed=53)
    c = ar.Comm(device="cuda:0", max_ranks=R, max_ll_bytes_per_rank=1 << 12)
    _, sv = ar.rank_buffers(R, N, torch.float16, c.device)
    for r in range(R):
        sv[r].copy_(x[r])
    call = c.prepare(sv, None, "ll")
    note("prepared LL before close")
    call()
    torch.cuda.synchronize()
    assert_parity(torch.stack([t.cpu() for t in sv]), expect(orc, x), "prepared before close")
    c.close()
    with pytest.raises(ValueError):
        call()


def test_comm_on_cuda_without_index(orc):
    """Comm(device="cuda") is the current device: tensors on "cuda:0" match it."""
    torch.cuda.set_device(0)
    with ar.Comm(device="cuda", max_ranks=2, max_ll_bytes_per_rank=1 << 12) as c:
        assert c.device == torch.device("cuda", 0)
        x = inputs.make(2, 300, "bf16", "normal", seed=54)
        _, sv = ar.rank_buffers(2, 300, torch.bfloat16, "cuda:0")
        for r in range(2):
            sv[r].copy_(x[r])
        note("Comm(device='cuda') all_reduce")
        c.all_reduce(sv, protocol="hb")
        torch.cuda.synchronize()
        assert_parity(torch.stack([t.cpu() for t in sv]), expect(orc, x), "cuda without index")


def test_last_launch_record(orc):
    """arCommGetLastLaunch names the shape each call launched: the built-in
    LL shape (8-byte packets), the HB default (one workgroup per CU,
    non-temporal), the staged HB form (two kernels), a 16-byte-packet LL call
    only when asked for, and no change for a call that enqueues nothing."""
    with ar.Comm(device="cuda:0", max_ranks=8, max_ll_bytes_per_rank=1 << 20) as c:
        assert c.last_launch() is None
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        x = inputs.make(8, 1 << 10, "bf16", "uniform", seed=55)
        run_allreduce(c, x, "ll")
        rec = c.last_launch()
        assert rec["protocol"] == ar.arProtocol.arProtoLL and rec["packetBytes"] == 8
        assert (rec["grid"], rec["threads"], rec["kernels"]) == (8, 256, 1)
        y = inputs.make(8, 1 << 19, "bf16", "uniform", seed=56)
        run_allreduce(c, y, "hb")
        rec = c.last_launch()
        assert rec["protocol"] == ar.arProtocol.arProtoHB and rec["nonTemporal"] == 1
        # one workgroup per CU, rounded down to whole chunks, at most the 32
        # tiles of 256 vectors that each of the 8 interleaved chunks has
        assert (rec["grid"], rec["threads"], rec["staged"]) == (
            min(max(cus // 8, 1), 32) * 8, 256, 0)
        c.set_option(ar.arOption.arOptHBStaged, 1)
        run_allreduce(c, y, "hb")
        assert c.last_launch()["kernels"] == 2 and c.last_launch()["staged"] == 1
        c.set_option(ar.arOption.arOptHBStaged, 0)
        c.set_option(ar.arOption.arOptLLPacketBytes, 16)
        run_allreduce(c, x, "ll")
        assert c.last_launch()["packetBytes"] == 16
        before = c.last_launch()
        rc = ar.arAllReduce([0] * 8, [0] * 8, 0, ar.arDataType.arBfloat16, ar.arRedOp.arSum, 8,
                            ar.arProtocol.arProtoLL, c.handle,
                            torch.cuda.current_stream().cuda_stream)
        assert rc == ar.arResult.arSuccess and c.last_launch() == before


# ---- shapes, tails and rank counts --------------------------------------------
@pytest.mark.parametrize("R", [3, 8, 12, 16, 24, 32])
@pytest.mark.parametrize("kib", [2, 8, 64, 128, 256, 512, 1024])
def test_ll_default_shape_table(comm, orc, R, kib):
    """LL at its built-in default launch shape (no tuning, no shape options) in
    each rank class of the default table (up to 8, 9-16, 17-32 ranks) and at
    sizes spanning its columns, including the 128-workgroup-per-rank
    entries; one element short of each power of two, so every size ends in a
    partial packet or vector."""
    N = kib * 512 - 1
    x = inputs.make(R, N, "bf16", "normal", seed=3000 + R * 7 + kib)
    check(comm, orc, x, "ll", what=f"ll default shape R={R} {kib} KiB")
    check(comm, orc, x, "ll", inplace=True, what=f"ll default shape in place R={R} {kib} KiB")



@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8, 13, 16, 24, 32])
@pytest.mark.parametrize("N", [1, 2, 3, 7, 9, 1023, 1025, 65536 + 5])
@pytest.mark.parametrize("protocol", ["ll", "hb"])
def test_tails_and_rank_counts(comm, orc, dtype, R, N, protocol):
    x = inputs.make(R, N, dtype, "normal", seed=1000 + R * 31 + N)
    check(comm, orc, x, protocol)


@pytest.mark.parametrize("R", [6, 7, 9, 15, 17, 31])
@pytest.mark.parametrize("kib", [2, 256, 1024])
def test_generic_rank_tables(comm, orc, R, kib):
    """A rank count without a kernel of its own runs the next larger table (4,
    8, 16 or 32 slots) with the count at run time: LL and HB at the edges of
    each table, LL's word-packet and three-element-packet sizes, one element
    short of a power of two (a partial last packet and vector)."""
    N = kib * 512 - 1
    x = inputs.make(R, N, "bf16", "normal", seed=6000 + R * 13 + kib)
    for protocol in ("ll", "hb"):
        check(comm, orc, x, protocol, what=f"{protocol} generic table R={R} {kib} KiB")


@functools.lru_cache(maxsize=2)
def _wave_bound_case(R, extra):
    N = (16 << 20) // 2 + extra
    x = inputs.make(R, N, "bf16", "int4", seed=7000 + R + extra)
    exact = torch.zeros(N, dtype=torch.int32)
    for r in range(R):
        exact += x[r].to(torch.int32)
    return x, exact


@pytest.mark.parametrize("inplace", [False, True], ids=["out", "inplace"])
@pytest.mark.parametrize("extra", [0, 8], ids=["at_bound", "one_vector_over"])
@pytest.mark.parametrize("R", [24, 32])
def test_hb_wave_table_size_bound(comm, orc, R, extra, inplace):
    """32-slot tables (32 ranks, and 24 on the generic table) run the HB kernel
    that reads the rank table from a wave-held copy up to 16 MiB per rank and
    the scalar-table kernel above: bf16 integers at exactly 16 MiB per rank and
    one 16-byte vector more, exact sums on every element of every rank, the
    oracle on sampled columns."""
    x, exact = _wave_bound_case(R, extra)
    note(f"hb wave-table bound R={R} extra={extra} inplace={inplace}")
    got = run_allreduce(comm, x, "hb", inplace=inplace)
    exact_b = exact.to(torch.bfloat16)
    for r in range(R):
        assert torch.equal(got[r], exact_b), f"rank {r}"
    g = torch.Generator().manual_seed(98)
    idx = torch.randint(0, x.shape[1], (1 << 16,), generator=g)
    idx[0] = x.shape[1] - 1
    assert_parity(got[:, idx].contiguous(), expect(orc, x[:, idx].contiguous()),
                  f"hb wave-table bound R={R} extra={extra} inplace={inplace} sampled")

@pytest.mark.parametrize("nt", [0, 1])
@pytest.mark.parametrize("unroll", [1, 2, 4])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("R", [1, 2, 3, 4, 5, 8, 13, 16, 24, 32])
def test_hb_access_policy_and_unroll(comm, orc, nt, unroll, dtype, R):
    """Each access policy (non-temporal, or ordinary cached loads and stores,
    which the tuner picks where a message fits the last-level cache) and each
    vectors-per-lane count is a separate instantiation of the HB kernel: every
    rank table and dtype, with a ragged tail and several tiles."""
    x = inputs.make(R, 70_001, dtype, "outliers", seed=4000 + 7 * R + unroll)
    try:
        comm.set_option(ar.arOption.arOptHBNonTemporal, nt)
        comm.set_option(ar.arOption.arOptHBUnroll, unroll)
        check(comm, orc, x, "hb", what=f"hb nt={nt} R={R} {dtype} unroll {unroll}")
        check(comm, orc, x, "hb", inplace=True, what=f"hb nt={nt} in place R={R} {dtype}")
    finally:
        comm.set_option(ar.arOption.arOptHBNonTemporal, -1)
        comm.set_option(ar.arOption.arOptHBUnroll, 0)


@pytest.mark.parametrize("protocol", ["ll", "hb"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_several_hb_tiles_and_ragged_chunks(comm, orc, protocol, dtype):
    # spans many tiles per chunk; N % R != 0 and N % 8 != 0
    x = inputs.make(8, 3 * 262144 + 12345, dtype, "outliers", seed=21)
    if protocol == "ll":
        x = x[:, : (1 << 20) // x.element_size()].contiguous()
    check(comm, orc, x, protocol)


@pytest.mark.parametrize("protocol", ["ll", "hb"])
def test_in_place_equals_out_of_place(comm, orc, protocol):
    x = inputs.make(8, 100_000, "bf16", "normal", seed=7)
    a = run_allreduce(comm, x, protocol)
    b = run_allreduce(comm, x, protocol, inplace=True)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert_parity(b, expect(orc, x), "in place")


@pytest.mark.parametrize("protocol", ["ll", "hb"])
def test_repeat_is_bitwise_deterministic(comm, protocol):
    x = inputs.make(8, 300_001, "fp16", "normal", seed=8)
    a = run_allreduce(comm, x, protocol)
    b = run_allreduce(comm, x, protocol)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ---- special values --------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("protocol", ["ll", "hb"])
def test_exhaustive_value_set_three_ranks(comm, protocol, dtype):
    """Every 3-rank column over the signed-zero/subnormal/tie/inf/NaN value set,
    against the exact rational model."""
    cols, want = pins._exhaustive_cols(dtype, 3)
    x = from_bits(pins.to_array(cols, dtype).view(np.uint32 if dtype == "fp32" else np.uint16),
                  dtype)
    got = run_allreduce(comm, x, protocol)
    for r in range(3):
        pins.assert_same_bits(bits(got[r]), want, dtype, f"value set {dtype} rank {r}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("R", [5, 7, 12, 24])
@pytest.mark.parametrize("protocol", ["ll", "hb"])
def test_generic_tables_special_values(comm, orc, protocol, R, dtype):
    """Rank counts without a kernel of their own (the slots of the table past the
    count load -0 and add it, an exact identity, in HB's flat order) over
    signed zeros, all-negative-zero columns, subnormals, cancellation and
    overflow, with one entry in a hundred an infinity or a NaN: bit-exact
    against the oracle (NaNs by class)."""
    rng = np.random.default_rng(700 + 13 * R)
    cols = pins.mixed_bits(rng, dtype, 8192 + 5, R)
    fmt = em.FORMATS[dtype]
    sign = 1 << (fmt.ebits + fmt.mbits)
    inf = ((1 << fmt.ebits) - 1) << fmt.mbits
    qnan = inf | (1 << (fmt.mbits - 1)) | 1
    kind = rng.integers(0, 3, cols.shape)
    special = np.where(kind == 0, inf, np.where(kind == 1, inf | sign, qnan))
    cols = np.where(rng.random(cols.shape) < 0.01, special, cols).astype(cols.dtype)
    x = from_bits(np.ascontiguousarray(cols.T), dtype)
    check(comm, orc, x, protocol, what=f"{protocol} generic table special values R={R} {dtype}")

@pytest.mark.parametrize("protocol", ["ll", "hb"])
def test_hand_cases(comm, protocol):
    for dtype, ins, out in pins.load_hand_cases():
        x = from_bits(pins.to_array([ins], dtype).view(
            np.uint32 if dtype == "fp32" else np.uint16), dtype)
        got = run_allreduce(comm, x, protocol)
        for r in range(len(ins)):
            pins.assert_same_bits(bits(got[r]), np.array([out]), dtype,
                                  f"hand case {dtype} {[hex(v) for v in ins]}")


@pytest.mark.parametrize("protocol", ["ll", "hb"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_signed_zeros_and_one_hot(comm, protocol, dtype):
    R, N = 8, 4096
    fmt = em.FORMATS[dtype]
    top = fmt.ebits + fmt.mbits
    npdt = np.uint32 if dtype == "fp32" else np.uint16
    neg = np.full((R, N), 1 << top, dtype=npdt)
    got = bits(run_allreduce(comm, from_bits(neg, dtype), protocol))
    assert np.all(got == (1 << top)), "all -0 must give -0"
    rng = np.random.default_rng(5)
    vals = pins.random_bits(rng, dtype, (N,), emin=-10, emax=10)
    hot = rng.integers(0, R, N)
    x = np.zeros((R, N), dtype=npdt)
    x[hot, np.arange(N)] = vals
    got = bits(run_allreduce(comm, from_bits(x, dtype), protocol))
    for r in range(R):
        assert np.array_equal(got[r], vals)


# ---- launch configurations do not change the bits -----------------------------
@pytest.mark.parametrize("opt,values", [
    (ar.arOption.arOptHBUnroll, [1, 2, 4]),
    (ar.arOption.arOptHBNonTemporal, [0, 1, -1]),
    (ar.arOption.arOptHBBlocks, [8, 40, 256, 2048]),
    (ar.arOption.arOptHBThreads, [64, 512, 1024]),
    (ar.arOption.arOptHBChunkLayout, [0, 1]),
])
def test_hb_tuning_options_keep_bits(comm, orc, opt, values):
    x = inputs.make(8, 1_000_003, "bf16", "outliers", seed=31)
    want = expect(orc, x)
    old = comm.get_option(opt)
    try:
        for v in values:
            comm.set_option(opt, v)
            assert_parity(run_allreduce(comm, x, "hb"), want, f"{opt.name}={v}")
    finally:
        comm.set_option(opt, old)


@pytest.mark.parametrize("opt,values", [
    (ar.arOption.arOptLLThreads, [64, 128, 512, 1024]),
    (ar.arOption.arOptLLBlocksPerRank, [1, 3, 16, 64]),
])
def test_ll_tuning_options_keep_bits(comm, orc, opt, values):
    x = inputs.make(8, 200_003, "bf16", "outliers", seed=32)
    want = expect(orc, x)
    old = comm.get_option(opt)
    try:
        for v in values:
            comm.set_option(opt, v)
            assert_parity(run_allreduce(comm, x, "ll"), want, f"{opt.name}={v}")
    finally:
        comm.set_option(opt, old)


@pytest.mark.parametrize("protocol", ["ll", "hb", "auto"])
def test_count_zero_touches_nothing(comm, protocol):
    from gpu_util import CODES, PROTO
    _, sv = ar.rank_buffers(8, 64, torch.bfloat16, "cuda")
    plane, rv = ar.rank_buffers(8, 64, torch.bfloat16, "cuda")
    plane.view(torch.uint8).fill_(0xA5)
    before = plane.clone()
    rc = ar.arAllReduce([t.data_ptr() for t in sv], [t.data_ptr() for t in rv], 0,
                        CODES["bf16"], ar.arRedOp.arSum, 8, PROTO[protocol], comm.handle,
                        torch.cuda.current_stream().cuda_stream)
    assert rc == ar.arResult.arSuccess
    torch.cuda.synchronize()
    assert torch.equal(plane.view(torch.uint8), before.view(torch.uint8))


@pytest.mark.parametrize("staged", [0, 1])
def test_hb_beyond_4_gib_per_rank(comm, orc, staged):
    """2^31 + 5 bf16 per rank (> 4 GiB, 64-bit offsets, ragged tail), R = 2.

    Integer inputs in [-4, 4] from a seeded CPU generator pattern: every output
    is checked against the exact sum on the GPU in slices, and ~1M sampled
    columns (the last 4096 included) against the oracle."""
    R, N = 2, (1 << 31) + 5
    note(f"HB R={R} N={N} bf16 > 4 GiB per rank, staged={staged}")
    g = torch.Generator().manual_seed(77)
    period = torch.randint(-4, 5, (R, 1 << 20), generator=g, dtype=torch.int8)
    _, sv = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    _, rv = ar.rank_buffers(R, N, torch.bfloat16, "cuda")
    pd = period.to("cuda")
    step = 1 << 20
    for r in range(R):  # rank r: its own random period, tiled
        for a in range(0, N, step):
            b = min(a + step, N)
            sv[r][a:b].copy_(pd[r, : b - a])
    from gpu_util import CODES, PROTO
    old = comm.get_option(ar.arOption.arOptHBStaged)
    comm.set_option(ar.arOption.arOptHBStaged, staged)
    try:
        rc = ar.arAllReduce([t.data_ptr() for t in sv], [t.data_ptr() for t in rv], N,
                            CODES["bf16"], ar.arRedOp.arSum, R, PROTO["hb"], comm.handle,
                            torch.cuda.current_stream().cuda_stream)
        assert rc == ar.arResult.arSuccess
        torch.cuda.synchronize()
    finally:
        comm.set_option(ar.arOption.arOptHBStaged, old)
    big = 1 << 28
    for a in range(0, N, big):
        b = min(a + big, N)
        want = sv[0][a:b].float() + sv[1][a:b].float()
        for r in range(R):
            assert torch.equal(rv[r][a:b].float(), want), f"rank {r} slice at {a}"
    idx = torch.cat([torch.randint(0, N, (1 << 20,), generator=g),
                     torch.arange(N - 4096, N)])
    xs = torch.stack([t[idx.to("cuda")].cpu() for t in sv])
    got = torch.stack([t[idx.to("cuda")].cpu() for t in rv])
    assert_parity(got, expect(orc, xs), "> 4 GiB per rank, sampled")
    del sv, rv
    torch.cuda.empty_cache()


@pytest.mark.parametrize("protocol", ["ll", "hb", "auto"])
def test_comm_all_reduce_convenience(comm, orc, protocol):
    x = inputs.make(8, 10_007, "bf16", "normal", seed=2024)
    want = expect(orc, x)
    send = [t.to("cuda") for t in x]
    recv = [torch.empty_like(t) for t in send]
    note(f"Comm.all_reduce {protocol}")
    out = comm.all_reduce(send, recv, protocol=protocol)
    torch.cuda.synchronize()
    assert_parity(torch.stack([t.cpu() for t in out]), want, f"all_reduce {protocol}")
    comm.all_reduce(send, protocol=protocol)  # in place
    torch.cuda.synchronize()
    assert_parity(torch.stack([t.cpu() for t in send]), want, f"all_reduce {protocol} in place")


def test_comm_all_reduce_rejects_bad_tensors(comm):
    a = [torch.zeros(64, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    with pytest.raises(ValueError):
        comm.all_reduce([a[0], a[1].to(torch.float16)])
    with pytest.raises(ValueError):
        comm.all_reduce(a, [a[0]])
    with pytest.raises(ValueError):
        comm.all_reduce([a[0], torch.zeros(128, dtype=torch.bfloat16, device="cuda")[::2]])
    with pytest.raises(ValueError):
        comm.all_reduce([a[0], torch.zeros(64, dtype=torch.bfloat16)])
    with pytest.raises(ar.ArError):  # 16-bit x 3 = 6 bytes apart: not 16-byte aligned
        base = torch.zeros(256, dtype=torch.bfloat16, device="cuda")
        comm.all_reduce([base[0:64], base[3:67]], [base[128:192], base[192:256]])
