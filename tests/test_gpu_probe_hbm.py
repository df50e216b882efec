"""The HBM ceiling probe (tests/gpu_probe/hbm_ceiling.hip), on the GPU.

The probe is a measurement aid for bench.py --only ceilings: the HB kernel's
memory traffic without its arithmetic.  These tests check that each of its
modes touches exactly the data it claims to -- every vector of every stream,
at a size that leaves a ragged last tile -- so that its timings measure the
traffic they are quoted for.
"""
import ctypes
from pathlib import Path

import numpy as np
import pytest
import torch

from gpu_util import note

pytestmark = pytest.mark.gpu

LIB = Path(__file__).resolve().parent / "gpu_probe" / "libhbm_ceiling.so"
NVEC = 100_003        # vectors per stream: many tiles and a ragged last one
GRID, THREADS = 64, 256


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not LIB.exists():
        raise RuntimeError(f"{LIB} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(str(LIB))
    vp = ctypes.c_void_p
    lib.hbm_ceiling_run.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), vp, ctypes.c_uint64,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.hbm_ceiling_run.restype = ctypes.c_int
    lib.hbm_ceiling_run_n.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), vp, ctypes.c_uint64,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.hbm_ceiling_run_n.restype = ctypes.c_int
    return lib


def _ptrs(plane):
    return (ctypes.c_void_p * 8)(*[plane[j].data_ptr() for j in range(8)])


def _run(probe, src, dst, sink, mode, grid=GRID, threads=THREADS):
    note(f"hbm ceiling probe mode {mode} grid {grid} x {threads}")
    rc = probe.hbm_ceiling_run(_ptrs(src), _ptrs(dst), sink.data_ptr() if sink is not None else None,
                               NVEC, mode, grid, threads, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return rc


def _planes():
    g = torch.Generator().manual_seed(7)
    host = torch.randint(-2**31, 2**31 - 1, (8, NVEC * 4), generator=g, dtype=torch.int64)
    src = host.to(torch.int32).cuda()
    return host.to(torch.int32), src


def test_copy_out_of_place(probe):
    host, src = _planes()
    dst = torch.zeros_like(src)
    assert _run(probe, src, dst, None, 2) == 0
    assert torch.equal(dst.cpu(), host)
    assert torch.equal(src.cpu(), host)


def test_copy_in_place_leaves_data(probe):
    host, src = _planes()
    assert _run(probe, src, src, None, 2) == 0
    assert torch.equal(src.cpu(), host)


@pytest.mark.parametrize("mode", [1, 3])
def test_write_pattern(probe, mode):
    _, dst = _planes()
    assert _run(probe, dst, dst, None, mode) == 0
    i = np.arange(NVEC, dtype=np.uint64)
    chunk = (i // THREADS) % 8
    want = np.stack([i & 0xFFFFFFFF, i >> 32, chunk, np.full(NVEC, 0x9E3779B9, np.uint64)],
                    axis=1).astype(np.uint32)
    got = dst.cpu().numpy().view(np.uint32).reshape(8, NVEC, 4)
    for j in range(8):
        assert np.array_equal(got[j], want), f"stream {j}"


def test_read_folds_every_vector(probe):
    host, src = _planes()
    sink = torch.zeros(GRID * THREADS * 4, dtype=torch.int32, device="cuda")
    assert _run(probe, src, src, sink, 0) == 0
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32).reshape(-1, 4), axis=0)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32).reshape(-1, 4), axis=0)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("grid,threads,mode", [(7, 256, 0), (0, 256, 1), (64, 100, 2),
                                               (64, 2048, 2), (64, 256, 4), (64, 256, -1)])
def test_bad_launch_shapes_are_refused(probe, grid, threads, mode):
    _, src = _planes()
    assert _run(probe, src, src, None, mode, grid, threads) == -1


@pytest.mark.parametrize("streams", [16, 32])
def test_more_streams_out_of_place_copy_and_read(probe, streams):
    """The 16- and 32-stream forms (the R = 16 / 32 workloads' shapes): an
    out-of-place copy moves every vector of every stream, and a read folds
    every vector into the sink."""
    g = torch.Generator().manual_seed(8)
    host = torch.randint(-2**31, 2**31 - 1, (streams, NVEC * 4), generator=g,
                         dtype=torch.int64).to(torch.int32)
    src = host.cuda()
    dst = torch.zeros_like(src)
    vp = ctypes.c_void_p
    sp = (vp * streams)(*[src[j].data_ptr() for j in range(streams)])
    dp = (vp * streams)(*[dst[j].data_ptr() for j in range(streams)])
    grid = 4 * streams
    note(f"hbm ceiling probe {streams} streams: copy out of place, read")
    assert probe.hbm_ceiling_run_n(sp, dp, None, NVEC, 2, grid, THREADS, streams,
                                   torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst.cpu(), host)
    sink = torch.zeros(grid * THREADS * 4, dtype=torch.int32, device="cuda")
    assert probe.hbm_ceiling_run_n(sp, sp, sink.data_ptr(), NVEC, 0, grid, THREADS, streams,
                                   torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32).reshape(-1, 4), axis=0)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32).reshape(-1, 4), axis=0)
    assert np.array_equal(got, want)
    for bad_streams, bad_grid, bad_threads in ((streams, grid + 1, THREADS), (12, grid, THREADS),
                                               (streams, grid, 1024)):
        assert probe.hbm_ceiling_run_n(sp, dp, None, NVEC, 2, bad_grid, bad_threads, bad_streams,
                                       torch.cuda.current_stream().cuda_stream) == -1
