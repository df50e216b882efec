"""Helpers for the GPU tests: run the HIP all-reduce through the C ABI and
compare with the oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import all_reduce_amd as ar
import pins

CODES = {"bf16": ar.arDataType.arBfloat16, "fp16": ar.arDataType.arFloat16,
         "fp32": ar.arDataType.arFloat32}
PROTO = {"ll": ar.arProtocol.arProtoLL, "hb": ar.arProtocol.arProtoHB,
         "auto": ar.arProtocol.arProtoAuto}
TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def dtype_name(t: torch.Tensor) -> str:
    return {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}[t.dtype]


def bits(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> numpy bit patterns (uint16 for 16-bit types, uint32 for fp32)."""
    t = t.contiguous()
    if t.dtype == torch.float32:
        return t.numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def oracle_view(t: torch.Tensor) -> np.ndarray:
    """CPU tensor -> the array form the oracle takes."""
    b = bits(t)
    return b.view(np.float32) if t.dtype == torch.float32 else b


def from_bits(b: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "fp32":
        return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint32).view(np.float32))
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16))
    return t.view(TORCH[dtype])


def note(msg: str):
    """Name the case on stderr before it touches the GPU."""
    sys.stderr.write(f"[gpu case] {msg}\n")
    sys.stderr.flush()


def run_allreduce(comm: ar.Comm, x: torch.Tensor, protocol: str, inplace: bool = False,
                  stream=None) -> torch.Tensor:
    """All-reduce the rows of CPU tensor ``x`` (R, N) on the GPU via arAllReduce.

    Inputs go into one rank plane (rank r at base + r * stride); outputs into a
    second plane filled with a poison pattern first (unless in place).  Returns
    the (R, N) outputs on the CPU."""
    R, N = x.shape
    dt = dtype_name(x)
    note(f"{protocol} R={R} N={N} {dt} inplace={inplace}")
    _, sv = ar.rank_buffers(R, N, x.dtype, comm.device)
    for r in range(R):
        sv[r].copy_(x[r])
    if inplace:
        rv = sv
    else:
        plane, rv = ar.rank_buffers(R, N, x.dtype, comm.device)
        plane.view(torch.uint8).fill_(0xA5)
    s = torch.cuda.current_stream(comm.device) if stream is None else stream
    rc = ar.arAllReduce([t.data_ptr() for t in sv], [t.data_ptr() for t in rv], N, CODES[dt],
                        ar.arRedOp.arSum, R, PROTO[protocol], comm.handle, s.cuda_stream)
    assert rc == ar.arResult.arSuccess, ar.arGetErrorString(rc)
    torch.cuda.synchronize(comm.device)
    return torch.stack([t.cpu() for t in rv])


def expect(orc, x: torch.Tensor) -> np.ndarray:
    """Oracle output bits (R, N) for CPU input ``x``."""
    out = orc.allreduce(oracle_view(x), dtype_name(x), nthreads=16)
    return out.view(np.uint32) if x.dtype == torch.float32 else out.view(np.uint16)


def assert_parity(got: torch.Tensor, want_bits: np.ndarray, what: str):
    dt = dtype_name(got)
    g = bits(got)
    for r in range(g.shape[0]):
        pins.assert_same_bits(g[r], want_bits[r], dt, f"{what} rank {r}")
