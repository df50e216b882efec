"""CPU oracle for the sum all-reduce over R rank buffers -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library under
``all_reduce_amd/`` never imports it, and this package imports nothing from
there: the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, OpenMP over elements); this
module only builds it with gcc and marshals numpy arrays through ctypes.
16-bit element types (bf16, fp16) travel as ``uint16`` bit patterns, fp32 as
``float32``.

What the oracle computes, per element i (see the header of ``oracle.c``):
``a = x_0[i]; a = fl32(a + x_j[i]) for j = 1..R-1; y = rne(a); out_r[i] = y``.
SUM and the dtypes float/float16/bfloat16 follow the runtime guards of the
SGLang MSCCL++ all-reduce guide (blog.gitcode.com), section 4.3; the fixed
rank order, fp32 accumulator and RNE narrowing are the reading taken where the
pages are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "oracle.c"
LIBRARY = HERE / "liboracle.so"

BF16, FP16, FP32 = 0, 1, 2
DTYPES = {"bf16": BF16, "fp16": FP16, "fp32": FP32}

CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared",
          "-fPIC", "-std=c11", "-Wall", "-Wextra"]


def build(source: Path = SOURCE, output: Path = LIBRARY) -> Path:
    """Compile ``source`` (the oracle, or a test's modified copy) with gcc."""
    output = Path(output)
    tmp = output.with_name(output.name + f".tmp{os.getpid()}")
    cmd = ["gcc", *CFLAGS, str(source), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    os.replace(tmp, output)
    return output


class Oracle:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: Path | str = LIBRARY):
        self.path = Path(path)
        lib = ctypes.CDLL(str(self.path))
        vpp = ctypes.POINTER(ctypes.c_void_p)
        lib.oracle_allreduce.argtypes = [vpp, vpp, ctypes.c_size_t, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int]
        lib.oracle_allreduce.restype = ctypes.c_int
        lib.oracle_allreduce_timed.argtypes = lib.oracle_allreduce.argtypes
        lib.oracle_allreduce_timed.restype = ctypes.c_double
        for name in ("oracle_rne_bf16_array", "oracle_rne_fp16_array"):
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
            fn.restype = None
        lib.oracle_allreduce_grouped.argtypes = [vpp, vpp, ctypes.c_size_t, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_allreduce_grouped.restype = ctypes.c_int
        lib.oracle_widen_fp16_array.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_size_t]
        lib.oracle_widen_fp16_array.restype = None
        self.lib = lib

    # -- converters -------------------------------------------------------
    def rne_bf16(self, x: np.ndarray, nthreads: int = 1) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_rne_bf16_array(x.ctypes.data, out.ctypes.data, x.size, nthreads)
        return out

    def rne_fp16(self, x: np.ndarray, nthreads: int = 1) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_rne_fp16_array(x.ctypes.data, out.ctypes.data, x.size, nthreads)
        return out

    def widen_fp16(self, h: np.ndarray) -> np.ndarray:
        h = np.ascontiguousarray(h, dtype=np.uint16)
        out = np.empty(h.shape, dtype=np.float32)
        self.lib.oracle_widen_fp16_array(h.ctypes.data, out.ctypes.data, h.size)
        return out

    # -- the all-reduce ---------------------------------------------------
    @staticmethod
    def _ptrs(arrays):
        return (ctypes.c_void_p * len(arrays))(*[a.ctypes.data for a in arrays])

    def allreduce_into(self, send: list[np.ndarray], recv: list[np.ndarray],
                       dtype: str, nthreads: int = 1, timed: bool = False):
        """Sum all-reduce of ``send`` rows into ``recv`` rows (may alias).

        Returns the call's wall time in seconds when ``timed`` is set."""
        code = DTYPES[dtype]
        want = np.float32 if code == FP32 else np.uint16
        count = send[0].size
        for a in (*send, *recv):
            if a.dtype != want or a.size != count or not a.flags.c_contiguous:
                raise ValueError("oracle: rank arrays must be contiguous, same size, "
                                 f"dtype {np.dtype(want)}")
        if len(send) != len(recv) or not send:
            raise ValueError("oracle: need as many recv as send arrays, at least one")
        sp, rp = self._ptrs(send), self._ptrs(recv)
        if timed:
            t = self.lib.oracle_allreduce_timed(sp, rp, count, code, len(send), nthreads)
            if t < 0:
                raise RuntimeError("oracle_allreduce failed")
            return t
        if self.lib.oracle_allreduce(sp, rp, count, code, len(send), nthreads) != 0:
            raise RuntimeError("oracle_allreduce failed")
        return None

    def allreduce_grouped(self, x: np.ndarray, dtype: str, group: int,
                          nthreads: int = 1) -> np.ndarray:
        """Hierarchical order: groups of ``group`` consecutive ranks summed first
        (binary32), then the group partials in group order; one rounding."""
        x = np.ascontiguousarray(x)
        out = np.empty_like(x)
        code = DTYPES[dtype]
        want = np.float32 if code == FP32 else np.uint16
        if x.dtype != want:
            raise ValueError(f"oracle: dtype {np.dtype(want)} expected")
        sp, rp = self._ptrs(list(x)), self._ptrs(list(out))
        if self.lib.oracle_allreduce_grouped(sp, rp, x.shape[1], code, x.shape[0], group,
                                             nthreads) != 0:
            raise ValueError("oracle_allreduce_grouped: bad arguments")
        return out

    def allreduce(self, x: np.ndarray, dtype: str, nthreads: int = 1) -> np.ndarray:
        """``x`` has shape (R, N); returns a new (R, N) array of outputs."""
        x = np.ascontiguousarray(x)
        out = np.empty_like(x)
        self.allreduce_into(list(x), list(out), dtype, nthreads)
        return out


_default: Oracle | None = None


def load() -> Oracle:
    """The oracle as built from ``oracle.c``; builds it first if it is missing."""
    global _default
    if _default is None:
        if not LIBRARY.exists() or LIBRARY.stat().st_mtime < SOURCE.stat().st_mtime:
            build()
        _default = Oracle(LIBRARY)
    return _default
