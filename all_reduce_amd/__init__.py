"""Python binding of the MI355X sum all-reduce over R simulated ranks.

The functions named ``ar*`` are the C ABI of ``include/ar_allreduce.h``, one
for one, over ctypes: arguments are marshalled and the result code is
returned, nothing else happens here.  :class:`Comm` and :func:`rank_buffers`
are conveniences on top for torch tensors; torch supplies device memory and
streams only.  Every step of the all-reduce runs in the HIP kernels of
``libar_allreduce.so``; there is no other implementation to fall back to, so a
missing library raises instead of running anything.
"""
from __future__ import annotations

import ctypes
from enum import IntEnum
from pathlib import Path
from typing import Sequence

LIBRARY = Path(__file__).resolve().parent / "_lib" / "libar_allreduce.so"
HEADER = Path(__file__).resolve().parent.parent / "include" / "ar_allreduce.h"


class arResult(IntEnum):
    arSuccess = 0
    arInvalidArgument = 1
    arUnsupported = 2
    arInvalidUsage = 3
    arHipError = 4
    arTimeout = 5
    arInternalError = 6


class arDataType(IntEnum):
    arBfloat16 = 0
    arFloat16 = 1
    arFloat32 = 2


class arRedOp(IntEnum):
    arSum = 0


class arProtocol(IntEnum):
    arProtoLL = 0
    arProtoHB = 1
    arProtoAuto = 2


class arOption(IntEnum):
    arOptPollTimeoutUs = 0
    arOptLLBlocksPerRank = 1
    arOptHBBlocks = 2
    arOptHBNonTemporal = 3
    arOptDebugFlagSkew = 4
    arOptHBUnroll = 5
    arOptLLThreads = 6
    arOptHBThreads = 7
    arOptHBChunkLayout = 8
    arOptNodeRanks = 9
    arOptLLPacketBytes = 10
    arOptHBStaged = 11
    arOptLLFlagScheme = 12
    arOptDebugSeqStart = 13
    arOptTuneFreshInputs = 14
    arOptLLDense = 15


AR_MAX_RANKS = 32
AR_NOALLOC_SCRATCH_BYTES = 64 << 20


class arTunedShape(ctypes.Structure):
    """Mirror of arTunedShape_t."""
    _fields_ = [("tuned", ctypes.c_int), ("threads", ctypes.c_int), ("blocks", ctypes.c_int),
                ("packetBytes", ctypes.c_int), ("nonTemporal", ctypes.c_int),
                ("us", ctypes.c_float)]


class arLaunchInfo(ctypes.Structure):
    """Mirror of arLaunchInfo_t."""
    _fields_ = [("protocol", ctypes.c_int), ("kernels", ctypes.c_int), ("grid", ctypes.c_uint),
                ("threads", ctypes.c_uint), ("packetBytes", ctypes.c_int),
                ("nonTemporal", ctypes.c_int), ("nodeRanks", ctypes.c_int),
                ("staged", ctypes.c_int), ("packetPayloadBytes", ctypes.c_int)]


class ArError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = arResult(code)
        super().__init__(f"{where}: {arGetErrorString(code)}")


_lib = None


def library() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIBRARY.exists():
        raise RuntimeError(f"{LIBRARY} is missing: build it with `python -m all_reduce_amd.build`")
    lib = ctypes.CDLL(str(LIBRARY))
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "arCommCreate": ([ctypes.POINTER(vp), i32, i32, sz], i32),
        "arCommDestroy": ([vp], i32),
        "arCommReset": ([vp, vp], i32),
        "arCommGetAsyncError": ([vp, ctypes.POINTER(i32)], i32),
        "arCommSetOption": ([vp, i32, i64], i32),
        "arCommGetOption": ([vp, i32, ctypes.POINTER(i64)], i32),
        "arAllReduce": ([ctypes.POINTER(vp), ctypes.POINTER(vp), sz, i32, i32, i32, i32, vp, vp], i32),
        "arCommTune": ([vp, i32, i32, sz, vp], i32),
        "arCommGetTunedShape": ([vp, i32, i32, i32, sz, i32, ctypes.POINTER(arTunedShape)], i32),
        "arCommGetLastLaunch": ([vp, ctypes.POINTER(arLaunchInfo)], i32),
        "arCommSetWorkspace": ([vp, vp, sz], i32),
        "arAllReduceNoAlloc": ([ctypes.POINTER(vp), ctypes.POINTER(vp), sz, i32, i32, i32, i32,
                                vp], i32),
        "arGetErrorString": ([i32], ctypes.c_char_p),
        "arGetVersion": ([], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


# ---- the C ABI, one Python function per entry point -----------------------
def arGetErrorString(result: int) -> str:
    return library().arGetErrorString(int(result)).decode()


def arGetVersion() -> int:
    return library().arGetVersion()


def arCommCreate(device: int, max_ranks: int, max_ll_bytes_per_rank: int):
    """Returns (result code, communicator handle or None)."""
    h = ctypes.c_void_p()
    r = library().arCommCreate(ctypes.byref(h), device, max_ranks, max_ll_bytes_per_rank)
    return r, (h.value if r == 0 else None)


def arCommDestroy(comm) -> int:
    return library().arCommDestroy(comm)


def arCommReset(comm, stream) -> int:
    return library().arCommReset(comm, stream)


def arCommGetAsyncError(comm):
    """Returns (result code, recorded asynchronous error)."""
    e = ctypes.c_int(0)
    r = library().arCommGetAsyncError(comm, ctypes.byref(e))
    return r, e.value


def arCommSetOption(comm, option: int, value: int) -> int:
    return library().arCommSetOption(comm, int(option), int(value))


def arCommGetOption(comm, option: int):
    v = ctypes.c_int64(0)
    r = library().arCommGetOption(comm, int(option), ctypes.byref(v))
    return r, v.value


def arCommTune(comm, dtype: int, nranks: int, max_bytes_per_rank: int, stream) -> int:
    return library().arCommTune(comm, int(dtype), nranks, max_bytes_per_rank, stream)


def arCommGetTunedShape(comm, dtype: int, nranks: int, protocol: int, bytes_per_rank: int,
                        in_place: int = 0):
    """Returns (result code, arTunedShape)."""
    shape = arTunedShape()
    r = library().arCommGetTunedShape(comm, int(dtype), nranks, int(protocol), bytes_per_rank,
                                      int(in_place), ctypes.byref(shape))
    return r, shape


def arCommSetWorkspace(comm, workspace, nbytes: int) -> int:
    """``workspace`` a device pointer as an integer, or None with 0."""
    return library().arCommSetWorkspace(comm, workspace, nbytes)


def arCommGetLastLaunch(comm):
    """Returns (result code, arLaunchInfo)."""
    info = arLaunchInfo()
    r = library().arCommGetLastLaunch(comm, ctypes.byref(info))
    return r, info


def _pointer_array(ptrs: Sequence[int] | None, nranks: int):
    """ctypes array of device pointers, NULL-padded to ``nranks`` entries so the
    library never reads past it (it rejects nranks > AR_MAX_RANKS before reading
    any pointer, and reports a NULL entry as arInvalidArgument)."""
    if ptrs is None:
        return None
    n = max(1, len(ptrs), min(max(int(nranks), 0), AR_MAX_RANKS))
    return (ctypes.c_void_p * n)(*ptrs)


def arAllReduce(sendbufs: Sequence[int] | None, recvbufs: Sequence[int] | None, count: int,
                dtype: int, op: int, nranks: int, protocol: int, comm, stream) -> int:
    """Device pointers as integers; ``None`` passes a NULL array."""
    s = _pointer_array(sendbufs, nranks)
    d = _pointer_array(recvbufs, nranks)
    return library().arAllReduce(s, d, count, int(dtype), int(op), nranks, int(protocol),
                                 comm, stream)


def arAllReduceNoAlloc(sendbufs: Sequence[int] | None, recvbufs: Sequence[int] | None,
                       count: int, dtype: int, op: int, nranks: int, node_ranks: int,
                       stream) -> int:
    """Device pointers as integers; ``None`` passes a NULL array."""
    s = _pointer_array(sendbufs, nranks)
    d = _pointer_array(recvbufs, nranks)
    return library().arAllReduceNoAlloc(s, d, count, int(dtype), int(op), nranks,
                                        int(node_ranks), stream)


# ---- torch conveniences ---------------------------------------------------
def _torch():
    import torch
    return torch


def dtype_code(dtype) -> arDataType:
    torch = _torch()
    table = {torch.bfloat16: arDataType.arBfloat16, torch.float16: arDataType.arFloat16,
             torch.float32: arDataType.arFloat32}
    if dtype not in table:
        raise ArError(arResult.arUnsupported, f"dtype {dtype}")
    return table[dtype]


def protocol_code(protocol) -> arProtocol:
    if isinstance(protocol, str):
        return {"ll": arProtocol.arProtoLL, "hb": arProtocol.arProtoHB,
                "auto": arProtocol.arProtoAuto}[protocol.lower()]
    return arProtocol(protocol)


def rank_buffers(nranks: int, count: int, dtype, device, align: int = 256):
    """One allocation holding ``nranks`` buffers of ``count`` elements.

    Rank r's buffer starts at ``base + r * stride`` with the stride rounded up
    to ``align`` bytes.  Returns (plane, views): ``plane`` is the
    (nranks, stride_elems) tensor, ``views[r]`` rank r's ``count`` elements."""
    torch = _torch()
    es = torch.empty((), dtype=dtype).element_size()
    stride = -(-max(count, 1) * es // align) * align // es
    plane = torch.empty((nranks, stride), dtype=dtype, device=device)
    return plane, [plane[r, :count] for r in range(nranks)]


class Comm:
    """Owns an ``arComm_t`` on one device; ``all_reduce`` over torch tensors."""

    def __init__(self, device=None, max_ranks: int = AR_MAX_RANKS,
                 max_ll_bytes_per_rank: int = 1 << 20):
        torch = _torch()
        dev = torch.device("cuda") if device is None else torch.device(device)
        if dev.type != "cuda":
            raise ValueError(f"a communicator needs a GPU device, not {dev}")
        # "cuda" without an index means the current device; resolve it now, so
        # that tensors on "cuda:<i>" compare equal to the communicator's device.
        dev = torch.device("cuda", dev.index if dev.index is not None
                           else torch.cuda.current_device())
        self.device = dev
        r, h = arCommCreate(dev.index, max_ranks, max_ll_bytes_per_rank)
        if r != 0:
            raise ArError(r, "arCommCreate")
        self.handle = h
        self.max_ranks = max_ranks
        self.max_ll_bytes_per_rank = max_ll_bytes_per_rank
        self._workspace = None

    def close(self):
        """Free the communicator after the device has finished the work using it."""
        if self.handle is not None:
            _torch().cuda.synchronize(self.device)
            r = arCommDestroy(self.handle)
            self.handle = None
            if r != 0:
                raise ArError(r, "arCommDestroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _stream(self, stream):
        torch = _torch()
        s = torch.cuda.current_stream(self.device) if stream is None else stream
        return s.cuda_stream

    def set_option(self, option, value: int):
        r = arCommSetOption(self.handle, option, value)
        if r != 0:
            raise ArError(r, "arCommSetOption")

    def get_option(self, option) -> int:
        r, v = arCommGetOption(self.handle, option)
        if r != 0:
            raise ArError(r, "arCommGetOption")
        return v

    def tune(self, dtype, nranks: int, max_bytes_per_rank: int, stream=None):
        """Measure launch shapes per power-of-two size (see arCommTune)."""
        r = arCommTune(self.handle, dtype_code(dtype), nranks, max_bytes_per_rank,
                       self._stream(stream))
        if r != 0:
            raise ArError(r, "arCommTune")

    def tuned_shape(self, dtype, nranks: int, protocol, bytes_per_rank: int,
                    in_place: bool = False):
        """(threads, blocks, us, packet_bytes, non_temporal) stored for that size
        and mode -- threads and blocks 0 when the built-in default won;
        packet_bytes 8 or 16 for LL, 0 for HB; non_temporal 1 or 0 for HB, 0 for
        LL -- or None if never tuned."""
        r, s = arCommGetTunedShape(self.handle, dtype_code(dtype), nranks,
                                   protocol_code(protocol), bytes_per_rank, 1 if in_place else 0)
        if r != 0:
            raise ArError(r, "arCommGetTunedShape")
        return None if s.tuned == 0 else (s.threads, s.blocks, s.us, s.packetBytes, s.nonTemporal)

    def set_workspace(self, workspace):
        """Attach a device tensor (256-byte aligned, on the communicator's
        device) as the staged two-level form's workspace, or None to detach.
        The tensor is kept alive while attached."""
        if workspace is None:
            r = arCommSetWorkspace(self.handle, None, 0)
        else:
            if not workspace.is_contiguous() or workspace.device != self.device:
                raise ValueError("the workspace must be a contiguous tensor on the "
                                 "communicator's device")
            r = arCommSetWorkspace(self.handle, workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size())
        if r != 0:
            raise ArError(r, "arCommSetWorkspace")
        self._workspace = workspace

    def last_launch(self) -> dict | None:
        """The shape of the communicator's most recent launch (see
        arCommGetLastLaunch) as a dict, or None before the first one."""
        r, info = arCommGetLastLaunch(self.handle)
        if r != 0:
            raise ArError(r, "arCommGetLastLaunch")
        if info.protocol < 0:
            return None
        return {name: getattr(info, name) for name, _ in info._fields_}

    def reset(self, stream=None):
        r = arCommReset(self.handle, self._stream(stream))
        if r != 0:
            raise ArError(r, "arCommReset")

    def async_error(self) -> arResult:
        r, e = arCommGetAsyncError(self.handle)
        if r != 0:
            raise ArError(r, "arCommGetAsyncError")
        return arResult(e)

    def all_reduce(self, send, recv=None, protocol="auto", stream=None):
        """Sum all-reduce of the tensors in ``send`` into ``recv`` (default: in place).

        ``protocol`` is "ll", "hb" or "auto" (the tuned faster one; HB where
        nothing was tuned)."""
        send, recv = self._check_ranks(send, recv)
        t0 = send[0]
        r = arAllReduce([t.data_ptr() for t in send], [t.data_ptr() for t in recv],
                        t0.numel(), dtype_code(t0.dtype), arRedOp.arSum, len(send),
                        protocol_code(protocol), self.handle, self._stream(stream))
        if r != 0:
            raise ArError(r, "arAllReduce")
        return recv

    def prepare(self, send, recv=None, protocol="auto", stream=None) -> "PreparedAllReduce":
        """``all_reduce(send, recv, protocol, stream)`` with its arguments
        marshalled once, for a loop that reduces the same buffers again and
        again without a graph.  The stream is fixed here (default: the current
        stream now); the tensors are kept alive by the returned call."""
        send, recv = self._check_ranks(send, recv)
        return PreparedAllReduce(self, send, recv, protocol_code(protocol), self._stream(stream))

    def _check_ranks(self, send, recv):
        if recv is None:
            recv = send
        if len(send) != len(recv) or not send:
            raise ValueError("need one receive tensor per send tensor")
        t0 = send[0]
        for t in (*send, *recv):
            if t.device != self.device:
                raise ValueError(f"tensor on {t.device}, communicator on {self.device}")
            if t.dtype != t0.dtype or t.numel() != t0.numel():
                raise ValueError("all rank tensors need the same dtype and size")
            if not t.is_contiguous():
                raise ValueError("rank tensors must be contiguous")
        return list(send), list(recv)


class PreparedAllReduce:
    """One ``arAllReduce`` call whose arguments (pointer arrays, count, dtype,
    protocol, stream) were marshalled once: calling it is a single foreign
    call.  Made by ``Comm.prepare``.  The communicator's handle is read at each
    call, so a call after ``Comm.close()`` raises instead of passing a freed
    communicator to the library."""

    __slots__ = ("_fn", "_head", "_tail", "_comm", "_keep")

    def __init__(self, comm, send, recv, protocol, stream):
        n = len(send)
        t0 = send[0]
        self._fn = library().arAllReduce
        self._head = (_pointer_array([t.data_ptr() for t in send], n),
                      _pointer_array([t.data_ptr() for t in recv], n),
                      t0.numel(), int(dtype_code(t0.dtype)), int(arRedOp.arSum), n,
                      int(protocol))
        self._tail = stream
        self._comm = comm
        self._keep = (send, recv)

    def __call__(self):
        h = self._comm.handle
        if h is None:
            raise ValueError("the communicator of this prepared call was closed")
        r = self._fn(*self._head, h, self._tail)
        if r != 0:
            raise ArError(r, "arAllReduce")
