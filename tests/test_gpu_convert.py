"""The kernels' fp32 -> bf16/fp16 narrowing on the GPU, over all 2^32 inputs.

The kernels narrow with gfx950's packed convert instructions; this runs the
same device code (ar::Bf16::narrow / ar::Fp16::narrow, through a test-only
probe library) on every binary32 pattern and compares with the oracle's
integer RNE converter, itself pinned exhaustively to torch's CPU ``.to()``.
NaNs are compared by class.
"""
import ctypes
from pathlib import Path

import numpy as np
import pytest
import torch

from gpu_util import note

pytestmark = pytest.mark.gpu
PROBE = Path(__file__).resolve().parent / "gpu_probe" / "libconvert_probe.so"


@pytest.fixture(scope="module")
def probe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not PROBE.exists():
        pytest.fail(f"{PROBE} not built (python -m all_reduce_amd.build)")
    lib = ctypes.CDLL(str(PROBE))
    lib.probe_narrow.argtypes = [ctypes.c_int, ctypes.c_uint32, ctypes.c_uint64,
                                 ctypes.c_void_p, ctypes.c_void_p]
    lib.probe_narrow.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_narrowing_all_patterns(probe, orc, dtype):
    step = 1 << 28
    inf = 0x7F80 if dtype == "bf16" else 0x7C00
    conv = orc.rne_bf16 if dtype == "bf16" else orc.rne_fp16
    out = torch.empty(step, dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for start in range(0, 1 << 32, step):
        note(f"narrow {dtype} patterns {start:#x}..+{step:#x}")
        assert probe.probe_narrow(0 if dtype == "bf16" else 1, start, step, out.data_ptr(),
                                  stream) == 0
        got = out.cpu()
        base = start - (1 << 32) if start >= 1 << 31 else start
        pats = torch.arange(step, dtype=torch.int32).add_(base).view(torch.float32)
        want = torch.from_numpy(conv(pats.numpy(), nthreads=16).view(np.int16))
        gn = (got & 0x7FFF) > inf
        wn = (want & 0x7FFF) > inf
        bad = (gn != wn) | (~gn & ~wn & (got != want))
        nbad = int(bad.sum())
        if nbad:
            i = int(bad.nonzero()[0])
            raise AssertionError(f"{dtype}: {nbad} mismatches from {start:#x}; first pattern "
                                 f"{(start + i) & 0xFFFFFFFF:#010x}: gpu {int(got[i]) & 0xFFFF:#06x}"
                                 f" oracle {int(want[i]) & 0xFFFF:#06x}")
