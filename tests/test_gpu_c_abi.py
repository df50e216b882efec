"""A plain C99 program calls the C ABI on the GPU: device memory from the HIP
runtime, no Python in the loop.  It checks every output element of LL, HB and
arProtoAuto calls, out of place and in place, against exact integer sums."""
import subprocess

import pytest
import torch

from c_abi import build as cbuild

pytestmark = pytest.mark.gpu


def test_plain_c_caller_on_the_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    exe = cbuild.HERE / "abi_device.bin"
    assert exe.exists(), "tests/c_abi/abi_device.bin is built by __graft_entry__.build()"
    print("[gpu case] plain C caller, R=8 bf16 N=100003", flush=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr
