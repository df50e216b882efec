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


def test_plain_c_caller_times_eager_calls():
    """--time: after the same checks, the host's cost per eager call from C
    (the smallest call, and LL / HB at 8 ranks x 2 KiB)."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import re
    exe = cbuild.HERE / "abi_device.bin"
    print("[gpu case] plain C caller, eager timing", flush=True)
    res = subprocess.run([str(exe), "--time"], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0 and res.stdout.strip().endswith("ok"), res.stdout + res.stderr
    m = re.search(r"hb_1rank_16B ([\d.]+) ll_8x2KiB ([\d.]+) hb_8x2KiB ([\d.]+)", res.stdout)
    assert m, res.stdout
    assert all(0 < float(v) < 1000 for v in m.groups())
