"""Build the two plain-C callers of the C ABI with gcc (test infrastructure).

``abi_host.bin`` uses only the library's host-side answers; ``abi_device.bin``
also uses the HIP runtime API for device memory and runs all-reduces on the
GPU.  Both link the library built by ``all_reduce_amd.build``.
"""
from __future__ import annotations

import subprocess
from pathlib import Path

HERE = Path(__file__).resolve().parent
ROOT = HERE.parent.parent
LIBDIR = ROOT / "all_reduce_amd" / "_lib"
ROCM = Path("/opt/rocm")
CFLAGS = ["-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", f"-I{ROOT / 'include'}"]
LINK = [f"-L{LIBDIR}", "-lar_allreduce", f"-Wl,-rpath,{LIBDIR}", "-Wl,-rpath,$ORIGIN/../../all_reduce_amd/_lib"]


def build() -> list[Path]:
    out = []
    host = HERE / "abi_host.bin"
    subprocess.run(["gcc", *CFLAGS, str(HERE / "abi_host.c"), "-o", str(host), *LINK],
                   check=True, capture_output=True, text=True)
    out.append(host)
    dev = HERE / "abi_device.bin"
    subprocess.run(["gcc", *CFLAGS, f"-I{ROCM / 'include'}", "-D__HIP_PLATFORM_AMD__",
                    str(HERE / "abi_device.c"), "-o", str(dev), *LINK,
                    f"-L{ROCM / 'lib'}", "-lamdhip64", f"-Wl,-rpath,{ROCM / 'lib'}"],
                   check=True, capture_output=True, text=True)
    out.append(dev)
    return out


if __name__ == "__main__":
    for p in build():
        print("built", p)
