"""Build the HIP library ``_lib/libar_allreduce.so`` for gfx950 with hipcc.

Every ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in
parallel), then linked into one shared library exporting the C ABI of
``include/ar_allreduce.h``.  Compiled in-tree so that the library travels with
the source tree.  Usage: ``python -m all_reduce_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
from pathlib import Path

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
CSRC = PKG / "csrc"
BUILD = PKG / "_build"
LIBDIR = PKG / "_lib"
LIBRARY = LIBDIR / "libar_allreduce.so"
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: no v_pk_*_f32 in generated code.  No fast-math, no
# contraction, binary32 denormals kept: the sums must round exactly as IEEE
# binary32 additions in rank order.
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=off", "-fno-fast-math",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{ROOT / 'include'}", f"-I{CSRC}",
]


def _compile(src: Path, obj: Path, extra: list[str]) -> None:
    cmd = [HIPCC, *HIP_FLAGS, *extra, "-c", str(src), "-o", str(obj)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{res.stdout}\n{res.stderr}")


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> Path:
    """Compile every HIP source and link the library; returns its path."""
    extra = list(extra_flags or [])
    BUILD.mkdir(exist_ok=True)
    LIBDIR.mkdir(exist_ok=True)
    sources = sorted(CSRC.glob("*.hip"))
    if not sources:
        raise RuntimeError(f"no HIP sources under {CSRC}")
    objs = [BUILD / (s.stem + ".o") for s in sources]
    jobs = min(len(sources), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as pool:
        list(pool.map(lambda so: _compile(so[0], so[1], extra), zip(sources, objs)))
    tmp = LIBRARY.with_name(LIBRARY.name + f".tmp{os.getpid()}")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *map(str, objs), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIBRARY)
    if verbose:
        print(f"built {LIBRARY}")
    return LIBRARY


PROBE_SRC = ROOT / "tests" / "gpu_probe" / "convert_probe.hip"
PROBE_LIB = ROOT / "tests" / "gpu_probe" / "libconvert_probe.so"
CEILING_SRC = ROOT / "tests" / "gpu_probe" / "hbm_ceiling.hip"
CEILING_LIB = ROOT / "tests" / "gpu_probe" / "libhbm_ceiling.so"


def _build_shared(src: Path, lib: Path, verbose: bool) -> Path:
    tmp = lib.with_name(lib.name + f".tmp{os.getpid()}")
    cmd = [HIPCC, *HIP_FLAGS, "-shared", str(src), "-o", str(tmp)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src.name}:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def build_probe(verbose: bool = False) -> Path:
    """The GPU probes (same flags): the test-only converter probe, and the HBM
    ceiling probe that bench.py --only ceilings times.  Returns the former."""
    _build_shared(CEILING_SRC, CEILING_LIB, verbose)
    return _build_shared(PROBE_SRC, PROBE_LIB, verbose)


if __name__ == "__main__":
    build(verbose=True)
    build_probe(verbose=True)
