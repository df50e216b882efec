"""Host-side code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

* The oracle (plain C) is rebuilt with gcc's sanitizers and driven through
  every entry point by ``tests/sanitize/oracle_driver.c``: all dtypes, rank
  counts 1..32, ragged sizes, the grouped order, the converters.
* The C ABI layer (``api.hip``, the host logic: validation, option handling,
  error strings) is rebuilt with the sanitizers on its host side only
  (``-Xarch_host``), linked with the library's other objects, and driven by
  ``tests/sanitize/abi_driver.c``: every entry point with a NULL communicator,
  communicator creation without a usable GPU, and thousands of randomised
  argument sets with out-of-range enums and exactly sized pointer arrays.
No GPU is used.
"""
import os
import shutil
import subprocess
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
SAN = ROOT / "tests" / "sanitize"
CLANG = Path("/opt/rocm/llvm/bin/clang")
HIPCC = Path(os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc"))
ENV = {"PATH": "/usr/bin:/bin", "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=0",
       "UBSAN_OPTIONS": "print_stacktrace=1"}


def run(cmd, **kw):
    res = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert res.returncode == 0, f"{cmd[0]}: {res.stdout[-3000:]}\n{res.stderr[-3000:]}"
    return res


def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_san"
    run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
         "-ffp-contract=off", "-fno-fast-math", str(ROOT / "oracle" / "oracle.c"),
         str(SAN / "oracle_driver.c"), "-o", str(exe), "-lm"])
    res = run([str(exe)], env=ENV, timeout=300)
    assert res.stdout.strip() == "ok", res.stdout


def test_abi_host_side_under_asan_and_ubsan(tmp_path):
    if not CLANG.exists():
        pytest.skip("clang from the ROCm toolchain is not installed")
    build = ROOT / "all_reduce_amd" / "_build"
    others = [build / f"{s.stem}.o" for s in sorted((ROOT / "all_reduce_amd" / "csrc").glob("*.hip"))
              if s.stem != "api"]
    if not all(o.exists() for o in others):
        pytest.skip("library objects missing: run the build first")
    api = tmp_path / "api_san.o"
    run([str(HIPCC), "--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
         "-Wno-unused-command-line-argument", f"-I{ROOT / 'include'}",
         f"-I{ROOT / 'all_reduce_amd' / 'csrc'}", "-c",
         str(ROOT / "all_reduce_amd" / "csrc" / "api.hip"), "-o", str(api)])
    lib = tmp_path / "libar_san.so"
    run([str(HIPCC), "--offload-arch=gfx950", "-shared", "-fPIC", str(api),
         *map(str, others), "-o", str(lib)])
    exe = tmp_path / "abi_san"
    run([str(CLANG), "-std=c99", "-g", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", f"-I{ROOT / 'include'}", str(SAN / "abi_driver.c"),
         f"-L{tmp_path}", "-lar_san", f"-Wl,-rpath,{tmp_path}", "-Wl,-rpath,/opt/rocm/lib",
         "-o", str(exe)])
    env = dict(ENV, ASAN_OPTIONS="detect_leaks=0")  # the HIP runtime keeps its own state
    res = run([str(exe)], env=env, timeout=300)
    assert res.stdout.strip() == "ok", res.stdout
