"""The C ABI library on the host: symbols, constants and argument validation.

No GPU is needed: the library loads without one, and every argument check of
``arAllReduce`` runs before any HIP call.  The reason a call was rejected is
read from the library's ``AR_DEBUG=1`` log in a child process.
"""
import json
import re
import ctypes
import subprocess
import sys

import pytest

import all_reduce_amd as ar

HEADER = ar.HEADER.read_text()


def declared_functions():
    body = re.sub(r"/\*.*?\*/", "", HEADER, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(ar[A-Z]\w*)\s*\(", body, re.M)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) == 14, names
    lib = ar.library()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    exported = subprocess.run(["nm", "-D", "--defined-only", str(ar.LIBRARY)],
                              capture_output=True, text=True, check=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", exported, re.M), n


def test_enums_match_header():
    for enum in (ar.arResult, ar.arDataType, ar.arRedOp, ar.arProtocol, ar.arOption):
        for member in enum:
            m = re.search(rf"\b{member.name}\s*=\s*(\d+)", HEADER)
            assert m and int(m.group(1)) == member.value, member
    assert int(re.search(r"#define AR_MAX_RANKS (\d+)", HEADER).group(1)) == ar.AR_MAX_RANKS
    m = re.search(r"#define AR_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", HEADER)
    assert int(m.group(1)) << int(m.group(2)) == ar.AR_NOALLOC_SCRATCH_BYTES


def test_version_and_error_strings():
    want = int(re.search(r"#define AR_VERSION (\d+)", HEADER).group(1))
    assert ar.arGetVersion() == want
    for code in ar.arResult:
        assert ar.arGetErrorString(code).startswith(code.name)
    assert "unknown" in ar.arGetErrorString(99)


# Each case: (label, kwargs for arAllReduce, expected code, expected log text)
A = 0x7F0000000000  # 16-byte aligned fake device addresses; never dereferenced
L = 4096            # bytes per rank for count 2048 bf16
CASES = [
    ("bad dtype", dict(dtype=3), "arUnsupported", "dtype"),
    ("bad op", dict(op=1), "arUnsupported", "arSum"),
    ("zero ranks", dict(nranks=0), "arUnsupported", "nranks"),
    ("33 ranks", dict(nranks=33), "arUnsupported", "nranks"),
    ("bad protocol", dict(protocol=3), "arInvalidArgument", "protocol"),
    ("NULL send array", dict(send=None), "arInvalidArgument", "NULL buffer array"),
    ("NULL recv array", dict(recv=None), "arInvalidArgument", "NULL buffer array"),
    ("NULL rank pointer", dict(send=[A, 0]), "arInvalidArgument", "NULL rank buffer"),
    ("misaligned", dict(send=[A + 8, A + L]), "arInvalidArgument", "16-byte aligned"),
    ("recv overlaps other send", dict(recv=[A + L, A + 3 * L]), "arInvalidArgument",
     "overlaps a send buffer"),
    ("recv partially overlaps own send", dict(recv=[A + 16, A + 3 * L]), "arInvalidArgument",
     "overlaps a send buffer"),
    ("recv overlap each other", dict(recv=[A + 4 * L, A + 4 * L + 16]), "arInvalidArgument",
     "receive buffers overlap"),
    ("count overflow", dict(count=1 << 62), "arInvalidArgument", "count too large"),
    # valid arguments: reaches the communicator check
    ("valid out of place", dict(), "arInvalidArgument", "NULL comm"),
    ("valid in place", dict(recv=[A, A + L]), "arInvalidArgument", "NULL comm"),
    ("sends may overlap", dict(send=[A, A], recv=[A + 4 * L, A + 5 * L]), "arInvalidArgument",
     "NULL comm"),
    ("count zero", dict(count=0, send=None, recv=None), "arSuccess", None),
    # fewer pointers than ranks: the binding pads with NULL, the library rejects
    ("short pointer list", dict(nranks=4), "arInvalidArgument", "NULL rank buffer"),
]

CHILD = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import all_reduce_amd as ar
for label, kw in json.loads(sys.argv[2]):
    args = dict(send=[0x7F0000000000, 0x7F0000000000 + 4096],
                recv=[0x7F0000000000 + 2 * 4096, 0x7F0000000000 + 3 * 4096],
                count=2048, dtype=0, op=0, nranks=2, protocol=1)
    args.update(kw)
    sys.stderr.write(f"@@{label}\n"); sys.stderr.flush()
    r = ar.arAllReduce(args["send"], args["recv"], args["count"], args["dtype"], args["op"],
                       args["nranks"], args["protocol"], None, None)
    sys.stderr.flush()
    print(json.dumps([label, r]), flush=True)
"""


@pytest.fixture(scope="module")
def validation_results():
    payload = json.dumps([(c[0], c[1]) for c in CASES])
    res = subprocess.run([sys.executable, "-c", CHILD, str(ar.HEADER.parent.parent), payload],
                         capture_output=True, text=True, env={"AR_DEBUG": "1", "PATH": "/usr/bin:/bin"},
                         timeout=120)
    assert res.returncode == 0, res.stderr
    codes = dict(json.loads(line) for line in res.stdout.splitlines())
    logs = {}
    for part in res.stderr.split("@@")[1:]:
        label, _, text = part.partition("\n")
        logs[label] = text
    return codes, logs


@pytest.mark.parametrize("label,kw,code,why", CASES, ids=[c[0] for c in CASES])
def test_validation(validation_results, label, kw, code, why):
    codes, logs = validation_results
    assert codes[label] == ar.arResult[code], (label, codes[label])
    if why is not None:
        assert why in logs[label], logs[label]
    else:
        assert logs[label].strip() == ""


def test_comm_arguments_checked_before_the_device():
    r, h = ar.arCommCreate(0, 0, 1024)
    assert r == ar.arResult.arInvalidArgument and h is None
    r, h = ar.arCommCreate(0, 33, 1024)
    assert r == ar.arResult.arInvalidArgument
    assert ar.arCommDestroy(None) == ar.arResult.arInvalidArgument
    assert ar.arCommReset(None, None) == ar.arResult.arInvalidArgument
    assert ar.arCommSetOption(None, 0, 1) == ar.arResult.arInvalidArgument
    assert ar.arCommGetOption(None, 0)[0] == ar.arResult.arInvalidArgument
    assert ar.arCommGetAsyncError(None)[0] == ar.arResult.arInvalidArgument
    assert ar.arCommTune(None, 0, 8, 1 << 20, None) == ar.arResult.arInvalidArgument
    assert ar.arCommGetTunedShape(None, 0, 8, 0, 1024)[0] == ar.arResult.arInvalidArgument


def test_comm_create_without_a_gpu_reports_hip_error():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    r, h = ar.arCommCreate(0, 8, 1 << 20)
    assert r == ar.arResult.arHipError and h is None


def test_python_helpers():
    import torch
    assert ar.protocol_code("LL") == ar.arProtocol.arProtoLL
    assert ar.protocol_code("hb") == ar.arProtocol.arProtoHB
    assert ar.protocol_code("auto") == ar.arProtocol.arProtoAuto
    assert ar.dtype_code(torch.bfloat16) == ar.arDataType.arBfloat16
    assert ar.dtype_code(torch.float32) == ar.arDataType.arFloat32
    with pytest.raises(ar.ArError):
        ar.dtype_code(torch.int32)


def test_plain_c_caller_host_side():
    """The header compiles as C99 and a C program linked to the library gets
    the host-side answers (no GPU needed)."""
    from c_abi import build as cbuild
    exe = cbuild.HERE / "abi_host.bin"
    if not exe.exists() or exe.stat().st_mtime < ar.LIBRARY.stat().st_mtime:
        cbuild.build()
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0 and res.stdout.strip() == "ok", res.stdout + res.stderr


def test_binding_mirrors_the_c_layout():
    """The ctypes mirrors of arTunedShape_t and arLaunchInfo_t have the C
    structs' sizes and field offsets, and the enums are int-sized as the binding assumes."""
    from c_abi import build as cbuild
    exe = cbuild.HERE / "abi_host.bin"
    if not exe.exists() or exe.stat().st_mtime < ar.LIBRARY.stat().st_mtime:
        cbuild.build()
    res = subprocess.run([str(exe), "layout"], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0, res.stdout + res.stderr
    shape_line, info_line, enum_line = res.stdout.strip().splitlines()
    for line, m in ((shape_line, ar.arTunedShape), (info_line, ar.arLaunchInfo)):
        words = line.split()
        c_layout = {words[i]: int(words[i + 1]) for i in range(0, len(words), 2)}
        py_layout = {words[0]: ctypes.sizeof(m)}
        py_layout.update({name: getattr(m, name).offset for name, _ in m._fields_})
        assert py_layout == c_layout
    words = enum_line.split()
    assert all(int(words[i + 1]) == ctypes.sizeof(ctypes.c_int) for i in range(0, len(words), 2))
