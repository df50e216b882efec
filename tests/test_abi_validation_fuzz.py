"""Randomised check of arAllReduce's argument validation (host only, no GPU).

A seeded generator draws dtypes, ops, rank counts, protocols, counts and
pointer layouts (aligned, misaligned, NULL, overlapping, in place, partly in
place).  With a NULL communicator the library must give, for each case, the
result code and the AR_DEBUG reason that the documented rules of
include/ar_allreduce.h give, checked in the header's order.  Pointers are
never dereferenced: validation runs before any HIP call.
"""
import json
import random
import subprocess
import sys

import all_reduce_amd as ar

SIZE_MAX = (1 << 64) - 1
ELEM = {0: 2, 1: 2, 2: 4}


def expected(case):
    """(result name, reason substring) for one case, from the header's rules."""
    dtype, op, nranks, proto, count, send, recv = (case[k] for k in
                                                   ("dtype", "op", "nranks", "proto",
                                                    "count", "send", "recv"))
    if dtype not in (0, 1, 2):
        return "arUnsupported", "dtype"
    if op != 0:
        return "arUnsupported", "arSum"
    if not 1 <= nranks <= 32:
        return "arUnsupported", "nranks"
    if proto not in (0, 1, 2):
        return "arInvalidArgument", "protocol"
    if count == 0:
        return "arSuccess", None
    if count > SIZE_MAX // 8:
        return "arInvalidArgument", "count too large"
    if send is None or recv is None:
        return "arInvalidArgument", "NULL buffer array"
    n = count * ELEM[dtype]
    pad = lambda lst: (lst + [0] * nranks)[:nranks]  # the binding NULL-pads short lists
    s_, d_ = pad(send), pad(recv)
    for r in range(nranks):
        s, d = s_[r], d_[r]
        if s == 0 or d == 0:
            return "arInvalidArgument", "NULL rank buffer"
        if (s | d) & 15:
            return "arInvalidArgument", "16-byte aligned"
        if s > (1 << 64) - 1 - n or d > (1 << 64) - 1 - n:
            return "arInvalidArgument", "wraps"
    over = lambda a, b: a < b + n and b < a + n
    for r in range(nranks):
        d = d_[r]
        for q in range(nranks):
            s = s_[q]
            if q == r and s == d:
                continue
            if over(d, s):
                return "arInvalidArgument", "overlaps a send buffer"
            if q != r and over(d, d_[q]):
                return "arInvalidArgument", "receive buffers overlap"
    return "arInvalidArgument", "NULL comm"


def draw(rng):
    nranks = rng.choice([0, 1, 2, 3, 4, 8, 16, 32, 33, rng.randint(1, 32)])
    dtype = rng.choice([0, 1, 2, 2, 1, 0, 3])
    op = rng.choice([0] * 9 + [1])
    proto = rng.choice([0, 1, 2, 2, 1, 0, 3])
    count = rng.choice([0, 1, 7, 1024, 4096, rng.randint(1, 1 << 20), (1 << 62), (1 << 61) + 3])
    base = 0x7F0000000000
    span = 1 << 24  # room per slot for the largest ordinary count
    slots = rng.choice([4, 12, 40])  # fewer slots: more buffers collide
    def ptr():
        kind = rng.random()
        if kind < 0.03:
            return 0
        if kind < 0.05:
            return (1 << 64) - 4096  # aligned, just below the top of the address space
        off = rng.choice([0] * 12 + [8, 4, 16, 32])
        return base + rng.randint(0, slots) * span + off
    send = [ptr() for _ in range(max(nranks, 0) + rng.choice([0, 0, 0, 0, -1]))]
    if rng.random() < 0.3:
        recv = list(send)  # in place
        if recv and rng.random() < 0.3:
            recv[rng.randrange(len(recv))] = ptr()
    else:
        recv = [ptr() for _ in range(len(send))]
    if rng.random() < 0.02:
        send = None
    if rng.random() < 0.02:
        recv = None
    if rng.random() < 0.05 and send:
        send = [s + 2 for s in send]  # misaligned by an element
    return dict(dtype=dtype, op=op, nranks=nranks, proto=proto, count=count, send=send, recv=recv)


CHILD = r"""
import json, sys
sys.path.insert(0, sys.argv[1])
import all_reduce_amd as ar
for c in json.loads(sys.stdin.read()):
    sys.stderr.write("@@\n"); sys.stderr.flush()
    r = ar.arAllReduce(c["send"], c["recv"], c["count"], c["dtype"], c["op"], c["nranks"],
                       c["proto"], None, None)
    sys.stderr.flush()
    print(r, flush=True)
"""


def test_validation_matches_the_rules():
    rng = random.Random(2026)
    cases = [draw(rng) for _ in range(3000)]
    res = subprocess.run([sys.executable, "-c", CHILD, str(ar.HEADER.parent.parent)],
                         input=json.dumps(cases), capture_output=True, text=True,
                         env={"AR_DEBUG": "1", "PATH": "/usr/bin:/bin"}, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    codes = [int(x) for x in res.stdout.split()]
    reasons = res.stderr.split("@@\n")[1:]
    assert len(codes) == len(cases) == len(reasons)
    seen = set()
    for c, code, why in zip(cases, codes, reasons):
        want, text = expected(c)
        assert ar.arResult(code).name == want, (c, ar.arResult(code).name, why)
        if text is None:
            assert why.strip() == "", (c, why)
        else:
            assert text in why, (c, why)
        seen.add((want, text))
    # the generator reaches every rule
    assert len(seen) == 13, sorted(seen, key=str)
