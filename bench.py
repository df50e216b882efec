#!/usr/bin/env python3
"""Benchmark of the MI355X sum all-reduce over R = 8 simulated ranks (one GPU).

Prints one JSON line on stdout (a markdown table goes to stderr).

What is timed (inputs resident in HBM before every timed region):

* LL sweep -- R = 8 bf16, 2^k elements per rank for k = 10..19 (2 KiB to
  1 MiB), uniform[-1, 1].  As in the SGLang MSCCL++ benchmark ("SGLang 中的
  MSCCL++ All-Reduce 基准测试与推理集成指南", blog.gitcode.com, section 3.3):
  10 calls captured in one graph, ``--warmup`` untimed replays, then
  ``--steps`` replays inside one HIP event pair; latency per call = elapsed /
  (steps * 10).  The HB protocol is timed the same way at every size, and LL
  vs HB at the decode shape 64 x 8192 with N(0, 1) values.
* HB prefill -- R = 8 bf16, 8192 x 8192 elements per rank (128 MiB), N(0, 1)
  with 0.1 % of entries x1000, in place.  The roofline figure uses ``--steps``
  launches back to back inside one event pair (the kernel's average launch
  duration; each call streams 2 GiB, far more than the 256 MB last-level
  cache).  Also reported ("cold"): ``--warmup`` + ``--steps`` calls each inside
  its own event pair, with the inputs restored from a pristine copy and 512 MiB
  written to flush the last-level cache before each (untimed).
* cpu_baseline -- the CPU oracle (plain C, OpenMP) timed on this host on the
  same LL sweep inputs, a bounded sample.

``value`` is the mean LL latency per call over the sweep in microseconds
(lower is better).  Every timed configuration is first checked bit for bit
against the oracle.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

METRIC = "all-reduce µs @2KiB–1MiB (R=8, hipGraph) + effective HBM GB/s vs peak"
HBM_PEAK_GBPS = 8000.0
CALLS_PER_GRAPH = 10
SWEEP = list(range(10, 20))


def log(msg: str):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--only", choices=["all", "sweep", "prefill", "copy"], default="all",
                    help="run one part (for profiler passes)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle checks")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        log(f"bench.py: --gpus {args.gpus} is not supported. This build runs on one GPU: "
            "the R ranks are simulated as R buffers in one GPU's HBM, so there is no "
            "multi-GPU run to launch.")
        return 2
    if args.steps < 1 or args.warmup < 0:
        log("bench.py: --steps must be >= 1 and --warmup >= 0")
        return 2

    import numpy as np
    import torch

    import all_reduce_amd as ar
    from all_reduce_amd import inputs

    if not torch.cuda.is_available():
        log("bench.py: no GPU visible")
        return 1
    ar.library()  # fails loudly if the HIP library is not built
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    comm = ar.Comm(device=dev, max_ranks=8, max_ll_bytes_per_rank=1 << 20)
    R = 8
    codes = {"ll": ar.arProtocol.arProtoLL, "hb": ar.arProtocol.arProtoHB}

    def launch(sv, rv, n, proto):
        rc = ar.arAllReduce([t.data_ptr() for t in sv], [t.data_ptr() for t in rv], n,
                            ar.arDataType.arBfloat16, ar.arRedOp.arSum, len(sv), codes[proto],
                            comm.handle, torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise ar.ArError(rc, "arAllReduce")

    orc = None
    if not args.no_parity or not args.no_cpu:
        import oracle
        orc = oracle.load()

    def bits16(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def parity(x_cpu, rv):
        if args.no_parity:
            return None
        want = orc.allreduce(bits16(x_cpu), "bf16", nthreads=len(os.sched_getaffinity(0)))
        got = np.stack([bits16(t) for t in rv])
        return bool(np.array_equal(got, want))

    def graph_time(sv, rv, n, proto):
        """µs per call: 10 calls per graph, warmup replays, then steps replays."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                launch(sv, rv, n, proto)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(CALLS_PER_GRAPH):
                launch(sv, rv, n, proto)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1000.0 / (args.steps * CALLS_PER_GRAPH)
        del g
        return us

    result = {}
    rows = []

    # ---- LL sweep (and HB at the same sizes) ------------------------------
    sweep_rows = []
    if args.only in ("all", "sweep"):
        for k in SWEEP:
            case = inputs.sweep(k)
            n = case["count"]
            x = inputs.make(**case)
            _, sv = ar.rank_buffers(R, n, torch.bfloat16, dev)
            _, rv = ar.rank_buffers(R, n, torch.bfloat16, dev)
            for r in range(R):
                sv[r].copy_(x[r])
            row = {"bytes_per_rank": 2 * n, "elems_per_rank": n}
            for proto in ("ll", "hb"):
                launch(sv, rv, n, proto)
                torch.cuda.synchronize()
                row[f"{proto}_parity"] = parity(x, rv)
                us = graph_time(sv, rv, n, proto)
                row[f"{proto}_us"] = round(us, 3)
                row[f"{proto}_gbps"] = round(2 * R * 2 * n / (us * 1e-6) / 1e9, 1)
            sweep_rows.append(row)
            log(f"sweep 2^{k}: LL {row['ll_us']:.2f} us  HB {row['hb_us']:.2f} us")
        if comm.async_error() != ar.arResult.arSuccess:
            raise RuntimeError("LL wait timed out during the sweep")
        result["ll_sweep"] = sweep_rows

        # decode shape, LL vs HB
        case = inputs.WORKLOADS["C3"]
        n = case["count"]
        x = inputs.make(**case)
        _, sv = ar.rank_buffers(R, n, torch.bfloat16, dev)
        _, rv = ar.rank_buffers(R, n, torch.bfloat16, dev)
        for r in range(R):
            sv[r].copy_(x[r])
        dec = {"elems_per_rank": n, "tokens": 64, "hidden": 8192}
        for proto in ("ll", "hb"):
            launch(sv, rv, n, proto)
            torch.cuda.synchronize()
            dec[f"{proto}_parity"] = parity(x, rv)
            dec[f"{proto}_us"] = round(graph_time(sv, rv, n, proto), 3)
        result["decode_64x8192"] = dec
        log(f"decode 64x8192: LL {dec['ll_us']:.2f} us  HB {dec['hb_us']:.2f} us")
        del sv, rv

    # ---- HB prefill, in place, 128 MiB per rank -----------------------------
    if args.only in ("all", "prefill"):
        case = inputs.WORKLOADS["C4"]
        n = case["count"]
        log("prefill: generating 8 x 64M bf16 inputs")
        x = inputs.make(**case)
        plane, sv = ar.rank_buffers(R, n, torch.bfloat16, dev)
        backup = torch.empty_like(plane)
        for r in range(R):
            sv[r].copy_(x[r])
        backup.copy_(plane)
        evict = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        launch(sv, sv, n, "hb")
        torch.cuda.synchronize()
        pre = {"elems_per_rank": n, "bytes_per_rank": 2 * n, "in_place": True}
        pre["parity"] = parity(x, sv)
        del x
        times = []
        for i in range(args.warmup + args.steps):
            plane.copy_(backup)
            evict.fill_(i & 0xFF)
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            launch(sv, sv, n, "hb")
            t1.record()
            torch.cuda.synchronize()
            if i >= args.warmup:
                times.append(t0.elapsed_time(t1) * 1000.0)
        b_alg = 2 * R * 2 * n
        mean_us = statistics.fmean(times)
        pre["us_mean_cold"] = round(mean_us, 2)
        pre["us_median_cold"] = round(statistics.median(times), 2)
        pre["us_min_cold"] = round(min(times), 2)
        # The kernel's average launch duration: steps launches back to back
        # inside one event pair (each call reads 1 GiB and writes 1 GiB, four
        # times the last-level cache, so little survives from call to call).
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            launch(sv, sv, n, "hb")
        t1.record()
        torch.cuda.synchronize()
        avg_us = t0.elapsed_time(t1) * 1000.0 / args.steps
        pre["us_per_launch"] = round(avg_us, 2)
        pre["gbps"] = round(b_alg / (avg_us * 1e-6) / 1e9, 1)
        pre["gbps_cold"] = round(b_alg / (mean_us * 1e-6) / 1e9, 1)
        result["hb_prefill"] = pre
        traffic = _counter_traffic()
        result["roofline"] = {
            "bound": "hbm", "achieved": pre["gbps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(pre["gbps"] / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, "
                            "copy-calibrated)" if traffic is not None else None,
            "kernel": "hb_twoshot<Bf16, R=8>", "bytes_per_launch": b_alg,
            "us_per_launch": pre["us_per_launch"],
        }
        log(f"prefill HB in place: {pre['us_per_launch']:.1f} us per launch, {pre['gbps']:.0f} GB/s "
            f"({100 * pre['gbps'] / HBM_PEAK_GBPS:.1f}% of 8 TB/s), parity {pre['parity']}")
        del plane, backup, evict, sv

    # ---- plain device copy, for context --------------------------------------
    if args.only in ("all", "copy"):
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1000.0 / args.steps
        result["device_copy_1GiB"] = {"us": round(us, 1),
                                      "gbps": round(2 * (1 << 30) / (us * 1e-6) / 1e9, 1)}
        del src, dst

    # ---- oracle on this host's cores -----------------------------------------
    if not args.no_cpu and sweep_rows:
        cores = len(os.sched_getaffinity(0))
        per_size = []
        t_start = time.perf_counter()
        for k in SWEEP:
            case = inputs.sweep(k)
            xb = bits16(inputs.make(**case))
            out = np.empty_like(xb)
            reps, spent = 0, 0.0
            while spent < 1.0 and reps < 2000:
                spent += orc.allreduce_into(list(xb), list(out), "bf16", nthreads=cores,
                                            timed=True)
                reps += 1
            per_size.append(spent / reps * 1e6)
        result["cpu_baseline"] = {
            "value": round(statistics.fmean(per_size), 2), "unit": "us", "cores": cores,
            "kind": "oracle",
            "sample": (f"the oracle (plain C, OpenMP, {cores} threads) on the same LL sweep "
                       "inputs, R=8 bf16 2^10..2^19 elements per rank, each size repeated for "
                       "about 1 s; mean µs per call over the 10 sizes"),
            "per_size_us": [round(v, 2) for v in per_size],
            "host_cpu": _cpu_model(),
            "wall_s": round(time.perf_counter() - t_start, 1),
        }
        log(f"oracle on {cores} threads: mean {result['cpu_baseline']['value']:.1f} us per call")

    if comm.async_error() != ar.arResult.arSuccess:
        raise RuntimeError("an LL wait timed out")
    comm.close()

    # ---- report ---------------------------------------------------------------
    value = statistics.fmean(r["ll_us"] for r in sweep_rows) if sweep_rows else None
    line = {
        "metric": METRIC,
        "value": round(value, 3) if value is not None else None,
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": (round(sum(r["ll_us"] for r in sweep_rows) * CALLS_PER_GRAPH / 1000.0, 4)
                        if sweep_rows else None),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": ("R=8 simulated ranks, bf16: LL one-shot sweep 2^10..2^19 elements "
                         "per rank (2 KiB-1 MiB), 10 calls per hipGraph; HB two-shot in place "
                         "at 8192x8192 per rank (128 MiB) for the HBM roofline"),
            "nranks": R, "calls_per_graph": CALLS_PER_GRAPH,
            "parallelism": "1 GPU, ranks simulated in HBM",
        },
    }
    line.update(result)
    print(json.dumps(line), flush=True)
    _markdown(line)
    return 0


def _sources_digest() -> str:
    """sha256 over the HB kernel's sources, to tie counter readings to them."""
    import hashlib
    from pathlib import Path
    csrc = Path(__file__).resolve().parent / "all_reduce_amd" / "csrc"
    h = hashlib.sha256()
    for name in ("hb_twoshot.hip", "ar_device.hpp", "ar_internal.hpp"):
        h.update((csrc / name).read_bytes())
    return h.hexdigest()


def _counter_traffic():
    """HBM bytes per launch of the prefill HB kernel from the committed counter
    summary, or None when that summary was taken from other kernel sources."""
    from pathlib import Path
    path = Path(__file__).resolve().parent / "profiles" / "hb_twoshot_bf16_r8_128MiB_counters.txt"
    if not path.exists():
        return None
    fields = {}
    for line in path.read_text().splitlines():
        if ":" in line and not line.startswith(("#", " ")):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    if fields.get("source_sha256") != _sources_digest():
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _cpu_model() -> str:
    try:
        for l in open("/proc/cpuinfo"):
            if l.startswith("model name"):
                return l.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _markdown(line: dict):
    rows = line.get("ll_sweep", [])
    if rows:
        log("\n| bytes/rank | LL µs | LL GB/s | HB µs | HB GB/s | parity |")
        log("|---:|---:|---:|---:|---:|:---:|")
        for r in rows:
            log(f"| {r['bytes_per_rank']} | {r['ll_us']:.2f} | {r['ll_gbps']:.0f} | "
                f"{r['hb_us']:.2f} | {r['hb_gbps']:.0f} | {r['ll_parity']}/{r['hb_parity']} |")


if __name__ == "__main__":
    sys.exit(main())
