#!/usr/bin/env python3
"""Benchmark of the MI355X sum all-reduce over R simulated ranks (one GPU).

Prints one JSON line on stdout; a markdown table goes to stderr.

Default run (inputs resident in HBM before every timed region; the built-in
launch shapes, so that a profiled run of the same command launches the shapes
the line reports; ``--tune`` first runs the start-up tuning of the guide's
section 4.4, arCommTune for bf16 R = 8 up to 128 MiB per rank):

* LL sweep -- R = 8 bf16, 2^k elements per rank for k = 10..19 (2 KiB to
  1 MiB), uniform[-1, 1].  As in the SGLang MSCCL++ benchmark ("SGLang 中的
  MSCCL++ All-Reduce 基准测试与推理集成指南", blog.gitcode.com, section 3.3):
  10 calls captured in one graph, ``--warmup`` untimed replays, then
  ``--steps`` replays inside one HIP event pair; latency per call = elapsed /
  (steps * 10).  Untimed passes over every size and protocol come first (for
  at least 2 s), so no size is timed as the first use of anything, nor while
  the GPU comes out of idle; four more timed passes
  per size give a median beside the guide's figure.  Each size also gets the
  guide's eager timing (2 warm-up calls, then the mean of 10 back-to-back
  calls) for LL and HB, through prepared calls (arguments marshalled once),
  and a timing-only plain-torch row (stack, fp32 sum, cast, copy to every
  rank).  Every row names the launch shape it ran (arCommGetLastLaunch).
* LL vs HB at the decode shape 64 x 8192 with N(0, 1) values.
* C1 -- R = 8, 1024 bf16: one out-of-place call of each protocol.
* HB prefill -- R = 8 bf16, 8192 x 8192 elements per rank (128 MiB), N(0, 1)
  with 0.1 % of entries x1000, in place.  The roofline figure uses ``--steps``
  launches back to back inside one event pair (the kernel's average launch
  duration; each call streams 2 GiB, far more than the 256 MB last-level
  cache).  Also reported ("cold"): ``--warmup`` + ``--steps`` calls each inside
  its own event pair, with the inputs restored from a pristine copy and 512 MiB
  written to flush the last-level cache before each (untimed).
* C5 -- R = 16 and 32, integers -4..4: 2^18 fp16 per rank (graph-replayed,
  HB and LL) and 4096 x 7168 fp32 per rank (112 MiB, HB back to back, out of
  place), HB with chunk = N/R beside the interleaved default layout.
* graph_floor_us -- the per-call cost of a graph-replayed one-rank, 16-byte
  call (one workgroup), to split LL latency into launch floor and protocol;
  ll_mean_above_floor_us is the sweep's mean LL latency minus it (the floor
  differs from machine to machine, the protocol's share much less).
* cpu_baseline -- the CPU oracle (plain C, OpenMP) timed on this host on the
  same LL sweep inputs, a bounded sample (per size the median of 3 runs of
  0.5 s of calls on all threads, and of 0.25 s on one thread).
* hbm_ceilings -- what the memory system delivers for the HB prefill's access
  shape without its arithmetic (tests/gpu_probe/hbm_ceiling.hip): 8 streams of
  128 MiB read only, written only (with non-temporal or ordinary stores), or
  copied, with HB's tile mapping and 128-bit accesses, best of a few launch
  shapes; HB in place is compared with the bound its equal read and write
  bytes imply.

``value`` is the mean LL latency per call over the sweep in microseconds
(lower is better), from the guide's single timed pass per size;
``value_median_passes`` the same from the per-size medians.  Every timed
configuration is first checked bit for bit against the oracle.

``--configs`` adds every named workload (R = 8 small, the sweep, decode,
prefill, and R = 16 / 32 with integer data in fp16 and fp32) as rows of one
table, plus the hierarchical order (nodes of 8) and the staged HB forms at
their shapes: µs per call, effective GB/s (2 * R * bytes per rank / time),
share of the 8 TB/s HBM peak, HBM GB/s from the committed rocprofv3 counter
summaries where one covers the kernel, the oracle's time at 1 and at all
host threads and its own GB/s, parity.

``--only {sweep, prefill, copy, c5, c5b, hier, ll_variants, ceilings}`` runs
one part alone (for profiler passes; c5b is the fp32 R = 16 / 32 workload at
112 MiB per rank, hier the same in the two-level order, fused and staged).
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
MEDIAN_PASSES = 5
SWEEP = list(range(10, 20))
EAGER_WARMUP, EAGER_CALLS = 2, 10
C5B_BYTES = 4096 * 7168 * 4  # bytes per rank of the fp32 4096 x 7168 workload
C5B_COUNTERS = "hb_twoshot_fp32_r16_r32_112MiB_counters.txt"


def log(msg: str):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--only", choices=["all", "sweep", "prefill", "copy", "c5", "c5b", "hier",
                                       "ll_variants", "ceilings"],
                    default="all", help="run one part (for profiler passes and ablations)")
    ap.add_argument("--configs", action="store_true",
                    help="also measure every named workload and print the full table")
    ap.add_argument("--tune", action="store_true",
                    help="run the start-up tuning (arCommTune) first, as SGLang's integration "
                         "does; by default the built-in launch shapes are timed")
    ap.add_argument("--sizes", default=None,
                    help="with --only ll_variants: comma-separated log2 element counts to run "
                         "(default: the whole sweep, 10..19)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle checks")
    return ap.parse_args()


class Bench:
    """Timing helpers around one communicator; all calls go through arAllReduce."""

    def __init__(self, args):
        import numpy as np
        import torch

        import all_reduce_amd as ar

        self.np, self.torch, self.ar, self.args = np, torch, ar, args
        ar.library()  # fails loudly if the HIP library is not built
        self.dev = torch.device("cuda", 0)
        torch.cuda.set_device(self.dev)
        self.comm = ar.Comm(device=self.dev, max_ranks=32, max_ll_bytes_per_rank=1 << 20)
        self.codes = {"ll": ar.arProtocol.arProtoLL, "hb": ar.arProtocol.arProtoHB}
        self.dtypes = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}
        self.threads = len(os.sched_getaffinity(0))
        self.orc = None
        if not args.no_parity or not args.no_cpu:
            import oracle
            self.orc = oracle.load()

    # -- buffers and calls ------------------------------------------------
    def planes(self, x):
        R, n = x.shape
        _, sv = self.ar.rank_buffers(R, n, x.dtype, self.dev)
        for r in range(R):
            sv[r].copy_(x[r])
        _, rv = self.ar.rank_buffers(R, n, x.dtype, self.dev)
        return sv, rv

    def launch(self, sv, rv, n, proto):
        dt = self.ar.dtype_code(sv[0].dtype)
        rc = self.ar.arAllReduce([t.data_ptr() for t in sv], [t.data_ptr() for t in rv], n, dt,
                                 self.ar.arRedOp.arSum, len(sv), self.codes[proto],
                                 self.comm.handle, self.torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise self.ar.ArError(rc, "arAllReduce")

    def events(self):
        E = self.torch.cuda.Event
        return E(enable_timing=True), E(enable_timing=True)

    # -- parity and the oracle ----------------------------------------------
    def bits(self, t):
        t = t.contiguous()
        if t.dtype == self.torch.float32:
            return t.cpu().numpy().view(self.np.uint32)
        return t.view(self.torch.int16).cpu().numpy().view(self.np.uint16)

    def oracle_in(self, x):
        b = self.bits(x)
        return b.view(self.np.float32) if x.dtype == self.torch.float32 else b

    def dname(self, t):
        return {v: k for k, v in self.dtypes.items()}[t.dtype]

    def parity(self, x, rv, sample=None):
        """Outputs bit-equal to the oracle's (optionally on sampled columns)."""
        if self.args.no_parity:
            return None
        torch, np = self.torch, self.np
        if sample is not None:
            x = x[:, sample].contiguous()
            got = np.stack([self.bits(t[sample.to(t.device)]) for t in rv])
        else:
            got = np.stack([self.bits(t) for t in rv])
        want = self.orc.allreduce(self.oracle_in(x), self.dname(x), nthreads=self.threads)
        want = want.view(np.uint32) if x.dtype == torch.float32 else want.view(np.uint16)
        return bool(np.array_equal(got, want))

    def oracle_ms(self, x, nthreads, reps=3):
        if self.args.no_cpu:
            return None
        xi = self.oracle_in(x)
        out = self.np.empty_like(xi)
        ts = [self.orc.allreduce_into(list(xi), list(out), self.dname(x), nthreads=nthreads,
                                      timed=True) for _ in range(reps)]
        return round(statistics.median(ts) * 1e3, 3)

    # -- timings ------------------------------------------------------------
    def graph_passes(self, sv, rv, n, proto, passes=1, call=None, check=None):
        """µs per call: 10 calls per graph, warmup replays, then ``passes``
        timed passes of steps replays, each inside its own event pair.
        ``call`` (optional) makes one call on the current stream instead of
        arAllReduce with the communicator.  With ``check`` (out of place
        only), the outputs are zeroed after capture, the graph is replayed
        once, and ``check()`` (the oracle comparison) is kept in
        ``last_graph_parity`` before the warm-up replays."""
        torch = self.torch
        one = call if call is not None else (lambda: self.launch(sv, rv, n, proto))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(2):
                one()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(CALLS_PER_GRAPH):
                one()
        self.last_graph_parity = None
        if check is not None:
            for t in rv:
                t.zero_()
            g.replay()
            torch.cuda.synchronize()
            self.last_graph_parity = check()
        for _ in range(self.args.warmup):
            g.replay()
        torch.cuda.synchronize()
        times = []
        for _ in range(passes):
            t0, t1 = self.events()
            t0.record()
            for _ in range(self.args.steps):
                g.replay()
            t1.record()
            torch.cuda.synchronize()
            times.append(t0.elapsed_time(t1) * 1000.0 / (self.args.steps * CALLS_PER_GRAPH))
        del g
        return times

    def graph_us(self, sv, rv, n, proto):
        """µs per call of one timed pass (see graph_passes)."""
        return self.graph_passes(sv, rv, n, proto)[0]

    def launch_record(self, protocol):
        """The launch shape of the communicator's last call, for the line."""
        rec = self.comm.last_launch()
        keys = ("grid", "threads", "packetBytes", "packetPayloadBytes") if protocol == "ll" else \
            ("grid", "threads", "nonTemporal", "kernels")
        return {k: rec[k] for k in keys}

    def eager_us(self, fn):
        """2 warm-up calls, then the mean of 10 back-to-back calls.  The library
        calls come prepared (``Comm.prepare``: arguments marshalled once), as a
        framework holds them for its fixed buffers."""
        for _ in range(EAGER_WARMUP):
            fn()
        self.torch.cuda.synchronize()
        t0, t1 = self.events()
        t0.record()
        for _ in range(EAGER_CALLS):
            fn()
        t1.record()
        self.torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1000.0 / EAGER_CALLS

    def torch_fn(self, sv, rv):
        """Timing-only plain-torch all-reduce: stack, fp32 sum, cast, copy out."""
        torch = self.torch

        def fn():
            y = torch.stack(sv).float().sum(0).to(sv[0].dtype)
            for t in rv:
                t.copy_(y)
        return fn

    def back_to_back_us(self, sv, rv, n, proto, reps, call=None):
        one = call if call is not None else (lambda: self.launch(sv, rv, n, proto))
        t0, t1 = self.events()
        t0.record()
        for _ in range(reps):
            one()
        t1.record()
        self.torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1000.0 / reps

    def cold_us(self, plane, backup, sv, rv, n, proto, calls, warmup):
        """Per-call events; inputs restored and the last-level cache flushed first."""
        torch = self.torch
        evict = torch.empty(512 << 20, dtype=torch.uint8, device=self.dev)
        times = []
        for i in range(warmup + calls):
            if backup is not None:
                plane.copy_(backup)
            evict.fill_(i & 0xFF)
            torch.cuda.synchronize()
            t0, t1 = self.events()
            t0.record()
            self.launch(sv, rv, n, proto)
            t1.record()
            torch.cuda.synchronize()
            if i >= warmup:
                times.append(t0.elapsed_time(t1) * 1000.0)
        del evict
        return times


def gbps(R, n, esize, us):
    return round(2 * R * n * esize / (us * 1e-6) / 1e9, 1)


def main():
    args = parse()
    if args.gpus != 1:
        log(f"bench.py: --gpus {args.gpus} is not supported. This library runs on one GPU: "
            "the R ranks are simulated as R buffers in one GPU's HBM, so there is no "
            "multi-GPU run to launch.")
        return 2
    if args.steps < 1 or args.warmup < 0:
        log("bench.py: --steps must be >= 1 and --warmup >= 0")
        return 2

    import torch

    from all_reduce_amd import inputs

    if not torch.cuda.is_available():
        log("bench.py: no GPU visible")
        return 1
    B = Bench(args)
    R = 8
    result = {}

    # Start-up tuning (--tune), as SGLang's MSCCL++ integration does (guide
    # section 4.4): every power-of-two size of the bf16 R = 8 workloads, both
    # protocols.  By default the built-in shapes are timed, so that a profiled
    # run of the same command launches exactly the shapes this line reports.
    if args.tune and args.only in ("all", "sweep", "prefill"):
        t0 = time.perf_counter()
        B.comm.tune(torch.bfloat16, R, 128 << 20)
        result["tuning"] = {"dtype": "bf16", "nranks": R, "max_bytes_per_rank": 128 << 20,
                            "wall_s": round(time.perf_counter() - t0, 2)}
        log(f"arCommTune bf16 R=8 up to 128 MiB per rank: {result['tuning']['wall_s']} s")

    # ---- LL sweep (HB, eager and plain torch at the same sizes) -------------
    sweep_rows = []
    if args.only in ("all", "sweep"):
        # Untimed passes over every size and protocol first (graphs captured
        # and replayed, eager calls), repeated for at least 2 s, so that no
        # size is timed as the first use of a buffer size, a graph shape or a
        # kernel, nor while the GPU is still coming out of idle (on some
        # machines the first timed size ran up to 1 us slow after a single
        # short pass).
        warm_inputs = [inputs.make(**inputs.sweep(k)) for k in SWEEP]
        t_warm = time.perf_counter()
        while True:
            for xw in warm_inputs:
                sv, rv = B.planes(xw)
                n = xw.shape[1]
                for proto in ("ll", "hb"):
                    B.graph_passes(sv, rv, n, proto)
                    B.eager_us(B.comm.prepare(sv, rv, proto))
                del sv, rv
            torch.cuda.synchronize()
            if time.perf_counter() - t_warm >= 2.0:
                break
        del warm_inputs
        for k in SWEEP:
            case = inputs.sweep(k)
            n = case["count"]
            x = inputs.make(**case)
            sv, rv = B.planes(x)
            row = {"bytes_per_rank": 2 * n, "elems_per_rank": n}
            for proto in ("ll", "hb"):
                B.launch(sv, rv, n, proto)
                torch.cuda.synchronize()
                row[f"{proto}_launch"] = B.launch_record(proto)
                row[f"{proto}_parity"] = B.parity(x, rv)
                # the first pass is the guide's protocol (--steps replays in one
                # event pair); four more give the median beside it.  The graph's
                # own first replay is checked against the oracle too.
                times = B.graph_passes(sv, rv, n, proto, passes=MEDIAN_PASSES,
                                       check=lambda: B.parity(x, rv))
                row[f"{proto}_parity_graph"] = B.last_graph_parity
                row[f"{proto}_us"] = round(times[0], 3)
                row[f"{proto}_us_median"] = round(statistics.median(times), 3)
                row[f"{proto}_gbps"] = gbps(R, n, 2, times[0])
                row[f"{proto}_eager_us"] = round(B.eager_us(B.comm.prepare(sv, rv, proto)), 3)
            row["torch_eager_us"] = round(B.eager_us(B.torch_fn(sv, rv)), 3)
            sweep_rows.append(row)
            log(f"sweep 2^{k}: LL {row['ll_us']:.2f} (median {row['ll_us_median']:.2f}) us  "
                f"HB {row['hb_us']:.2f} (median {row['hb_us_median']:.2f}) us (graph); "
                f"eager LL {row['ll_eager_us']:.2f} HB {row['hb_eager_us']:.2f} "
                f"torch {row['torch_eager_us']:.2f}; LL {row['ll_launch']}")
        if B.comm.async_error() != B.ar.arResult.arSuccess:
            raise RuntimeError("LL wait timed out during the sweep")
        result["ll_sweep"] = sweep_rows

        case = inputs.WORKLOADS["C3"]
        n = case["count"]
        x = inputs.make(**case)
        sv, rv = B.planes(x)
        dec = {"elems_per_rank": n, "tokens": 64, "hidden": 8192}
        for proto in ("ll", "hb"):
            B.launch(sv, rv, n, proto)
            torch.cuda.synchronize()
            dec[f"{proto}_launch"] = B.launch_record(proto)
            dec[f"{proto}_parity"] = B.parity(x, rv)
            times = B.graph_passes(sv, rv, n, proto, passes=MEDIAN_PASSES,
                                   check=lambda: B.parity(x, rv))
            dec[f"{proto}_parity_graph"] = B.last_graph_parity
            dec[f"{proto}_us"] = round(times[0], 3)
            dec[f"{proto}_us_median"] = round(statistics.median(times), 3)
        result["decode_64x8192"] = dec
        log(f"decode 64x8192: LL {dec['ll_us']:.2f} us  HB {dec['hb_us']:.2f} us")
        del sv, rv

        # The per-call floor of a graph-replayed launch: a one-rank, 16-byte
        # HB call (one workgroup, one vector), for the latency breakdown.
        x = inputs.make(1, 8, "bf16", "uniform", seed=0)
        sv, rv = B.planes(x)
        # Minimum of five measurements: a lone one-workgroup graph has read up
        # to 4.5 us on some runs where every real call of the sweep ran faster.
        result["graph_floor_us"] = round(min(B.graph_us(sv, rv, 8, "hb") for _ in range(5)), 3)
        result["ll_mean_above_floor_us"] = round(
            statistics.fmean(r["ll_us"] for r in sweep_rows) - result["graph_floor_us"], 3)
        log(f"graph-replayed launch floor: {result['graph_floor_us']:.2f} us per call")
        del sv, rv

    # ---- C1: R = 8, 1024 bf16, one out-of-place call -------------------------
    if args.only in ("all", "sweep"):
        result["c1"] = run_c1(B, inputs)

    # ---- HB prefill, in place, 128 MiB per rank -----------------------------
    if args.only in ("all", "prefill"):
        case = inputs.WORKLOADS["C4"]
        n = case["count"]
        log("prefill: generating 8 x 64M bf16 inputs")
        x = inputs.make(**case)
        plane, sv = B.ar.rank_buffers(R, n, torch.bfloat16, B.dev)
        for r in range(R):
            sv[r].copy_(x[r])
        backup = plane.clone()
        B.launch(sv, sv, n, "hb")
        torch.cuda.synchronize()
        pre = {"elems_per_rank": n, "bytes_per_rank": 2 * n, "in_place": True,
               "launch": B.launch_record("hb")}
        pre["parity"] = B.parity(x, sv)
        if args.configs:
            pre["oracle_ms_1"] = B.oracle_ms(x, 1, reps=1)
            pre["oracle_ms_T"] = B.oracle_ms(x, B.threads, reps=1)
        del x
        times = B.cold_us(plane, backup, sv, sv, n, "hb", args.steps, args.warmup)
        b_alg = 2 * R * 2 * n
        mean_us = statistics.fmean(times)
        pre["us_mean_cold"] = round(mean_us, 2)
        pre["us_median_cold"] = round(statistics.median(times), 2)
        pre["us_min_cold"] = round(min(times), 2)
        # The kernel's average launch duration: steps launches back to back
        # inside one event pair.
        avg_us = B.back_to_back_us(sv, sv, n, "hb", args.steps)
        pre["us_per_launch"] = round(avg_us, 2)
        # The same calls graph-replayed (10 per graph, timed like the sweep).
        pre["us_graph"] = round(B.graph_us(sv, sv, n, "hb"), 2)
        pre["gbps"] = gbps(R, n, 2, avg_us)
        pre["gbps_cold"] = gbps(R, n, 2, mean_us)
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
        log(f"prefill HB in place: {pre['us_per_launch']:.1f} us per launch "
            f"({pre['us_graph']:.1f} graph-replayed), {pre['gbps']:.0f} GB/s "
            f"({100 * pre['gbps'] / HBM_PEAK_GBPS:.1f}% of 8 TB/s), parity {pre['parity']}")
        del plane, backup, sv

    # ---- plain device copy, for context --------------------------------------
    if args.only in ("all", "copy"):
        src = torch.empty(1 << 30, dtype=torch.uint8, device=B.dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(args.warmup):
            dst.copy_(src)
        torch.cuda.synchronize()
        t0, t1 = B.events()
        t0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        t1.record()
        torch.cuda.synchronize()
        us = t0.elapsed_time(t1) * 1000.0 / args.steps
        result["device_copy_1GiB"] = {"us": round(us, 1),
                                      "gbps": round(2 * (1 << 30) / (us * 1e-6) / 1e9, 1)}
        del src, dst

    # ---- C5: R = 16 / 32, fp16 2^18 and fp32 4096 x 7168 integers -----------
    # (--only c5b: the fp32 part alone, for the profiler's counter passes)
    if args.only in ("all", "c5", "c5b"):
        if args.tune:
            for R5 in (16, 32):
                if args.only != "c5b":
                    B.comm.tune(torch.float16, R5, 1 << 19)
                B.comm.tune(torch.float32, R5, C5B_BYTES)
        result["c5"] = run_c5(B, inputs, fp16=args.only != "c5b")

    # ---- two-level order at the fp32 C5b shapes alone (for profiler passes) --
    if args.only == "hier":
        result["hier"] = run_hier(B, inputs, ((16, "fp32"), (32, "fp32")))

    # ---- HBM ceilings of the HB access pattern, beside HB itself -------------
    if args.only in ("all", "ceilings"):
        ceil = run_ceilings(B, args)
        rd = ceil["read"]["best_gbps"]
        wr = max(ceil["write"]["best_gbps"], ceil["write, ordinary stores"]["best_gbps"])
        mixed = 2.0 / (1.0 / rd + 1.0 / wr)   # equal bytes read and written, one after the other
        hb = ceil["hb in place"]["gbps"]
        result["hbm_ceilings"] = {
            "read_gbps": rd, "write_gbps": wr,
            "copy_in_place_gbps": ceil["copy in place"]["best_gbps"],
            "copy_out_of_place_gbps": ceil["copy out of place"]["best_gbps"],
            "read_write_bound_gbps": round(mixed, 1),
            "hb_in_place_gbps": hb, "hb_frac_of_read_write_bound": round(hb / mixed, 4),
            "note": "HB's access shape without its arithmetic (tests/gpu_probe/hbm_ceiling.hip), "
                    "best of 6 launch shapes per pattern; reads non-temporal, writes the "
                    "better of non-temporal and ordinary stores; the read/write bound combines "
                    "the read-only and write-only ceilings for equal bytes"}
        if args.only == "ceilings":
            result["ceilings"] = ceil
        result["hbm_ceilings_c5b"] = run_c5b_ceilings(B, args)

    # ---- LL flag scheme x packet width at the default shape, over the sweep ---
    if args.only == "ll_variants":
        opt = B.ar.arOption
        rows = []
        for k in ([int(v) for v in args.sizes.split(",")] if args.sizes else SWEEP):
            case = inputs.sweep(k)
            n = case["count"]
            x = inputs.make(**case)
            sv, rv = B.planes(x)
            row = {"bytes_per_rank": 2 * n}
            for scheme, sname in ((0, "cleared"), (1, "sequenced")):
                for width in (8, 16):
                    B.comm.set_option(opt.arOptLLFlagScheme, scheme)
                    B.comm.set_option(opt.arOptLLPacketBytes, width)
                    B.launch(sv, rv, n, "ll")
                    torch.cuda.synchronize()
                    key = f"{sname}_{width}"
                    row[f"{key}_parity"] = B.parity(x, rv)
                    row[f"{key}_us"] = round(B.graph_us(sv, rv, n, "ll"), 3)
            B.comm.set_option(opt.arOptLLFlagScheme, 0)
            B.comm.set_option(opt.arOptLLPacketBytes, 0)
            rows.append(row)
            log("ll_variants 2^%d: " % k + "  ".join(
                f"{key[:-3]} {v:.2f}" for key, v in row.items() if key.endswith("_us")))
            del sv, rv
        if B.comm.async_error() != B.ar.arResult.arSuccess:
            raise RuntimeError("LL wait timed out during the LL variant sweep")
        result["ll_variants"] = rows
        for key in [k for k in rows[0] if k.endswith("_us")]:
            result[f"ll_variants_mean_{key}"] = round(statistics.mean(r[key] for r in rows), 3)

    # ---- every named workload as one table ----------------------------------
    if args.configs and args.only == "all":
        result["configs"] = run_configs(B, inputs, sweep_rows, result)

    # ---- oracle on this host's cores -----------------------------------------
    if not args.no_cpu and sweep_rows:
        cores = B.threads
        t_start = time.perf_counter()

        def per_call_us(xb, out, nthreads, seconds):
            """One run: calls repeated for ``seconds`` of timed work; µs per call."""
            reps, spent = 0, 0.0
            while spent < seconds:
                spent += B.orc.allreduce_into(list(xb), list(out), "bf16", nthreads=nthreads,
                                              timed=True)
                reps += 1
            return spent / reps * 1e6

        per_size, per_size_1 = [], []
        for k in SWEEP:
            xb = B.oracle_in(inputs.make(**inputs.sweep(k)))
            out = B.np.empty_like(xb)
            per_size.append(statistics.median(per_call_us(xb, out, cores, 0.5)
                                              for _ in range(3)))
            per_size_1.append(statistics.median(per_call_us(xb, out, 1, 0.25)
                                                for _ in range(3)))
        result["cpu_baseline"] = {
            "value": round(statistics.fmean(per_size), 2), "unit": "us", "cores": cores,
            "kind": "oracle",
            "sample": (f"the oracle (plain C, OpenMP) on the same LL sweep inputs, R=8 bf16 "
                       f"2^10..2^19 elements per rank; per size the median of 3 runs, each "
                       f"repeating the call for 0.5 s of timed work on {cores} threads (0.25 s "
                       f"on 1 thread); mean µs per call over the 10 sizes"),
            "per_size_us": [round(v, 2) for v in per_size],
            "value_1_thread": round(statistics.fmean(per_size_1), 2),
            "per_size_us_1_thread": [round(v, 2) for v in per_size_1],
            "host_cpu": _cpu_model(),
            "wall_s": round(time.perf_counter() - t_start, 1),
        }
        log(f"oracle: mean {result['cpu_baseline']['value']:.1f} us per call on {cores} threads, "
            f"{result['cpu_baseline']['value_1_thread']:.1f} us on 1 thread")

    if B.comm.async_error() != B.ar.arResult.arSuccess:
        raise RuntimeError("an LL wait timed out")
    B.comm.close()

    value = statistics.fmean(r["ll_us"] for r in sweep_rows) if sweep_rows else None
    if sweep_rows:
        result["value_median_passes"] = round(
            statistics.fmean(r["ll_us_median"] for r in sweep_rows), 3)
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
            "element_type": "bf16", "accumulate": "f32 in rank order, one RNE rounding",
            "parallelism": "1 GPU, ranks simulated in HBM",
            "tuned": args.tune,
        },
    }
    line.update(result)
    print(json.dumps(line), flush=True)
    _markdown(line)
    return 0


def run_c1(B, inputs):
    """C1: R = 8, 1024 bf16 uniform[-1, 1], one out-of-place call of each
    protocol: its parity, its own time (one event pair around the single
    eager call, launch included) and the eager mean of 10 prepared calls."""
    torch = B.torch
    case = inputs.WORKLOADS["C1"]
    x = inputs.make(**case)
    n = case["count"]
    sv, rv = B.planes(x)
    out = {"nranks": case["nranks"], "elems_per_rank": n, "bytes_per_rank": 2 * n}
    for proto in ("ll", "hb"):
        for t in rv:
            t.view(torch.int16).fill_(-23131)  # 0xA5A5: no call result has these bits everywhere
        torch.cuda.synchronize()
        t0, t1 = B.events()
        t0.record()
        B.launch(sv, rv, n, proto)
        t1.record()
        torch.cuda.synchronize()
        out[f"{proto}_single_call_us"] = round(t0.elapsed_time(t1) * 1000.0, 3)
        out[f"{proto}_launch"] = B.launch_record(proto)
        out[f"{proto}_parity"] = B.parity(x, rv)
        out[f"{proto}_eager_us"] = round(B.eager_us(B.comm.prepare(sv, rv, proto)), 3)
    log(f"C1: LL {out['ll_single_call_us']:.2f} us single call ({out['ll_eager_us']:.2f} eager "
        f"mean), HB {out['hb_single_call_us']:.2f} ({out['hb_eager_us']:.2f}), parity "
        f"{out['ll_parity']}/{out['hb_parity']}")
    del sv, rv
    return out


def run_c5(B, inputs, fp16=True):
    """C5: R = 16 and 32 simulated ranks with integers -4..4, HB two-shot with
    chunk = N/R (the configured layout) beside the interleaved default:
    C5a 2^18 fp16 per rank, graph-replayed (plus LL at the same size; the
    runs' timing passes taken in turn), and C5b 4096 x 7168 fp32 per rank
    (112 MiB), back-to-back launches, out of place, with the cold per-call
    mean and median beside them (last-level cache flushed before each call).
    Each row checks the
    oracle (C5b on 2^20 sampled columns), that all R outputs are equal, and
    that rank 0's equals the exact integer sum."""
    torch = B.torch
    O = B.ar.arOption
    rows = []
    cases = ([("C5a", R, "fp16") for R in (16, 32)] if fp16 else []) + \
        [("C5b", R, "fp32") for R in (16, 32)]
    for name, R, dtype in cases:
        case = inputs.integer_case(R, dtype)
        n = case["count"]
        es = 4 if dtype == "fp32" else 2
        log(f"{name} R={R}: generating {R} x {n} {dtype} inputs")
        x = inputs.make(**case)
        exact = torch.zeros(n, dtype=torch.int32)
        for r in range(R):
            exact += x[r].to(torch.int32)
        exact = exact.to(x.dtype).to(B.dev)
        sv, rv = B.planes(x)
        sample = None if name == "C5a" else torch.randint(
            0, n, (1 << 20,), generator=torch.Generator().manual_seed(99))
        runs = [("hb", 0, "chunk N/R"), ("hb", 1, "interleaved tiles")]
        if name == "C5a":
            runs.append(("ll", 1, "-"))
        checked = {}
        for proto, layout, lname in runs:
            B.comm.set_option(O.arOptHBChunkLayout, layout)
            try:
                for t in rv:
                    t.view(torch.int16 if es == 2 else torch.int32).fill_(-23131)
                B.launch(sv, rv, n, proto)
                torch.cuda.synchronize()
                rec = B.launch_record(proto)
                par = B.parity(x, rv, sample=sample)
                same = all(torch.equal(rv[r], rv[0]) for r in range(1, R))
                checked[lname, proto] = (rec, par, same and torch.equal(rv[0], exact))
            finally:
                B.comm.set_option(O.arOptHBChunkLayout, 1)
        timed = {key: [] for key in checked}
        if name == "C5a":
            # graph-replayed passes taken in turn across the runs, so that no
            # run is timed only in the state the previous one left behind;
            # one untimed round first (the first pass after the parity checks
            # read up to 0.6 us slow)
            for rnd in range(MEDIAN_PASSES + 1):
                for proto, layout, lname in runs:
                    B.comm.set_option(O.arOptHBChunkLayout, layout)
                    try:
                        t = B.graph_passes(sv, rv, n, proto)
                        if rnd > 0:
                            timed[lname, proto] += t
                    finally:
                        B.comm.set_option(O.arOptHBChunkLayout, 1)
        for proto, layout, lname in runs:
            rec, par, ex = checked[lname, proto]
            if name == "C5a":
                # the median: single passes at this size scatter by up to
                # 0.5 us with the state the previous run left
                times = timed[lname, proto]
                us, med, mode = statistics.median(times), times[0], "graph, median"
            else:
                # back to back, and per call with the last-level cache flushed
                # before each one (the prefill's cold protocol; out of place,
                # so nothing is restored)
                B.comm.set_option(O.arOptHBChunkLayout, layout)
                try:
                    for _ in range(B.args.warmup):
                        B.launch(sv, rv, n, proto)
                    us = B.back_to_back_us(sv, rv, n, proto, B.args.steps)
                    cold = B.cold_us(None, None, sv, rv, n, proto, B.args.steps, B.args.warmup)
                finally:
                    B.comm.set_option(O.arOptHBChunkLayout, 1)
                med, mode = None, "back-to-back"
            g = gbps(R, n, es, us)
            row = {"config": name, "R": R, "dtype": dtype, "elems_per_rank": n,
                   "bytes_per_rank": n * es, "proto": proto, "chunk_layout": lname,
                   "mode": mode, "us": round(us, 3),
                   "us_first_pass": None if med is None else round(med, 3), "gbps": g,
                   "pct_of_peak": round(100 * g / HBM_PEAK_GBPS, 2), "parity": par,
                   "exact_integer_sums": ex, "launch": rec}
            if name == "C5b":
                row["us_cold_mean"] = round(statistics.fmean(cold), 2)
                row["us_cold_median"] = round(statistics.median(cold), 2)
            rows.append(row)
            log(f"{name} R={R} {dtype} {proto} ({lname}): {us:.2f} us, {g:.0f} GB/s "
                f"({100 * g / HBM_PEAK_GBPS:.1f}% of 8 TB/s), parity {par}, exact {ex}")
        del x, sv, rv, exact
    return rows


def run_hier(B, inputs, cases):
    """The two-level order in nodes of 8 ranks at the C5 shapes: the flat fused
    kernel, the fused kernel folding the two-level order in registers, the
    staged two-level form (node partials in a workspace, a kernel boundary,
    the fold across nodes), the same form through arAllReduceNoAlloc where its
    partials fit the library's 64 MiB static scratch, and LL in nodes of 8 at
    the fp16 size.  Each is checked against the grouped oracle (the flat one
    against the oracle; fp32 on 2^20 sampled columns) and the exact integer
    sums; graph-replayed at the fp16 size (the median of passes taken in turn
    across the forms), back to back at the fp32 one."""
    torch, ar = B.torch, B.ar
    O = ar.arOption
    rows = []
    ws = None
    for R, dtype in cases:
        case = inputs.integer_case(R, dtype)
        n = case["count"]
        es = 4 if dtype == "fp32" else 2
        x = inputs.make(**case)
        exact = torch.zeros(n, dtype=torch.int32)
        for r in range(R):
            exact += x[r].to(torch.int32)
        exact = exact.to(x.dtype).to(B.dev)
        sv, rv = B.planes(x)
        small = n <= (1 << 18)
        sample = None if small else torch.randint(
            0, n, (1 << 20,), generator=torch.Generator().manual_seed(98))
        want = want_flat = None
        if not B.args.no_parity:
            xs = B.oracle_in(x if sample is None else x[:, sample].contiguous())
            cast = (lambda a: a.view(B.np.uint32)) if dtype == "fp32" else \
                (lambda a: a.view(B.np.uint16))
            want = cast(B.orc.allreduce_grouped(xs, dtype, 8, nthreads=B.threads))
            want_flat = cast(B.orc.allreduce(xs, dtype, nthreads=B.threads))
        del x
        need = (R // 8) * ((n * 4 + 255) // 256 * 256)
        if ws is None or ws.numel() < need:
            ws = None
            ws = torch.empty(need, dtype=torch.uint8, device=B.dev)
        B.comm.set_workspace(ws)
        sp, rp = [t.data_ptr() for t in sv], [t.data_ptr() for t in rv]
        code = ar.dtype_code(sv[0].dtype)

        def no_alloc():
            rc = ar.arAllReduceNoAlloc(sp, rp, n, code, ar.arRedOp.arSum, R, 8,
                                       torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise ar.ArError(rc, "arAllReduceNoAlloc")
        forms = [("hb", "flat", {}, None), ("hb", "fused, nodes of 8", {O.arOptNodeRanks: 8}, None),
                 ("hb", "staged two-level, nodes of 8",
                  {O.arOptNodeRanks: 8, O.arOptHBStaged: 1}, None)]
        if need <= ar.AR_NOALLOC_SCRATCH_BYTES:
            forms.append(("hb", "no-alloc two-level, nodes of 8", {}, no_alloc))
        if small:
            forms.append(("ll", "LL, nodes of 8", {O.arOptNodeRanks: 8}, None))
        checked = {}
        for proto, form, opts, call in forms:
            for o, v in opts.items():
                B.comm.set_option(o, v)
            try:
                for t in rv:
                    t.view(torch.int16 if es == 2 else torch.int32).fill_(-23131)
                (call or (lambda: B.launch(sv, rv, n, proto)))()
                torch.cuda.synchronize()
                rec = B.comm.last_launch() if call is None else None
                par = None
                if want is not None:
                    got = B.np.stack([B.bits(t if sample is None else t[sample.to(t.device)])
                                      for t in rv])
                    par = bool(B.np.array_equal(got, want_flat if form == "flat" else want))
                ex = all(torch.equal(rv[r], rv[0]) for r in range(1, R)) and \
                    torch.equal(rv[0], exact)
                checked[form] = (rec, par, ex)
            finally:
                for o in opts:
                    B.comm.set_option(o, 0)
        timed = {form: [] for _, form, _, _ in forms}
        if small:
            # graph passes in turn across the forms after one untimed round, so
            # that no form is timed only in the state the previous one left
            for rnd in range(MEDIAN_PASSES + 1):
                for proto, form, opts, call in forms:
                    for o, v in opts.items():
                        B.comm.set_option(o, v)
                    try:
                        t = B.graph_passes(sv, rv, n, proto, call=call)
                        if rnd > 0:
                            timed[form] += t
                    finally:
                        for o in opts:
                            B.comm.set_option(o, 0)
        for proto, form, opts, call in forms:
            rec, par, ex = checked[form]
            if small:
                us, first, mode = statistics.median(timed[form]), timed[form][0], "graph"
            else:
                for o, v in opts.items():
                    B.comm.set_option(o, v)
                try:
                    for _ in range(B.args.warmup):
                        (call or (lambda: B.launch(sv, rv, n, proto)))()
                    us = B.back_to_back_us(sv, rv, n, proto, B.args.steps, call=call)
                finally:
                    for o in opts:
                        B.comm.set_option(o, 0)
                first, mode = None, "back-to-back"
            g = gbps(R, n, es, us)
            rows.append({"R": R, "dtype": dtype, "elems_per_rank": n, "proto": proto,
                         "form": form, "mode": mode if not small else "graph, median",
                         "us": round(us, 3), "us_first_pass": None if first is None else round(first, 3),
                         "gbps": g, "pct_of_peak": round(100 * g / HBM_PEAK_GBPS, 2),
                         "parity": par, "exact_integer_sums": ex,
                         "kernels": rec["kernels"] if rec else 2})
            log(f"{dtype} R={R} {form}: {us:.2f} us, {g:.0f} GB/s, parity {par}, exact {ex}")
        B.comm.set_workspace(None)
        del sv, rv, exact
    return rows


def run_configs(B, inputs, sweep_rows, result):
    """Rows for every named workload (see the module docstring)."""
    torch = B.torch
    O = B.ar.arOption
    T = B.threads
    rows = []

    # HBM bytes per launch measured by rocprofv3 for the HBM-bound rows (fused
    # HB at full size), from the committed counter summaries
    counted = {("C4 8192x8192 in place", "hb"): _counter_traffic(),
               ("C5b R=16", "hb"): _counter_traffic(C5B_COUNTERS, "hbm_bytes_per_launch_r16"),
               ("C5b R=32", "hb"): _counter_traffic(C5B_COUNTERS, "hbm_bytes_per_launch_r32")}

    def add(name, R, dtype, n, proto, mode, us, parity, o1=None, oT=None):
        es = 4 if dtype == "fp32" else 2
        g = gbps(R, n, es, us)
        hbm = counted.get((name, proto)) if mode in ("back-to-back", "cold", "graph") else None
        rows.append({"config": name, "R": R, "dtype": dtype, "elems_per_rank": n,
                     "bytes_per_rank": n * es, "proto": proto, "mode": mode,
                     "us_per_call": round(us, 2), "gbps": g,
                     "pct_of_peak": round(100 * g / HBM_PEAK_GBPS, 2),
                     "counter_gbps": round(hbm / (us * 1e3), 1) if hbm else None,
                     "oracle_ms_1": o1, "oracle_ms_T": oT,
                     "oracle_gbps_T": round(2 * R * n * es / (oT * 1e6), 2) if oT else None,
                     "parity": parity})

    # C1: R=8, 1024 bf16, eager calls of each protocol
    case = inputs.WORKLOADS["C1"]
    x = inputs.make(**case)
    sv, rv = B.planes(x)
    o1, oT = B.oracle_ms(x, 1), B.oracle_ms(x, T)
    for proto in ("ll", "hb"):
        B.launch(sv, rv, case["count"], proto)
        torch.cuda.synchronize()
        par = B.parity(x, rv)
        us = B.eager_us(B.comm.prepare(sv, rv, proto))
        add("C1", 8, "bf16", case["count"], proto, "eager", us, par, o1, oT)
    # C2: the sweep, from the rows already measured
    for k, r in zip(SWEEP, sweep_rows):
        x = inputs.make(**inputs.sweep(k))
        o1, oT = B.oracle_ms(x, 1), B.oracle_ms(x, T)
        for proto in ("ll", "hb"):
            add(f"C2 2^{k}", 8, "bf16", r["elems_per_rank"], proto, "graph", r[f"{proto}_us"],
                r[f"{proto}_parity"], o1, oT)
            add(f"C2 2^{k}", 8, "bf16", r["elems_per_rank"], proto, "eager",
                r[f"{proto}_eager_us"], r[f"{proto}_parity"], o1, oT)
        add(f"C2 2^{k}", 8, "bf16", r["elems_per_rank"], "torch", "eager",
            r["torch_eager_us"], None, o1, oT)
    # C3: decode shape
    d = result.get("decode_64x8192")
    if d:
        x = inputs.make(**inputs.WORKLOADS["C3"])
        o1, oT = B.oracle_ms(x, 1), B.oracle_ms(x, T)
        for proto in ("ll", "hb"):
            add("C3 64x8192", 8, "bf16", d["elems_per_rank"], proto, "graph", d[f"{proto}_us"],
                d[f"{proto}_parity"], o1, oT)
    # C4: prefill, from the measured rows
    p = result.get("hb_prefill")
    if p:
        add("C4 8192x8192 in place", 8, "bf16", p["elems_per_rank"], "hb", "back-to-back",
            p["us_per_launch"], p["parity"], p.get("oracle_ms_1"), p.get("oracle_ms_T"))
        add("C4 8192x8192 in place", 8, "bf16", p["elems_per_rank"], "hb", "cold",
            p["us_mean_cold"], p["parity"], p.get("oracle_ms_1"), p.get("oracle_ms_T"))
        add("C4 8192x8192 in place", 8, "bf16", p["elems_per_rank"], "hb", "graph",
            p["us_graph"], p["parity"], p.get("oracle_ms_1"), p.get("oracle_ms_T"))
    # C5a / C5b: the rows measured by run_c5 (both chunk layouts), with the
    # oracle timed on the same inputs
    oracle_times = {}
    for row in result.get("c5", []):
        key = (row["config"], row["R"], row["dtype"])
        if key not in oracle_times:
            x = inputs.make(**inputs.integer_case(row["R"], row["dtype"]))
            reps = 3 if row["config"] == "C5a" else 1
            oracle_times[key] = (B.oracle_ms(x, 1, reps=reps), B.oracle_ms(x, T, reps=reps))
            del x
        o1, oT = oracle_times[key]
        name = f"{row['config']} R={row['R']}"
        if row["proto"] == "hb" and row["chunk_layout"] == "chunk N/R":
            name += " chunk N/R"
        add(name, row["R"], row["dtype"], row["elems_per_rank"], row["proto"], row["mode"],
            row["us"], None if row["parity"] is None else
            (row["parity"] and row["exact_integer_sums"]), o1, oT)

    # NEXT-2: the two-level order (nodes of 8 ranks) at the C5 shapes: the
    # fused kernel folding it in registers, the staged two-level form, the
    # no-alloc entry point where its partials fit, LL at the fp16 size
    for row in run_hier(B, inputs, ((16, "fp16"), (32, "fp16"), (16, "fp32"), (32, "fp32"))):
        name = f"{'C5a' if row['dtype'] == 'fp16' else 'C5b'} R={row['R']} {row['form']}"
        add(name, row["R"], row["dtype"], row["elems_per_rank"], row["proto"], row["mode"],
            row["us"], None if row["parity"] is None else
            (row["parity"] and row["exact_integer_sums"]))

    # HB5 ablation: the staged two-shot (reduce-scatter into the owner, kernel
    # boundary, all-gather from the owner) beside the fused rows above
    B.comm.set_option(O.arOptHBStaged, 1)
    try:
        for name, case, mode in (("C3 64x8192", inputs.WORKLOADS["C3"], "graph"),
                                 ("C4 8192x8192 in place", inputs.WORKLOADS["C4"], "back-to-back"),
                                 ("C5b R=32", inputs.integer_case(32, "fp32"), "back-to-back")):
            x = inputs.make(**case)
            R, n, dtype = case["nranks"], case["count"], case["dtype"]
            in_place = "in place" in name
            sv, rv = B.planes(x)
            if in_place:
                rv = sv
            B.launch(sv, rv, n, "hb")
            torch.cuda.synchronize()
            sample = None if n <= (1 << 20) else torch.randint(
                0, n, (1 << 20,), generator=torch.Generator().manual_seed(97))
            par = B.parity(x, rv, sample=sample)
            us = (B.graph_us(sv, rv, n, "hb") if mode == "graph"
                  else B.back_to_back_us(sv, rv, n, "hb", B.args.steps))
            add(f"{name} staged", R, dtype, n, "hb", f"{mode}, staged", us, par)
            del x, sv, rv
            log(f"staged {name} done")
    finally:
        B.comm.set_option(O.arOptHBStaged, 0)

    log("\n| config | R | dtype | elems/rank | bytes/rank | proto | mode | µs/call | eff. GB/s | "
        "% of 8 TB/s | counter GB/s | oracle ms (1 thr) | oracle ms (T thr) | oracle GB/s (T thr) | "
        "parity |")
    log("|---|---:|---|---:|---:|---|---|---:|---:|---:|---:|---:|---:|---:|:---:|")
    for r in rows:
        cg = "—" if r["counter_gbps"] is None else f"{r['counter_gbps']:.0f}"
        log(f"| {r['config']} | {r['R']} | {r['dtype']} | {r['elems_per_rank']} | "
            f"{r['bytes_per_rank']} | {r['proto']} | {r['mode']} | {r['us_per_call']:.2f} | "
            f"{r['gbps']:.0f} | {r['pct_of_peak']:.1f} | {cg} | {r['oracle_ms_1']} | "
            f"{r['oracle_ms_T']} | {r['oracle_gbps_T']} | {r['parity']} |")
    log(f"(T = {T} host threads)")
    return rows


def run_ceilings(B, args):
    """The HB prefill's memory traffic without its arithmetic: the ceiling
    probe (tests/gpu_probe/hbm_ceiling.hip) reads, writes or copies 8 streams
    of 128 MiB with HB's tile mapping and 128-bit non-temporal accesses, over
    a few launch shapes; HB itself runs on the same planes in place and out of
    place.  GB/s counts the bytes each pattern must move."""
    import ctypes
    from pathlib import Path
    torch, ar = B.torch, B.ar
    lib_path = Path(__file__).resolve().parent / "tests" / "gpu_probe" / "libhbm_ceiling.so"
    if not lib_path.exists():
        raise RuntimeError(f"{lib_path} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(str(lib_path))
    vp = ctypes.c_void_p
    lib.hbm_ceiling_run.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), vp, ctypes.c_uint64,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.hbm_ceiling_run.restype = ctypes.c_int
    lib.hbm_ceiling_run_n.argtypes = [ctypes.POINTER(vp), ctypes.POINTER(vp), vp, ctypes.c_uint64,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp]
    lib.hbm_ceiling_run_n.restype = ctypes.c_int
    B.ceiling_lib = lib
    R, n = 8, 8192 * 8192                      # bf16 elements per rank: 128 MiB
    nvec = n * 2 // 16
    src = torch.empty((R, n), dtype=torch.bfloat16, device=B.dev).normal_()
    dst = torch.empty_like(src)
    shapes = [(256, 256), (512, 256), (1024, 256), (2048, 256), (256, 512), (512, 128)]
    sink = torch.empty(max(g * t for g, t in shapes) * 4, dtype=torch.int32, device=B.dev)
    sp = (vp * 8)(*[src[j].data_ptr() for j in range(R)])
    dp = (vp * 8)(*[dst[j].data_ptr() for j in range(R)])
    gib = 1 << 30
    patterns = [("read", 0, sp, gib), ("write", 1, dp, gib),
                ("write, ordinary stores", 3, dp, gib), ("copy in place", 2, sp, 2 * gib),
                ("copy out of place", 2, dp, 2 * gib)]

    def timed(fn, reps):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        t0, t1 = B.events()
        t0.record()
        for _ in range(reps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1000.0 / reps

    out = {}
    for name, mode, d, nbytes in patterns:
        by_shape = {}
        for g, t in shapes:
            def fn(mode=mode, d=d, g=g, t=t):
                rc = lib.hbm_ceiling_run(sp, d, sink.data_ptr(), nvec, mode, g, t,
                                         torch.cuda.current_stream().cuda_stream)
                if rc != 0:
                    raise RuntimeError("hbm_ceiling_run refused its launch")
            us = timed(fn, args.steps)
            by_shape[f"{g}x{t}"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        best = max(by_shape, key=by_shape.get)
        out[name] = {"best_gbps": by_shape[best], "best_shape": best, "gbps_by_shape": by_shape}
        log(f"ceiling {name}: best {by_shape[best]:.0f} GB/s at {best}")
    opt = ar.arOption.arOptHBBlocks
    cus = torch.cuda.get_device_properties(B.dev).multi_processor_count
    for name, d, blocks in (("hb in place", sp, 0), ("hb out of place", dp, 0),
                            ("hb out of place, 2 workgroups per CU", dp, 2 * cus)):
        srcs = [src[j].data_ptr() for j in range(R)]
        dsts = [src[j].data_ptr() if d is sp else dst[j].data_ptr() for j in range(R)]

        def fn(srcs=srcs, dsts=dsts):
            rc = ar.arAllReduce(srcs, dsts, n, ar.arDataType.arBfloat16, ar.arRedOp.arSum, R,
                                ar.arProtocol.arProtoHB, B.comm.handle,
                                torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise ar.ArError(rc, "arAllReduce")
        B.comm.set_option(opt, blocks)
        try:
            us = timed(fn, args.steps)
        finally:
            B.comm.set_option(opt, 0)
        out[name] = {"us": round(us, 2), "gbps": round(2 * gib / (us * 1e-6) / 1e9, 1),
                     "shape": f"{blocks} workgroups x default threads" if blocks else "default"}
        log(f"{name}: {us:.1f} us, {out[name]['gbps']:.0f} GB/s")
    del src, dst, sink
    return out


def run_c5b_ceilings(B, args):
    """The C5b shape's memory ceilings: R = 16 and 32 streams of 112 MiB
    (fp32 4096 x 7168 per rank) read only, written only (non-temporal or
    ordinary stores), and copied out of place (2R streams, HB's access shape
    at that R), with HB's tile mapping, best of a few launch shapes; HB itself
    out of place on the same planes at its default shape.  GB/s counts the
    bytes each pattern must move."""
    import ctypes
    torch, ar = B.torch, B.ar
    lib = B.ceiling_lib
    n = 4096 * 7168
    nvec = n * 4 // 16
    shapes = [(256, 256), (512, 256), (1024, 256), (256, 128), (512, 128), (256, 512)]
    out = {}
    for R in (16, 32):
        src = torch.empty((R, n), dtype=torch.float32, device=B.dev).normal_()
        dst = torch.empty_like(src)
        sink = torch.empty(max(g * t for g, t in shapes) * 4, dtype=torch.int32, device=B.dev)
        sp = (ctypes.c_void_p * R)(*[src[j].data_ptr() for j in range(R)])
        dp = (ctypes.c_void_p * R)(*[dst[j].data_ptr() for j in range(R)])
        one = R * n * 4
        res = {}
        for name, mode, d, nbytes in (("read", 0, sp, one), ("write", 1, dp, one),
                                      ("write, ordinary stores", 3, dp, one),
                                      ("copy out of place", 2, dp, 2 * one)):
            best = 0.0
            # the probe holds R vectors per lane: at most 512 threads at 16
            # streams and 256 at 32, as the HB kernel
            for g, t in [(g, t) for g, t in shapes if t <= (256 if R >= 32 else 512)]:
                def fn(mode=mode, d=d, g=g, t=t):
                    rc = lib.hbm_ceiling_run_n(sp, d, sink.data_ptr(), nvec, mode, g, t, R,
                                               torch.cuda.current_stream().cuda_stream)
                    if rc != 0:
                        raise RuntimeError("hbm_ceiling_run_n refused its launch")
                us = _timed(B, fn, args.steps)
                best = max(best, nbytes / (us * 1e-6) / 1e9)
            res[name] = round(best, 1)
        srcs = [src[j].data_ptr() for j in range(R)]
        dsts = [dst[j].data_ptr() for j in range(R)]

        def hb():
            rc = ar.arAllReduce(srcs, dsts, n, ar.arDataType.arFloat32, ar.arRedOp.arSum, R,
                                ar.arProtocol.arProtoHB, B.comm.handle,
                                torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise ar.ArError(rc, "arAllReduce")
        hb_gbps = 2 * one / (_timed(B, hb, args.steps) * 1e-6) / 1e9
        wr = max(res["write"], res["write, ordinary stores"])
        bound = 2.0 / (1.0 / res["read"] + 1.0 / wr)
        out[f"r{R}"] = {"read_gbps": res["read"], "write_gbps": wr,
                        "copy_out_of_place_gbps": res["copy out of place"],
                        "read_write_bound_gbps": round(bound, 1),
                        "hb_out_of_place_gbps": round(hb_gbps, 1),
                        "hb_frac_of_peak": round(hb_gbps / HBM_PEAK_GBPS, 4),
                        "hb_frac_of_copy": round(hb_gbps / res["copy out of place"], 4),
                        "hb_frac_of_read_write_bound": round(hb_gbps / bound, 4)}
        log(f"C5b ceilings R={R}: read {res['read']:.0f}, write {wr:.0f}, copy out of place "
            f"{res['copy out of place']:.0f}, read/write bound {bound:.0f}; HB {hb_gbps:.0f} GB/s "
            f"({100 * hb_gbps / res['copy out of place']:.1f}% of the copy)")
        del src, dst, sink
    return out


def _timed(B, fn, reps):
    for _ in range(2):
        fn()
    B.torch.cuda.synchronize()
    t0, t1 = B.events()
    t0.record()
    for _ in range(reps):
        fn()
    t1.record()
    B.torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1000.0 / reps


def _sources_digest() -> str:
    """sha256 over what the HB kernel is compiled from (its source file, the
    device header it includes, the compiler flags without include paths), to
    tie counter readings to that kernel."""
    import hashlib
    from pathlib import Path
    from all_reduce_amd import build
    csrc = Path(__file__).resolve().parent / "all_reduce_amd" / "csrc"
    h = hashlib.sha256()
    for name in ("hb_twoshot.hip", "ar_device.hpp"):
        h.update((csrc / name).read_bytes())
    h.update(" ".join(f for f in build.HIP_FLAGS if not f.startswith("-I")).encode())
    return h.hexdigest()


def _counter_traffic(summary="hb_twoshot_bf16_r8_128MiB_counters.txt",
                     key="hbm_bytes_per_launch"):
    """HBM bytes per launch of an HB kernel from a committed counter summary
    under profiles/, or None when that summary is missing or was taken from
    other kernel sources."""
    from pathlib import Path
    path = Path(__file__).resolve().parent / "profiles" / summary
    if not path.exists():
        return None
    fields = {}
    for line in path.read_text().splitlines():
        if ":" in line and not line.startswith(("#", " ")):
            k, _, val = line.partition(":")
            fields[k.strip()] = val.strip()
    if fields.get("source_sha256") != _sources_digest():
        return None
    try:
        return int(fields[key])
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
        log("\n| bytes/rank | LL graph µs (median of 5) | HB graph µs (median of 5) | LL eager µs | "
            "HB eager µs | torch eager µs | LL GB/s | HB GB/s | LL grid x threads | "
            "parity LL/HB |")
        log("|---:|---:|---:|---:|---:|---:|---:|---:|---|:---:|")
        for r in rows:
            ll = r["ll_launch"]
            log(f"| {r['bytes_per_rank']} | {r['ll_us']:.2f} ({r['ll_us_median']:.2f}) | "
                f"{r['hb_us']:.2f} ({r['hb_us_median']:.2f}) | "
                f"{r['ll_eager_us']:.2f} | {r['hb_eager_us']:.2f} | {r['torch_eager_us']:.2f} | "
                f"{r['ll_gbps']:.0f} | {r['hb_gbps']:.0f} | {ll['grid']} x {ll['threads']} | "
                f"{r['ll_parity']}/{r['hb_parity']} |")
    c5 = line.get("c5", [])
    if c5:
        log("\n| config | R | dtype | proto | chunk layout | mode | µs | GB/s | % of 8 TB/s | "
            "parity | exact sums |")
        log("|---|---:|---|---|---|---|---:|---:|---:|:---:|:---:|")
        for r in c5:
            log(f"| {r['config']} | {r['R']} | {r['dtype']} | {r['proto']} | {r['chunk_layout']} | "
                f"{r['mode']} | {r['us']:.2f} | {r['gbps']:.0f} | {r['pct_of_peak']:.1f} | "
                f"{r['parity']} | {r['exact_integer_sums']} |")


if __name__ == "__main__":
    sys.exit(main())
