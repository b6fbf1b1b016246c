#!/usr/bin/env python3
"""Benchmark of the MoE expert operation of a verification pass on one MI355X.

Metric: achieved HBM GB/s of the expert operation and its fraction of the
8 TB/s peak, against pass size n = 1..8, for the per-slot and the deduplicating
kernel; the bandwidth ratio r(n) = beta_dedup / beta_slot, the byte share
u(n) = E_dedup / E_slot, the saving S(n) = t_slot - t_dedup and the crossover n
(Lan, arXiv:2610.34440, Sections 1-3).

Headline workload: the Qwen3-30B-A3B-shaped layer (N = 128 experts, top-8,
d_model = 2048, d_ff = 768, bf16) 48 times back to back per pass, each layer with
its own weights, its own Zipf(s = 1.1) routing trace and its own activations; a
pass of n tokens copies the ids of the same n consecutive token positions from
every layer's trace.  One step = for each n = 1..8, one such window run by both
kernels.  Timing protocol (Lan Section 2, Table 1 and its caption; App. E): every
timed pass runs after a read-only 1 GiB flush (the 256 MB Infinity Cache would
otherwise hold a small pass; a flush that also writes leaves dirty lines whose
write-back competes with the timed reads), between two HIP events on the launch
stream; each window is timed `--reps` times and its median kept; per n the
median and quartiles over windows are reported, and beta, r and u come from bytes
and median times summed over windows (and layers).  Bytes are requested expert
bytes: n m w per-slot, X(n) w deduplicating (w = 3 d d_ff 2 B).

The other workloads (same protocol, compact r(n), u(n) and crossover in the
headline line): the DeepSeek-V2-Lite-shaped layer (uniform and correlated
routing), the Mixtral-8x7B-shaped layer (uniform and repeat-0.6 routing) and the
32-node draft tree on a Qwen3-shaped layer.

The last stdout line is one compact JSON object (a few KB); the full record, with
the per-window data and the further sections (HIP graph replay, chosen-id fits and
bounds, dispatch, router, shared experts, subtree selection), is written to
`--out`.  Progress goes to stderr.
"""
import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = "expert-op achieved HBM GB/s & % peak vs pass size n=1..8; dedup r(n), crossover n"
SCRUB_BYTES = 1 << 30
COPY_BYTES = 1 << 28
A_GRID = [i / 21.0 for i in range(22)]  # acceptance values of the best-draft-length staircase
HEADLINE = "qwen3x48"
WORKLOADS = ("qwen3x48", "tree", "dsv2lite", "mixtral")
PMC_TREES = 8          # seeded trees in a counter run
ORACLE_LAYERS = 2      # headline layers whose plain weights stay resident for the oracle's sample
HOST_WINDOWS = 6       # windows per n offered to the oracle's timed sample
MAX_POOL = 16          # host threads for the oracle: one GPU's share of the host's cores
TRACE_TOKENS = 4096    # tokens per routing trace
FULL_RECORD = os.path.join("gpurun_out", "bench_full.json")
WEIGHT_LAYOUT = "tiled"  # moe_pack_tiled: 16-row x 64-byte blocks, waves on interleaved K steps


def progress(msg):
    """A stage of the run has finished (stderr; stdout carries only the JSON line)."""
    print("[bench] %s" % msg, file=sys.stderr, flush=True)


class HipEvents:
    """Raw hipEvent_t handles (torch's Event only sees torch's own streams)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.pool = []

    def make(self, k):
        out = []
        for _ in range(k):
            e = ctypes.c_void_p()
            assert self.h.hipEventCreate(ctypes.byref(e)) == 0
            self.pool.append(e)
            out.append(e.value)
        return out

    def record(self, ev, stream):
        assert self.h.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0

    def ms(self, a, b):
        self.h.hipEventSynchronize(ctypes.c_void_p(b))
        f = ctypes.c_float()
        assert self.h.hipEventElapsedTime(ctypes.byref(f), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return float(f.value)


class Clock:
    """Times launches on the bench stream: the read-only flush, an event, the
    launches, an event; `median_us` takes the median over repetitions."""

    def __init__(self, torch, stream, scrub=True):
        self.torch = torch
        self.ev = HipEvents()
        self.e = self.ev.make(2)
        self.stream = stream
        self.sh = stream.cuda_stream
        self.scrub = scrub
        self.buf = torch.ones(SCRUB_BYTES // 4, dtype=torch.float32, device="cuda")
        self.out = torch.empty((), dtype=torch.float32, device="cuda")

    def flush(self):
        self.torch.sum(self.buf, dim=0, out=self.out)  # reads 1 GiB, writes 4 bytes

    def once_us(self, fn):
        if self.scrub:
            self.flush()
        self.ev.record(self.e[0], self.sh)
        fn()
        self.ev.record(self.e[1], self.sh)
        return self.ev.ms(self.e[0], self.e[1]) * 1e3

    def median_us(self, fn, reps):
        return float(np.median([self.once_us(fn) for _ in range(reps)]))


def load_layout(layer):
    """The layer in the layout the timed runs use: all three matrices tiled when
    d and d_ff are whole 64-byte steps, else W_down packed."""
    step = 32 if layer.dtype.itemsize == 2 else 16
    if layer.d % step == 0 and layer.d_ff % step == 0:
        return layer.tiled_copy()
    return layer.packed_copy()


def source_hash():
    h = hashlib.sha256()
    for p in ("expert_ffn_amd/csrc/expert_kernel.h", "expert_ffn_amd/csrc/expert_launch.hip",
              "expert_ffn_amd/csrc/moe_expert.hip"):
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ aggregation

def per_n_rows(recs, nvals):
    """Per n: bytes and (median) times summed over the timed windows give beta per
    kernel, r = beta_dedup / beta_slot and u = E_dedup / E_slot (Lan Section 2, Table 1
    caption); the median and quartiles are over the windows' times."""
    rows = []
    for n in nvals:
        R = [r for r in recs if r["n"] == n]
        bs, bd = sum(r["bytes_slot"] for r in R), sum(r["bytes_dedup"] for r in R)
        ts, td = sum(r["t_slot_ms"] for r in R) / 1e3, sum(r["t_dedup_ms"] for r in R) / 1e3
        gs, gd = bs / ts / 1e9, bd / td / 1e9
        rows.append(dict(n=n, windows=len(R), gbps_slot=round(gs, 1), gbps_dedup=round(gd, 1),
                         frac_slot=round(gs / PEAK_HBM_GBPS, 4), frac_dedup=round(gd / PEAK_HBM_GBPS, 4),
                         r=round(gd / gs, 4), u=round(bd / bs, 4),
                         us_slot=round(ts / len(R) * 1e6, 2), us_dedup=round(td / len(R) * 1e6, 2),
                         bytes_slot=bs / len(R), bytes_dedup=bd / len(R),
                         mean_U=round(sum(r["U"] for r in R) / len(R), 2),
                         **{"%s_us_%s" % (stat, k): v for k in ("slot", "dedup")
                            for stat, v in zip(("median", "q1", "q3"),
                                               np.round(np.percentile([r["t_%s_ms" % k] * 1e3 for r in R],
                                                                      [50, 25, 75]), 2).tolist())}))
    return rows


def crossover_of(rows):
    """Smallest n >= 2 from which the deduplicating kernel stays faster, i.e. the
    saving t_slot - t_dedup is positive at that n and every larger one (0: none)."""
    cross = 0
    for r in reversed(rows):
        if r["n"] < 2 or r["us_slot"] - r["us_dedup"] <= 0:
            break
        cross = r["n"]
    return cross


def strip_bytes(rows):
    return [{k: v for k, v in r.items() if not k.startswith("bytes_")} for r in rows]


def compact(rows, keys=("r", "u")):
    """Arrays over n of the named per-n fields."""
    return {k: [r[k] for r in rows] for k in keys}


def kernel_totals(recs, kind, launches_per_pass=1):
    """Summed requested bytes and summed (median) times of one kernel over the timed
    passes, and the average per launch."""
    b = sum(r["bytes_" + kind] for r in recs)
    s = sum(r["t_%s_ms" % kind] for r in recs) / 1e3
    nl = len(recs) * launches_per_pass
    return dict(bytes=b, seconds=s, launches=nl, gbps=b / s / 1e9, avg_launch_us=s / nl * 1e6,
                bytes_per_launch=b / nl)


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline(passes, budget_s, max_threads=MAX_POOL):
    """The oracle, as it stands, on host cores over a bounded sample of passes.

    `passes` = [(weights (W_gate, W_up, W_down), x, ids, w, dtype, requested bytes)].
    First on one thread until `budget_s` has passed, then the same passes spread
    over a thread pool of the process's cores (at most `max_threads`, one pass per
    thread at a time; the C call releases the GIL), whose results must be bitwise
    equal to the single-thread ones.  `value` is the pool's rate, `cores` its
    thread count."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    t0 = time.perf_counter()
    nbytes = 0
    ys = []
    for (W, x, ids, w, dt, nb) in passes:
        ys.append(oracle.moe_ffn(*W, x, ids, w, dt))
        nbytes += nb
        if time.perf_counter() - t0 > budget_s:
            break
    dt1 = time.perf_counter() - t0
    done = len(ys)
    cores = max(1, min(len(os.sched_getaffinity(0)), max_threads))
    t1 = time.perf_counter()
    with ThreadPoolExecutor(cores) as pool:
        ya = list(pool.map(lambda p: oracle.moe_ffn(*p[0], p[1], p[2], p[3], p[4]), passes[:done]))
    dt_all = time.perf_counter() - t1
    same = all(np.array_equal(a, b) for a, b in zip(ys, ya))
    if not same:
        raise RuntimeError("oracle results differ between one thread and %d threads" % cores)
    return {"value": round(nbytes / dt_all / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": "%d passes, requested per-slot weight bytes / wall time of the C oracle (double "
                      "accumulate), one pass per thread on %d threads" % (done, cores),
            "seconds": round(dt_all, 2), "bitwise_equal_to_one_thread": same,
            "one_thread": {"value": round(nbytes / dt1 / 1e9, 4), "seconds": round(dt1, 2)},
            "nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "cpu": _cpu_model()}


# ------------------------------------------------------------------ counters and profiles

PMC_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc {counter} -d $R/gpurun_out/pmc_{tag} "
           "-o run --output-format csv -- python3 $R/bench.py --pmc-pass > $R/gpurun_out/pmc_{tag}.log   "
           "(R = repository root)")
PROF_CMD = ("rocprofv3 --kernel-trace --stats -d gpurun_out/prof_qwen3x48 -o run --output-format csv -- "
            "python3 bench.py --workloads qwen3x48 --no-extras --steps 4 --warmup 1 --reps 2 "
            "--out gpurun_out/prof_full.json > gpurun_out/prof_bench_qwen3x48.json")


def _counter_rows(path):
    import csv
    return list(csv.DictReader(open(path)))


def traffic_from(fetch_csv, write_csv, kernel="slot"):
    """HBM bytes per launch of one kernel ("slot" or "dedup", told apart by the
    kernel's mode template argument) from two counter runs of `--pmc-pass`.

    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by what the same
    counter reads for the run's device copy of COPY_BYTES (read and written once),
    then averaged over the kernel's launches, like the achieved figure."""
    tag = "k_expert<true, %d," % (0 if kernel == "slot" else 1)
    out = {}
    for name, path in (("fetch", fetch_csv), ("write", write_csv)):
        rows = _counter_rows(path)
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        cal = max(copy)  # the 256 MiB device copy is the largest copy of the run
        factor = COPY_BYTES / (cal * 1024.0)
        ke = [float(r["Counter_Value"]) for r in rows if tag in r["Kernel_Name"]]
        out[name] = dict(copy_kib=cal, factor=factor, kernel_kib=ke, bytes=[v * 1024.0 * factor for v in ke])
    n = len(out["fetch"]["bytes"])
    assert n == len(out["write"]["bytes"]) and n > 0
    per_launch = (sum(out["fetch"]["bytes"]) + sum(out["write"]["bytes"])) / n
    return out, per_launch


def _workloads_of(order):
    seen = []
    for p in order:
        if p["workload"] not in seen:
            seen.append(p["workload"])
    return seen


def write_traffic_summary(fetch_csv, write_csv, pass_json, out_dir=None):
    """profiles/traffic_k_expert.md from the two counter runs of `--pmc-pass`: per
    workload, kernel and n the launches' fetched and written bytes against the
    algorithmic bytes (n m w per-slot, U w deduplicating), and per workload and kernel
    the counted bytes per launch (the headline's are the roofline's `traffic`)."""
    info = [json.loads(l) for l in open(pass_json) if l.startswith('{"pmc_pass"')][-1]
    lines = ["# HBM traffic of k_expert per launch: every workload of the bench, both kernels",
             "", "Commands (one GPU; FETCH_SIZE and WRITE_SIZE in separate runs), then on any host:", "", "```",
             PMC_CMD.format(counter="FETCH_SIZE", tag="fetch"), PMC_CMD.format(counter="WRITE_SIZE", tag="write"),
             "python3 bench.py --traffic-from gpurun_out/pmc_fetch/run_counter_collection.csv "
             "gpurun_out/pmc_write/run_counter_collection.csv gpurun_out/pmc_fetch.log", "```", "",
             "One window per (routing, n) (the headline: one window per n, 48 layers; the tree: %d seeded trees), each "
             "launch after the 1 GiB read flush. Algorithmic bytes: n m w per-slot, U w deduplicating (U distinct "
             "experts of the layer)." % PMC_TREES, ""]
    rec = {"source_hash": info["source_hash"], "per_launch": {}}
    data = {}
    for kernel in ("slot", "dedup"):
        order = [p for p in info["pmc_pass"] if p["kernel"] == kernel]
        out, _ = traffic_from(fetch_csv, write_csv, kernel=kernel)
        assert len(order) == len(out["fetch"]["bytes"]), (kernel, len(order), len(out["fetch"]["bytes"]))
        data[kernel] = (order, out)
    out = data["slot"][1]
    lines += ["Calibration: the run's device copy of %d bytes reads %.1f KiB FETCH_SIZE and %.1f KiB WRITE_SIZE, so "
              "the counters are scaled by %.4f and %.4f." % (COPY_BYTES, out["fetch"]["copy_kib"],
                                                             out["write"]["copy_kib"], out["fetch"]["factor"],
                                                             out["write"]["factor"]), ""]
    for wl in _workloads_of(info["pmc_pass"]):
        lines += ["## %s" % wl, "",
                  "| n | launches | mean U | per-slot alg. MB | fetched MB | fetched / alg. | written MB | "
                  "dedup alg. MB | fetched MB | fetched / alg. | written MB |",
                  "|---|---|---|---|---|---|---|---|---|---|---|"]
        rec["per_launch"][wl] = {}
        cells = {}
        for kernel in ("slot", "dedup"):
            order, out = data[kernel]
            idx = [i for i, p in enumerate(order) if p["workload"] == wl]
            if not idx:
                continue
            for n in sorted(set(order[i]["n"] for i in idx)):
                ii = [i for i in idx if order[i]["n"] == n]
                alg = sum(order[i]["bytes"] for i in ii) / len(ii)
                fb = sum(out["fetch"]["bytes"][i] for i in ii) / len(ii)
                wb = sum(out["write"]["bytes"][i] for i in ii) / len(ii)
                cells.setdefault(n, {"launches": len(ii), "U": sum(order[i]["U"] for i in ii) / len(ii)})
                cells[n][kernel] = (alg, fb, wb)
            cnt = sum(out["fetch"]["bytes"][i] + out["write"]["bytes"][i] for i in idx) / len(idx)
            rec["per_launch"][wl][kernel] = {"bytes": round(cnt, 1), "launches": len(idx),
                                             "algorithmic": round(sum(order[i]["bytes"] for i in idx) / len(idx), 1),
                                             "fetched_over_algorithmic": round(
                                                 sum(out["fetch"]["bytes"][i] for i in idx) /
                                                 sum(order[i]["bytes"] for i in idx), 4)}
        for n in sorted(cells):
            c = cells[n]
            row = ["%d" % n, "%d" % c["launches"], "%.2f" % c["U"]]
            for kernel in ("slot", "dedup"):
                if kernel in c:
                    a, f, w = c[kernel]
                    row += ["%.1f" % (a / 1e6), "%.1f" % (f / 1e6), "%.3f" % (f / a), "%.2f" % (w / 1e6)]
                else:
                    row += ["-"] * 4
            lines.append("| " + " | ".join(row) + " |")
        lines += [""] + ["Per launch, %s kernel: %.2f MB counted (fetched + written) for %.2f MB algorithmic." % (
            kernel, v["bytes"] / 1e6, v["algorithmic"] / 1e6) for kernel, v in rec["per_launch"][wl].items()] + [""]
    rec["fetch_factor"] = round(out["fetch"]["factor"], 4)
    rec["write_factor"] = round(out["write"]["factor"], 4)
    lines += ["traffic-json: " + json.dumps(rec)]
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), "traffic_k_expert.md")
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)
    return path


def read_traffic(kernel="slot", workload=HEADLINE):
    """Counted HBM bytes per launch from the committed counter summary, if it was
    taken on this kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic_k_expert.md")
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic-json: "):
            rec = json.loads(line[len("traffic-json: "):])
            if rec.get("source_hash") == source_hash():
                return rec["per_launch"].get(workload, {}).get(kernel, {}).get("bytes")
    return None


SQ_A = ("SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_BUSY_CYCLES "
        "SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_INSTS_MFMA GRBM_GUI_ACTIVE")
SQ_B = ("SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_LDS SQ_INSTS_VALU SQ_INST_CYCLES_VMEM_RD SQ_INSTS_SALU "
        "SQ_CYCLES GRBM_GUI_ACTIVE")
SQ_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc {counters} -d $R/gpurun_out/pmc_{tag} "
          "-o run --output-format csv -- python3 $R/bench.py --pmc-pass > $R/gpurun_out/pmc_{tag}.log")


def _per_dispatch(path, tag):
    """{dispatch id: {counter: value, "_us": duration}} of the dispatches whose kernel
    name contains `tag`, in dispatch order."""
    import collections
    d = collections.OrderedDict()
    for r in _counter_rows(path):
        if tag not in r["Kernel_Name"]:
            continue
        key = int(r.get("Dispatch_Id") or r.get("Correlation_Id"))
        e = d.setdefault(key, {})
        e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if "Start_Timestamp" in r and r["Start_Timestamp"]:
            e["_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000
    return list(d.values())


def write_sq_summary(csv_a, csv_b, pass_json, out_dir=None):
    """profiles/k_expert_sq_counters.md: instruction-level counters of the `--pmc-pass`
    launches, averaged per (workload, kernel), with the share of wave cycles spent
    waiting, the MFMA work against the dense bf16 peak and the VALU activity."""
    info = [json.loads(l) for l in open(pass_json) if l.startswith('{"pmc_pass"')][-1]
    lines = ["# k_expert instruction-level counters: every workload of the bench, both kernels", "",
             "Two counter runs over the launches of the traffic summary, then on any host (R = repository root):", "",
             "```", SQ_CMD.format(counters=SQ_A, tag="sqa"), SQ_CMD.format(counters=SQ_B, tag="sqb"),
             "python3 bench.py --sq-summary gpurun_out/pmc_sqa/run_counter_collection.csv "
             "gpurun_out/pmc_sqb/run_counter_collection.csv gpurun_out/pmc_sqa.log", "```", "",
             "Averages per launch. wait share = SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES (the share of wave cycles spent "
             "waiting on operands); MFMA share = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops / duration / 2.5 PFLOP/s "
             "(dense bf16 peak); VALU per wave = SQ_INSTS_VALU / SQ_WAVES; LDS conflict share = "
             "SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS. Source hash %s." % info["source_hash"], "",
             "| workload | kernel | launches | µs | waves | wait share | MFMA share | VALU per wave | LDS conflict share |",
             "|---|---|---|---|---|---|---|---|---|"]
    out = {}
    for kernel, mode in (("slot", 0), ("dedup", 1)):
        order = [p for p in info["pmc_pass"] if p["kernel"] == kernel]
        A = _per_dispatch(csv_a, "k_expert<true, %d," % mode)
        B = _per_dispatch(csv_b, "k_expert<true, %d," % mode)
        assert len(A) == len(B) == len(order), (kernel, len(A), len(B), len(order))
        for wl in _workloads_of(order):
            idx = [i for i, p in enumerate(order) if p["workload"] == wl]

            def avg(X, c):
                return sum(X[i].get(c, 0.0) for i in idx) / len(idx)
            us = avg(A, "_us")
            wait = avg(A, "SQ_WAIT_INST_ANY") / max(avg(A, "SQ_WAVE_CYCLES"), 1.0)
            mfma = avg(A, "SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512 / max(us * 1e-6, 1e-12) / 2.5e15
            valu = avg(B, "SQ_INSTS_VALU") / max(avg(A, "SQ_WAVES"), 1.0)
            lds = avg(B, "SQ_LDS_BANK_CONFLICT") / max(avg(B, "SQ_ACTIVE_INST_LDS"), 1.0)
            out.setdefault(wl, {})[kernel] = dict(us=us, wait=wait, mfma=mfma)
            lines.append("| %s | %s | %d | %.1f | %.0f | %.3f | %.4f | %.0f | %.4f |" % (
                wl, kernel, len(idx), us, avg(A, "SQ_WAVES"), wait, mfma, valu, lds))
    lines += ["", "sq-json: " + json.dumps({"source_hash": info["source_hash"], "per_launch": out})]
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), "k_expert_sq_counters.md")
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)
    return path


def launch_gaps(disp):
    """Launch gaps of the expert kernels from kernel-trace dispatches (start ns, end ns,
    name): for every pair of dispatches adjacent in start order that are launches of
    the same k_expert kernel (a pass's layers back to back), the idle time from the
    first's end to the second's start.  Returns {kernel: (gaps, gap ns, busy ns)},
    busy = the durations of the dispatches that follow a gap."""
    import re
    out = {}
    disp = sorted(disp)
    for (s0, e0, k0), (s1, e1, k1) in zip(disp, disp[1:]):
        m0, m1 = re.search(r"k_expert<[^>]*>", k0), re.search(r"k_expert<[^>]*>", k1)
        if not m0 or not m1 or m0.group(0) != m1.group(0):
            continue
        n, g, busy = out.get(m0.group(0), (0, 0, 0))
        out[m0.group(0)] = (n + 1, g + max(0, s1 - e0), busy + (e1 - s1))
    return out


def write_profile_summary(prof_dir, bench_json):
    """profiles/k_expert_qwen3x48.md: short summary of a `rocprofv3 --kernel-trace
    --stats` run of this bench on the headline workload, with the bench line's event
    figures of the same run beside the trace's."""
    import collections
    import re
    trace = [f for f in os.listdir(prof_dir) if f.endswith("kernel_trace.csv")][0]
    stats = [f for f in os.listdir(prof_dir) if f.endswith("kernel_stats.csv")][0]
    d = collections.defaultdict(list)
    disp = []  # (start, end, kernel) of every dispatch, for the launch gaps
    for r in _counter_rows(os.path.join(prof_dir, trace)):
        disp.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]))
        m = re.search(r"(k_\w+)(<[^>]*>)?", r["Kernel_Name"])
        if not m:
            continue
        key = (m.group(1) + (m.group(2) or ""), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))
        d[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000)
    gaps = launch_gaps(disp)
    b = [json.loads(l) for l in open(bench_json) if l.startswith('{"metric"')][-1]
    lines = ["# k_expert (per-slot and deduplicating), qwen3-shaped layer x48 per pass, zipf routing, n = 1..8",
             "", "Command (from the repository root, one MI355X):", "", "```", PROF_CMD, "```", "",
             "## rocprofv3 --stats (all kernels of the run)", "", "| kernel | calls | avg us | % of GPU time |",
             "|---|---|---|---|"]
    for r in _counter_rows(os.path.join(prof_dir, stats)):
        m = re.search(r"(k_\w+<[^>]*>|k_\w+)", r["Name"])
        short = m.group(1) if m else r["Name"].split("(")[0][:60]
        lines.append("| `%s` | %s | %.2f | %.2f |" % (short, r["Calls"], float(r["AverageNs"]) / 1000,
                                                      float(r["Percentage"])))
    lines += ["", "## Per-launch durations of the expert kernels by grid size (kernel trace)", "",
              "| kernel | workgroups | launches | avg us | min us | max us |", "|---|---|---|---|---|---|"]
    for k in sorted(d):
        v = d[k]
        lines.append("| `%s` | %d | %d | %.2f | %.2f | %.2f |" % (k[0], k[1], len(v), sum(v) / len(v), min(v), max(v)))
    rf = b["roofline"]
    lines += ["", "## Bench line of the same run (HIP events on the launch stream)", ""]
    for kernel, mode in (("slot", 0), ("dedup", 1)):
        tr = [v for k, vs in d.items() if k[0].startswith("k_expert<true, %d" % mode) for v in vs]
        kk = rf["kernels"][kernel]
        lines.append("- %s kernel: avg %.2f us per launch by events (median of reps, 48 launches per pass, launch "
                     "gaps included), %.2f us by the kernel trace (%d launches, every rep and warm-up window); "
                     "%.0f algorithmic bytes per launch; achieved %.1f GB/s = %.3f of 8 TB/s" % (
                         kernel, kk["avg_launch_us"], sum(tr) / max(len(tr), 1), len(tr),
                         kk["bytes_per_launch"], kk["achieved"], kk["frac"]))
    lines += ["- value: %.1f GB/s (all passes, both kernels); roofline kernel: %s" % (b["value"], rf["kernel"]),
              "- source hash %s" % b.get("source_hash"), "",
              "## Launch gaps (kernel trace)", "",
              "Launches of one kernel back to back in a pass (one launch per layer, 48 per pass): the idle time",
              "between one launch's end and the next one's start, over the busy time plus those gaps.", "",
              "| kernel | gaps | mean gap us | launch-gap share |", "|---|---|---|---|"]
    for name, (n_gap, gap_ns, busy_ns) in sorted(gaps.items()):
        lines.append("| `%s` | %d | %.2f | %.4f |" % (name, n_gap, gap_ns / max(n_gap, 1) / 1000,
                                                     gap_ns / max(gap_ns + busy_ns, 1)))
    path = os.path.join(ROOT, "profiles", "k_expert_%s.md" % HEADLINE)
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)


# ------------------------------------------------------------------ step model, extras

def step_model_section(efa, spec, rows, shared_us, layers=1):
    """The step-time model fed by the measured times of one routing: E_p(n) is the
    mean requested bytes of a pass, beta_p(n) = E_p(n) / measured time (fixed work
    folded in, phi = 0), D = the shared experts' bytes read once per pass with
    beta_D = D / their measured time, t0 = h = 0; k*(a) over 22 acceptance values."""
    nmax = len(rows)
    E = [[r["bytes_slot"] for r in rows], [r["bytes_dedup"] for r in rows]]
    beta = [[r["bytes_slot"] / (r["us_slot"] * 1e-6) for r in rows],
            [r["bytes_dedup"] / (r["us_dedup"] * 1e-6) for r in rows]]
    D = float(spec.n_shared * spec.expert_bytes)
    beta_D = D / (sum(shared_us) / len(shared_us) * 1e-6) if D > 0 and shared_us else 1.0
    mW = layers * spec.m * spec.expert_bytes  # expert bytes of one token over the layers of a pass
    out = efa.step_time_model(nmax, A_GRID, mW, E, beta, D=D, beta_D=beta_D)
    return {"inputs": {"m_W": mW, "D": D, "beta_D_GBps": round(beta_D / 1e9, 1),
                       "t0": 0.0, "h": 0.0, "phi": "folded into the measured times"},
            "a": [round(a, 4) for a in A_GRID],
            "kstar_slot": out["kstar"][0].tolist(), "kstar_dedup": out["kstar"][1].tolist(),
            "speedup_slot": [round(v, 4) for v in out["speedup"][0].tolist()],
            "speedup_dedup": [round(v, 4) for v in out["speedup"][1].tolist()],
            "a0": [round(v, 5) for v in out["a0"].tolist()],
            "step_points_slot": [round(v, 5) for v in out["step_point"][0][1:].tolist()],
            "step_points_dedup": [round(v, 5) for v in out["step_point"][1][1:].tolist()],
            "tau_us_slot": [round(v * 1e6, 2) for v in out["tau"][0].tolist()],
            "tau_us_dedup": [round(v * 1e6, 2) for v in out["tau"][1].tolist()],
            "crossover_model": out["crossover"]}


def chosen_id_section(args, efa, routing, spec, layer, ws, clock, recs, per_kind, x_of):
    """Passes with chosen ids (U distinct experts among n m slots, from heavy
    repetition to none, n = 2..9), the fits of Eq. (4) and Eq. (E.1) through the
    library, the re-read cost c_re/c_u, each fit's median relative error on the
    timed windows of trace routing (epsilon, the larger of the two) and the Table 2
    factors applied to the measured passes."""
    import torch
    m, N, b = spec.m, spec.N, spec.expert_bytes
    rows = []
    for n in range(2, 10):
        Us = sorted(set(int(round(v)) for v in np.linspace(m, min(n * m, N), 6)))
        x = x_of(n)
        y = torch.empty(n, spec.d, dtype=torch.float32, device="cuda")
        for U in Us:
            for rep in range(3):
                tr = routing.chosen_pass(N, m, n, U, routing.rng_for(args.seed, 0, "chosen", 1000 * n + 10 * U + rep))
                ids = torch.from_numpy(tr.ids).cuda()
                w = torch.from_numpy(tr.w).cuda()
                t = {k: clock.median_us(lambda: fn(layer, x, ids, w, y=y, ws=ws), 3) * 1e-6
                     for k, fn in (("slot", efa.expert_perslot), ("dedup", efa.expert_dedup))}
                rows.append((n, U, t["slot"], t["dedup"]))
    n_c = np.array([r[0] for r in rows]); U_c = np.array([r[1] for r in rows])
    cs = efa.fit_times(efa.MOE_KIND_SLOT, n_c, U_c, m, np.array([r[2] for r in rows]), b)
    cd = efa.fit_times(efa.MOE_KIND_DEDUP, n_c, U_c, m, np.array([r[3] for r in rows]), b)
    out = {"workload": "passes with chosen ids, n = 2..9, U from m to min(n m, N) (6 values), 3 passes each, "
                       "median of 3 timed runs after the flush",
           "passes": [dict(n=int(r[0]), U=int(r[1]), t_slot_us=round(r[2] * 1e6, 2), t_dedup_us=round(r[3] * 1e6, 2))
                      for r in rows],
           "fit_slot": {"t_op_us": cs[0] * 1e6, "c_u_s_per_GB": cs[1] * 1e9, "c_re_s_per_GB": cs[2] * 1e9,
                        "reread_cost": cs[2] / cs[1]},
           "fit_dedup": {"t_op_us": cd[0] * 1e6, "c_g_s_per_GB": cd[1] * 1e9, "c_t_us_per_token": cd[2] * 1e6}}
    if recs is None:
        return out
    # each fit's relative error on the timed windows (n >= 2)
    win = [r for r in recs if r["n"] >= 2]
    nw = np.array([r["n"] for r in win], np.float64); Uw = np.array([r["U"] for r in win], np.float64)
    pred_s = cs[0] + cs[1] * Uw * b + cs[2] * (nw * m - Uw) * b
    pred_d = cd[0] + cd[1] * Uw * b + cd[2] * nw
    meas_s = np.array([r["t_slot_ms"] * 1e-3 for r in win]); meas_d = np.array([r["t_dedup_ms"] * 1e-3 for r in win])
    eps_s = float(np.median(np.abs(pred_s - meas_s) / meas_s))
    eps_d = float(np.median(np.abs(pred_d - meas_d) / meas_d))
    eps = max(eps_s, eps_d)
    out.update(eps_slot=eps_s, eps_dedup=eps_d, eps=eps, windows=len(win))
    if eps < 0.5:
        f = efa.error_bounds(eps)
        out["bounds"] = f
        dec = {}
        for kind, pk in per_kind.items():
            rows_k = []
            for row in pk["per_n"]:
                if row["n"] < 2:
                    continue
                S = row["us_slot"] - row["us_dedup"]
                rows_k.append(dict(n=row["n"], faster_kernel_decided=bool(abs(math.log(row["r"]) - math.log(row["u"]))
                                                                         > f["faster_margin"]),
                                   saving_us=round(S, 2),
                                   saving_bound_us=round(f["time_factor"] * (row["us_slot"] + row["us_dedup"]), 2)))
            sm = pk["step_model"]
            stable = []
            for key in ("tau_us_slot", "tau_us_dedup"):
                V = [sm["tau_us_slot"][0]] + sm[key][1:]  # V(0) = the per-slot tau(1), V(k) = tau_p(k+1)
                cnt = 0
                for a in A_GRID:
                    T = [sum(a ** i for i in range(k + 1)) / V[k] for k in range(len(V))]
                    ks = int(np.argmax(T))
                    cnt += all(T[i] < f["regret_factor"] * T[ks] for i in range(len(T)) if i != ks)
                stable.append(cnt)
            dec[kind] = {"per_n": rows_k, "kstar_certain_slot": stable[0], "kstar_certain_dedup": stable[1],
                         "a_points": len(A_GRID)}
        out["decisions"] = dec
    return out


def dispatch_section(efa, layer, ws, ys, passes, kinds, nvals, warmup, per_kind, clock):
    """The crossover-driven switch (moe_expert_auto) on held-out windows: the crossover
    comes from the timed windows' measured S(n); the warm-up windows, never used for
    it, are run by both kernels and by the switch, each after the flush."""
    out = {"workload": "warm-up windows of each routing (not used for the crossover), n = 1..%d" % nvals[-1]}
    held = list(range(warmup)) or [0]
    for kind, _ in kinds:
        c = int(per_kind[kind]["crossover"])
        tot = {"slot": 0.0, "dedup": 0.0, "auto": 0.0, "best": 0.0}
        for n in nvals:
            for s_ in held:
                p = passes[(kind, n, s_)]
                t = {"slot": clock.once_us(lambda: efa.expert_perslot(layer, p["x"], p["ids"], p["w"], y=ys[n], ws=ws)),
                     "dedup": clock.once_us(lambda: efa.expert_dedup(layer, p["x"], p["ids"], p["w"], y=ys[n], ws=ws)),
                     "auto": clock.once_us(lambda: efa.expert_auto(layer, p["x"], p["ids"], p["w"], c, y=ys[n],
                                                                   ws=ws))}
                for k in ("slot", "dedup", "auto"):
                    tot[k] += t[k]
                tot["best"] += min(t["slot"], t["dedup"])
        out[kind] = {"crossover": c, **{k + "_us_total": round(v, 1) for k, v in tot.items()},
                     "auto_over_best": round(tot["auto"] / tot["best"], 4),
                     "auto_over_slot": round(tot["auto"] / tot["slot"], 4),
                     "auto_over_dedup": round(tot["auto"] / tot["dedup"], 4)}
    return out


def router_section(args, efa, synth, spec, passes, kinds, nvals, clock):
    """The router ahead of the expert operation (two launches: logits, then top-m and
    softmax) on the layer's own activations, after the flush, events around both."""
    from synth.device import to_torch
    wr = to_torch(synth.router_weights(spec, args.seed))
    us = []
    for n in nvals:
        x = passes[(kinds[0][0], n, 0)]["x"]
        out = efa.router_topk(wr, x, spec.m)
        us.append(round(clock.median_us(lambda: efa.router_topk(wr, x, spec.m, out=out), 5), 2))
    nb = spec.N * spec.d * 2
    return {"workload": "router of the layer: logits of N=%d experts over d=%d (bf16), top-%d and softmax, n = 1..%d"
                        % (spec.N, spec.d, spec.m, nvals[-1]),
            "launches": 2, "us_per_n": us, "router_bytes": nb,
            "GBps_per_n": [round((nb + n * spec.d * 2) / (t * 1e-6) / 1e9, 1) for n, t in zip(nvals, us)]}


def tree_selection(args, efa, routing, spec, layer, x, y, ws, clock, ntrees, dedup_fit):
    """The verification subtree of each seeded 32-node tree chosen by reward over
    predicted cycle time (SpecFit Eq. (5), moe_tree_select, K = 7), with the cycle time
    calibrated from the deduplicating kernel's fit on chosen ids on the same layer
    (beta = c_g w per union expert, b_k = t_op + c_t (k + 1)); the selected tokens are
    then run through the dedup kernel and timed, next to the 7 nodes of highest
    cumulative probability (the plain rule for a 7-node budget)."""
    import torch
    t_op, c_g, c_t = dedup_fit
    K = 7
    w_exp = spec.expert_bytes
    beta = c_g * w_exp
    b = [max(t_op + c_t * (k + 1), 1e-9) for k in range(K + 1)]
    rows = []
    for i in range(1, ntrees + 1):
        parent, ttr = routing.tree_routing(spec.N, spec.m, 0.5, routing.rng_for(args.seed, 0, "tree", i))
        p = routing.tree_commit_probs(parent, routing.rng_for(args.seed, 0, "tree", 1000 + i))
        bm = efa.expert_bitmaps(ttr.ids[:, None, :], spec.N)
        s = efa.tree_select(parent, p, bm, K, b, beta)
        top = sorted(range(1, 32), key=lambda v: (-p[v], v))[:K]
        res = {}
        for name, nodes in (("selected", [0] + s["ids"]), ("top7", [0] + sorted(top))):
            ids = torch.from_numpy(np.ascontiguousarray(ttr.ids[nodes])).cuda()
            w = torch.from_numpy(np.ascontiguousarray(ttr.w[nodes])).cuda()
            n = len(nodes)
            t = clock.median_us(lambda: efa.expert_dedup(layer, x[:n], ids, w, y=y[:n], ws=ws), 3) * 1e-6
            R = 1.0 + float(sum(p[v] for v in nodes[1:]))
            U = len(set(ttr.ids[nodes].reshape(-1).tolist()))
            res[name] = dict(nodes=n - 1, R=R, U=U, t_meas=t, t_pred=b[n - 1] + beta * U)
        rows.append(res)

    def mean(k, f):
        return float(np.mean([r[k][f] for r in rows]))
    out = {"workload": "%d seeded 32-node trees, commit probabilities per tree, K = 7, one qwen3-shaped layer"
                       % ntrees, "beta_us_per_union_expert": beta * 1e6, "b_us": [v * 1e6 for v in b]}
    for k in ("selected", "top7"):
        out[k] = {"nodes": mean(k, "nodes"), "R": mean(k, "R"), "U": mean(k, "U"),
                  "t_meas_us": mean(k, "t_meas") * 1e6, "t_pred_us": mean(k, "t_pred") * 1e6,
                  "R_per_ms_measured": float(np.mean([r[k]["R"] / r[k]["t_meas"] for r in rows])) * 1e-3,
                  "pred_rel_err_median": float(np.median([abs(r[k]["t_pred"] - r[k]["t_meas"]) / r[k]["t_meas"]
                                                          for r in rows]))}
    return out


# ------------------------------------------------------------------ workloads

def xdev(torch, spec, shape, key):
    """Activations ~ N(0, 1) rounded to bf16, from torch's seeded device generator."""
    g = torch.Generator(device="cuda")
    g.manual_seed(int(key) & ((1 << 63) - 1))
    return torch.randn(*shape, spec.d, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)


def qwen3x48(args, torch, efa, synth, routing, clock, nvals, full):
    """The headline workload: the Qwen3-shaped layer x48 back to back per pass."""
    from synth.device import device_layer_weights
    spec = synth.CONFIGS["qwen3"]
    L, T = spec.layers, TRACE_TOKENS
    t_setup = time.perf_counter()
    layers, plain = [], []
    for l in range(L):
        w = device_layer_weights(spec, args.seed, l)
        layers.append(efa.Layer(*w, m=spec.m).tiled_copy())  # weight-load time: tiled layout
        if l < ORACLE_LAYERS:
            plain.append(w)
        del w
    traces = [routing.make_trace(spec, "zipf", T, seed=args.seed, layer=l, s=1.1) for l in range(L)]
    torch.cuda.synchronize()
    progress("qwen3 x48: %d layers on the device (%.1f s)" % (L, time.perf_counter() - t_setup))
    S = args.warmup + args.steps
    w_exp = spec.expert_bytes
    sh = clock.sh
    lib = efa.lib()
    vp = ctypes.c_void_p
    descs = [l.desc() for l in layers]
    ws = layers[0].workspace(nvals[-1])
    # inputs resident in HBM before timing: per n, ids / w of every (window, layer) and
    # activations of every (window, layer); per-layer outputs
    dev = {}
    for n in nvals:
        starts = routing.window_starts(T, n, S, seed=args.seed)
        ids = np.stack([np.stack([routing.window(traces[l], int(starts[s]), n)[0] for l in range(L)])
                        for s in range(S)]).astype(np.int32)
        ww = np.stack([np.stack([routing.window(traces[l], int(starts[s]), n)[1] for l in range(L)])
                       for s in range(S)]).astype(np.float32)
        U = np.array([[len(set(ids[s, l].reshape(-1).tolist())) for l in range(L)] for s in range(S)])
        dev[n] = dict(ids_h=ids, w_h=ww, U=U, ids=torch.from_numpy(ids).cuda(), w=torch.from_numpy(ww).cuda(),
                      x=xdev(torch, spec, (S, L, n), 1000 + n),
                      y=torch.empty(L, n, spec.d, dtype=torch.float32, device="cuda"))

    def argsets(n, s, y=None, stream=None):
        """Prebuilt C-ABI arguments of the 48 launches of window s (so that they queue
        faster than they run)."""
        D = dev[n]
        nm = n * spec.m
        yp = (y if y is not None else D["y"]).data_ptr()
        st = stream if stream is not None else sh
        return [(ctypes.byref(descs[l]), ctypes.byref(layers[l]._weights),
                 vp(D["x"].data_ptr() + ((s * L + l) * n * spec.d) * 2),
                 vp(D["ids"].data_ptr() + (s * L + l) * nm * 4), vp(D["w"].data_ptr() + (s * L + l) * nm * 4),
                 n, vp(yp + l * n * spec.d * 4), None, vp(ws.data_ptr()), ws.numel(), vp(st)) for l in range(L)]

    def run_all(fn, sets):
        for a in sets:
            rc = fn(*a)
            if rc != 0:
                raise RuntimeError("expert call failed: status %d" % rc)

    if args.pmc_pass:
        # Counter run: one window per n, each kernel once per pass after the flush;
        # then the 32-node tree on layer 0 (a few seeded trees)
        order = []
        for kname, fn in (("slot", lib.moe_expert_perslot), ("dedup", lib.moe_expert_dedup)):
            for n in nvals:
                s = args.warmup
                clock.flush()
                run_all(fn, argsets(n, s))
                for l in range(L):
                    Ul = int(dev[n]["U"][s, l])
                    order.append(dict(workload=HEADLINE, kernel=kname, n=n, layer=l, U=Ul,
                                      bytes=(n * spec.m if kname == "slot" else Ul) * w_exp))
        x = xdev(torch, spec, (32,), 77)
        y = torch.empty(32, spec.d, dtype=torch.float32, device="cuda")
        ws32 = layers[0].workspace(32)
        for i in range(PMC_TREES):
            _, ttr = routing.tree_routing(spec.N, spec.m, 0.5, routing.rng_for(args.seed, 0, "tree", 100000 + i))
            ids, w = torch.from_numpy(ttr.ids).cuda(), torch.from_numpy(ttr.w).cuda()
            U = len(set(ttr.ids.reshape(-1).tolist()))
            for kname, fn in (("slot", efa.expert_perslot), ("dedup", efa.expert_dedup)):
                clock.flush()
                fn(layers[0], x, ids, w, y=y, ws=ws32)
                order.append(dict(workload="tree", kernel=kname, n=32, layer=0, U=U,
                                  bytes=(32 * spec.m if kname == "slot" else U) * w_exp))
        torch.cuda.synchronize()
        return {"pmc_order": order}

    recs = []
    for n in nvals:
        for s in range(S):
            sets = argsets(n, s)
            ts = clock.median_us(lambda: run_all(lib.moe_expert_perslot, sets), args.reps)
            td = clock.median_us(lambda: run_all(lib.moe_expert_dedup, sets), args.reps)
            if s >= args.warmup:
                Us = dev[n]["U"][s]
                recs.append(dict(n=n, window=s, U=float(Us.mean()), bytes_slot=L * n * spec.m * w_exp,
                                 bytes_dedup=int(Us.sum()) * w_exp, t_slot_ms=ts / 1e3, t_dedup_ms=td / 1e3))
    torch.cuda.synchronize()
    progress("qwen3 x48: %d windows x %d n timed, %d reps each" % (args.steps, len(nvals), args.reps))
    rows = per_n_rows(recs, nvals)
    res = {"workload": "qwen3-shaped layer x48 back to back per pass (N=128, m=8, d=2048, d_ff=768, bf16), "
                       "zipf(s=1.1) routing per layer, %d windows per n, median of %d reps" % (args.steps, args.reps),
           "per_n": strip_bytes(rows), "crossover": crossover_of(rows),
           "step_model": step_model_section(efa, spec, rows, [], layers=L), "recs": recs, "rows": rows}

    # the oracle's sample: windows of this workload on the first layers, before the
    # weights go (plain copies of those layers on the host)
    from synth.device import from_torch_bf16
    host = [tuple(from_torch_bf16(t) for t in plain[l]) for l in range(ORACLE_LAYERS)]
    cpu_passes = []
    for s in range(args.warmup, args.warmup + min(HOST_WINDOWS, args.steps)):
        for n in nvals:
            for l in range(ORACLE_LAYERS):
                D = dev[n]
                cpu_passes.append((host[l], from_torch_bf16(D["x"][s, l]), D["ids_h"][s, l], D["w_h"][s, l], "bf16",
                                   n * spec.m * w_exp))
    res["cpu_passes"] = cpu_passes
    res["cpu_sample"] = ("windows of the same workload (layers 0..%d of the 48, every n = 1..%d in turn, window by "
                         "window)" % (ORACLE_LAYERS - 1, nvals[-1]))
    del plain

    if full and not args.no_extras:
        # The same 48 launches as HIP graphs (one capture per n and kernel over the
        # static id / weight buffers, which each window's launches read at run time),
        # replayed on the bench stream and checked bitwise against the eager launches.
        cap = torch.cuda.Stream()  # default priority
        grecs = []
        for n in nvals:
            yg = torch.empty(L, n, spec.d, dtype=torch.float32, device="cuda")
            graphs = {}
            torch.cuda.synchronize()
            for kname, fn in (("slot", lib.moe_expert_perslot), ("dedup", lib.moe_expert_dedup)):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    run_all(fn, argsets(n, args.warmup, y=yg, stream=cap.cuda_stream))
                graphs[kname] = g
            torch.cuda.synchronize()
            sets = argsets(n, args.warmup)
            row = {"n": n}
            for kname, fn in (("slot", lib.moe_expert_perslot), ("dedup", lib.moe_expert_dedup)):
                row[kname + "_eager_us"] = round(clock.median_us(lambda: run_all(fn, sets), 3), 1)
                row[kname + "_graph_us"] = round(clock.median_us(lambda: graphs[kname].replay(), 3), 1)
                assert torch.equal(dev[n]["y"], yg), "graph replay differs from the eager launches (%s)" % kname
            grecs.append(row)
            del graphs
        res["hip_graph"] = {"what": "the 48 launches of a pass captured once per n and kernel and replayed; us per "
                                    "pass of 48 layers, median of 3 (one window), checked bitwise against the eager "
                                    "launches", "per_n": grecs}
        progress("qwen3 x48: hip graph replay done")
    res["layer0"] = layers[0]
    del layers
    return res


def time_windows(args, efa, clock, layer, passes, kinds, nvals, ws, ys, w_exp, m):
    """Both kernels on every prepared window of every routing: median of reps each."""
    recs = []
    for kind, _ in kinds:
        for n in nvals:
            for s in range(args.warmup + args.steps):
                p = passes[(kind, n, s)]
                ts = clock.median_us(lambda: efa.expert_perslot(layer, p["x"], p["ids"], p["w"], y=ys[n], ws=ws),
                                     args.reps)
                td = clock.median_us(lambda: efa.expert_dedup(layer, p["x"], p["ids"], p["w"], y=ys[n], ws=ws),
                                     args.reps)
                if s >= args.warmup:
                    recs.append(dict(kind=kind, n=n, window=s, U=p["U"], bytes_slot=n * m * w_exp,
                                     bytes_dedup=p["U"] * w_exp, t_slot_ms=ts / 1e3, t_dedup_ms=td / 1e3))
    return recs


def prepare_windows(args, torch, synth, routing, spec, kinds, nvals, host_x=True):
    """Device inputs of every (routing, n, window) of a single-layer workload."""
    from synth.device import to_torch
    passes = {}
    S = args.warmup + args.steps
    for ki, (kind, kw) in enumerate(kinds):
        tr = routing.make_trace(spec, kind, TRACE_TOKENS, seed=args.seed, **kw)
        for n in nvals:
            starts = routing.window_starts(TRACE_TOKENS, n, S, seed=args.seed + 17 * ki)
            xs = None if host_x else xdev(torch, spec, (S, n), 2000 + 100 * ki + n)
            for s in range(S):
                ids, w = routing.window(tr, int(starts[s]), n)
                x = to_torch(synth.pass_x(spec, args.seed, 0, 10000 * ki + 100 * n + s, n)) if host_x else xs[s]
                passes[(kind, n, s)] = dict(x=x, ids=torch.from_numpy(ids).cuda(), w=torch.from_numpy(w).cuda(),
                                            ids_h=ids, w_h=w, U=len(set(ids.reshape(-1).tolist())))
    return passes


def pmc_single_layer(args, torch, efa, synth, routing, clock, nvals, name):
    """Counter run of a single-layer workload: one window per (routing, n), each
    kernel once after the flush; returns what ran, in dispatch order."""
    from synth.device import device_layer_weights
    spec = synth.CONFIGS[name]
    kinds = {"dsv2lite": [("uniform", {}), ("correlated", {"p": 0.5})],
             "mixtral": [("uniform", {}), ("correlated", {"p": 0.6})]}[name]
    layer = load_layout(efa.Layer(*device_layer_weights(spec, args.seed, 0), m=spec.m))
    one = argparse.Namespace(**{**vars(args), "steps": 1, "warmup": 0})
    passes = prepare_windows(one, torch, synth, routing, spec, kinds, nvals, host_x=False)
    ws = layer.workspace(nvals[-1])
    order = []
    for kind, _ in kinds:
        for n in nvals:
            p = passes[(kind, n, 0)]
            y = torch.empty(n, spec.d, dtype=torch.float32, device="cuda")
            for kname, fn in (("slot", efa.expert_perslot), ("dedup", efa.expert_dedup)):
                clock.flush()
                fn(layer, p["x"], p["ids"], p["w"], y=y, ws=ws)
                order.append(dict(workload="%s_%s" % (name, kind), kernel=kname, n=n, layer=0, U=p["U"],
                                  bytes=(n * spec.m if kname == "slot" else p["U"]) * spec.expert_bytes))
    torch.cuda.synchronize()
    del layer
    return order


def dsv2lite(args, torch, efa, synth, routing, clock, nvals):
    """The DeepSeek-V2-Lite-shaped layer, uniform and correlated routing; with the
    extras: shared experts, router, dispatch, chosen-id fits and bounds."""
    from synth.device import to_torch
    spec = synth.CONFIGS["dsv2lite"]
    kinds = [("uniform", {}), ("correlated", {"p": 0.5})]
    host_w = synth.layer_weights(spec, args.seed)
    layer = load_layout(efa.Layer(*(to_torch(a) for a in host_w), m=spec.m))
    passes = prepare_windows(args, torch, synth, routing, spec, kinds, nvals)
    ws = layer.workspace(nvals[-1])
    ys = {n: torch.empty(n, spec.d, dtype=torch.float32, device="cuda") for n in nvals}
    torch.cuda.synchronize()
    recs = time_windows(args, efa, clock, layer, passes, kinds, nvals, ws, ys, spec.expert_bytes, spec.m)
    progress("dsv2lite timed")
    out = {"workload": "deepseek-v2-lite-shaped layer (N=64 top-6, d=2048, d_ff=1408, bf16), uniform and correlated "
                       "(p=0.5) routing, %d windows per n, median of %d reps" % (args.steps, args.reps)}
    # the shared experts' pass (read once per pass whatever the routing): D(n) of the step model
    shared_us, fused = [], None
    if not args.no_extras:
        sh_host = synth.layer_weights(spec, args.seed, shared=True)
        shl = load_layout(efa.Layer(*(to_torch(a) for a in sh_host), m=spec.n_shared))
        sws = shl.workspace(nvals[-1])
        for n in nvals:
            sids = torch.arange(spec.n_shared, dtype=torch.int32, device="cuda").repeat(n, 1).contiguous()
            sw = torch.ones(n, spec.n_shared, dtype=torch.float32, device="cuda")
            x = passes[(kinds[0][0], n, 0)]["x"]
            shared_us.append(clock.median_us(lambda: efa.expert_dedup(shl, x, sids, sw, y=ys[n], ws=sws), 5))
        # the same experts in the routed call itself (one launch): routed alone and
        # routed + shared on the same windows, paired, both kernels
        fl = efa.Layer(layer.w_gate, layer.w_up, layer.w_down, m=spec.m, packed=layer.packed, tiled=layer.tiled,
                       shared=(shl.w_gate, shl.w_up, shl.w_down))
        fws = fl.workspace(nvals[-1])
        fused = {"routed_slot": [], "fused_slot": [], "routed_dedup": [], "fused_dedup": []}
        for n in nvals:
            for kname, fn in (("slot", efa.expert_perslot), ("dedup", efa.expert_dedup)):
                tr_, tf_ = [], []
                for s_ in range(min(4, args.warmup + args.steps)):
                    p = passes[(kinds[0][0], n, s_)]
                    tr_.append(clock.once_us(lambda: fn(layer, p["x"], p["ids"], p["w"], y=ys[n], ws=ws)))
                    tf_.append(clock.once_us(lambda: fn(fl, p["x"], p["ids"], p["w"], y=ys[n], ws=fws)))
                fused["routed_" + kname].append(round(float(np.median(tr_)), 2))
                fused["fused_" + kname].append(round(float(np.median(tf_)), 2))
        out["shared_experts"] = {"workload": "%d always-on shared experts, weight 1, every token: one deduplicating "
                                             "call per pass (the D(n) bytes of the step model)" % spec.n_shared,
                                 "us_per_n": [round(v, 2) for v in shared_us], "bytes": spec.n_shared * spec.expert_bytes,
                                 "in_call": dict(workload="the same experts computed in the routed launch (desc "
                                                          "n_shared); routed alone vs routed + shared, paired on "
                                                          "%s windows, median of 4" % kinds[0][0],
                                                 **{k + "_us": v for k, v in fused.items()})}
        del shl, fl, fws
    per_kind = {}
    for kind, _ in kinds:
        rows = per_n_rows([r for r in recs if r["kind"] == kind], nvals)
        per_kind[kind] = dict(per_n=strip_bytes(rows), crossover=crossover_of(rows),
                              step_model=step_model_section(efa, spec, rows, shared_us))
        if fused is not None:
            # D/beta_D from the time the shared experts add to the routed launch
            marg = [f - r for k in ("slot", "dedup") for f, r in zip(fused["fused_" + k], fused["routed_" + k])]
            per_kind[kind]["step_model_shared_in_call"] = step_model_section(
                efa, spec, rows, [max(sum(marg) / len(marg), 1e-3)])
    out["results"] = per_kind
    if not args.no_extras:
        out["router"] = router_section(args, efa, synth, spec, passes, kinds, nvals, clock)
        out["dispatch"] = dispatch_section(efa, layer, ws, ys, passes, kinds, nvals, args.warmup, per_kind, clock)
        ws9 = layer.workspace(9)
        out["chosen_ids"] = chosen_id_section(args, efa, routing, spec, layer, ws9, clock, recs, per_kind,
                                              lambda n: to_torch(synth.pass_x(spec, args.seed, 0, 77000 + n, n)))
        progress("dsv2lite extras done")
    return out, per_kind


def mixtral(args, torch, efa, synth, routing, clock, nvals):
    """The Mixtral-shaped layer, uniform and repeat-0.6 routing (device weights)."""
    from synth.device import device_layer_weights
    spec = synth.CONFIGS["mixtral"]
    kinds = [("uniform", {}), ("correlated", {"p": 0.6})]
    layer = load_layout(efa.Layer(*device_layer_weights(spec, args.seed, 0), m=spec.m))
    passes = prepare_windows(args, torch, synth, routing, spec, kinds, nvals, host_x=False)
    ws = layer.workspace(nvals[-1])
    ys = {n: torch.empty(n, spec.d, dtype=torch.float32, device="cuda") for n in nvals}
    torch.cuda.synchronize()
    recs = time_windows(args, efa, clock, layer, passes, kinds, nvals, ws, ys, spec.expert_bytes, spec.m)
    per_kind = {}
    for kind, _ in kinds:
        rows = per_n_rows([r for r in recs if r["kind"] == kind], nvals)
        per_kind[kind] = dict(per_n=strip_bytes(rows), crossover=crossover_of(rows))
    del layer
    return {"workload": "mixtral-shaped layer (N=8 top-2, d=4096, d_ff=14336, bf16), uniform and repeat p=0.6 "
                        "routing, %d windows per n, median of %d reps" % (args.steps, args.reps),
            "results": per_kind}, per_kind


def tree(args, torch, efa, synth, routing, clock, layer):
    """The 32-node draft tree on one Qwen3-shaped layer: seeded trees, both kernels."""
    spec = synth.CONFIGS["qwen3"]
    ntrees = args.steps
    y = torch.empty(32, spec.d, dtype=torch.float32, device="cuda")
    ws32 = layer.workspace(32)
    x = xdev(torch, spec, (32,), 77)
    recs = []
    for i in range(args.warmup + ntrees):
        _, ttr = routing.tree_routing(spec.N, spec.m, 0.5, routing.rng_for(args.seed, 0, "tree", 100000 + i))
        ids, w = torch.from_numpy(ttr.ids).cuda(), torch.from_numpy(ttr.w).cuda()
        U = len(set(ttr.ids.reshape(-1).tolist()))
        ts = clock.median_us(lambda: efa.expert_perslot(layer, x, ids, w, y=y, ws=ws32), args.reps)
        td = clock.median_us(lambda: efa.expert_dedup(layer, x, ids, w, y=y, ws=ws32), args.reps)
        if i >= args.warmup:
            recs.append(dict(n=32, U=U, bytes_slot=32 * spec.m * spec.expert_bytes, bytes_dedup=U * spec.expert_bytes,
                             t_slot_ms=ts / 1e3, t_dedup_ms=td / 1e3))
    row = per_n_rows(recs, [32])[0]
    out = {"workload": "32-node ancestor-closed draft tree (1+1+2+4+8+16, children reuse parent experts with p=0.5) on "
                       "one qwen3-shaped layer, %d seeded trees, median of %d reps" % (ntrees, args.reps),
           **{k: v for k, v in row.items() if not k.startswith("bytes_")},
           "bytes_slot": row["bytes_slot"], "bytes_dedup_mean": row["bytes_dedup"]}
    if not args.no_extras:
        # NEXT-3: subtree selection, calibrated by the dedup kernel's chosen-id fit on this layer
        ws9 = layer.workspace(9)
        fit = chosen_id_section(args, efa, routing, spec, layer, ws9, clock, None, None,
                                lambda n: xdev(torch, spec, (n,), 78000 + n))
        out["chosen_id_fit"] = {k: fit[k] for k in ("fit_slot", "fit_dedup")}
        fd = fit["fit_dedup"]
        out["selection"] = tree_selection(args, efa, routing, spec, layer, x, y, ws32, clock, ntrees,
                                          (fd["t_op_us"] * 1e-6, fd["c_g_s_per_GB"] * 1e-9,
                                           fd["c_t_us_per_token"] * 1e-6))
    return out


def _r4(v):
    return [round(float(x), 4) for x in v]


def headline_line(args, head, others, cpu, nvals, launches_per_pass, full_path):
    """The compact final line: the headline workload's per-n figures, the roofline of
    its dominant kernel with the per-n and n = 1 fractions of both kernels, the oracle
    baseline, and r(n), u(n), crossover and n = 1 fractions of the other workloads."""
    recs, rows = head["recs"], head["rows"]
    tot_bytes = sum(r["bytes_slot"] + r["bytes_dedup"] for r in recs)
    tot_s = sum(r["t_slot_ms"] + r["t_dedup_ms"] for r in recs) / 1e3
    kt = {k: kernel_totals(recs, k, launches_per_pass) for k in ("slot", "dedup")}
    dom = max(kt, key=lambda k: kt[k]["seconds"])
    kernels = {}
    for k in ("slot", "dedup"):
        kernels[k] = {"achieved": round(kt[k]["gbps"], 1), "frac": round(kt[k]["gbps"] / PEAK_HBM_GBPS, 4),
                      "avg_launch_us": round(kt[k]["avg_launch_us"], 3),
                      "bytes_per_launch": round(kt[k]["bytes_per_launch"], 1), "launches": kt[k]["launches"],
                      "traffic": read_traffic(k)}
    roofline = {"bound": "hbm", "achieved": kernels[dom]["achieved"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": kernels[dom]["frac"], "traffic": kernels[dom]["traffic"],
                "kernel": "k_expert %s (one launch per layer; the kernel with the most time)" % (
                    "per-slot" if dom == "slot" else "deduplicating"),
                "frac_n1_slot": rows[0]["frac_slot"], "frac_n1_dedup": rows[0]["frac_dedup"],
                "frac_per_n_slot": [r["frac_slot"] for r in rows], "frac_per_n_dedup": [r["frac_dedup"] for r in rows],
                "kernels": kernels}
    sm = head["step_model"]
    line = {"metric": METRIC, "value": round(tot_bytes / tot_s / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(tot_s * 1e3 / args.steps, 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "qwen3-30b-a3b-shaped MoE layer x48 back to back per pass (N=128 top-8, d=2048, "
                                   "d_ff=768, bf16 weights, fp32 accumulate), zipf(s=1.1) routing per layer, n=1..%d, "
                                   "per-slot and dedup kernels" % nvals[-1],
                       "layers": 48, "windows_per_n": args.steps, "reps_per_window": args.reps,
                       "weight_layout": WEIGHT_LAYOUT, "launches_per_layer": 1,
                       "scrub_bytes": 0 if args.no_scrub else SCRUB_BYTES},
            "roofline": roofline, "cpu_baseline": cpu,
            "per_n": {"n": list(nvals), "us_slot": [r["us_slot"] for r in rows],
                      "us_dedup": [r["us_dedup"] for r in rows], "gbps_slot": [r["gbps_slot"] for r in rows],
                      "gbps_dedup": [r["gbps_dedup"] for r in rows], "r": [r["r"] for r in rows],
                      "u": [r["u"] for r in rows], "U": [r["mean_U"] for r in rows]},
            "crossover": head["crossover"],
            "staircase": {"kstar_slot": sm["kstar_slot"], "kstar_dedup": sm["kstar_dedup"],
                          "crossover_model": sm["crossover_model"]},
            "others": others, "full_record": full_path, "source_hash": source_hash()}
    return line


def other_summary(per_kind):
    out = {}
    for kind, pk in per_kind.items():
        rows = pk["per_n"]
        out[kind] = {"r": _r4(r["r"] for r in rows), "u": _r4(r["u"] for r in rows), "cross": pk["crossover"],
                     "frac_n1": [rows[0]["frac_slot"], rows[0]["frac_dedup"]],
                     "frac_n8": [rows[-1]["frac_slot"], rows[-1]["frac_dedup"]]}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=16, help="timed windows per n (and seeded trees)")
    ap.add_argument("--warmup", type=int, default=2, help="untimed windows per n before the timed ones")
    ap.add_argument("--reps", type=int, default=3, help="timed runs of each window; the median is kept")
    ap.add_argument("--nmax", type=int, default=8)
    ap.add_argument("--seed", type=int, default=2026)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-scrub", action="store_true")
    ap.add_argument("--workloads", default=",".join(WORKLOADS),
                    help="comma list of %s (the headline, qwen3x48, always runs)" % ",".join(WORKLOADS))
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the further sections (graph replay, fits, dispatch, router, shared experts, selection)")
    ap.add_argument("--out", default=FULL_RECORD, help="where the full record (JSON) goes")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="for a counter run: one window per n of the headline workload, both kernels, each pass "
                         "after the 1 GiB read flush, then a 256 MiB device copy; prints what ran")
    ap.add_argument("--traffic-from", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "PASS_LOG"),
                    help="write profiles/traffic_k_expert.md from two counter runs (no GPU)")
    ap.add_argument("--sq-summary", nargs=3, metavar=("SQA_CSV", "SQB_CSV", "PASS_LOG"),
                    help="write profiles/k_expert_sq_counters.md from two counter runs (no GPU)")
    ap.add_argument("--profile-summary", nargs=2, metavar=("PROF_DIR", "BENCH_JSON"),
                    help="write profiles/k_expert_qwen3x48.md from a kernel-trace run (no GPU)")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic_summary(*args.traffic_from)
        return
    if args.profile_summary:
        write_profile_summary(*args.profile_summary)
        return
    if args.sq_summary:
        write_sq_summary(*args.sq_summary)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the expert operation here runs on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    wl = [w for w in args.workloads.split(",") if w]
    bad = [w for w in wl if w not in WORKLOADS]
    if bad or args.steps < 1 or args.reps < 1 or args.warmup < 0:
        ap.error("bad --workloads / --steps / --reps / --warmup")

    import torch
    import expert_ffn_amd as efa
    import synth
    from synth import routing

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    clock = Clock(torch, stream, scrub=not args.no_scrub)
    nvals = list(range(1, args.nmax + 1))
    assert efa.kernels_per_call(efa.MOE_KIND_SLOT) == 1 and efa.kernels_per_call(efa.MOE_KIND_DEDUP) == 1
    t_all = time.perf_counter()

    head = qwen3x48(args, torch, efa, synth, routing, clock, nvals, full=True)
    if args.pmc_pass:  # counter run: the other single-layer workloads, then the calibration copy
        order = head["pmc_order"]
        del head
        torch.cuda.empty_cache()
        order += pmc_single_layer(args, torch, efa, synth, routing, clock, nvals, "dsv2lite")
        torch.cuda.empty_cache()
        order += pmc_single_layer(args, torch, efa, synth, routing, clock, nvals, "mixtral")
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_pass": order, "flush_read_bytes": SCRUB_BYTES, "copy_bytes": COPY_BYTES,
                          "source_hash": source_hash()}))
        return
    full = {"headline": {k: v for k, v in head.items() if k not in ("recs", "rows", "cpu_passes", "cpu_sample",
                                                                     "layer0")},
            "headline_windows": head["recs"]}
    others = {}
    if "tree" in wl:
        full["tree"] = tree(args, torch, efa, synth, routing, clock, head["layer0"])
        t = full["tree"]
        others["tree"] = {"r": t["r"], "u": t["u"], "U": t["mean_U"], "us_slot": t["us_slot"],
                          "us_dedup": t["us_dedup"], "frac": [t["frac_slot"], t["frac_dedup"]]}
        progress("tree done")
    del head["layer0"]
    torch.cuda.empty_cache()
    cpu = cpu_baseline(head.pop("cpu_passes"), args.cpu_budget)
    cpu["sample"] += "; " + head["cpu_sample"]
    progress("cpu baseline done")
    if "dsv2lite" in wl:
        full["dsv2lite"], pk = dsv2lite(args, torch, efa, synth, routing, clock, nvals)
        others.update({"dsv2lite_" + k: v for k, v in other_summary(pk).items()})
        torch.cuda.empty_cache()
    if "mixtral" in wl:
        full["mixtral"], pk = mixtral(args, torch, efa, synth, routing, clock, nvals)
        others.update({"mixtral_" + ("p0.6" if k == "correlated" else k): v for k, v in other_summary(pk).items()})
        progress("mixtral done")
        torch.cuda.empty_cache()
    line = headline_line(args, head, others, cpu, nvals, 48, args.out)
    full["line"] = line
    full["wall_s"] = round(time.perf_counter() - t_all, 1)
    if args.out:
        os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
        with open(args.out, "w") as f:
            json.dump(full, f, default=lambda o: o.tolist() if hasattr(o, "tolist") else str(o))
    print(json.dumps(line, separators=(",", ":")))


if __name__ == "__main__":
    main()
