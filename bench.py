#!/usr/bin/env python3
"""Benchmark of the MoE expert operation of a verification pass on one MI355X.

Metric: achieved HBM GB/s of the expert operation and its fraction of the
8 TB/s peak, against pass size n = 1..8, for the per-slot and the deduplicating
kernel; the bandwidth ratio r(n) = beta_dedup / beta_slot, the byte share
u(n) = E_dedup / E_slot, the saving S(n) = t_slot - t_dedup and the crossover n
(Lan, arXiv:2610.34440, Sections 1-3).

One step = for each routing kind of the layer and each n = 1..8, one pass copied
from a window of the routing trace, run once by each kernel.  Every pass is timed
alone with HIP events on the launch stream, after a read-only 1 GiB cache flush
(the 256 MB Infinity Cache would otherwise hold a whole pass; a flush that also
writes would leave dirty lines whose write-back competes with the timed reads).  Bytes are requested
expert bytes: n m w per-slot, X(n) w deduplicating (w = 3 d d_ff 2 B).
beta, r and u are from bytes and times summed over the timed passes.

Prints one JSON line.
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


class HipEvents:
    """Raw hipEvent_t handles (torch's Event only sees torch's own streams)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]
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


WEIGHT_LAYOUT = "tiled"  # moe_pack_tiled: 16-row x 64-byte blocks, waves on interleaved K steps


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


HOST_WINDOWS = 6  # windows per (routing, n) offered to the oracle's timed sample


def cpu_baseline(spec, host_w, passes, budget_s, max_threads=16):
    """The oracle, as it stands, on host cores over a bounded sample of passes: once on
    one thread, then the same passes spread over the process's cores (one pass per
    thread at a time; the C call releases the GIL), whose results must be bitwise
    equal to the single-thread ones."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    t0 = time.perf_counter()
    nbytes = 0
    ys = []
    for (x_h, ids, w) in passes:
        ys.append(oracle.moe_ffn(*host_w, x_h, ids, w, spec.dtype))
        nbytes += ids.size * spec.expert_bytes
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    done = len(ys)
    cores = max(1, min(len(os.sched_getaffinity(0)), max_threads))
    t1 = time.perf_counter()
    with ThreadPoolExecutor(cores) as pool:
        ya = list(pool.map(lambda p: oracle.moe_ffn(*host_w, p[0], p[1], p[2], spec.dtype), passes[:done]))
    dt_all = time.perf_counter() - t1
    same = all(np.array_equal(a, b) for a, b in zip(ys, ya))
    if not same:
        raise RuntimeError("oracle results differ between one thread and %d threads" % cores)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d passes (windows of the same traces, every n and routing in turn), %.1f s, requested per-slot weight bytes / "
                      "wall time, single-threaded C oracle (double accumulate)" % (done, dt),
            "all_cores": {"value": round(nbytes / dt_all / 1e9, 4), "unit": "GB/s", "cores": cores,
                          "seconds": round(dt_all, 2), "bitwise_equal_to_one_thread": same,
                          "how": "the same passes, one per thread at a time"},
            "cpu": _cpu_model()}


PMC_CMD = ("cd /tmp && export TMPDIR=/tmp && timeout -s KILL 300 rocprofv3 --pmc {counter} -d $R/gpurun_out/pmc_{tag} "
           "-o run --output-format csv -- python3 $R/bench.py --pmc-pass   (R = repository root)")
PROF_CMD = ("rocprofv3 --kernel-trace --stats -d gpurun_out/prof -o run --output-format csv -- "
            "python3 bench.py --no-extras > gpurun_out/prof_bench.json")


def progress(msg):
    """A stage of the run has finished (stderr; stdout carries only the JSON line)."""
    print("[bench] %s" % msg, file=sys.stderr, flush=True)


def prof_cmd(config):
    """The kernel-trace command whose summary profiles/k_expert_<config>_n1-8.md holds."""
    if config == "dsv2lite":
        return PROF_CMD
    return ("rocprofv3 --kernel-trace --stats -d gpurun_out/prof_%s -o run --output-format csv -- "
            "python3 bench.py --config %s --no-extras > gpurun_out/prof_bench_%s.json" % (config, config, config))


def _counter_rows(path):
    import csv
    return list(csv.DictReader(open(path)))


def traffic_from(fetch_csv, write_csv, config, kernel="slot"):
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


def write_traffic_summary(fetch_csv, write_csv, config, pass_json, out_dir=None):
    info = [json.loads(l) for l in open(pass_json) if l.startswith('{"pmc_pass"')][-1]
    out, per_launch = traffic_from(fetch_csv, write_csv, config)
    slot_pass = [p for p in info["pmc_pass"] if p.get("kernel", "slot") == "slot"]
    dedup_pass = [p for p in info["pmc_pass"] if p.get("kernel") == "dedup"]
    alg = [p["bytes"] for p in slot_pass]
    n = len(alg)
    assert n == len(out["fetch"]["bytes"])
    rec = {"kernel": "k_expert per-slot", "config": config, "launches": n,
           "bytes_per_launch": round(per_launch, 1), "algorithmic_bytes_per_launch": round(sum(alg) / n, 1),
           "fetch_factor": round(out["fetch"]["factor"], 4), "write_factor": round(out["write"]["factor"], 4),
           "source_hash": info["source_hash"]}
    lines = ["# HBM traffic of the per-slot k_expert launches, %s-shaped layer, n = 1..8, uniform + correlated" % config,
             "", "Commands (one GPU; FETCH_SIZE and WRITE_SIZE in separate runs), then on any host:", "", "```",
             PMC_CMD.format(counter="FETCH_SIZE", tag="fetch"), PMC_CMD.format(counter="WRITE_SIZE", tag="write"),
             "python3 bench.py --traffic-from gpurun_out/pmc_fetch/run_counter_collection.csv "
             "gpurun_out/pmc_write/run_counter_collection.csv gpurun_out/pmc.log", "```", "",
             "Calibration: the run's device copy of %d bytes reads %.1f KiB FETCH_SIZE and %.1f KiB WRITE_SIZE, so "
             "the counters are scaled by %.4f and %.4f." % (COPY_BYTES, out["fetch"]["copy_kib"],
                                                             out["write"]["copy_kib"], out["fetch"]["factor"],
                                                             out["write"]["factor"]),
             "", "| routing | n | algorithmic MB | fetched MB (scaled) | written MB (scaled) | fetched / algorithmic |",
             "|---|---|---|---|---|---|"]
    for i, p in enumerate(slot_pass):
        fb, wb = out["fetch"]["bytes"][i], out["write"]["bytes"][i]
        lines.append("| %s | %d | %.1f | %.1f | %.2f | %.3f |" % (p["kind"], p["n"], p["bytes"] / 1e6, fb / 1e6,
                                                                 wb / 1e6, fb / p["bytes"]))
    lines += ["", "Per launch (average over the %d launches): %.1f MB counted, %.1f MB algorithmic." % (
        n, per_launch / 1e6, sum(alg) / n / 1e6)]
    if dedup_pass:
        dout, dper = traffic_from(fetch_csv, write_csv, config, kernel="dedup")
        assert len(dedup_pass) == len(dout["fetch"]["bytes"])
        lines += ["", "The deduplicating kernel on the same passes: U distinct experts, each to be read once "
                  "(algorithmic U w).", "",
                  "| routing | n | U | algorithmic MB | fetched MB (scaled) | written MB (scaled) | "
                  "fetched / algorithmic |", "|---|---|---|---|---|---|---|"]
        for i, p in enumerate(dedup_pass):
            fb, wb = dout["fetch"]["bytes"][i], dout["write"]["bytes"][i]
            lines.append("| %s | %d | %d | %.1f | %.1f | %.2f | %.3f |" % (
                p["kind"], p["n"], p["U"], p["bytes"] / 1e6, fb / 1e6, wb / 1e6, fb / p["bytes"]))
        dalg = sum(p["bytes"] for p in dedup_pass) / len(dedup_pass)
        lines += ["", "Per dedup launch (average over the %d launches): %.1f MB counted, %.1f MB algorithmic." % (
            len(dedup_pass), dper / 1e6, dalg / 1e6)]
        rec["dedup_bytes_per_launch"] = round(dper, 1)
        rec["dedup_algorithmic_bytes_per_launch"] = round(dalg, 1)
    lines += ["", "traffic-json: " + json.dumps(rec)]
    path = os.path.join(out_dir or os.path.join(ROOT, "profiles"), "traffic_k_expert_perslot_%s.md" % config)
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)
    return path


def read_traffic(config):
    """bytes per launch from the committed counter summary, if it is for this kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic_k_expert_perslot_%s.md" % config)
    if not os.path.exists(path):
        return None
    for line in open(path):
        if line.startswith("traffic-json: "):
            rec = json.loads(line[len("traffic-json: "):])
            if rec.get("source_hash") == source_hash():
                return rec["bytes_per_launch"]
    return None


def write_profile_summary(prof_dir, bench_json, config):
    """Short markdown summary of a `rocprofv3 --kernel-trace --stats` run of this bench."""
    import collections
    import re
    trace = [f for f in os.listdir(prof_dir) if f.endswith("kernel_trace.csv")][0]
    stats = [f for f in os.listdir(prof_dir) if f.endswith("kernel_stats.csv")][0]
    d = collections.defaultdict(list)
    for r in _counter_rows(os.path.join(prof_dir, trace)):
        m = re.search(r"(k_\w+)(<[^>]*>)?", r["Kernel_Name"])
        if not m:
            continue
        key = (m.group(1) + (m.group(2) or ""), int(r["Grid_Size_X"]) // int(r["Workgroup_Size_X"]))
        d[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000)
    b = [json.loads(l) for l in open(bench_json) if l.startswith('{"metric"')][-1]
    lines = ["# k_expert (per-slot and deduplicating), %s-shaped layer, n = 1..8, uniform + correlated routing" % config,
             "", "Command (from the repository root, one MI355X):", "", "```", prof_cmd(config), "```", "",
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
    # the per-slot bf16 kernel without shared experts (the last template flag), as timed
    slot = [v for k, vs in d.items() if k[0].startswith("k_expert<true, 0") and k[0].endswith("false>") for v in vs]
    rf = b["roofline"]
    lines += ["", "## Bench line of the same run (HIP events on the launch stream)", "",
              "- value: %.1f GB/s (all passes, both kernels)" % b["value"],
              "- per-slot kernel: avg %.2f us per launch by events, %.2f us by the kernel trace (%d launches, "
              "warm-up included); %.0f algorithmic bytes per launch; achieved %.1f GB/s = %.3f of 8 TB/s" % (
                  rf["avg_launch_us"], sum(slot) / max(len(slot), 1), len(slot), rf["algorithmic_bytes_per_launch"],
                  rf["achieved"], rf["frac"]),
              "- deduplicating kernel: avg %.2f us, achieved %.1f GB/s" % (rf["dedup_kernel"]["avg_launch_us"],
                                                                           rf["dedup_kernel"]["achieved"]),
              "- source hash %s" % b.get("source_hash")]
    path = os.path.join(ROOT, "profiles", "k_expert_%s_n1-8.md" % config)
    open(path, "w").write("\n".join(lines) + "\n")
    print(path)


def dispatch_section(args, efa, layer, ws, ys, passes, kinds, nvals, per_kind, flush, ev, stream):
    """The crossover-driven switch (moe_expert_auto) on held-out windows: the crossover
    comes from the timed windows' measured S(n); the warm-up windows, never used for
    it, are run by both kernels and by the switch, each after the flush."""
    e2 = ev.make(2)
    out = {"workload": "warm-up windows of each routing (not used for the crossover), n = 1..%d" % nvals[-1]}
    held = [s_ for s_ in range(args.warmup)] or [0]
    for kind, _ in kinds:
        c = int(per_kind[kind]["crossover"])
        tot = {"slot": 0.0, "dedup": 0.0, "auto": 0.0, "best": 0.0}
        for n in nvals:
            for s_ in held:
                p = passes[(kind, n, s_)]
                t = {}
                for name, call in (("slot", lambda: efa.expert_perslot(layer, p["x"], p["ids"], p["w"], y=ys[n], ws=ws,
                                                                       stream=stream)),
                                   ("dedup", lambda: efa.expert_dedup(layer, p["x"], p["ids"], p["w"], y=ys[n], ws=ws,
                                                                      stream=stream)),
                                   ("auto", lambda: efa.expert_auto(layer, p["x"], p["ids"], p["w"], c, y=ys[n], ws=ws,
                                                                    stream=stream))):
                    flush()
                    ev.record(e2[0], stream.cuda_stream)
                    call()
                    ev.record(e2[1], stream.cuda_stream)
                    t[name] = ev.ms(e2[0], e2[1]) * 1e3
                for k in ("slot", "dedup", "auto"):
                    tot[k] += t[k]
                tot["best"] += min(t["slot"], t["dedup"])
        out[kind] = {"crossover": c, **{k + "_us_total": round(v, 1) for k, v in tot.items()},
                     "auto_over_best": round(tot["auto"] / tot["best"], 4),
                     "auto_over_slot": round(tot["auto"] / tot["slot"], 4),
                     "auto_over_dedup": round(tot["auto"] / tot["dedup"], 4)}
    return out


def router_section(args, efa, synth, spec, passes, kinds, nvals, flush, ev, stream):
    """The router ahead of the expert operation (two launches: logits, then top-m and
    softmax) on the layer's own activations, after the flush, events around both."""
    import torch
    from synth.device import to_torch
    wr = to_torch(synth.router_weights(spec, args.seed))
    e2 = ev.make(2)
    us = []
    for n in nvals:
        x = passes[(kinds[0][0], n, 0)]["x"]
        out = efa.router_topk(wr, x, spec.m, stream=stream)
        tl = []
        for _ in range(5):
            flush()
            ev.record(e2[0], stream.cuda_stream)
            efa.router_topk(wr, x, spec.m, out=out, stream=stream)
            ev.record(e2[1], stream.cuda_stream)
            tl.append(ev.ms(e2[0], e2[1]) * 1e3)
        us.append(round(float(np.median(tl)), 2))
    nb = spec.N * spec.d * 2
    return {"workload": "router of the layer: logits of N=%d experts over d=%d (bf16), top-%d and softmax, n = 1..%d"
                        % (spec.N, spec.d, spec.m, nvals[-1]),
            "launches": 2, "us_per_n": us, "router_bytes": nb,
            "GBps_per_n": [round((nb + n * spec.d * 2) / (t * 1e-6) / 1e9, 1) for n, t in zip(nvals, us)]}


def chosen_id_section(args, efa, routing, spec, layer, ws, ys, flush, ev, stream, recs, per_kind, x_of):
    """Passes with chosen ids (U distinct experts among n m slots, from heavy
    repetition to none, n = 2..9), the fits of Eq. (4) and Eq. (E.1) through the
    library, the re-read cost c_re/c_u, each fit's median relative error on the
    timed windows of recorded-style routing (epsilon, the larger of the two) and
    the Table 2 factors applied to the measured passes."""
    import torch
    m, N, b = spec.m, spec.N, spec.expert_bytes
    e2 = ev.make(2)
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
                t = {}
                for kname, fn in (("slot", efa.expert_perslot), ("dedup", efa.expert_dedup)):
                    tl = []
                    for _ in range(3):
                        flush()
                        fn(layer, x, ids, w, y=y, ws=ws, stream=stream, events=e2)
                        tl.append(ev.ms(e2[0], e2[1]) * 1e-3)
                    t[kname] = float(np.median(tl))
                rows.append((n, U, t["slot"], t["dedup"]))
    n_c = np.array([r[0] for r in rows]); U_c = np.array([r[1] for r in rows])
    cs = efa.fit_times(efa.MOE_KIND_SLOT, n_c, U_c, m, np.array([r[2] for r in rows]), b)
    cd = efa.fit_times(efa.MOE_KIND_DEDUP, n_c, U_c, m, np.array([r[3] for r in rows]), b)
    # each fit's relative error on the timed windows (n >= 2)
    win = [r for r in recs if r["n"] >= 2]
    nw = np.array([r["n"] for r in win], np.float64); Uw = np.array([r["U"] for r in win], np.float64)
    pred_s = cs[0] + cs[1] * Uw * b + cs[2] * (nw * m - Uw) * b
    pred_d = cd[0] + cd[1] * Uw * b + cd[2] * nw
    meas_s = np.array([r["t_slot_ms"] * 1e-3 for r in win]); meas_d = np.array([r["t_dedup_ms"] * 1e-3 for r in win])
    eps_s = float(np.median(np.abs(pred_s - meas_s) / meas_s))
    eps_d = float(np.median(np.abs(pred_d - meas_d) / meas_d))
    eps = max(eps_s, eps_d)
    out = {"workload": "passes with chosen ids, n = 2..9, U from m to min(n m, N) (6 values), 3 passes each, "
                       "median of 3 timed runs after the flush",
           "passes": [dict(n=int(r[0]), U=int(r[1]), t_slot_us=round(r[2] * 1e6, 2), t_dedup_us=round(r[3] * 1e6, 2))
                      for r in rows],
           "fit_slot": {"t_op_us": cs[0] * 1e6, "c_u_s_per_GB": cs[1] * 1e9, "c_re_s_per_GB": cs[2] * 1e9,
                        "reread_cost": cs[2] / cs[1]},
           "fit_dedup": {"t_op_us": cd[0] * 1e6, "c_g_s_per_GB": cd[1] * 1e9, "c_t_us_per_token": cd[2] * 1e6},
           "eps_slot": eps_s, "eps_dedup": eps_d, "eps": eps, "windows": len(win)}
    if eps < 0.5:
        f = efa.error_bounds(eps)
        out["bounds"] = f
        dec = {}
        for kind, pk in per_kind.items():
            per_n = pk["per_n"]
            rows_k = []
            for row in per_n:
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


A_GRID = [i / 21.0 for i in range(22)]  # acceptance values of the best-draft-length staircase


def step_model_section(efa, spec, rows, shared_us, layers=1):
    """The step-time model fed by the measured times of one routing: E_p(n) is the
    mean requested bytes of a pass, beta_p(n) = E_p(n) / measured kernel time (fixed
    work folded in, phi = 0), D = the shared experts' bytes read once per pass with
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


def per_n_rows(recs, nvals):
    rows = []
    for n in nvals:
        R = [r for r in recs if r["n"] == n]
        bs, bd = sum(r["bytes_slot"] for r in R), sum(r["bytes_dedup"] for r in R)
        ts, td = sum(r["t_slot_ms"] for r in R) / 1e3, sum(r["t_dedup_ms"] for r in R) / 1e3
        gs, gd = bs / ts / 1e9, bd / td / 1e9
        rows.append(dict(n=n, gbps_slot=round(gs, 1), gbps_dedup=round(gd, 1),
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
    """Smallest n >= 2 from which the deduplicating kernel stays faster (0: none)."""
    cross = 0
    for r in reversed(rows):
        if r["n"] < 2 or r["us_slot"] - r["us_dedup"] <= 0:
            break
        cross = r["n"]
    return cross


def strip_bytes(rows):
    return [{k: v for k, v in r.items() if not k.startswith("bytes_")} for r in rows]


def tree_selection(args, efa, routing, spec, layer, x, y, ws, timed, w_exp, ntrees, dedup_fit):
    """The verification subtree of each seeded 32-node tree chosen by reward over
    predicted cycle time (SpecFit Eq. (5), moe_tree_select, K = 7), with the cycle time
    calibrated from the deduplicating kernel's fit on chosen ids (beta = c_g w per
    union expert, b_k = t_op + c_t (k + 1)); the selected tokens are then run through
    the dedup kernel and timed, next to the 7 nodes of highest cumulative
    probability (the plain rule for a 7-node budget)."""
    import torch
    if dedup_fit is None:
        return None
    t_op, c_g, c_t = dedup_fit
    K = 7
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
            t = float(np.median([timed(lambda: efa.expert_dedup(layer, x[:n], ids, w, y=y[:n], ws=ws))
                                 for _ in range(3)])) * 1e-3
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


def extra_configs(args, torch, efa, synth, routing, ev, flush, stream, dedup_fit=None):
    """The other workloads: the Qwen3-30B-A3B-shaped layer 48 times back to back per
    pass (zipf routing), the 32-node draft tree on that layer, and the
    Mixtral-8x7B-shaped layer (uniform and repeat-0.6 routing).  Weights from the
    seeded device generator.  Each pass timed alone after the read flush."""
    from synth.device import device_layer_weights
    out = {}
    e2 = ev.make(2)
    sh = stream.cuda_stream

    def xdev(spec, n, key):
        g = torch.Generator(device="cuda")
        g.manual_seed(key)
        return torch.randn(n, spec.d, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)

    def timed(fn):
        flush()
        ev.record(e2[0], sh)
        fn()
        ev.record(e2[1], sh)
        return ev.ms(e2[0], e2[1])

    # ---- Qwen3-shaped: 48 layers back to back ----
    spec = synth.CONFIGS["qwen3"]
    L = spec.layers
    layers = [load_layout(efa.Layer(*device_layer_weights(spec, args.seed, l), m=spec.m)) for l in range(L)]
    T = 1024
    traces = [routing.make_trace(spec, "zipf", T, seed=args.seed, layer=l, s=1.1) for l in range(L)]
    ws = layers[0].workspace(8)
    w_exp = spec.expert_bytes
    reps = 3
    qrows = []
    recs = []
    lib = efa.lib()
    vp = ctypes.c_void_p
    descs = [l.desc() for l in layers]

    def argsets(n, x, dev, y):  # prebuilt C-ABI arguments, so 48 launches queue faster than they run
        return [(ctypes.byref(descs[l]), ctypes.byref(layers[l]._weights), vp(x.data_ptr()), vp(dev[l][0].data_ptr()),
                 vp(dev[l][1].data_ptr()), n, vp(y.data_ptr()), None, vp(ws.data_ptr()), ws.numel(), vp(sh))
                for l in range(L)]

    def run_all(fn, sets):
        for a in sets:
            assert fn(*a) == 0

    # The same 48 launches also as HIP graphs (one capture per n and kernel over
    # static id / weight buffers that each window is copied into), replayed on the
    # bench stream: the serving form, with no host launch work per layer.
    cap_stream = torch.cuda.Stream()  # default priority
    grecs = []
    for n in range(1, 9):
        starts = routing.window_starts(T, n, reps + 1, seed=args.seed)
        y = torch.empty(n, spec.d, dtype=torch.float32, device="cuda")
        yg = torch.empty(n, spec.d, dtype=torch.float32, device="cuda")
        x = xdev(spec, n, 1000 + n)
        dev = [(torch.zeros(n, spec.m, dtype=torch.int32, device="cuda"),
                torch.zeros(n, spec.m, dtype=torch.float32, device="cuda")) for _ in range(L)]
        sets = argsets(n, x, dev, y)
        graphs = {}
        for rp in range(reps + 1):
            win = [routing.window(traces[l], int(starts[rp]), n) for l in range(L)]
            for (di, dw), (i, w) in zip(dev, win):
                di.copy_(torch.from_numpy(i))
                dw.copy_(torch.from_numpy(w))
            U = [len(set(i.reshape(-1).tolist())) for i, _ in win]
            if not graphs:  # capture on the first window (the kernels' ids are read at run time)
                torch.cuda.synchronize()
                for kname, fn in (("slot", lib.moe_expert_perslot), ("dedup", lib.moe_expert_dedup)):
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g, stream=cap_stream):
                        gsets = [a[:6] + (vp(yg.data_ptr()),) + a[7:10] + (vp(cap_stream.cuda_stream),)
                                 for a in sets]
                        run_all(fn, gsets)
                    graphs[kname] = g
                torch.cuda.synchronize()
            ts = timed(lambda: run_all(lib.moe_expert_perslot, sets))
            tgs = timed(lambda: graphs["slot"].replay())
            assert torch.equal(y, yg), "graph replay differs from the eager launches (per-slot)"
            td = timed(lambda: run_all(lib.moe_expert_dedup, sets))
            tgd = timed(lambda: graphs["dedup"].replay())
            assert torch.equal(y, yg), "graph replay differs from the eager launches (dedup)"
            if rp > 0:
                recs.append(dict(n=n, U=sum(U) / L, bytes_slot=L * n * spec.m * w_exp, bytes_dedup=sum(U) * w_exp,
                                 t_slot_ms=ts, t_dedup_ms=td))
                grecs.append(dict(n=n, slot_eager_us=ts * 1e3, slot_graph_us=tgs * 1e3, dedup_eager_us=td * 1e3,
                                  dedup_graph_us=tgd * 1e3))
        del graphs
    qrows = per_n_rows(recs, range(1, 9))
    out["qwen3_x48"] = {"workload": "qwen3-shaped layer x48 back to back per pass (N=128, m=8, d=2048, d_ff=768, "
                                    "bf16), zipf(s=1.1) routing per layer, %d passes per n" % reps,
                        "per_n": strip_bytes(qrows), "crossover": crossover_of(qrows),
                        "step_model": step_model_section(efa, spec, qrows, [], layers=L),
                        "hip_graph": {"what": "the 48 launches of a pass captured once per n and kernel, replayed "
                                              "after each window is copied into the captured id/weight buffers; "
                                              "us per pass of 48 layers, median of %d windows" % reps,
                                      "per_n": [{k: (round(float(np.median([r[k] for r in grecs if r["n"] == n])), 1)
                                                     if k != "n" else n)
                                                 for k in ("n", "slot_eager_us", "slot_graph_us", "dedup_eager_us",
                                                           "dedup_graph_us")} for n in range(1, 9)]}}

    progress("qwen3 x48 done")
    # ---- 32-node draft tree on one Qwen3-shaped layer ----
    tl = layers[0]
    trecs = []
    ntrees = 32
    y = torch.empty(32, spec.d, dtype=torch.float32, device="cuda")
    ws32 = tl.workspace(32)
    x = xdev(spec, 32, 77)
    for i in range(ntrees + 1):
        _, ttr = routing.tree_routing(spec.N, spec.m, 0.5, routing.rng_for(args.seed, 0, "tree", i))
        ids, w = torch.from_numpy(ttr.ids).cuda(), torch.from_numpy(ttr.w).cuda()
        U = len(set(ttr.ids.reshape(-1).tolist()))
        ts = timed(lambda: efa.expert_perslot(tl, x, ids, w, y=y, ws=ws32, stream=stream))
        td = timed(lambda: efa.expert_dedup(tl, x, ids, w, y=y, ws=ws32, stream=stream))
        if i > 0:
            trecs.append(dict(n=32, U=U, bytes_slot=32 * spec.m * w_exp, bytes_dedup=U * w_exp, t_slot_ms=ts,
                              t_dedup_ms=td))
    trow = per_n_rows(trecs, [32])[0]
    sel = tree_selection(args, efa, routing, spec, tl, x, y, ws32, timed, w_exp, ntrees, dedup_fit)
    out["tree"] = {"workload": "32-node ancestor-closed draft tree (1+1+2+4+8+16, children reuse parent experts "
                               "with p=0.5) on one qwen3-shaped layer, %d seeded trees" % ntrees,
                   **{k: v for k, v in trow.items() if not k.startswith("bytes_")},
                   "bytes_slot": trow["bytes_slot"], "bytes_dedup_mean": trow["bytes_dedup"], "selection": sel}
    del layers, tl
    torch.cuda.empty_cache()

    progress("tree done")
    # ---- Mixtral-shaped ----
    spec = synth.CONFIGS["mixtral"]
    ml = load_layout(efa.Layer(*device_layer_weights(spec, args.seed, 0), m=spec.m))
    wsm = ml.workspace(8)
    w_exp = spec.expert_bytes
    mix = {}
    for kind, kw in (("uniform", {}), ("correlated", {"p": 0.6})):
        tr = routing.make_trace(spec, kind, T, seed=args.seed, **kw)
        mrecs = []
        for n in range(1, 9):
            starts = routing.window_starts(T, n, reps + 1, seed=args.seed + 5)
            y = torch.empty(n, spec.d, dtype=torch.float32, device="cuda")
            x = xdev(spec, n, 2000 + n)
            for rp in range(reps + 1):
                i_h, w_h = routing.window(tr, int(starts[rp]), n)
                ids, w = torch.from_numpy(i_h).cuda(), torch.from_numpy(w_h).cuda()
                ts = timed(lambda: efa.expert_perslot(ml, x, ids, w, y=y, ws=wsm, stream=stream))
                td = timed(lambda: efa.expert_dedup(ml, x, ids, w, y=y, ws=wsm, stream=stream))
                if rp > 0:
                    U = len(set(i_h.reshape(-1).tolist()))
                    mrecs.append(dict(n=n, U=U, bytes_slot=n * spec.m * w_exp, bytes_dedup=U * w_exp, t_slot_ms=ts,
                                      t_dedup_ms=td))
        rows = per_n_rows(mrecs, range(1, 9))
        mix[kind] = {"per_n": strip_bytes(rows), "crossover": crossover_of(rows)}
    out["mixtral"] = {"workload": "mixtral-shaped layer (N=8, m=2, d=4096, d_ff=14336, bf16), %d passes per n" % reps,
                      **mix}
    del ml
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="dsv2lite", choices=["dsv2lite", "qwen3", "mixtral"])
    ap.add_argument("--nmax", type=int, default=8)
    ap.add_argument("--seed", type=int, default=2026)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-scrub", action="store_true")
    ap.add_argument("--details", default="", help="write per-pass records (JSONL) here")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the other workloads (qwen3 x48, draft tree, mixtral) after the headline one")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="for a counter run: one step of per-slot passes (both routings, n=1..nmax), each after "
                         "the 1 GiB read flush, then a 256 MiB device copy; prints what ran")
    ap.add_argument("--traffic-from", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "PASS_LOG"),
                    help="write profiles/traffic_k_expert_perslot_<config>.md from two counter runs (no GPU)")
    ap.add_argument("--profile-summary", nargs=2, metavar=("PROF_DIR", "BENCH_JSON"),
                    help="write profiles/k_expert_<config>_n1-8.md from a kernel-trace run (no GPU)")
    args = ap.parse_args()
    if args.traffic_from:
        write_traffic_summary(args.traffic_from[0], args.traffic_from[1], args.config, args.traffic_from[2])
        return
    if args.profile_summary:
        write_profile_summary(*args.profile_summary, args.config)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the expert operation here runs on a single MI355X and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import expert_ffn_amd as efa
    import synth
    from synth import routing
    from synth.device import to_torch

    torch.cuda.set_device(0)
    spec = synth.CONFIGS[args.config]
    kinds = {"dsv2lite": [("uniform", {}), ("correlated", {"p": 0.5})],
             "qwen3": [("zipf", {"s": 1.1})],
             "mixtral": [("uniform", {}), ("correlated", {"p": 0.6})]}[args.config]
    T = 4096
    t_setup = time.perf_counter()
    host_w = synth.layer_weights(spec, args.seed)
    # weights in the tiled layout (moe_pack_tiled), done once at weight-load time
    layer = load_layout(efa.Layer(*(to_torch(a) for a in host_w), m=spec.m))
    progress("%s layer on the device (%.1f s)" % (args.config, time.perf_counter() - t_setup))
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    nsteps_total = args.warmup + args.steps
    nvals = list(range(1, args.nmax + 1))

    # inputs resident in HBM before timing: one window per (kind, n, step)
    passes = {}
    host_passes = []
    for ki, (kind, kw) in enumerate(kinds):
        tr = routing.make_trace(spec, kind, T, seed=args.seed, **kw)
        for n in nvals:
            starts = routing.window_starts(T, n, nsteps_total, seed=args.seed + 17 * ki)
            for s in range(nsteps_total):
                ids, w = routing.window(tr, int(starts[s]), n)
                x_h = synth.pass_x(spec, args.seed, 0, 10000 * ki + 100 * n + s, n)
                dev = (to_torch(x_h), torch.from_numpy(ids).cuda(), torch.from_numpy(w).cuda())
                passes[(kind, n, s)] = dict(x=dev[0], ids=dev[1], w=dev[2], ids_h=ids,
                                            U=len(set(ids.reshape(-1).tolist())))
                if s < HOST_WINDOWS:
                    host_passes.append(((s, ki, n), (x_h, ids, w)))
    # the oracle's sample: window by window, each over both routings and every n
    host_passes = [p for _, p in sorted(host_passes, key=lambda e: e[0])]
    ws = layer.workspace(nvals[-1])  # zero-filled once; serves every n
    ys = {n: torch.empty(n, spec.d, dtype=torch.float32, device="cuda") for n in nvals}
    scrub = torch.ones(SCRUB_BYTES // 4, dtype=torch.float32, device="cuda")
    scrub_out = torch.empty((), dtype=torch.float32, device="cuda")

    def flush():
        torch.sum(scrub, dim=0, out=scrub_out)  # reads 1 GiB, writes 4 bytes
    info = torch.zeros(3, dtype=torch.int32, device="cuda")
    ev = HipEvents()
    nk = efa.kernels_per_call(efa.MOE_KIND_SLOT)
    assert nk == 1 and efa.kernels_per_call(efa.MOE_KIND_DEDUP) == 1
    ev_slot = ev.make(2)
    ev_dedup = ev.make(2)
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup

    w_exp = spec.expert_bytes
    recs = []

    def run_step(s, record):
        for kind, _ in kinds:
            for n in nvals:
                p = passes[(kind, n, s)]
                if not args.no_scrub:
                    flush()
                efa.expert_perslot(layer, p["x"], p["ids"], p["w"], y=ys[n], ws=ws, stream=stream, events=ev_slot)
                t_slot = ev.ms(ev_slot[0], ev_slot[1])
                if not args.no_scrub:
                    flush()
                efa.expert_dedup(layer, p["x"], p["ids"], p["w"], y=ys[n], ws=ws, info=info, stream=stream,
                                 events=ev_dedup)
                t_dedup = ev.ms(ev_dedup[0], ev_dedup[1])
                if record:
                    recs.append(dict(kind=kind, n=n, step=s, U=p["U"], bytes_slot=n * spec.m * w_exp,
                                     bytes_dedup=p["U"] * w_exp, t_slot_ms=t_slot, t_dedup_ms=t_dedup))

    if args.pmc_pass:
        # Counter run: the flush (a plain read of SCRUB_BYTES) and a device copy
        # (COPY_BYTES read and written) calibrate FETCH_SIZE and WRITE_SIZE; the
        # per-slot launches in between are the ones the bench times.
        # (then the deduplicating kernel on the same passes: it reads each of the U
        # distinct experts once)
        order = []
        for kname, fn in (("slot", efa.expert_perslot), ("dedup", efa.expert_dedup)):
            for kind, _ in kinds:
                for n in nvals:
                    p = passes[(kind, n, args.warmup)]
                    U = len(set(p["ids"].cpu().numpy().ravel().tolist()))
                    flush()
                    fn(layer, p["x"], p["ids"], p["w"], y=ys[n], ws=ws, stream=stream)
                    order.append(dict(kernel=kname, kind=kind, n=n, U=U,
                                      bytes=(n * spec.m if kname == "slot" else U) * w_exp))
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_pass": order, "flush_read_bytes": SCRUB_BYTES, "copy_bytes": COPY_BYTES,
                          "source_hash": source_hash()}))
        return

    for s in range(args.warmup):
        run_step(s, False)
    torch.cuda.synchronize()
    progress("%d warm-up steps done" % args.warmup)
    t_wall = time.perf_counter()
    for s in range(args.warmup, nsteps_total):
        run_step(s, True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    progress("%d timed steps done (%.3f s)" % (args.steps, wall))

    # the shared experts' pass (read once per pass whatever the routing): D(n) of the step model
    shared_us = []
    if spec.n_shared:
        sh_host = synth.layer_weights(spec, args.seed, shared=True)
        shl = load_layout(efa.Layer(*(to_torch(a) for a in sh_host), m=spec.n_shared))
        sws = shl.workspace(nvals[-1])
        e2 = ev.make(2)
        for n in nvals:
            sids = torch.arange(spec.n_shared, dtype=torch.int32, device="cuda").repeat(n, 1).contiguous()
            sw = torch.ones(n, spec.n_shared, dtype=torch.float32, device="cuda")
            x = passes[(kinds[0][0], n, 0)]["x"]
            tl = []
            for rep in range(4):
                flush()
                efa.expert_dedup(shl, x, sids, sw, y=ys[n], ws=sws, stream=stream, events=e2)
                tl.append(ev.ms(e2[0], e2[1]) * 1e3)
            shared_us.append(sorted(tl[1:])[1])
        # the same experts computed in the routed call itself (one launch): routed
        # alone and routed + shared on the same windows, paired, both kernels
        fl = efa.Layer(layer.w_gate, layer.w_up, layer.w_down, m=spec.m, packed=layer.packed, tiled=layer.tiled,
                       shared=(shl.w_gate, shl.w_up, shl.w_down))
        fws = fl.workspace(nvals[-1])
        fused = {"routed_slot": [], "fused_slot": [], "routed_dedup": [], "fused_dedup": []}
        for n in nvals:
            for kname, fn in (("slot", efa.expert_perslot), ("dedup", efa.expert_dedup)):
                tr_, tf_ = [], []
                for s_ in range(min(4, nsteps_total)):
                    p = passes[(kinds[0][0], n, s_)]
                    flush()
                    fn(layer, p["x"], p["ids"], p["w"], y=ys[n], ws=ws, stream=stream, events=e2)
                    tr_.append(ev.ms(e2[0], e2[1]) * 1e3)
                    flush()
                    fn(fl, p["x"], p["ids"], p["w"], y=ys[n], ws=fws, stream=stream, events=e2)
                    tf_.append(ev.ms(e2[0], e2[1]) * 1e3)
                fused["routed_" + kname].append(round(float(np.median(tr_)), 2))
                fused["fused_" + kname].append(round(float(np.median(tf_)), 2))
        del shl, fl, fws

    # aggregate (bytes and times summed over the timed passes)
    per_kind = {}
    for kind, _ in kinds:
        rows = per_n_rows([r for r in recs if r["kind"] == kind], nvals)
        per_kind[kind] = dict(per_n=strip_bytes(rows), crossover=crossover_of(rows),
                              step_model=step_model_section(efa, spec, rows, shared_us))
        if spec.n_shared:
            # D/beta_D from the time the shared experts add to the routed launch
            marg = [f - r for k in ("slot", "dedup") for f, r in zip(fused["fused_" + k], fused["routed_" + k])]
            per_kind[kind]["step_model_shared_in_call"] = step_model_section(
                efa, spec, rows, [max(sum(marg) / len(marg), 1e-3)])

    tot_bytes = sum(r["bytes_slot"] + r["bytes_dedup"] for r in recs)
    tot_s = sum(r["t_slot_ms"] + r["t_dedup_ms"] for r in recs) / 1e3
    value = tot_bytes / tot_s / 1e9
    ms_per_step = tot_s * 1e3 / args.steps

    # dominant kernel: the per-slot launch (one fused kernel per pass)
    n_launch = len(recs)
    slot_bytes = sum(r["bytes_slot"] for r in recs)
    slot_s = sum(r["t_slot_ms"] for r in recs) / 1e3
    dd_bytes = sum(r["bytes_dedup"] for r in recs)
    dd_s = sum(r["t_dedup_ms"] for r in recs) / 1e3
    achieved = slot_bytes / slot_s / 1e9
    traffic = read_traffic(args.config)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic,
                "kernel": "k_expert<bf16, per-slot> (whole operation, one launch)", "launches": n_launch,
                "avg_launch_us": round(slot_s / n_launch * 1e6, 3),
                "algorithmic_bytes_per_launch": round(slot_bytes / n_launch, 1),
                "dedup_kernel": {"achieved": round(dd_bytes / dd_s / 1e9, 1),
                                 "avg_launch_us": round(dd_s / n_launch * 1e6, 3),
                                 "algorithmic_bytes_per_launch": round(dd_bytes / n_launch, 1)}}

    cpu = cpu_baseline(spec, host_w, host_passes, args.cpu_budget)
    progress("cpu baseline done")
    extras = {}
    if not args.no_extras and args.config == "dsv2lite":
        ws9 = layer.workspace(9)
        extras["router"] = router_section(args, efa, synth, spec, passes, kinds, nvals, flush, ev, stream)
        progress("router done")
        extras["dispatch"] = dispatch_section(args, efa, layer, ws, ys, passes, kinds, nvals, per_kind, flush, ev,
                                              stream)
        progress("dispatch done")
        extras["chosen_ids"] = chosen_id_section(
            args, efa, routing, spec, layer, ws9, ys, flush, ev, stream, recs, per_kind,
            lambda n: to_torch(synth.pass_x(spec, args.seed, 0, 77000 + n, n)))
        progress("chosen-id fits done")
        del ws9
    if spec.n_shared:
        extras["shared_experts"] = {"workload": "%d always-on shared experts, weight 1, every token: one "
                                                "deduplicating call per pass (the D(n) bytes of the step model)"
                                                % spec.n_shared, "us_per_n": [round(v, 2) for v in shared_us],
                                    "bytes": spec.n_shared * spec.expert_bytes,
                                    "in_call": dict(workload="the same experts computed in the routed launch "
                                                             "(desc n_shared); routed alone vs routed + shared, "
                                                             "paired on %s windows, median of 4" % kinds[0][0],
                                                    **{k + "_us": v for k, v in fused.items()})}
    if not args.no_extras and args.config == "dsv2lite":
        del passes, layer
        torch.cuda.empty_cache()
        fit = extras.get("chosen_ids", {}).get("fit_dedup")
        dfit = None if fit is None else (fit["t_op_us"] * 1e-6, fit["c_g_s_per_GB"] * 1e-9,
                                         fit["c_t_us_per_token"] * 1e-6)
        extras.update(extra_configs(args, torch, efa, synth, routing, ev, flush, stream, dedup_fit=dfit))

    out = {"metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "%s-shaped MoE layer expert op, n=1..%d, routing %s" % (
               args.config, nvals[-1], "+".join(k for k, _ in kinds)),
               "N": spec.N, "m": spec.m, "d_model": spec.d, "d_ff": spec.d_ff, "weight_layout": WEIGHT_LAYOUT,
               "passes_per_step": len(kinds) * len(nvals) * 2,
               "launches_per_pass": {"slot": efa.kernels_per_call(efa.MOE_KIND_SLOT),
                                     "dedup": efa.kernels_per_call(efa.MOE_KIND_DEDUP)},
               "scrub_bytes": 0 if args.no_scrub else SCRUB_BYTES},
           "roofline": roofline, "cpu_baseline": cpu, "results": per_kind, "extras": extras,
           "wall_s_timed": round(wall, 3), "setup_s": round(setup_s, 1), "source_hash": source_hash()}
    if args.details:
        with open(args.details, "w") as f:
            for r in recs:
                f.write(json.dumps(r) + "\n")
    print(json.dumps(out))


if __name__ == "__main__":
    main()
