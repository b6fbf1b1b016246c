"""The bench's host-side bookkeeping (no GPU).

* Counters: FETCH_SIZE / WRITE_SIZE rows of a counter run are calibrated by the run's
  device copy, split by kernel (per-slot, deduplicating) and averaged per launch; the
  summary file carries the per-launch figures and the kernel source hash.
* Aggregation (Lan Section 2, Table 1 caption): beta, r and u from bytes and times
  summed over windows; the crossover as the smallest n from which the saving stays
  positive; both against records computed by hand.
* The final line: compact (a few KB), with the fields the metric needs.
* Launch gaps from a kernel trace: idle time between back-to-back launches of one
  expert kernel, against a hand-made trace.
"""
import csv
import json

import bench

SLOT = "void moe_k::k_expert<true, 0, 1, 2, true, 1, 2, false>(moe_k::Args)"
DEDUP = "void moe_k::k_expert<true, 1, 1, 2, true, 1, 2, false>(moe_k::Args)"
COPY = "__amd_rocclr_copyBuffer"


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Value": value})


def _runs(tmp_path):
    kib = bench.COPY_BYTES / 1024.0
    # the copy reads half its bytes in FETCH_SIZE (factor 2) and all in WRITE_SIZE (factor 1);
    # a smaller copy earlier in the run must not be taken for the calibration
    fetch = [(COPY, 10.0), (SLOT, 1000.0), (SLOT, 3000.0), (DEDUP, 500.0), (COPY, kib / 2)]
    write = [(COPY, 10.0), (SLOT, 4.0), (SLOT, 8.0), (DEDUP, 2.0), (COPY, kib)]
    fp, wp = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _csv(fp, fetch)
    _csv(wp, write)
    return str(fp), str(wp)


def test_traffic_is_calibrated_and_split_by_kernel(tmp_path):
    fp, wp = _runs(tmp_path)
    out, per_launch = bench.traffic_from(fp, wp)
    assert abs(out["fetch"]["factor"] - 2.0) < 1e-12 and abs(out["write"]["factor"] - 1.0) < 1e-12
    assert out["fetch"]["bytes"] == [1000 * 1024 * 2.0, 3000 * 1024 * 2.0]
    assert per_launch == ((1000 + 3000) * 2 + (4 + 8)) * 1024 / 2
    dout, dper = bench.traffic_from(fp, wp, kernel="dedup")
    assert dout["fetch"]["bytes"] == [500 * 1024 * 2.0] and dper == (500 * 2 + 2) * 1024


def test_traffic_summary_records_per_launch_figures(tmp_path):
    fp, wp = _runs(tmp_path)
    passes = [dict(workload="qwen3x48", kernel="slot", n=1, layer=0, U=8, bytes=2_000_000),
              dict(workload="tree", kernel="slot", n=32, layer=0, U=15, bytes=6_000_000),
              dict(workload="qwen3x48", kernel="dedup", n=1, layer=0, U=8, bytes=1_000_000)]
    log = tmp_path / "pmc.log"
    log.write_text("noise\n" + json.dumps({"pmc_pass": passes, "source_hash": "abc"}) + "\n")
    path = bench.write_traffic_summary(fp, wp, str(log), out_dir=str(tmp_path))
    rec = json.loads([l for l in open(path) if l.startswith("traffic-json: ")][0][len("traffic-json: "):])
    assert rec["source_hash"] == "abc"
    q, t = rec["per_launch"]["qwen3x48"], rec["per_launch"]["tree"]
    assert q["slot"]["launches"] == 1 and t["slot"]["launches"] == 1 and q["dedup"]["launches"] == 1
    assert q["slot"]["bytes"] == (1000 * 2 + 4) * 1024 and t["slot"]["bytes"] == (3000 * 2 + 8) * 1024
    assert q["slot"]["algorithmic"] == 2_000_000 and q["slot"]["fetched_over_algorithmic"] == round(
        1000 * 2 * 1024 / 2_000_000, 4)
    assert q["dedup"]["bytes"] == (500 * 2 + 2) * 1024 and q["dedup"]["algorithmic"] == 1_000_000
    assert "tree" in open(path).read()


def test_cpu_baseline_one_thread_and_all_cores():
    """The oracle timing: one thread, then the same passes on a thread pool; the record
    carries both rates, the thread count, nproc and the CPU model, and the pooled results
    are bitwise those of one thread (a mismatch raises)."""
    import synth
    from synth import routing
    spec = synth.layer_spec("tiny", N=8, m=2, d=64, d_ff=128, dtype="bf16")
    W = synth.layer_weights(spec, 5)
    passes = []
    for p, n in enumerate((1, 3, 5, 8)):
        tr = routing.uniform_trace(8, 2, n, routing.rng_for(5, 0, "uniform", p))
        passes.append((W, synth.pass_x(spec, 5, 0, p, n), tr.ids, tr.w, "bf16", n * 2 * spec.expert_bytes))
    rec = bench.cpu_baseline(passes, 60.0, max_threads=4)
    assert rec["kind"] == "oracle" and rec["value"] > 0 and rec["unit"] == "GB/s"
    assert rec["sample"].startswith("4 passes")
    assert rec["bitwise_equal_to_one_thread"] is True
    assert 1 <= rec["cores"] <= 4 and rec["one_thread"]["value"] > 0
    assert rec["nproc"] >= 1 and isinstance(rec["cpu"], str) and rec["cpu"]


def _rec(n, U, ts_us, td_us, m=8, w=100_000):
    return dict(n=n, U=U, bytes_slot=n * m * w, bytes_dedup=U * w, t_slot_ms=ts_us / 1e3, t_dedup_ms=td_us / 1e3)


def test_per_n_rows_sums_bytes_and_times():
    """beta_p = summed bytes / summed times over the windows of one n; r = beta_dedup /
    beta_slot; u = E_dedup / E_slot; quartiles over the windows' times (by hand)."""
    recs = [_rec(2, 10, 2.0, 1.0), _rec(2, 14, 4.0, 3.0), _rec(2, 12, 3.0, 5.0), _rec(1, 8, 1.0, 1.25)]
    rows = bench.per_n_rows(recs, [1, 2])
    r1, r2 = rows
    # n = 1: 800 kB in 1 us per-slot (800 GB/s), 800 kB in 1.25 us dedup (640 GB/s)
    assert r1["windows"] == 1 and r1["gbps_slot"] == 800.0 and r1["gbps_dedup"] == 640.0
    assert r1["r"] == 0.8 and r1["u"] == 1.0 and r1["frac_slot"] == 0.1
    # n = 2: per-slot 3 x 1.6 MB in 9 us, dedup (1.0 + 1.4 + 1.2) MB in 9 us
    assert r2["windows"] == 3 and r2["bytes_slot"] == 1_600_000 and r2["bytes_dedup"] == 1_200_000
    assert r2["gbps_slot"] == round(4.8e6 / 9e-6 / 1e9, 1) and r2["gbps_dedup"] == 400.0
    assert r2["r"] == 0.75 and r2["u"] == 0.75
    assert r2["us_slot"] == 3.0 and r2["us_dedup"] == 3.0 and r2["mean_U"] == 12.0
    assert (r2["q1_us_slot"], r2["median_us_slot"], r2["q3_us_slot"]) == (2.5, 3.0, 3.5)
    assert (r2["q1_us_dedup"], r2["median_us_dedup"], r2["q3_us_dedup"]) == (2.0, 3.0, 4.0)


def test_crossover_is_where_the_saving_stays_positive():
    def rows(S):  # S[n] = t_slot - t_dedup for n = 1..len(S)
        return [dict(n=i + 1, us_slot=10.0 + s, us_dedup=10.0) for i, s in enumerate(S)]
    assert bench.crossover_of(rows([0, -1, 2, 3, 1])) == 3
    assert bench.crossover_of(rows([0, 1, 2, 3])) == 2
    assert bench.crossover_of(rows([5, 1, -2, 3, 0])) == 0     # S(5) = 0 is not a saving
    assert bench.crossover_of(rows([5, 1, 2, -1, 3])) == 5
    assert bench.crossover_of(rows([-1])) == 0                  # n = 1 alone has no crossover


def test_headline_line_is_compact_and_complete():
    """The final stdout line: at most 4 KB, with value = summed bytes / summed times over
    both kernels, ms_per_step = summed times / steps, the roofline of the kernel with the
    most time (its per-n and n = 1 fractions for both kernels) and the oracle baseline."""
    import argparse
    recs = [_rec(n, 8 + 3 * (n - 1), 20.0 * n, 12.0 * n + 10, m=8, w=9_437_184 * 48) for n in range(1, 9)
            for _ in range(20)]
    rows = bench.per_n_rows(recs, list(range(1, 9)))
    head = {"recs": recs, "rows": rows, "crossover": bench.crossover_of(rows),
            "step_model": {"kstar_slot": [0] * 22, "kstar_dedup": [1] * 22, "crossover_model": 2}}
    pk = {"uniform": {"per_n": rows, "crossover": 5}, "correlated": {"per_n": rows, "crossover": 2}}
    others = {("dsv2lite_" + k): v for k, v in bench.other_summary(pk).items()}
    others.update({("mixtral_" + k): v for k, v in bench.other_summary(pk).items()})
    others["tree"] = {"r": 0.6, "u": 0.33, "U": 85.2, "us_slot": 330.0, "us_dedup": 180.0, "frac": [0.9, 0.6]}
    cpu = {"value": 55.1, "unit": "GB/s", "cores": 16, "kind": "oracle", "sample": "x" * 300,
           "one_thread": {"value": 4.3, "seconds": 12.0}, "nproc": 256, "affinity": 16, "cpu": "some cpu model name",
           "seconds": 1.0, "bitwise_equal_to_one_thread": True}
    args = argparse.Namespace(steps=20, warmup=5, reps=3, no_scrub=False)
    line = bench.headline_line(args, head, others, cpu, list(range(1, 9)), 48, "gpurun_out/bench_full.json")
    text = json.dumps(line, separators=(",", ":"))
    assert len(text) <= 4096, len(text)
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
              "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in line, k
    tb = sum(r["bytes_slot"] + r["bytes_dedup"] for r in recs)
    ts = sum(r["t_slot_ms"] + r["t_dedup_ms"] for r in recs) / 1e3
    assert line["value"] == round(tb / ts / 1e9, 1) and line["ms_per_step"] == round(ts * 1e3 / 20, 4)
    rf = line["roofline"]
    assert rf["bound"] == "hbm" and rf["peak"] == 8000.0 and rf["unit"] == "GB/s"
    assert "per-slot" in rf["kernel"]  # the per-slot kernel has the more time here
    sb = sum(r["bytes_slot"] for r in recs) / (len(recs) * 48)
    st = sum(r["t_slot_ms"] for r in recs) / 1e3 / (len(recs) * 48)
    assert rf["achieved"] == round(sb / st / 1e9, 1) and rf["frac"] == round(sb / st / 1e9 / 8000.0, 4)
    assert rf["frac_n1_slot"] == rows[0]["frac_slot"] and rf["frac_n1_dedup"] == rows[0]["frac_dedup"]
    assert len(rf["frac_per_n_slot"]) == 8 and len(line["per_n"]["r"]) == 8
    assert line["cpu_baseline"]["kind"] == "oracle" and line["config"]["windows_per_n"] == 20


def test_bench_refuses_more_than_one_gpu():
    """One GPU is measured: --gpus above 1 exits with status 2 and says why, before any
    device work."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert p.returncode == 2
    assert "one GPU" in p.stderr and p.stdout == ""


def test_launch_gaps_between_back_to_back_expert_launches():
    """Gaps count only between adjacent launches of the same expert kernel, in start
    order; another kernel in between (the flush) breaks the run."""
    a = "void moe_k::k_expert<true, 0, 1, 2, true, 4, 2, false>(moe_k::Args)"
    b = "void moe_k::k_expert<true, 1, 1, 2, true, 4, 2, false>(moe_k::Args)"
    flush = "void at::native::reduce_kernel<512, 1>(...)"
    disp = [(100, 200, a), (210, 300, a), (330, 400, a),   # gaps 10 and 30; busy 90 + 70
            (400, 900, flush),
            (905, 1000, a),                                # after the flush: no gap counted
            (1000, 1100, b), (1100, 1150, b)]              # gap 0; busy 50
    g = bench.launch_gaps(list(reversed(disp)))            # (any input order)
    ka, kb = "k_expert<true, 0, 1, 2, true, 4, 2, false>", "k_expert<true, 1, 1, 2, true, 4, 2, false>"
    assert g == {ka: (2, 40, 160), kb: (1, 0, 50)}
