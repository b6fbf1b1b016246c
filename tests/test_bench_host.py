"""The bench's counter bookkeeping on the host (no GPU): FETCH_SIZE / WRITE_SIZE rows of
a counter run are calibrated by the run's device copy, split by kernel (per-slot,
deduplicating) and averaged per launch; the summary file carries the per-launch
figures and the kernel source hash."""
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
    out, per_launch = bench.traffic_from(fp, wp, "dsv2lite")
    assert abs(out["fetch"]["factor"] - 2.0) < 1e-12 and abs(out["write"]["factor"] - 1.0) < 1e-12
    assert out["fetch"]["bytes"] == [1000 * 1024 * 2.0, 3000 * 1024 * 2.0]
    assert per_launch == ((1000 + 3000) * 2 + (4 + 8)) * 1024 / 2
    dout, dper = bench.traffic_from(fp, wp, "dsv2lite", kernel="dedup")
    assert dout["fetch"]["bytes"] == [500 * 1024 * 2.0] and dper == (500 * 2 + 2) * 1024


def test_traffic_summary_records_per_launch_figures(tmp_path):
    fp, wp = _runs(tmp_path)
    passes = [dict(kernel="slot", kind="uniform", n=1, U=6, bytes=2_000_000),
              dict(kernel="slot", kind="uniform", n=2, U=11, bytes=6_000_000),
              dict(kernel="dedup", kind="uniform", n=2, U=11, bytes=1_000_000)]
    log = tmp_path / "pmc.log"
    log.write_text("noise\n" + json.dumps({"pmc_pass": passes, "source_hash": "abc"}) + "\n")
    path = bench.write_traffic_summary(fp, wp, "dsv2lite", str(log), out_dir=str(tmp_path))
    rec = json.loads([l for l in open(path) if l.startswith("traffic-json: ")][0][len("traffic-json: "):])
    assert rec["source_hash"] == "abc" and rec["launches"] == 2
    assert rec["bytes_per_launch"] == ((1000 + 3000) * 2 + (4 + 8)) * 1024 / 2
    assert rec["algorithmic_bytes_per_launch"] == 4_000_000
    assert rec["dedup_bytes_per_launch"] == (500 * 2 + 2) * 1024
    assert rec["dedup_algorithmic_bytes_per_launch"] == 1_000_000


def test_cpu_baseline_one_thread_and_all_cores():
    """The oracle timing: one thread, then the same passes on a thread pool; the record
    carries both rates, the thread count and the CPU model, and the pooled results are
    bitwise those of one thread (a mismatch raises)."""
    import synth
    from synth import routing
    spec = synth.layer_spec("tiny", N=8, m=2, d=64, d_ff=128, dtype="bf16")
    W = synth.layer_weights(spec, 5)
    passes = []
    for p, n in enumerate((1, 3, 5, 8)):
        tr = routing.uniform_trace(8, 2, n, routing.rng_for(5, 0, "uniform", p))
        passes.append((synth.pass_x(spec, 5, 0, p, n), tr.ids, tr.w))
    rec = bench.cpu_baseline(spec, W[:3], passes, 60.0, max_threads=4)
    assert rec["kind"] == "oracle" and rec["cores"] == 1 and rec["value"] > 0
    assert rec["sample"].startswith("4 passes")
    ac = rec["all_cores"]
    assert ac["bitwise_equal_to_one_thread"] is True
    assert 1 <= ac["cores"] <= 4 and ac["value"] > 0
    assert isinstance(rec["cpu"], str) and rec["cpu"]


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
