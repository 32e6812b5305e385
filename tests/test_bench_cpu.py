"""Host logic of bench.py: the counter summary and the traffic it feeds to the roofline."""

import csv

import bench


def _write_counters(path, counter, rows):
    cols = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        for i, (name, v) in enumerate(rows, 1):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def _k(name):
    return f"gqa::(anonymous namespace)::{name}(gqa::(anonymous namespace)::Params)"


def test_summarize_counters_scales_and_assigns_workloads(tmp_path, monkeypatch):
    copy = "__amd_rocclr_copyBuffer"
    # 1 MiB calibration; FETCH reads half the true size (scale 2), WRITE the true size (scale 1)
    per = bench.calls_per_workload(steps=1, warmup=1)  # warm-up, timed and profiled call
    fetch = [(copy, 512.0)] * 3 + [(_k("prefill_causal_fwd"), 100.0), (_k("prefill_merge"), 10.0)] * per
    for s in range(3):
        fetch += [(_k("paged_prepass"), 1.0), (_k("paged_fwd"), 20.0 + s)] * per
    for q in range(len(bench.VERIFY_QUERIES)):
        fetch += [(_k("verify_fwd"), 30.0 + q), (_k("verify_merge"), 3.0)] * per
    write = [(n, 2 * v if n == copy else v / 2) for n, v in fetch]
    _write_counters(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write_counters(tmp_path / "w.csv", "WRITE_SIZE", write)
    text = bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), steps=1, warmup=1,
                                    calib_mib=1, n_kv=128000)
    table = tmp_path / "t.md"
    table.write_text(text)
    monkeypatch.setattr(bench, "TRAFFIC_TABLE", str(table))
    t = bench.recorded_traffic()
    assert t[("prefill_causal_fwd", bench.prefill_workload(128000))] == (100 * 2 + 50) * 1024
    for s, sel in enumerate(bench.PAGED_SELECTIONS):
        assert t[("paged_fwd", bench.paged_workload(sel))] == ((20 + s) * 2 + (20 + s) / 2) * 1024
    for q, nq in enumerate(bench.VERIFY_QUERIES):
        assert t[("verify_fwd", bench.verify_workload(nq))] == ((30 + q) * 2 + (30 + q) / 2) * 1024


def test_recorded_traffic_is_dropped_when_sources_change(tmp_path, monkeypatch):
    table = tmp_path / "t.md"
    row = "| `prefill_causal_fwd` | `w` | 3 | 1.0 | 1.0 | 3,072 |\n"
    table.write_text(f"kernel source digest: `{bench.kernel_source_digest()}`\n\n" + row)
    monkeypatch.setattr(bench, "TRAFFIC_TABLE", str(table))
    assert bench.recorded_traffic() == {("prefill_causal_fwd", "w"): 3072}
    table.write_text("kernel source digest: `0000000000000000`\n\n" + row)
    assert bench.recorded_traffic() == {}


def test_committed_traffic_table_parses():
    # whether or not it is current, the committed table must be readable
    with open(bench.TRAFFIC_TABLE) as f:
        assert "kernel source digest:" in f.read()


def test_summarize_sweep_trace_assigns_points_in_order(tmp_path):
    """Dispatch i of a kernel belongs to sweep point i // calls_per_workload; only the calls after the
    warm-up (timed and profiled passes) are averaged."""
    import workloads

    points = (workloads.LONG_40K,) + workloads.SWEEP
    warmup, steps = 1, 2
    cols = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
    path = tmp_path / "trace.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=cols)
        w.writeheader()
        t = 0
        for i in range(len(points)):
            for j in range(bench.calls_per_workload(steps, warmup)):
                fwd = 10**9 if j < warmup else (i + 1) * 10**6 + j  # warm-up calls are slow and must be ignored
                w.writerow({"Kernel_Name": _k("prefill_causal_fwd"), "Start_Timestamp": t, "End_Timestamp": t + fwd})
                t += fwd
                w.writerow({"Kernel_Name": _k("prefill_merge"), "Start_Timestamp": t, "End_Timestamp": t + 30000})
                t += 30000
    rows = bench.summarize_sweep_trace(str(path), steps=steps, warmup=warmup).splitlines()[2:]
    assert len(rows) == len(points)
    for i, (cfg, row) in enumerate(zip(points, rows)):
        cells = [c.strip() for c in row.strip("|").split("|")]
        assert int(cells[0]) == cfg.n_kv
        assert float(cells[3]) == round(((i + 1) * 10**6 + 2.5) / 1e6, 4)  # mean of j = 1 .. 4
        assert float(cells[7]) == 30.0
