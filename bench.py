#!/usr/bin/env python3
"""Benchmark of libgqa on one MI355X.

Default workload: dense causal GQA prefill, Q = 8000 query rows at positions
120000..127999 of KV = 128000 keys, Hq = 6 query heads sharing Hkv = 1 K/V
head, D = 256, scale 1/16, fp16 in / fp16 out with fp32 accumulation, seeded
N(0,1) synthetic inputs resident in HBM.  One step is one gqa_prefill_causal
call (main kernel + log-sum-exp merge).  The metric is algorithmic TFLOP/s:
4 * D * Hq * (visible query-key pairs) per step over the measured step time.

Every workload runs W warm-up calls, then K timed calls with the library's
profiling off (the step time), then K more calls with it on (the main
kernel's time from HIP events, and the shader clock): recording the events
costs a few microseconds per call, which stays out of the step time.

Prints ONE JSON line.  Besides the driver's fields it carries
  roofline      the dominant kernel's achieved TFLOP/s (algorithmic FLOPs per
                launch / its average duration, timed with HIP events recorded
                by the library around that kernel on its stream) against the
                fp16 dense matrix-core peak; also the average shader clock those
                launches ran at (sampled by the kernel while profiling) and the
                fraction of the peak rescaled to that clock;
  cpu_baseline  the fp64 oracle timed on this host's cores for a bounded sample
                of query rows of the same workload, in the same unit;
  paths         the same measurement for the other workloads: the tiny causal
                prefill (Q = 256, KV = 1024), the KV = 40000 long prefill and the
                other points of the key sweep (48000..120000), the paged
                block-sparse prefill (S = 64/512/2048), the paged dense causal
                prefill (every block selected, pages of 16 and 784 tokens), the
                FP8 verifier tail (q = 2/4/8) and the varlen causal prefill of
                a chunked-prefill batch.

`roofline.traffic` is the HBM traffic per launch of that kernel, read from the
committed counter summary (profiles/hbm_traffic_per_launch.md) when the kernel
sources still hash to the digest recorded there, else null.  That summary is
written by `python bench.py --summarize-counters FETCH.csv WRITE.csv` from two
rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of
`bench.py --steps S --warmup W --no-cpu-baseline --copy-calibration-mib M`.

With --tiny it instead prints one such line for the tiny workload (Q = 256 at
positions 768..1023 of KV = 1024, launch-bound at this size).
With --sweep it instead prints one JSON line per point of the long-prefill
key sweep (Q = 8000 at the last positions of KV = 40000, 48000, ..., 128000),
each with the step time, the main kernel's time, TFLOP/s and fraction of the
fp16 peak, and the shader clock; the default single line is not printed then.

Usage: python bench.py [--gpus 1] [--steps K (50)] [--warmup W (20)] [--no-cpu-baseline] [--sweep]
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import re
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

PEAK_F16_TFLOPS = 2516.6  # 256 CUs x 2.4 GHz x 4096 dense fp16 FLOP/clk/CU
PEAK_CLOCK_MHZ = 2400.0
PEAK_HBM_GBS = 8000.0
# The long-prefill page's candidate at this workload (V100, FP16): 100.20284 ms.
PAGE_MS_Q8000_KV128000 = 100.20284
# Its two printed points of the key sweep (Test Result; other points are not printed).
PAGE_MS_SWEEP = {40000: 30.27579, 128000: PAGE_MS_Q8000_KV128000}


TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "hbm_traffic_per_launch.md")
PAGED_SELECTIONS = (64, 512, 2048)
PAGED_DENSE_PAGES = (16, 784)  # paged dense causal prefill: every block up to the diagonal selected
VERIFY_QUERIES = (1, 2, 4, 8)  # 1: the single-row tail


def prefill_workload(n_kv: int, nq: int = 8000) -> str:
    return f"causal_gqa_prefill_q{nq}_kv{n_kv}"


def paged_workload(select_tokens: int, tail: int = 1) -> str:
    return f"paged_sparse_q4096_page16_select{select_tokens}_tail{tail}"


def paged_dense_workload(page_size: int, tail: int = 1) -> str:
    return f"paged_dense_causal_q4096_page{page_size}_tail{tail}"


def varlen_workload() -> str:
    return "varlen_causal_prefill_batch8_kv4096to32768_q25pct"


def verify_workload(nq: int) -> str:
    return f"verify_fp8kv_q{nq}_ctx{workloads.VERIFY_CONTEXT}"


def kernel_source_digest() -> str:
    """Hash of the kernel sources and of the build script (its flags shape the code)."""
    h = hashlib.sha256()
    pkg = os.path.join(ROOT, "gqa_causal_flash_amd")
    csrc = os.path.join(pkg, "csrc")
    files = [os.path.join(csrc, n) for n in sorted(os.listdir(csrc)) if n.endswith((".hip", ".hpp", ".cpp", ".h"))]
    files.append(os.path.join(pkg, "build.py"))
    for f in files:
        h.update(os.path.basename(f).encode() + b"\0")
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_traffic() -> dict:
    """{(kernel, workload): HBM bytes per launch} from the committed counter summary,
    or {} when it was taken on other kernel sources than these."""
    try:
        with open(TRAFFIC_TABLE) as f:
            text = f.read()
    except OSError:
        return {}
    m = re.search(r"kernel source digest: `([0-9a-f]+)`", text)
    if not m or m.group(1) != kernel_source_digest():
        return {}
    out = {}
    for line in text.splitlines():
        cells = [c.strip().strip("`") for c in line.strip().strip("|").split("|")]
        if len(cells) == 6 and cells[5].replace(",", "").isdigit():
            out[(cells[0], cells[1])] = int(cells[5].replace(",", ""))
    return out


def _counter_rows(path: str, counter: str):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                m = re.search(r"gqa::\(anonymous namespace\)::(\w+)", r["Kernel_Name"])
                name = m.group(1) if m else r["Kernel_Name"].split("(")[0].split()[-1]
                rows.append((int(r["Dispatch_Id"]), name, float(r["Counter_Value"])))
    rows.sort()
    return rows


# kernel -> workload family, and the kernels a benchmark step of each family starts with
KERNEL_FAMILY = {"prefill_causal_fwd": "prefill", "prefill_merge": "prefill",
                 "paged_prepass": "paged", "paged_fwd": "paged", "paged_merge": "paged",
                 "verify_fwd": "verify", "verify_merge": "verify",
                 "prefill_varlen_prepass": "varlen", "prefill_causal_varlen": "varlen",
                 "prefill_merge_varlen": "varlen", "prefill_causal_e4m3": "e4m3"}
STEP_STARTS = {"prefill_causal_fwd", "paged_prepass", "verify_fwd", "prefill_varlen_prepass", "prefill_causal_e4m3"}


def family_labels(n_kv: int) -> dict:
    """The workloads of each family in the order main() runs them."""
    prefill_paths = [workloads.TINY, workloads.LONG_40K] + [c for c in workloads.SWEEP if c.n_kv != n_kv]
    return {"prefill": [prefill_workload(n_kv)] + [prefill_workload(c.n_kv, c.nq) for c in prefill_paths],
            "varlen": [varlen_workload()], "e4m3": [e4m3_workload(128000)],
            "paged": [paged_workload(s) for s in PAGED_SELECTIONS] + [paged_dense_workload(p) for p in PAGED_DENSE_PAGES],
            "verify": [verify_workload(q) for q in VERIFY_QUERIES]}


def assign_workloads(rows, per: int, n_kv: int):
    """Label (dispatch, kernel, value) rows of one default benchmark run with their workload.

    A step starts at one of STEP_STARTS, and each workload of a family makes
    `per` (warmup + steps) of them; kernels outside the families are dropped."""
    labels = family_labels(n_kv)
    count = {k: 0 for k in labels}
    cur = None
    for _, name, v in rows:
        if name in STEP_STARTS:
            cur = KERNEL_FAMILY[name]
            count[cur] += 1
        if cur is None or KERNEL_FAMILY.get(name) != cur:
            continue
        yield name, labels[cur][min((count[cur] - 1) // per, len(labels[cur]) - 1)], v


def calls_per_workload(steps: int, warmup: int) -> int:
    """Calls of each kernel that one benchmark workload makes (time_steps): the warm-up calls, the
    timed steps, and as many profiled calls."""
    return warmup + 2 * steps


def summarize_counters(fetch_csv: str, write_csv: str, steps: int, warmup: int, calib_mib: int, n_kv: int) -> str:
    """Markdown table of FETCH_SIZE / WRITE_SIZE per launch of every libgqa kernel.

    The three plain device copies of `calib_mib` MiB made before any workload are
    the known-size reference: each counter's scale factor is the copy's true byte
    count over what the counter reads for it.  Dispatches are assigned to
    workloads by the benchmark's fixed order (assign_workloads)."""
    per = calls_per_workload(steps, warmup)
    true_kib = calib_mib * 1024.0
    result, factors = {}, {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, counter)
        copies = [v for _, n, v in rows if n == "__amd_rocclr_copyBuffer"][:3]
        if len(copies) < 3 or max(copies) > 1.01 * min(copies):
            raise SystemExit(f"{path}: the first three copies do not look like the {calib_mib} MiB calibration: {copies}")
        factors[counter] = true_kib / (sum(copies) / 3)
        for name, wl, v in assign_workloads(rows, per, n_kv):
            result.setdefault((name, wl), {}).setdefault(counter, []).append(v)
    lines = [
        "| kernel | workload | dispatches | FETCH_SIZE (KiB, avg) | WRITE_SIZE (KiB, avg) | HBM bytes per launch |",
        "|---|---|---|---|---|---|",
    ]
    for (name, wl), c in result.items():
        f = sum(c.get("FETCH_SIZE", [0])) / max(1, len(c.get("FETCH_SIZE", [])))
        w = sum(c.get("WRITE_SIZE", [0])) / max(1, len(c.get("WRITE_SIZE", [])))
        nbytes = (f * factors["FETCH_SIZE"] + w * factors["WRITE_SIZE"]) * 1024
        lines.append(f"| `{name}` | `{wl}` | {len(c.get('FETCH_SIZE', []))} | {f:,.1f} | {w:,.1f} | {round(nbytes):,} |")
    head = (f"kernel source digest: `{kernel_source_digest()}`\n\n"
            f"calibration: plain device copy of {calib_mib} MiB; FETCH_SIZE scale {factors['FETCH_SIZE']:.4f}, "
            f"WRITE_SIZE scale {factors['WRITE_SIZE']:.4f}\n\n")
    return head + "\n".join(lines) + "\n"


def summarize_metrics(counter_csv: str, steps: int, warmup: int, n_kv: int) -> str:
    """Markdown table of every counter or derived metric of one rocprofv3 --pmc counter_collection.csv
    of the default benchmark (run with the given --steps/--warmup/--kv), averaged per kernel and workload."""
    per = calls_per_workload(steps, warmup)
    by_counter = {}
    with open(counter_csv, newline="") as f:
        for r in csv.DictReader(f):
            m = re.search(r"gqa::\(anonymous namespace\)::(\w+)", r["Kernel_Name"])
            if m:
                by_counter.setdefault(r["Counter_Name"], []).append(
                    (int(r["Dispatch_Id"]), m.group(1), float(r["Counter_Value"])))
    names = list(by_counter)
    result = {}
    for cn, rows in by_counter.items():
        rows.sort()
        for name, wl, v in assign_workloads(rows, per, n_kv):
            result.setdefault((name, wl), {}).setdefault(cn, []).append(v)
    lines = ["| kernel | workload | dispatches | " + " | ".join(names) + " |",
             "|---|---|---|" + "---|" * len(names)]
    for (name, wl), c in result.items():
        vals = [sum(c.get(n, [0.0])) / max(1, len(c.get(n, []))) for n in names]
        lines.append(f"| `{name}` | `{wl}` | {len(c.get(names[0], []))} | " + " | ".join(f"{v:.2f}" for v in vals) + " |")
    return "\n".join(lines) + "\n"


def summarize_trace(trace_csv: str, steps: int, warmup: int, n_kv: int) -> str:
    """Markdown table of the duration of every libgqa kernel per workload, from a rocprofv3
    --kernel-trace CSV of the default benchmark run with the given --steps/--warmup: average
    over all dispatches and over the timed ones (the 2 * steps after the warm-up of each workload:
    the timed pass and the profiled pass), min, max."""
    per = calls_per_workload(steps, warmup)
    rows = []
    with open(trace_csv, newline="") as f:
        for r in csv.DictReader(f):
            m = re.search(r"gqa::\(anonymous namespace\)::(\w+)", r["Kernel_Name"])
            if m:
                rows.append((int(r["Dispatch_Id"]), m.group(1), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    rows.sort()
    result = {}
    for name, wl, d in assign_workloads(rows, per, n_kv):
        result.setdefault((name, wl), []).append(d)
    lines = ["| kernel | workload | dispatches | average (us) | timed average (us) | min (us) | max (us) |",
             "|---|---|---|---|---|---|---|"]
    for (name, wl), ds in result.items():
        timed = ds[-2 * steps:]
        lines.append(f"| `{name}` | `{wl}` | {len(ds)} | {sum(ds) / len(ds) / 1e3:,.1f} | "
                     f"{sum(timed) / len(timed) / 1e3:,.1f} | {min(ds) / 1e3:,.1f} | {max(ds) / 1e3:,.1f} |")
    return "\n".join(lines) + "\n"


def summarize_sweep_trace(trace_csv: str, steps: int, warmup: int) -> str:
    """Markdown table of prefill_causal_fwd / prefill_merge durations per point of the key sweep.

    Reads a rocprofv3 --kernel-trace CSV of `bench.py --sweep --steps S --warmup W`: the sweep runs its
    points in order (KV = 40000, 48000, ..., 128000), each with calls_per_workload(S, W) calls, so
    dispatch i of a kernel belongs to point i // calls_per_workload(S, W).  The timed calls' kernel time
    is the average over the dispatches after the warm-up of each point."""
    per = calls_per_workload(steps, warmup)
    points = (workloads.LONG_40K,) + workloads.SWEEP
    dur = {"prefill_causal_fwd": [], "prefill_merge": []}
    with open(trace_csv, newline="") as f:
        for row in csv.DictReader(f):
            for k in dur:
                if f"::{k}" in row["Kernel_Name"]:
                    dur[k].append(int(row["End_Timestamp"]) - int(row["Start_Timestamp"]))
    for k, v in dur.items():
        if len(v) != per * len(points):
            raise SystemExit(f"{trace_csv}: {len(v)} dispatches of {k}, expected {per * len(points)}")
    lines = ["| KV | q_pos0 | FLOP | `prefill_causal_fwd` avg of timed (ms) | min (ms) | TFLOP/s | fraction of "
             f"{PEAK_F16_TFLOPS} | `prefill_merge` avg (us) |",
             "|---|---|---|---|---|---|---|---|"]
    for i, cfg in enumerate(points):
        fwd = dur["prefill_causal_fwd"][i * per + warmup:(i + 1) * per]
        mrg = dur["prefill_merge"][i * per + warmup:(i + 1) * per]
        ms = sum(fwd) / len(fwd) / 1e6
        fl = prefill_flops(cfg.nq, cfg.n_kv, cfg.q_pos0)
        tf = fl / (ms * 1e-3) / 1e12
        lines.append(f"| {cfg.n_kv} | {cfg.q_pos0} | {fl:.4e} | {ms:.4f} | {min(fwd) / 1e6:.4f} | {tf:.1f} | "
                     f"{tf / PEAK_F16_TFLOPS:.4f} | {sum(mrg) / len(mrg) / 1e3:.1f} |")
    return "\n".join(lines) + "\n"


def prefill_flops(nq: int, n_kv: int, q_pos0: int, hq: int = 6, d: int = 256) -> float:
    p0, p1 = q_pos0, q_pos0 + nq - 1
    pairs = (p0 + 1 + p1 + 1) * nq // 2
    return 4.0 * d * hq * pairs


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def numpy_blas() -> str:
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:
        return "unknown"


def time_steps(fn, steps: int, warmup: int):
    """Run fn warmup times, then time exactly `steps` calls (sync on both sides) with the library's
    profiling off: the wall time per step.  Then run `steps` more calls with profiling on: the main
    kernel's time per launch from the timing-only HIP events the library records around it on the
    call's stream, and the shader clock its workgroups sample.  Recording the events costs a few
    microseconds per call, so they stay out of the step time.

    Returns (wall ms per step, main-kernel ms per launch); the clock is left in time_steps.clock_mhz."""
    import torch

    import gqa_causal_flash_amd as g

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    g.gqa_profile_start()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    kms, kn = g.gqa_profile_stop()
    time_steps.clock_mhz = g.gqa_profile_clock_mhz()
    return wall, (kms / kn if kn else float("nan"))


def bench_prefill(cfg, steps, warmup, seed=0):
    import torch

    import gqa_causal_flash_amd as g

    q, k, v = workloads.causal_inputs(cfg.nq, cfg.n_kv, seed)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    o = torch.empty_like(dq)
    nbytes = g.gqa_prefill_causal_workspace_size(cfg.nq, cfg.n_kv, cfg.q_pos0)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")

    def step():
        g.gqa_prefill_causal(dq, dk, dv, cfg.q_pos0, cfg.scale, o=o, workspace=ws)

    ms, kms = time_steps(step, steps, warmup)
    flops = prefill_flops(cfg.nq, cfg.n_kv, cfg.q_pos0)
    return dict(ms=ms, kernel_ms=kms, flops=flops, host=(q, k, v), clock_mhz=time_steps.clock_mhz)


def sweep_point(cfg, steps, warmup):
    """One dense prefill workload: step and main-kernel times, TFLOP/s and fractions of the fp16 peak."""
    r = bench_prefill(cfg, steps, warmup)
    achieved = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
    clock = r["clock_mhz"]
    page_ms = PAGE_MS_SWEEP.get(cfg.n_kv)
    name = prefill_workload(cfg.n_kv, cfg.nq)
    return {
        "workload": name, "nq": cfg.nq, "n_kv": cfg.n_kv, "q_pos0": cfg.q_pos0,
        "flops": r["flops"], "steps": steps, "warmup": warmup,
        "ms_per_step": round(r["ms"], 4),
        "tflops_step": round(r["flops"] / (r["ms"] * 1e-3) / 1e12, 2),
        "kernel_ms": round(r["kernel_ms"], 4),
        "tflops_kernel": round(achieved, 2),
        "frac": round(achieved / PEAK_F16_TFLOPS, 4),
        "clock_mhz": round(clock, 1) if clock else None,
        "frac_at_clock": round(achieved / (PEAK_F16_TFLOPS * clock / PEAK_CLOCK_MHZ), 4) if clock else None,
        "page_ms_v100": page_ms,
        "roofline": {"kernel": "prefill_causal_fwd", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_F16_TFLOPS, 4),
                     "algorithmic_bytes": prefill_bytes(cfg),
                     "traffic": recorded_traffic().get(("prefill_causal_fwd", name))},
    }


def prefill_bytes(cfg) -> int:
    """Q, K, V and O of a dense prefill, each read or written once (fp16)."""
    return 2 * (2 * cfg.nq * cfg.hq * cfg.d + 2 * cfg.n_kv * cfg.hkv * cfg.d)


def cpu_baseline_prefill(cfg, host, seconds: float):
    """fp64 oracle on a sample of query rows spread over the workload, timed on this host: one worker
    process per host core (at most 16), each with single-threaded BLAS, each evaluating its share of the
    sampled rows with the unchanged oracle function."""
    from oracle import rowpool

    q, k, v = host
    rng = np.random.default_rng(7)
    procs = rowpool.host_cores()

    def run(n):
        rows = np.sort(rng.choice(cfg.nq, n, replace=False))
        t0 = time.perf_counter()
        rowpool.run_rows("prefill_causal", (q, k, v, cfg.q_pos0, cfg.scale), rows=rows, procs=procs)
        dt = time.perf_counter() - t0
        pairs = int((cfg.q_pos0 + rows + 1).sum())
        return dt, pairs, n

    n = 8 * procs
    dt, pairs, n = run(n)
    for _ in range(4):  # grow the sample until it takes about `seconds`
        if dt >= 0.6 * seconds or n >= cfg.nq:
            break
        n = int(min(cfg.nq, max(2 * n, n * seconds / max(dt, 1e-3))))
        dt, pairs, n = run(n)
    flops = 4.0 * cfg.d * cfg.hq * pairs
    return dict(
        value=flops / dt / 1e12,
        unit="TFLOP/s",
        cores=procs,
        kind="oracle",
        sample=f"{n} of {cfg.nq} query rows (x{cfg.hq} heads, all visible keys of each, up to {cfg.n_kv}) "
               f"in {dt:.1f} s of fp64 numpy, {procs} worker processes with single-threaded BLAS "
               f"(process start included)",
        cpu_model=host_cpu_model(),
        blas=numpy_blas(),
        processes=procs,
    )


def paged_visible_pairs(x) -> int:
    """Visible (query row, key) pairs of one head in a paged block-sparse workload."""
    offs = x.qblock_offsets
    total = 0
    for b in range(offs.size - 1):
        sel = np.unique(x.kv_block_ids[offs[b]:offs[b + 1]]).astype(np.int64)
        toks = (sel[:, None] * x.kv_block_tokens + np.arange(x.kv_block_tokens)).reshape(-1)
        toks = np.sort(toks[toks < x.live_len])
        r0, r1 = b * x.qblock_rows, min(x.q.shape[0], (b + 1) * x.qblock_rows)
        pos = x.q_pos0 + np.arange(r0, r1)
        total += int(np.searchsorted(toks, pos, side="right").sum())
    return total


def paged_bytes(x):
    """(algorithmic, gathered) bytes of a paged workload.  Algorithmic: every live K and V row that some
    query block selects, once (the union of the selections), plus Q and O.  Gathered: each query block's
    selected live rows counted per query block (what the kernel copies to LDS), plus Q and O."""
    ids = np.asarray(x.kv_block_ids, dtype=np.int64)
    live = np.clip(x.live_len - 4 * ids, 0, 4)  # live tokens of each selected 4-token block
    uniq = np.unique(ids)
    live_u = np.clip(x.live_len - 4 * uniq, 0, 4)
    row = 2 * 256 * 2  # one token of K and of V, fp16
    qo = 2 * x.q.nbytes
    return int(live_u.sum()) * row + qo, int(live.sum()) * row + qo


def roofline_mfma_or_hbm(kernel: str, flops: float, nbytes: int, kms: float) -> dict:
    """Roofline of a kernel that both multiplies and streams: the binding roof is the one whose time at
    peak is longer (matrix cores at the fp16 peak, or HBM at 8 TB/s); `achieved` and `frac` are given
    against it, and the other figure is kept beside it."""
    t_mfma = flops / (PEAK_F16_TFLOPS * 1e12)
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    tf = flops / (kms * 1e-3) / 1e12
    gbs = nbytes / (kms * 1e-3) / 1e9
    if t_hbm > t_mfma:
        r = {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(gbs / PEAK_HBM_GBS, 4), "tflops": round(tf, 2),
             "frac_of_fp16_peak": round(tf / PEAK_F16_TFLOPS, 4)}
    else:
        r = {"kernel": kernel, "bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_F16_TFLOPS,
             "unit": "TFLOP/s", "frac": round(tf / PEAK_F16_TFLOPS, 4), "GBps": round(gbs, 1),
             "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    r.update(algorithmic_bytes=int(nbytes), algorithmic_flops=flops,
             us_at_mfma_peak=round(t_mfma * 1e6, 2), us_at_hbm_peak=round(t_hbm * 1e6, 2))
    return r


def bench_paged(select_tokens, steps, warmup, tail=1, seed=0, dense_page_size=None):
    """Paged block-sparse prefill with S-token selections, or (dense_page_size set) the paged
    dense causal prefill with every block up to the diagonal selected over pages of that size."""
    import torch

    import gqa_causal_flash_amd as g

    if dense_page_size is None:
        x = workloads.paged_sparse_inputs(select_tokens=select_tokens, tail=tail, seed=seed)
        name = paged_workload(select_tokens, tail)
    else:
        x = workloads.paged_sparse_inputs(select_tokens=4, tail=tail, seed=seed, saturate=True,
                                          page_size=dense_page_size)
        name = paged_dense_workload(dense_page_size, tail)
    dev = {k: torch.from_numpy(np.ascontiguousarray(getattr(x, k))).cuda()
           for k in ("q", "k_cache", "v_cache", "page_table", "qblock_offsets", "kv_block_ids")}
    o = torch.empty_like(dev["q"])
    nbytes = g.gqa_prefill_paged_sparse_workspace_size(x.q.shape[0], x.kv_block_ids.size)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def step():
        g.gqa_prefill_paged_sparse(dev["q"], dev["k_cache"], dev["v_cache"], dev["page_table"],
                                   dev["qblock_offsets"], dev["kv_block_ids"], x.q_pos0, x.live_len, x.scale,
                                   o=o, workspace=ws)

    ms, kms = time_steps(step, steps, warmup)
    pairs = paged_visible_pairs(x)
    flops = 4.0 * 256 * 6 * pairs
    alg, gathered = paged_bytes(x)
    line = {
        "workload": name,
        "ms_per_step": round(ms, 4), "kernel_ms": round(kms, 4),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2), "visible_pairs_per_head": pairs,
        "roofline": dict(roofline_mfma_or_hbm("paged_fwd", flops, alg, kms),
                         gathered_bytes=gathered, gathered_GBps=round(gathered / (kms * 1e-3) / 1e9, 1),
                         traffic=recorded_traffic().get(("paged_fwd", name))),
    }
    if dense_page_size is None:
        line["page_ms_v100"] = {64: 1.010, 512: 3.204, 2048: 11.203}[select_tokens]
    return line


def bench_varlen(steps, warmup, seed=0):
    """Varlen causal prefill of a chunked-prefill batch: 8 requests with kv lengths uniform in
    [4096, 32768], each prefilling its last quarter (queries at the last positions)."""
    import torch

    import gqa_causal_flash_amd as g

    kv, ql = workloads.varlen_batch_lengths(seed)
    x = workloads.varlen_inputs(kv, ql, seed)
    q, k, v = (torch.from_numpy(a).cuda() for a in (x.q, x.k, x.v))
    cu_q, cu_kv = torch.from_numpy(x.cu_q).cuda(), torch.from_numpy(x.cu_kv).cuda()
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0], 6), dtype=torch.float32, device="cuda")
    ws = torch.empty(g.gqa_prefill_causal_varlen_workspace_size(len(kv), q.shape[0]), dtype=torch.uint8,
                     device="cuda")

    def step():
        g.gqa_prefill_causal_varlen(q, k, v, cu_q, cu_kv, x.scale, o=o, lse=lse, workspace=ws)

    ms, kms = time_steps(step, steps, warmup)
    pairs = int(sum(int(n) * (int(m) - int(n)) + int(n) * (int(n) + 1) // 2 for n, m in zip(ql, kv)))
    flops = 4.0 * 256 * 6 * pairs
    tf = flops / (kms * 1e-3) / 1e12
    return {
        "workload": varlen_workload(),
        "kv_lens": [int(a) for a in kv], "q_lens": [int(a) for a in ql],
        "ms_per_step": round(ms, 4), "kernel_ms": round(kms, 4),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "roofline": {"kernel": "prefill_causal_varlen", "bound": "mfma", "achieved": round(tf, 2),
                     "peak": PEAK_F16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_F16_TFLOPS, 4),
                     "traffic": recorded_traffic().get(("prefill_causal_varlen", varlen_workload()))},
    }


PEAK_F8_TFLOPS = 2 * PEAK_F16_TFLOPS  # dense fp8 matrix-core peak (5.0 PFLOP/s)
# Q K^T (half the FLOPs) on the fp8 matrix cores, P V (the other half) on the fp16 ones
PEAK_E4M3_PREFILL_TFLOPS = 1.0 / (0.5 / PEAK_F8_TFLOPS + 0.5 / PEAK_F16_TFLOPS)


def e4m3_workload(n_kv: int) -> str:
    return f"e4m3_gqa_prefill_q8000_kv{n_kv}"


def bench_e4m3(steps, warmup, n_kv=128000, seed=0):
    """Causal prefill over E4M3 Q/K/V (per-tensor scales) at Q=8000, with Q K^T on the fp8 matrix cores."""
    import torch

    import gqa_causal_flash_amd as g

    nq = 8000
    x = workloads.e4m3_prefill_inputs(nq, n_kv, seed)
    q8, k8, v8 = (torch.from_numpy(a).cuda() for a in (x.q_bytes, x.k_bytes, x.v_bytes))
    o = torch.empty((nq, 6, 256), dtype=torch.float16, device="cuda")
    ws = torch.empty(max(1, g.gqa_prefill_causal_workspace_size(nq, n_kv, x.q_pos0)), dtype=torch.uint8, device="cuda")

    def step():
        g.gqa_prefill_causal_e4m3(q8, x.q_scale, k8, x.k_scale, v8, x.v_scale, x.q_pos0, x.scale, o=o, workspace=ws)

    ms, kms = time_steps(step, steps, warmup)
    mhz = time_steps.clock_mhz
    flops = prefill_flops(nq, n_kv, x.q_pos0)
    tf = flops / (kms * 1e-3) / 1e12
    return {
        "workload": e4m3_workload(n_kv),
        "ms_per_step": round(ms, 4), "kernel_ms": round(kms, 4),
        "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
        "roofline": {"kernel": "prefill_causal_e4m3", "bound": "mfma", "achieved": round(tf, 2),
                     "peak": round(PEAK_E4M3_PREFILL_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(tf / PEAK_E4M3_PREFILL_TFLOPS, 4),
                     "peak_note": "Q K^T at the fp8 peak, P V at the fp16 peak",
                     "frac_of_fp16_peak": round(tf / PEAK_F16_TFLOPS, 4),
                     "clock_mhz": round(mhz, 1) if mhz else None,
                     "frac_at_clock": round(tf / (PEAK_E4M3_PREFILL_TFLOPS * mhz / PEAK_CLOCK_MHZ), 4) if mhz else None,
                     "algorithmic_bytes": nq * 6 * 256 + 2 * n_kv * 256 + 2 * nq * 6 * 256,
                     "traffic": recorded_traffic().get(("prefill_causal_e4m3", e4m3_workload(n_kv)))},
    }


def bench_verify(nq, steps, warmup, copies=3, seed=0):
    import torch

    import gqa_causal_flash_amd as g

    x = workloads.verify_inputs(nq, workloads.VERIFY_CONTEXT, seed)
    q = torch.from_numpy(x.q).cuda()
    kvs = [(torch.from_numpy(x.k_bytes).cuda(), torch.from_numpy(x.v_bytes).cuda())]
    for _ in range(copies - 1):  # independent copies so the 256 MiB last-level cache cannot serve them
        kvs.append((kvs[0][0].clone(), kvs[0][1].clone()))
    o = torch.empty_like(q)
    nbytes = g.gqa_verify_fp8kv_workspace_size(nq, workloads.VERIFY_CONTEXT)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    it = [0]

    def step():
        k, v = kvs[it[0] % copies]
        it[0] += 1
        g.gqa_verify_fp8kv(q, k, v, x.k_scale, x.v_scale, x.scale, o=o, workspace=ws)

    ms, kms = time_steps(step, steps, warmup)
    alg = 2 * x.k_bytes.nbytes + 2 * x.q.nbytes
    gbs = alg / (kms * 1e-3) / 1e9
    return {
        "workload": verify_workload(nq),
        "ms_per_step": round(ms, 4), "kernel_ms": round(kms, 4), "kv_copies_rotated": copies,
        "roofline": {"kernel": "verify_fwd", "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": alg,
                     "traffic": recorded_traffic().get(("verify_fwd", verify_workload(nq)))},
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 50 timed steps: the short paths (tens of microseconds per step) then average over a few ms per pass
    ap.add_argument("--steps", type=int, default=50)
    # the card takes tens of launches to settle (the first long prefills run up to 15 % slower)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--kv", type=int, default=workloads.HEADLINE.n_kv, help="key count of the prefill workload")
    ap.add_argument("--no-paths", action="store_true", help="skip the paged and verifier measurements")
    ap.add_argument("--tiny", action="store_true",
                    help="time the dense prefill of the tiny workload (Q=256 at positions 768..1023 of KV=1024) "
                         "and print one JSON line instead of the default line")
    ap.add_argument("--sweep", action="store_true",
                    help="time the dense prefill at every point of the key sweep (KV = 40000, 48000..128000) and "
                         "print one JSON line per point instead of the default line")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (3 times), as the known-size reference "
                         "for the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize-sweep-trace", metavar="TRACE_CSV",
                    help="print the per-point kernel times of a rocprofv3 --kernel-trace CSV of a --sweep run made "
                         "with the given --steps/--warmup, and exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_CSV",
                    help="print the per-workload kernel times of a rocprofv3 --kernel-trace CSV of a default run "
                         "made with the given --steps/--warmup/--kv, and exit")
    ap.add_argument("--summarize-metrics", metavar="COUNTER_CSV",
                    help="print every counter of a rocprofv3 --pmc counter_collection.csv of a default run made "
                         "with the given --steps/--warmup/--kv, averaged per kernel and workload, and exit")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the per-launch HBM traffic table from two rocprofv3 --pmc counter_collection.csv "
                         "files of a run made with the given --steps/--warmup/--kv/--copy-calibration-mib, and exit")
    args = ap.parse_args(argv)

    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.steps, args.warmup, args.kv), end="")
        return 0

    if args.summarize_metrics:
        print(summarize_metrics(args.summarize_metrics, args.steps, args.warmup, args.kv), end="")
        return 0

    if args.summarize_sweep_trace:
        print(summarize_sweep_trace(args.summarize_sweep_trace, args.steps, args.warmup), end="")
        return 0

    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters, steps=args.steps, warmup=args.warmup,
                                 calib_mib=args.copy_calibration_mib or 1024, n_kv=args.kv), end="")
        return 0

    if args.gpus != 1:
        print("bench.py: libgqa is a single-GPU library; this benchmark runs on exactly one GPU "
              "(--gpus 1); a sharded multi-GPU run is not part of it.", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1

    if args.tiny:
        print(json.dumps(sweep_point(workloads.TINY, args.steps, args.warmup)), flush=True)
        return 0

    if args.sweep:
        for cfg in (workloads.LONG_40K,) + workloads.SWEEP:
            print(json.dumps(sweep_point(cfg, args.steps, args.warmup)), flush=True)
        return 0

    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copy calibration: 3 x {n} bytes", file=sys.stderr)
    cfg = workloads.CausalConfig(prefill_workload(args.kv), nq=8000, n_kv=args.kv)
    r = bench_prefill(cfg, args.steps, args.warmup)
    value = r["flops"] / (r["ms"] * 1e-3) / 1e12
    achieved = r["flops"] / (r["kernel_ms"] * 1e-3) / 1e12
    line = {
        "metric": "causal GQA prefill TFLOP/s & ms (Q=8000,KV=128K) + % of fp16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(PAGE_MS_Q8000_KV128000 / r["ms"], 3) if cfg.n_kv == 128000 else None,
        "vs_baseline_note": "ratio to the long-prefill page's V100 candidate (100.20284 ms); context, not a target",
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "nq": cfg.nq, "n_kv": cfg.n_kv, "q_pos0": cfg.q_pos0, "hq": cfg.hq,
                   "hkv": cfg.hkv, "d": cfg.d, "scale": cfg.scale, "seed": 0, "pct_of_fp16_peak":
                   round(100 * value / PEAK_F16_TFLOPS, 2)},
        "roofline": {
            "kernel": "prefill_causal_fwd",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_F16_TFLOPS, 4),
            "kernel_ms": round(r["kernel_ms"], 4),
            # the same launches against the peak rescaled to the shader clock they ran at
            "clock_mhz": round(r["clock_mhz"], 1),
            "peak_at_clock": round(PEAK_F16_TFLOPS * r["clock_mhz"] / PEAK_CLOCK_MHZ, 1) if r["clock_mhz"] else None,
            "frac_at_clock": round(achieved / (PEAK_F16_TFLOPS * r["clock_mhz"] / PEAK_CLOCK_MHZ), 4)
            if r["clock_mhz"] else None,
            "algorithmic_bytes": prefill_bytes(cfg),
            "traffic": recorded_traffic().get(("prefill_causal_fwd", cfg.name)),
        },
    }
    if not args.no_paths:
        line["paths"] = {
            # the tiny workload (Q = 256 at 768..1023 of KV = 1024), the page's KV = 40000 point and the rest of
            # its key sweep (48000..120000; 128000 is the line's own workload)
            "prefill_tiny": [sweep_point(workloads.TINY, args.steps, args.warmup)],
            "prefill_long_40k": [sweep_point(workloads.LONG_40K, args.steps, args.warmup)],
            "prefill_sweep": [sweep_point(c, args.steps, args.warmup) for c in workloads.SWEEP if c.n_kv != cfg.n_kv],
            "paged_sparse": [bench_paged(sel, args.steps, args.warmup) for sel in PAGED_SELECTIONS],
            "paged_dense": [bench_paged(None, args.steps, args.warmup, dense_page_size=ps) for ps in PAGED_DENSE_PAGES],
            "verify_fp8kv": [bench_verify(nq, args.steps, args.warmup) for nq in VERIFY_QUERIES],
            "varlen": [bench_varlen(args.steps, args.warmup)],
            "e4m3_prefill": [bench_e4m3(args.steps, args.warmup)],
        }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(cfg, r["host"], args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
