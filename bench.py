"""Throughput of exact per-row top-k on one MI355X.

One step = one call of the selection over one batch of synthetic score rows
already resident in HBM.  Default workload: 128 rows x 1,048,576 fp32 scores,
k = 512 (even rows strictly ascending, odd rows quantized to 256 levels).
The timed region rotates over several copies of the batch (more bytes than
the 256 MB last-level cache) so every step reads cold HBM.

Prints one JSON line.  `value` is effective HBM read GB/s = 4 * (valid
scores) / (wall time per step).  `roofline` compares the selection kernel's
average duration (HIP events on the launch stream) with the 8 TB/s HBM peak.
`cpu_baseline` times the CPU oracle on the host cores over the same batch.
"""

from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
TRAFFIC_DIR = os.path.join(ROOT, "profiles")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(ROOT, "sparse_attention_indexer_row_amd", "csrc", "*"))):
        with open(p, "rb") as f:
            h.update(os.path.basename(p).encode())
            h.update(f.read())
    return h.hexdigest()


def load_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(TRAFFIC_DIR, f"topk_select_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t


PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -T -f csv -d {d} -o trace -- "
             "python3 bench.py --workload {w} --steps 20 --warmup 5 --no-cpu-baseline --no-probe",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -T -f csv -d {d} -o fetch -- "
             "python3 bench.py --workload {w} --profile-run --steps 5 --warmup 2",
    "write": "rocprofv3 --pmc WRITE_SIZE -T -f csv -d {d} -o write -- "
             "python3 bench.py --workload {w} --profile-run --steps 5 --warmup 2",
}
COPY_BYTES = 1 << 30   # one probe copy in --profile-run: 1 GiB read, 1 GiB written


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_profiles(workload: str, trace_dir: str, fetch_dir: str, write_dir: str) -> int:
    """Turns the three rocprofv3 runs of PROFILE_COMMANDS into the committed
    summaries: profiles/topk_select_<workload>_rocprof.md (kernel statistics)
    and profiles/topk_select_<workload>_traffic.json (HBM bytes per launch,
    scaled by the counters' reading for the 1 GiB probe copy)."""
    import numpy as np

    from sparse_attention_indexer_row_amd import workloads

    stats = _csv_rows(os.path.join(trace_dir, "trace_kernel_stats.csv"))
    trace = _csv_rows(os.path.join(trace_dir, "trace_kernel_trace.csv"))
    sel = [r for r in stats if r["Name"].startswith("select_kernel")]
    if not sel:
        print("no select_kernel in the kernel statistics", file=sys.stderr)
        return 1
    durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            for r in trace if r["Kernel_Name"].startswith("select_kernel")]

    def counter(dirname, prefix, name):
        rows = _csv_rows(os.path.join(dirname, f"{prefix}_counter_collection.csv"))
        pick = lambda kn: [float(r["Counter_Value"]) for r in rows
                           if r["Kernel_Name"].startswith(kn) and r["Counter_Name"] == name]
        return pick("select_kernel"), pick("probe_copy_kernel")

    f_sel, f_copy = counter(fetch_dir, "fetch", "FETCH_SIZE")
    w_sel, w_copy = counter(write_dir, "write", "WRITE_SIZE")
    if not (f_sel and f_copy and w_sel and w_copy):
        print("counter files lack select_kernel or probe_copy_kernel rows", file=sys.stderr)
        return 1
    fetch_scale = (COPY_BYTES / 1024) / float(np.mean(f_copy))
    write_scale = (COPY_BYTES / 1024) / float(np.mean(w_copy))
    fetch_b = float(np.mean(f_sel)) * 1024 * fetch_scale
    write_b = float(np.mean(w_sel)) * 1024 * write_scale
    w = workloads.make(workload)
    algo_read = 4 * w.valid_elements()
    algo_write = 8 * w.rows * w.k
    traffic = {
        "kernel": "select_kernel", "workload": workload,
        "kernel_source_sha256": kernel_source_hash(),
        "fetch_kib_per_dispatch": round(float(np.mean(f_sel)), 3),
        "write_kib_per_dispatch": round(float(np.mean(w_sel)), 3),
        "copy_bytes": COPY_BYTES,
        "copy_fetch_kib": round(float(np.mean(f_copy)), 3),
        "copy_write_kib": round(float(np.mean(w_copy)), 3),
        "fetch_scale": round(fetch_scale, 5), "write_scale": round(write_scale, 5),
        "bytes_per_launch": int(round(fetch_b + write_b)),
        "fetch_bytes_per_launch": int(round(fetch_b)),
        "write_bytes_per_launch": int(round(write_b)),
        "algorithmic_read_bytes": algo_read, "algorithmic_write_bytes": algo_write,
        "commands": {k: v.format(d="<dir>", w=workload) for k, v in PROFILE_COMMANDS.items()},
    }
    os.makedirs(TRAFFIC_DIR, exist_ok=True)
    with open(os.path.join(TRAFFIC_DIR, f"topk_select_{workload}_traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")
    lines = [f"# select_kernel, workload `{workload}`: rocprofv3 summary", "",
             f"Workload: {w.description}.", "",
             "Commands (run from the repository root; `<dir>` is any output directory):", ""]
    lines += [f"    {v.format(d='<dir>', w=workload)}" for v in PROFILE_COMMANDS.values()]
    lines += ["", "Kernel statistics (`--kernel-trace --stats`):", "",
              "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    lines += ["", f"select_kernel dispatch durations: mean {np.mean(durs):.1f} us, median "
              f"{np.median(durs):.1f} us over {len(durs)} dispatches (includes the warm-up and "
              f"parity launches).", "",
              "HBM traffic per select_kernel dispatch (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`):", "",
              f"- FETCH_SIZE {traffic['fetch_kib_per_dispatch']} KiB; the 1 GiB probe copy reads as "
              f"{traffic['copy_fetch_kib']} KiB, scale {traffic['fetch_scale']} -> "
              f"{fetch_b / 1e6:.1f} MB read (algorithmic {algo_read / 1e6:.1f} MB).",
              f"- WRITE_SIZE {traffic['write_kib_per_dispatch']} KiB; the 1 GiB probe copy writes as "
              f"{traffic['copy_write_kib']} KiB, scale {traffic['write_scale']} -> "
              f"{write_b / 1e6:.2f} MB written (algorithmic {algo_write / 1e6:.2f} MB of outputs).",
              f"- Total {traffic['bytes_per_launch'] / 1e6:.1f} MB per launch, "
              f"{traffic['bytes_per_launch'] / (algo_read + algo_write):.3f} x the algorithmic bytes.",
              "", f"Kernel sources: sha256 {traffic['kernel_source_sha256']}.", ""]
    with open(os.path.join(TRAFFIC_DIR, f"topk_select_{workload}_rocprof.md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 0


def host_cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="adverse",
                    choices=["small", "outlier", "one_row", "adverse", "ragged"])
    ap.add_argument("--copies", type=int, default=0,
                    help="input copies to rotate over (0: enough for >= 1.5 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--profile-run", action="store_true",
                    help="only the timed selection launches (for rocprofv3 counter runs)")
    ap.add_argument("--summarize-profiles", nargs=3, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ summaries from the rocprofv3 runs of PROFILE_COMMANDS")
    args = ap.parse_args()
    if args.summarize_profiles:
        return summarize_profiles(args.workload, *args.summarize_profiles)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(rows are independent, so more GPUs would each run this same single-GPU path)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from sparse_attention_indexer_row_amd import api, workloads

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    print(f"[bench] generating workload {args.workload}", file=sys.stderr, flush=True)
    w = workloads.make(args.workload)
    rows, n, k = w.rows, w.n, w.k
    valid = w.valid_elements()
    read_bytes = 4 * valid

    base = torch.from_numpy(w.scores).to(dev)
    lengths = torch.from_numpy(w.lengths).to(dev) if w.lengths is not None else None
    batch_bytes = base.numel() * 4
    copies = args.copies or max(2, -(-(3 << 29) // batch_bytes))
    inputs = [base] + [base.clone() for _ in range(copies - 1)]
    vals = torch.empty((rows, k), dtype=torch.float32, device=dev)
    idx = torch.empty((rows, k), dtype=torch.int32, device=dev)
    plan = api.topk_plan(rows, n, k)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        api.topk_select(inputs[i % copies], k, lengths, out=(vals, idx), stream=stream)

    # parity on sampled rows of copy 0 (the full-size parity test covers all rows)
    parity = None
    if not args.profile_run:
        import oracle
        step(0)
        torch.cuda.synchronize()
        sample = sorted({0, 1, rows // 2, rows - 1})
        sl = w.lengths[sample] if w.lengths is not None else None
        rv, ri = oracle.topk(w.scores[sample], k, sl)
        gv, gi = vals.cpu().numpy()[sample], idx.cpu().numpy()[sample]
        ok = np.array_equal(gi, ri) and np.array_equal(gv.view(np.uint32), rv.view(np.uint32))
        parity = f"bit-exact vs oracle on rows {sample}" if ok else "MISMATCH"
        if not ok:
            print("[bench] parity mismatch against the oracle", file=sys.stderr)

    for i in range(args.warmup):
        step(i + 1)
    torch.cuda.synchronize()

    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record(stream)
    for i in range(K):
        starts[i].record(stream)
        step(args.warmup + 1 + i)
        ends[i].record(stream)
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    total_ms = t_all0.elapsed_time(t_all1)
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    ms_per_step = total_ms / K
    kern_ms = float(np.mean(per_launch_ms))
    print(f"[bench] {K} steps: {ms_per_step * 1e3:.1f} us/step, kernel avg {kern_ms * 1e3:.1f} us, "
          f"median {np.median(per_launch_ms) * 1e3:.1f} us, wall {1e3 * (wall1 - wall0) / K:.1f} ms/step",
          file=sys.stderr, flush=True)

    if args.profile_run:
        # Counter calibration: a plain copy of a known size (1 GiB read, 1 GiB
        # written) profiled in the same run, so HBM byte counters can be
        # scaled by what they read for known traffic.
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        for _ in range(3):
            api.topk_probe_copy(src, dst, stream=stream)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 3 x {src.numel() * 4} bytes", file=sys.stderr, flush=True)
        return 0

    value = read_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = read_bytes / (kern_ms * 1e-3) / 1e9

    probe = None
    if not args.no_probe:
        # plain streaming read of 2 GiB with the same per-wave access pattern
        buf = torch.empty(1 << 29, dtype=torch.float32, device=dev)
        buf.fill_(1.0)
        sink = api.topk_probe_read(buf)
        for _ in range(2):
            api.topk_probe_read(buf, sink)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        reps = 5
        for _ in range(reps):
            api.topk_probe_read(buf, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        probe = (buf.numel() * 4 * reps) / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del buf

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cores = host_cores()
        sample_rows = rows
        t0 = time.perf_counter()
        oracle.topk(w.scores[:sample_rows], k, w.lengths[:sample_rows] if w.lengths is not None else None,
                    threads=cores)
        dt = time.perf_counter() - t0
        sample_valid = (sample_rows * n if w.lengths is None
                        else int(np.clip(w.lengths[:sample_rows], 0, n).sum()))
        cpu = {"value": round(4 * sample_valid / dt / 1e9, 3), "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": f"all {sample_rows} rows of the batch, one pass, {dt:.2f} s wall "
                         f"({sample_rows / dt:.1f} rows/s)"}

    traffic = load_traffic(args.workload)
    roofline = {
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic["bytes_per_launch"] if traffic else None,
    }
    out = {
        "metric": "effective HBM read GB/s (and rows/s) for top-512 of 1M fp32 scores/row",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.description, "rows": rows, "n": n, "k": k,
                   "read_bytes_per_step": read_bytes, "split": plan["split"],
                   "waves": plan["waves"], "input_copies": copies},
        "rows_per_s": round(rows / (ms_per_step * 1e-3), 1),
        "kernel_us_mean": round(kern_ms * 1e3, 2),
        "kernel_us_median": round(float(np.median(per_launch_ms)) * 1e3, 2),
        "read_probe_GBps": round(probe, 1) if probe else None,
        "parity": parity,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
