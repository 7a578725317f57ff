"""Throughput of exact per-row top-k on one MI355X.

One step = one call of the selection over one batch of synthetic score rows
already resident in HBM.  Default workload: 128 rows x 1,048,576 fp32 scores,
k = 512 (even rows strictly ascending, odd rows quantized to 256 levels).
The timed region rotates over several copies of the batch (more bytes than
the 256 MB last-level cache) so every step reads cold HBM.

Prints one JSON line.  `value` is effective HBM read GB/s = 4 * (valid
scores) / (time per step), the K steps timed back to back between two events
on the launch stream.  `roofline` compares the selection kernel's average
launch duration (each of K further launches between its own pair of events)
with the 8 TB/s HBM peak.  `cpu_baseline` times the CPU oracle on the host
cores over the same batch.
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


# Sources each bench path's kernels are built from; a traffic summary is
# stale once any of them changes.
SELECT_SOURCES = ["select_kernel.hip", "common.h", "wave_sort.h", "select_args.h"]
RADIX_SOURCES = ["pool_kernel.hip", "common.h", "internal.h", "select_args.h", "wave_sort.h"]
KERNEL_SOURCES = {
    "vocab": RADIX_SOURCES,
    "decode": ["decode_kernel.hip", "common.h", "internal.h", "select_args.h"],
    "pool": SELECT_SOURCES + ["pool_kernel.hip", "internal.h"],
    "pooled": RADIX_SOURCES,
    # topk_select routes these shapes to the radix selection (4 x 16K and
    # 64 x 128K at k = 512, 256 ragged rows at k = 2,048)
    "small": RADIX_SOURCES,
    "outlier": RADIX_SOURCES,
    "ragged": RADIX_SOURCES,
}


def kernel_source_hash(workload: str = "adverse") -> str:
    h = hashlib.sha256()
    names = KERNEL_SOURCES.get(workload, SELECT_SOURCES)
    for name in sorted(names):
        with open(os.path.join(ROOT, "sparse_attention_indexer_row_amd", "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()


def profile_target(workload: str):
    """(summary file stem, kernels one call launches, algorithmic read bytes,
    algorithmic write bytes) of a bench workload; host only, no GPU."""
    from sparse_attention_indexer_row_amd import workloads
    if workload == "decode":
        w = workloads.decode()
        rows, heads, dqk = w.q.shape
        return (traffic_stem(workload), ["decode_partial_kernel", "decode_combine_kernel"],
                decode_read_bytes(w), 4 * rows * heads * w.dv)
    if workload == "pooled":
        w = workloads.pooled()
        return (traffic_stem(workload),
                ["radix_select_kernel"],
                4 * w.pool_scores.size + 4 * w.pool_idx.size, 8 * w.rows * w.k)
    if workload == "pool":
        w = workloads.make("adverse")
        return (traffic_stem(workload), ["block_max8_kernel", "radix_select_kernel"],
                4 * w.valid_elements(), 8 * w.rows * POOL_KEEP)
    w = workloads.make(workload)
    if workload == "vocab" or routed_to_radix(w.rows, w.n, w.k, 256):
        return (traffic_stem(workload), ["radix_select_kernel"], 4 * w.valid_elements(),
                8 * w.rows * w.k)
    return (traffic_stem(workload), ["select_kernel"], 4 * w.valid_elements(), 8 * w.rows * w.k)


def routed_to_radix(rows: int, n: int, k: int, cus: int) -> bool:
    """Whether topk_select takes the radix path for this shape: the library's
    own plan (no launch), used to label the kernel a workload runs.  `cus`
    is kept for the callers; the plan queries the device itself."""
    from sparse_attention_indexer_row_amd import _lib, api
    return api.topk_plan(rows, n, k, for_select=True)["path"] == _lib.TOPK_PATH_RADIX


def decode_bound(q, kv, idx, scale, dv):
    """Per-element tolerance of the decode's parity check, in float64:
    2^-7 * sum_j p_j |v_jc| + 1e-6 with p the exact softmax of the selected
    positions -- twice what bf16-rounded softmax weights can move a convex
    combination (the same bound as the GPU tests')."""
    import numpy as np
    rows, heads, _ = q.shape
    n = kv.shape[0]
    out = np.full((rows, heads, dv), 1e-6)
    for r in range(rows):
        j = idx[r][(idx[r] >= 0) & (idx[r] < n)].astype(np.int64)
        if j.size == 0:
            continue
        keys = kv[j].astype(np.float64)
        logits = scale * (q[r].astype(np.float64) @ keys.T)
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        out[r] += 2.0 ** -7 * (p @ np.abs(keys[:, :dv]))
    return out


def decode_read_bytes(w) -> int:
    """Algorithmic bytes a decode call reads: each selected cache row once
    (bf16), the queries and the indices."""
    rows, heads, dqk = w.q.shape
    return 2 * w.idx.size * dqk + 2 * w.q.size + 4 * w.idx.size


def traffic_stem(workload: str) -> str:
    return {"pooled": "topk_pooled_select_pooled", "vocab": "topk_select_radix_vocab",
            "decode": "topk_sparse_decode_decode",
            "pool": "topk_block_pool_adverse"}.get(workload, f"topk_select_{workload}")


def load_traffic(workload: str):
    """HBM bytes per call from committed rocprofv3 counter runs, or None
    when the kernel sources changed since the counters were taken."""
    path = os.path.join(TRAFFIC_DIR, f"{traffic_stem(workload)}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_hash(workload):
        return None
    return t


PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -T -f csv -d {d} -o trace -- "
             "python3 bench.py --workload {w} --steps 20 --warmup 5 --no-cpu-baseline --no-probe "
             "--no-context",
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
    summaries: profiles/<entry point>_<workload>_rocprof.md (kernel
    statistics) and profiles/<entry point>_<workload>_traffic.json (HBM bytes
    per call, summed over the call's kernels and scaled by the counters'
    reading for the 1 GiB probe copy)."""
    import numpy as np

    stem, kernels, algo_read, algo_write = profile_target(workload)
    stats = _csv_rows(os.path.join(trace_dir, "trace_kernel_stats.csv"))
    trace = _csv_rows(os.path.join(trace_dir, "trace_kernel_trace.csv"))
    durs = {kn: [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                 for r in trace if r["Kernel_Name"].startswith(kn)] for kn in kernels}
    if not all(durs.values()):
        print(f"the kernel trace lacks one of {kernels}", file=sys.stderr)
        return 1

    def counter(dirname, prefix, name):
        rows = _csv_rows(os.path.join(dirname, f"{prefix}_counter_collection.csv"))
        pick = lambda kn: [float(r["Counter_Value"]) for r in rows
                           if r["Kernel_Name"].startswith(kn) and r["Counter_Name"] == name]
        return {kn: pick(kn) for kn in kernels}, pick("probe_copy_kernel")

    f_k, f_copy = counter(fetch_dir, "fetch", "FETCH_SIZE")
    w_k, w_copy = counter(write_dir, "write", "WRITE_SIZE")
    if not (all(f_k.values()) and f_copy and all(w_k.values()) and w_copy):
        print("counter files lack a kernel's or probe_copy_kernel's rows", file=sys.stderr)
        return 1
    fetch_scale = (COPY_BYTES / 1024) / float(np.mean(f_copy))
    write_scale = (COPY_BYTES / 1024) / float(np.mean(w_copy))
    f_kib = {kn: float(np.mean(v)) for kn, v in f_k.items()}
    w_kib = {kn: float(np.mean(v)) for kn, v in w_k.items()}
    fetch_b = sum(f_kib.values()) * 1024 * fetch_scale
    write_b = sum(w_kib.values()) * 1024 * write_scale
    traffic = {
        "kernels": kernels, "workload": workload,
        "kernel_source_sha256": kernel_source_hash(workload),
        "fetch_kib_per_dispatch": {kn: round(v, 3) for kn, v in f_kib.items()},
        "write_kib_per_dispatch": {kn: round(v, 3) for kn, v in w_kib.items()},
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
    with open(os.path.join(TRAFFIC_DIR, f"{stem}_traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
        f.write("\n")
    lines = [f"# {' + '.join(kernels)}, workload `{workload}`: rocprofv3 summary", "",
             "Commands (run from the repository root; `<dir>` is any output directory):", ""]
    lines += [f"    {v.format(d='<dir>', w=workload)}" for v in PROFILE_COMMANDS.values()]
    lines += ["", "Kernel statistics (`--kernel-trace --stats`):", "",
              "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| {r['Name']} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} |")
    lines.append("")
    for kn in kernels:
        lines.append(f"{kn} dispatch durations: mean {np.mean(durs[kn]):.1f} us, median "
                     f"{np.median(durs[kn]):.1f} us over {len(durs[kn])} dispatches (includes the "
                     f"warm-up and parity launches).")
    lines += ["", "HBM traffic per call (`--pmc FETCH_SIZE`, then `--pmc WRITE_SIZE`; KiB per "
              "dispatch of each kernel):", ""]
    for kn in kernels:
        lines.append(f"- {kn}: FETCH_SIZE {f_kib[kn]:.1f} KiB, WRITE_SIZE {w_kib[kn]:.1f} KiB")
    lines += [f"- The 1 GiB probe copy reads as {traffic['copy_fetch_kib']} KiB and writes as "
              f"{traffic['copy_write_kib']} KiB: scales {traffic['fetch_scale']} and "
              f"{traffic['write_scale']}.",
              f"- Read {fetch_b / 1e6:.1f} MB per call (algorithmic {algo_read / 1e6:.1f} MB); written "
              f"{write_b / 1e6:.2f} MB (algorithmic {algo_write / 1e6:.2f} MB of outputs).",
              f"- Total {traffic['bytes_per_launch'] / 1e6:.1f} MB per call, "
              f"{traffic['bytes_per_launch'] / (algo_read + algo_write):.3f} x the algorithmic bytes.",
              "", f"Kernel sources: sha256 {traffic['kernel_source_sha256']}.", ""]
    with open(os.path.join(TRAFFIC_DIR, f"{stem}_rocprof.md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))
    return 0


def host_cpu() -> dict:
    """The host's CPU model and logical CPU count, for the baseline's context."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count()}


def host_cores() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


METRIC_SELECT = "effective HBM read GB/s (and rows/s) for top-512 of 1M fp32 scores/row"


def median_us(torch, stream, call, n=30, warm=5):
    """Median of n HIP-event-timed calls on `stream` (call(i) for i = 0, 1, ...)."""
    import numpy as np
    for i in range(warm):
        call(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        call(warm + i)
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) * 1e3 for a, b in ev]))


def harmonic(n: int) -> float:
    return sum(1.0 / i for i in range(1, n + 1))


def headline_extras(dev, torch, api, workloads):
    """Context measured beside the headline line: topk_select on R rows of 1M
    N(0,1) scores for R = 64, 128, 256 (cold: two copies of each batch), and
    the other spec configurations (4 x 16K, 64 x 128K with outliers,
    1 x 1M, 256 ragged rows of <= 256K at k = 2,048) in microseconds per call,
    with torch.topk on the same rows."""
    import numpy as np
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev)
    sweep = {}
    for R in (64, 128, 256):
        gen.manual_seed(1000 + R)
        xs = [torch.randn((R, 1 << 20), generator=gen, device=dev) for _ in range(2)]
        t = median_us(torch, stream, lambda i: api.topk_select(xs[i % 2], 512, stream=stream))
        gbs = 4 * R * (1 << 20) / (t * 1e-6) / 1e9
        sweep[str(R)] = {"us_per_call": round(t, 1), "GBps": round(gbs, 1),
                         "frac_of_8TBps": round(gbs / HBM_PEAK_GBPS, 4),
                         "plan": {k: v for k, v in api.topk_plan(R, 1 << 20, 512,
                                                                 for_select=True).items()
                                  if k in ("split", "waves", "path")}}
        del xs
    configs = {}
    for label, name in (("C1", "small"), ("C2", "outlier"), ("C3", "one_row"), ("C5", "ragged")):
        w = workloads.make(name)
        base = torch.from_numpy(w.scores).to(dev)
        ln = torch.from_numpy(w.lengths).to(dev) if w.lengths is not None else None
        m = max(2, -(-(3 << 29) // (base.numel() * 4)))
        xs = [base] + [base.clone() for _ in range(m - 1)]
        t = median_us(torch, stream, lambda i: api.topk_select(xs[i % m], w.k, ln, stream=stream))
        entry = {"workload": w.description, "us_per_call": round(t, 1),
                 "GBps": round(4 * w.valid_elements() / (t * 1e-6) / 1e9, 1),
                 "path": "radix" if routed_to_radix(w.rows, w.n, w.k, 256) else "streaming"}
        if w.lengths is None:
            tk = median_us(torch, stream, lambda i: torch.topk(xs[i % m], w.k, dim=1), n=10)
            entry["torch_topk_us"] = round(tk, 1)
        configs[label] = entry
        del xs, base
    return {"rows_sweep_1M_normal_k512": sweep, "other_configs": configs}


def probe_sweep(torch, api, dev) -> dict:
    """Read-probe sweep: whole-chip rate over read shapes (threads, loads in
    flight per thread, plain or nontemporal loads, bytes per workgroup) and
    the rate with 1..256 compute units active (one 4 MiB workgroup per unit,
    kept alone on its unit by a 96 KiB LDS reservation).  Each rate is the
    median of 7 event-timed reads rotating over three 1 GiB buffers."""
    stream = torch.cuda.current_stream(dev)
    gib = 1 << 30
    bufs = [torch.ones(gib // 4, dtype=torch.float32, device=dev) for _ in range(3)]
    sink = torch.empty(1 << 16, dtype=torch.int32, device=dev)

    def rate(per, groups, threads, loads, nt, lds=0):
        t = median_us(torch, stream, lambda i: api.topk_probe_read_cfg(
            bufs[i % 3], per, groups, threads, loads, nt, lds, sink=sink, stream=stream),
            n=7, warm=2)
        return per * groups / (t * 1e-6) / 1e9, t

    shapes = []
    for per in (64 << 10, 4 << 20):
        for threads in (256, 512, 1024):
            for loads in (1, 2, 4, 8):
                if per % (16 * threads * loads):
                    continue
                for nt in (False, True):
                    gbs, t = rate(per, gib // per, threads, loads, nt)
                    shapes.append({"bytes_per_group": per, "threads": threads, "loads": loads,
                                   "nontemporal": nt, "GBps": round(gbs, 1)})
    cus = []
    for g in (1, 2, 4, 8, 16, 32, 64, 96, 128, 160, 192, 224, 256):
        gbs, t = rate(4 << 20, g, 1024, 4, True, 96 << 10)
        cus.append({"active_cus": g, "GBps": round(gbs, 1), "GBps_per_cu": round(gbs / g, 2)})
    best = max(shapes, key=lambda x: x["GBps"])
    return {"shapes": shapes, "active_cus": cus, "best": best,
            "best_frac_of_8TBps": round(best["GBps"] / HBM_PEAK_GBPS, 4)}


def write_probe_summary(res: dict) -> str:
    path = os.path.join(TRAFFIC_DIR, "read_probe_sweep.md")
    lines = ["# Streaming-read ceiling of MI355X: read-probe sweep", "",
             "Command (from the repository root): `python bench.py --probe-sweep`", "",
             "Whole chip, 1 GiB per read (median of 7, three rotating 1 GiB buffers):", "",
             "| bytes per workgroup | threads | loads in flight | nontemporal | GB/s |",
             "|---|---|---|---|---|"]
    for x in res["shapes"]:
        lines.append(f"| {x['bytes_per_group'] >> 10} KiB | {x['threads']} | {x['loads']} | "
                     f"{'yes' if x['nontemporal'] else 'no'} | {x['GBps']:.0f} |")
    b = res["best"]
    lines += ["", f"Best: {b['GBps']:.0f} GB/s ({res['best_frac_of_8TBps']:.3f} of 8 TB/s) with "
              f"{b['threads']} threads, {b['loads']} loads in flight, "
              f"{'nontemporal' if b['nontemporal'] else 'plain'} loads, "
              f"{b['bytes_per_group'] >> 10} KiB per workgroup.", "",
              "Active compute units (one 4 MiB workgroup of 1,024 threads per unit, four "
              "nontemporal loads in flight):", "",
              "| active CUs | GB/s | GB/s per CU |", "|---|---|---|"]
    for x in res["active_cus"]:
        lines.append(f"| {x['active_cus']} | {x['GBps']:.0f} | {x['GBps_per_cu']:.1f} |")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    return path
POOL_GROUP, POOL_KEEP, POOL_PINNED = 8, 2000, 16


def make_case(name, dev, np, torch, api, workloads):
    """Inputs, one step, its parity check and CPU baseline for a workload.
    The timed region rotates over enough input copies (>= 1.5 GiB) that
    every step reads cold HBM."""
    import oracle
    from sparse_attention_indexer_row_amd import _lib

    stream = torch.cuda.current_stream(dev)
    c = {}

    def rotate(base_list, batch_bytes):
        copies = max(2, -(-(3 << 29) // batch_bytes))
        return [base_list] + [[t.clone() for t in base_list] for _ in range(copies - 1)], copies

    if name == "decode":
        from oracle.decode import sparse_decode
        w = workloads.decode()
        rows, heads, dqk = w.q.shape
        q = torch.from_numpy(w.q).to(dev, dtype=torch.bfloat16)
        kv = torch.from_numpy(w.kv).to(dev, dtype=torch.bfloat16)
        # Each step gathers a different set of positions (the workload's and
        # more draws of the same recipe), so the rows a step reads were not
        # touched by the previous 23 steps (about 1.8 GB): cold HBM, not the
        # 256 MB last-level cache.
        sets = [w.idx] + [workloads.decode_positions(rows, w.kv.shape[0], w.idx.shape[1],
                                                     seed=w.seed + 1 + c) for c in range(23)]
        idx_sets = [torch.from_numpy(x).to(dev) for x in sets]
        out = torch.empty((rows, heads, w.dv), dtype=torch.float32, device=dev)

        def step(i):
            api.topk_sparse_decode(q, kv, idx_sets[i % len(idx_sets)], w.dv, w.scale, out=out,
                                   stream=stream)

        sample = sorted({r for r in (0, 1, rows // 2, rows - 1) if r < rows})

        def parity():
            got = out.cpu().numpy()
            ok = True
            for r in sample:
                want = sparse_decode(w.q[r:r + 1], w.kv, w.idx[r:r + 1], w.scale, w.dv)[0]
                bound = decode_bound(w.q[r:r + 1], w.kv, w.idx[r:r + 1], w.scale, w.dv)[0]
                ok = ok and bool(np.all(np.abs(got[r] - want) <= bound))
            return ok, sample

        def cpu(cores):
            t0 = time.perf_counter()
            sparse_decode(w.q, w.kv, w.idx, w.scale, w.dv)
            dt = time.perf_counter() - t0
            return dt, decode_read_bytes(w), f"all {rows} rows (float64 numpy)"

        c.update(rows=rows, read_bytes=decode_read_bytes(w), copies=len(idx_sets), step=step,
                 parity=parity,
                 cpu=cpu, cpu_cores=lambda cores: 1,
                 kernel="decode_partial_kernel + decode_combine_kernel (whole call)",
                 parity_kind="within 2^-7 sum_j p_j |v_jc| + 1e-6 of the float64 oracle, "
                             "per element",
                 metric="effective HBM read GB/s of gathered bf16 cache rows for sparse-attention "
                        "decode over 512 selected positions (16 heads, dqk 576, dv 512)",
                 config={"workload": w.description, "rows": rows, "heads": heads, "dqk": dqk,
                         "dv": w.dv, "k": int(w.idx.shape[1])})
        c["set_copies"] = lambda m: None
        return c

    if name == "pooled":
        w = workloads.pooled()
        base = [torch.from_numpy(w.pool_scores).to(dev), torch.from_numpy(w.pool_idx).to(dev)]
        inputs, copies = rotate(base, base[0].numel() * 4 + base[1].numel() * 4)
        vals = torch.empty((w.rows, w.k), dtype=torch.float32, device=dev)
        idx = torch.empty((w.rows, w.k), dtype=torch.int32, device=dev)

        def step(i):
            ps, pi = inputs[i % len(inputs)]
            api.topk_pooled_select(ps, pi, w.group, w.k, w.n, out=(vals, idx), stream=stream)

        def parity():
            sample = sorted({r for r in (0, 1, w.rows // 2, w.rows - 1) if r < w.rows})
            rv, ri = oracle.pooled_topk(w.pool_scores[sample], w.pool_idx[sample], w.group, w.k, w.n)
            gv, gi = vals.cpu().numpy()[sample], idx.cpu().numpy()[sample]
            return (np.array_equal(gi, ri) and np.array_equal(gv.view(np.uint32), rv.view(np.uint32)),
                    sample)

        def cpu(cores):
            t0 = time.perf_counter()
            oracle.pooled_topk(w.pool_scores, w.pool_idx, w.group, w.k, w.n)
            return time.perf_counter() - t0, 4 * w.pool_scores.size, f"all {w.rows} pooled rows"

        read = 4 * w.pool_scores.size
        c.update(rows=w.rows, read_bytes=read, copies=copies, step=step, parity=parity, cpu=cpu,
                 cpu_cores=lambda cores: 1,
                 kernel="radix_select_kernel",
                 metric="effective HBM read GB/s of pooled scores for top-512 inside "
                        "2,000-block pools (16,000 candidates per row)",
                 config={"workload": w.description, "rows": w.rows, "n": w.n, "k": w.k,
                         "group": w.group, "keep": w.keep})
        c["set_copies"] = lambda m: None
        return c

    wname = "adverse" if name == "pool" else name
    w = workloads.make(wname)
    rows, n, k = w.rows, w.n, w.k
    base = torch.from_numpy(w.scores).to(dev)
    lengths = torch.from_numpy(w.lengths).to(dev) if w.lengths is not None else None
    inputs, copies = rotate([base], base.numel() * 4)

    def set_copies(m):
        inputs[:] = [[base]] + [[base.clone()] for _ in range(m - 1)]

    sample = sorted({r for r in (0, 1, rows // 2, rows - 1) if r < rows})
    sl = w.lengths[sample] if w.lengths is not None else None
    if name == "pool":
        vals = torch.empty((rows, POOL_KEEP), dtype=torch.float32, device=dev)
        idx = torch.empty((rows, POOL_KEEP), dtype=torch.int32, device=dev)

        def step(i):
            api.topk_block_pool(inputs[i % len(inputs)][0], POOL_GROUP, POOL_KEEP, POOL_PINNED,
                                lengths, out=(vals, idx), stream=stream)

        def ref(x, ln, cores):
            return oracle.block_pool(x, POOL_GROUP, POOL_KEEP, POOL_PINNED, ln)

        kernel = "block_max8_kernel + radix_select_kernel (whole call)"
        metric = ("effective HBM read GB/s of 1M fp32 scores/row for the block-max pool "
                  f"(blocks of {POOL_GROUP}, {POOL_KEEP:,} kept, {POOL_PINNED} newest pinned)")
        config = {"workload": w.description + f"; block-max pool, blocks of {POOL_GROUP}, "
                  f"keep {POOL_KEEP}, {POOL_PINNED} pinned", "rows": rows, "n": n,
                  "group": POOL_GROUP, "keep": POOL_KEEP, "pinned": POOL_PINNED}
        cores_used = lambda cores: 1
    elif name == "vocab":
        vals = torch.empty((rows, k), dtype=torch.float32, device=dev)
        idx = torch.empty((rows, k), dtype=torch.int32, device=dev)

        def step(i):
            api.topk_select_radix(inputs[i % len(inputs)][0], k, lengths, out=(vals, idx),
                                  stream=stream)

        def ref(x, ln, cores):
            return oracle.topk(x, k, ln, threads=cores)

        kernel = "radix_select_kernel"
        metric = f"effective HBM read GB/s (and rows/s) for top-{k:,} of {n:,} fp32 scores/row"
        config = {"workload": w.description, "rows": rows, "n": n, "k": k}
        cores_used = lambda cores: cores
    else:
        vals = torch.empty((rows, k), dtype=torch.float32, device=dev)
        idx = torch.empty((rows, k), dtype=torch.int32, device=dev)

        def step(i):
            api.topk_select(inputs[i % len(inputs)][0], k, lengths, out=(vals, idx), stream=stream)

        def ref(x, ln, cores):
            return oracle.topk(x, k, ln, threads=cores)

        # topk_select takes the radix path on wide lists over many short
        # rows (the library's routing rule, mirrored here for the labels)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        routed = routed_to_radix(rows, n, k, cus)
        kernel = "radix_select_kernel" if routed else "select_kernel"
        metric = METRIC_SELECT
        plan = api.topk_plan(rows, n, k)
        config = {"workload": w.description, "rows": rows, "n": n, "k": k,
                  "path": "radix" if routed else "streaming"}
        if not routed:
            config.update(split=plan["split"], waves=plan["waves"])
        cores_used = lambda cores: cores

    def parity():
        rv, ri = ref(w.scores[sample], sl, 4)
        gv, gi = vals.cpu().numpy()[sample], idx.cpu().numpy()[sample]
        return (np.array_equal(gi, ri) and np.array_equal(gv.view(np.uint32), rv.view(np.uint32)),
                sample)

    def cpu(cores):
        t0 = time.perf_counter()
        ref(w.scores, w.lengths, cores)
        return (time.perf_counter() - t0, 4 * w.valid_elements(),
                f"all {rows} rows of the batch")

    def extras():
        """Per-row counts of scores that entered a tray and of threshold-raising
        selections (the schedule's own instrumentation, one extra call), and
        torch.topk on the same rows for context."""
        out = {}
        if name == "pool":
            return out
        # the oracle single-threaded on a few rows, beside the threaded baseline
        few = min(rows, 8)
        t0 = time.perf_counter()
        oracle.topk(w.scores[:few], k, w.lengths[:few] if w.lengths is not None else None,
                    threads=1)
        dt = time.perf_counter() - t0
        few_bytes = 4 * (few * n if w.lengths is None
                         else int(np.clip(w.lengths[:few], 0, n).sum()))
        out["cpu_single_thread"] = {"value": round(few_bytes / dt / 1e9, 3), "unit": "GB/s",
                                    "rows_per_s": round(few / dt, 1), "cores": 1,
                                    "sample": f"{few} rows, one pass, {dt:.2f} s wall"}
        if kernel == "select_kernel":
            st = torch.zeros((rows, 2), dtype=torch.int64, device=dev)
            ws = api.new_workspace(rows, n, k, plan["split"]) if plan["split"] > 1 else None
            api.topk_select_ex(base, k, lengths, stats=st, workspace=ws, stream=stream)
            torch.cuda.synchronize()
            e = st.cpu().numpy().astype(np.float64)
            st2 = torch.zeros((rows, 2), dtype=torch.int64, device=dev)
            if ws is not None:
                api.topk_workspace_init(ws)
            api.topk_select_ex(base, k, lengths, stats=st2, workspace=ws, stream=stream,
                               flags=_lib.TOPK_FLAG_NO_ESTIMATE)
            torch.cuda.synchronize()
            e2 = st2.cpu().numpy().astype(np.float64)
            S = plan["split"]
            nb = -(-n // 1024)
            bound = S * 1.5 * plan["tray_words"] * harmonic(max(1, nb // S))
            out["entrants"] = {"mean": round(float(e[:, 0].mean()), 1), "max": int(e[:, 0].max()),
                               "sorts_mean": round(float(e[:, 1].mean()), 2),
                               "sorts_max": int(e[:, 1].max()),
                               "no_estimate_mean": round(float(e2[:, 0].mean()), 1),
                               "no_estimate_max": int(e2[:, 0].max()),
                               "bound_1.5_B_H": round(bound, 1),
                               "pages_bound": 29000,
                               "per": "row (all segments of a split row); the bound sums "
                                      "1.5 x tray capacity x H(blocks per segment) over the "
                                      f"{S} segments"}
            if lengths is None:
                tv, _ = torch.topk(base, k, dim=1)
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(5):
                    torch.topk(base, k, dim=1)
                e1.record(stream)
                torch.cuda.synchronize()
                t_us = e0.elapsed_time(e1) / 5 * 1e3
                same = bool(torch.equal(tv.cpu(), vals.cpu()))
                out["torch_topk"] = {"us_per_call": round(t_us, 1),
                                     "GBps": round(4 * w.valid_elements() / (t_us * 1e-6) / 1e9, 1),
                                     "values_equal": same, "note": "context only"}
        return out

    c.update(rows=rows, read_bytes=4 * w.valid_elements(), copies=copies, step=step,
             parity=parity, cpu=cpu, cpu_cores=cores_used, kernel=kernel, metric=metric,
             config=config, set_copies=set_copies, extras=extras)
    return c


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="adverse",
                    choices=["small", "outlier", "one_row", "adverse", "ragged", "pool", "pooled",
                             "vocab", "decode"],
                    help="pool: topk_block_pool over the adverse rows (blocks of 8, keep 2,000, "
                         "16 pinned); pooled: topk_pooled_select over 2,000-block pools; "
                         "vocab: topk_select_radix, top-4,096 of 129,000-score rows; "
                         "decode: topk_sparse_decode over 512 selected positions per row")
    ap.add_argument("--copies", type=int, default=0,
                    help="input copies to rotate over (0: enough for >= 1.5 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--profile-run", action="store_true",
                    help="only the timed selection launches (for rocprofv3 counter runs)")
    ap.add_argument("--probe-sweep", action="store_true",
                    help="sweep the streaming-read probe and write profiles/read_probe_sweep.md")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the headline's context lines (rows sweep, other configs)")
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
    if args.probe_sweep:
        res = probe_sweep(torch, api, dev)
        print(f"[bench] wrote {write_probe_summary(res)}", file=sys.stderr, flush=True)
        print(json.dumps(res), flush=True)
        return 0

    stream = torch.cuda.current_stream(dev)
    print(f"[bench] generating workload {args.workload}", file=sys.stderr, flush=True)
    case = make_case(args.workload, dev, np, torch, api, workloads)
    rows, read_bytes, copies = case["rows"], case["read_bytes"], case["copies"]
    if args.copies:
        case["set_copies"](args.copies)
        copies = args.copies
    step = case["step"]

    # parity on sampled rows of copy 0 (the full-size parity tests cover all rows)
    parity = None
    if not args.profile_run:
        step(0)
        torch.cuda.synchronize()
        ok, sample = case["parity"]()
        parity = (f"{case.get('parity_kind', 'bit-exact vs oracle')} on rows {sample}" if ok
                  else "MISMATCH")
        if not ok:
            print("[bench] parity mismatch against the oracle", file=sys.stderr)

    for i in range(args.warmup):
        step(i + 1)
    torch.cuda.synchronize()

    # The timed region: K steps back to back, events only at its two ends (an
    # event pair around every launch would hold each launch until the one
    # before has ended and cost several microseconds a step).
    K = args.steps
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_all0.record(stream)
    for i in range(K):
        step(args.warmup + 1 + i)
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall1 = time.perf_counter()
    total_ms = t_all0.elapsed_time(t_all1)
    ms_per_step = total_ms / K
    # Launch durations (the roofline's): the same K steps once more, each
    # bracketed by its own pair of events on the launch stream.
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        starts[i].record(stream)
        step(args.warmup + 1 + K + i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    kern_ms = float(np.mean(per_launch_ms))
    print(f"[bench] {K} steps: {ms_per_step * 1e3:.1f} us/step, wall {1e3 * (wall1 - wall0) / K:.3f} "
          f"ms/step; launch durations over {K} more: mean {kern_ms * 1e3:.1f} us, median "
          f"{np.median(per_launch_ms) * 1e3:.1f} us", file=sys.stderr, flush=True)

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
        # the library's read probe (the sweep's best shape) over 2 GiB
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
        # Repeat the oracle's pass over the sample until about 15 s of CPU
        # work (wall time x threads) have run, at most 20 passes or 30 s.
        cores = host_cores()
        used = case["cpu_cores"](cores)
        total, passes, done_bytes = 0.0, 0, 0
        while True:
            dt, sample_bytes, sample = case["cpu"](cores)
            total += dt
            passes += 1
            done_bytes += sample_bytes
            if total * used >= 15.0 or passes >= 20 or total >= 30.0:
                break
        cpu = {"value": round(done_bytes / total / 1e9, 3), "unit": "GB/s", "cores": used,
               "kind": "oracle",
               "sample": f"{sample}, {passes} pass{'es' if passes > 1 else ''}, {total:.2f} s wall"}

    extra = {}
    if "extras" in case and not args.profile_run:
        extra = case["extras"]()
    context = None
    if args.workload == "adverse" and not args.no_context:
        context = headline_extras(dev, torch, api, workloads)

    traffic = load_traffic(args.workload)
    roofline = {
        "kernel": case["kernel"],
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": traffic["bytes_per_launch"] if traffic else None,
    }
    out = {
        "metric": case["metric"],
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
        "config": dict(case["config"], read_bytes_per_step=read_bytes, input_copies=copies),
        "rows_per_s": round(rows / (ms_per_step * 1e-3), 1),
        "kernel_us_mean": round(kern_ms * 1e3, 2),
        "kernel_us_median": round(float(np.median(per_launch_ms)) * 1e3, 2),
        "kernel_us_p10": round(float(np.percentile(per_launch_ms, 10)) * 1e3, 2),
        "kernel_us_p90": round(float(np.percentile(per_launch_ms, 90)) * 1e3, 2),
        "read_probe_GBps": round(probe, 1) if probe else None,
        "frac_of_read_probe": round(achieved / probe, 4) if probe else None,
        "entrants": extra.get("entrants"),
        "context": context,
        "torch_topk": extra.get("torch_topk"),
        "host": host_cpu(),
        "cpu_single_thread": extra.get("cpu_single_thread"),
        "parity": parity,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
