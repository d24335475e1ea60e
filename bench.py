"""Throughput of LSH-sampled decode attention on one MI355X.

The metric is decode query-heads per second: one step is one decode step of
every query head of the batch (query hash, bucket probe and collision count,
selection, 1/u-weighted attention over the selected keys, log-sum-exp merge)
against tables built at prefill.  The tables of every input copy are built
before the timed region, as prefill does; the build is timed on its own and
reported under ``breakdown.build`` (with the build + decode step), since it
runs once per sequence, not once per generated token.

Steps rotate over ``--copies`` independent input copies (keys, values,
tables, queries), so the decode never finds the previous step's K/V rows in
the 256 MB last-level cache.  ``value`` comes from eager launches of the
steps (``--launch graph``: from steps replayed from HIP graphs, one per
copy); both are timed and reported.
``roofline`` is the dominant decode kernel's fraction of the HBM peak on its
algorithmic bytes (per-dispatch HIP events on the library's stream, in a
separate eager pass) and, under ``roofline.decode``, the whole decode's.
``breakdown`` carries every kernel's figures, the measured selection, the
estimate's relative L2 error against exact attention (computed on the GPU by
the same kernels with every key in the exact set), the table build, a
centred-plant variant of the workload (sparse selection), the hybrid decode
and decode steps over a growing cache.  ``cpu_baseline`` times the fp64 CPU
oracle's decode on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4] [--launch graph|eager]
                       [--hybrid-sink S] [--hybrid-window W] [--headline-only] [--no-cpu-baseline]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
MFMA_F32_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA, TFLOP/s

BUILD_KERNELS = ("transpose_w", "project_codes", "chunk_sort", "chunk_insert")
DECODE_KERNELS = ("qhash", "decode")
KERNEL_SOURCES = {
    "transpose_w": ("build_kernels.hip",), "project_codes": ("build_kernels.hip",),
    "chunk_sort": ("build_kernels.hip",), "chunk_insert": ("build_kernels.hip",), "qhash": ("decode_kernels.hip",),
    "decode": ("attend_bf16.hip", "decode_roles.h"),
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4, help="workload id in workloads.CONFIGS (default: 128K GQA-8)")
    ap.add_argument("--copies", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline decode (profiling runs: every decode launch then has the "
                         "headline workload's shape and selection)")
    ap.add_argument("--hybrid-sink", type=int, default=4,
                    help="sink keys of the hybrid decode timed beside the plain one")
    ap.add_argument("--hybrid-window", type=int, default=1024,
                    help="recent-window keys of the hybrid decode timed beside the plain one")
    ap.add_argument("--launch", choices=("graph", "eager"), default="eager",
                    help="launch mode behind `value` (both are timed and reported; eager is the faster for the "
                         "two-launch decode)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    ap.add_argument("--ingest-counters", metavar="DIR",
                    help="no GPU work: read the rocprofv3 counter CSVs under DIR/fetch, DIR/write (FETCH_SIZE, "
                         "WRITE_SIZE of a bench run) and DIR/calib_fetch, DIR/calib_write (the same counters of "
                         "--copy-calibration) and write profiles/traffic_<workload>.json and .md")
    ap.add_argument("--ingest-pmc", metavar="DIR",
                    help="no GPU work: average every counter of the rocprofv3 --pmc CSVs under DIR (one pass per "
                         "subdirectory) over the launches of --pmc-kernel and write "
                         "profiles/pmc_<kernel>_<workload>.md")
    ap.add_argument("--pmc-kernel", default="project_codes", help="kernel kind for --ingest-pmc")
    ap.add_argument("--ingest-stats", metavar="DIR",
                    help="no GPU work: read the rocprofv3 --stats kernel CSV under DIR and write "
                         "profiles/kernel_stats_<workload>.md")
    return ap.parse_args()


def source_digest(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel] + ("lsh_device.h", "lsh_kernels.h"):
        with open(os.path.join(ROOT, "lsh_sampled_sparse_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None
    when there are none or the kernel source changed since they were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel)
    if not rec or rec.get("source_digest") != source_digest(kernel):
        return None
    return rec["bytes_per_launch"]


def copy_calibration():
    """A plain elementwise kernel (torch.neg over 2^28 fp32 = 1 GiB) that reads
    exactly 1 GiB and writes exactly 1 GiB: the reference against which the
    HBM byte counters (FETCH_SIZE, WRITE_SIZE) are scaled."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": 4 * n, "launches": 5, "kernel": "torch.neg fp32"}), flush=True)


# rocprofv3 kernel names -> the library's kernel kinds
KERNEL_PATTERNS = (("qhash_kernel", "qhash"), ("decode_bf16_kernel", "decode"), ("decode_f32_kernel", "decode"),
                   ("project_codes", "project_codes"), ("chunk_sort", "chunk_sort"), ("chunk_insert", "chunk_insert"),
                   ("transpose_w", "transpose_w"))


def _counter_values(d, counter):
    """(kernel name, value) of every dispatch in the counter CSVs under d."""
    import csv
    import glob
    rows = []
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no {counter} rows under {d}")
    return rows


def ingest_counters(d, workload):
    """HBM bytes per launch of every library kernel from two counter runs,
    scaled by what the same counters read for the 1 GiB copy."""
    calib = {}
    for counter, sub in (("FETCH_SIZE", "calib_fetch"), ("WRITE_SIZE", "calib_write")):
        vals = [v for name, v in _counter_values(os.path.join(d, sub), counter) if "neg" in name]
        if not vals:
            raise SystemExit(f"no copy kernel in {sub}")
        calib[counter] = sum(vals) / len(vals)
    scale = {"FETCH_SIZE": float(1 << 30) / calib["FETCH_SIZE"], "WRITE_SIZE": float(1 << 30) / calib["WRITE_SIZE"]}
    per = {}
    for counter, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        for name, v in _counter_values(os.path.join(d, sub), counter):
            kind = next((k for pat, k in KERNEL_PATTERNS if pat in name), None)
            if kind:
                per.setdefault(kind, {}).setdefault(counter, []).append(v * scale[counter])
    rec = {"_calibration": {
        "kernel": "torch.neg fp32 over 2^28 elements (reads 1 GiB, writes 1 GiB)",
        "FETCH_SIZE_KiB": round(calib["FETCH_SIZE"], 3), "WRITE_SIZE_KiB": round(calib["WRITE_SIZE"], 3),
        "fetch_per_counted": scale["FETCH_SIZE"] / 1024.0, "write_per_counted": scale["WRITE_SIZE"] / 1024.0}}
    for kind in sorted(per):
        f, w = per[kind].get("FETCH_SIZE", [0.0]), per[kind].get("WRITE_SIZE", [0.0])
        fb, wb = sum(f) / len(f), sum(w) / len(w)
        rec[kind] = {"bytes_per_launch": int(fb + wb), "fetch_bytes": int(fb), "write_bytes": int(wb),
                     "launches": len(f), "source_digest": source_digest(kind)}
    base = os.path.join(ROOT, "profiles", f"traffic_{workload}")
    with open(base + ".json", "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    lines = [f"# HBM traffic per launch: {workload}", "",
             "Commands (from the repository root, one MI355X; one counter per run):", "", "```",
             "rocprofv3 --pmc FETCH_SIZE -f csv -d <dir>/fetch -o run -- python3 bench.py --steps 3 --warmup 1 "
             "--no-cpu-baseline --headline-only",
             "rocprofv3 --pmc WRITE_SIZE -f csv -d <dir>/write -o run -- python3 bench.py --steps 3 --warmup 1 "
             "--no-cpu-baseline --headline-only",
             "rocprofv3 --pmc FETCH_SIZE -f csv -d <dir>/calib_fetch -o run -- python3 bench.py --copy-calibration",
             "rocprofv3 --pmc WRITE_SIZE -f csv -d <dir>/calib_write -o run -- python3 bench.py --copy-calibration",
             f"python3 bench.py --ingest-counters <dir>   # writes this file and traffic_{workload}.json",
             "```", "",
             f"Scaling: the 1 GiB elementwise copy reads {calib['FETCH_SIZE']:.4g} KiB of FETCH_SIZE and writes "
             f"{calib['WRITE_SIZE']:.4g} KiB of WRITE_SIZE, so one counted KiB stands for "
             f"{scale['FETCH_SIZE'] / 1024:.4g} KiB fetched and {scale['WRITE_SIZE'] / 1024:.4g} KiB written.", "",
             "| kernel | launches | fetch MB | write MB | total MB per launch |", "|---|---|---|---|---|"]
    for kind in sorted(per):
        r = rec[kind]
        lines.append(f"| {kind} | {r['launches']} | {r['fetch_bytes'] / 1e6:.1f} | {r['write_bytes'] / 1e6:.1f} | "
                     f"{r['bytes_per_launch'] / 1e6:.1f} |")
    with open(base + ".md", "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(json.dumps({k: v.get("bytes_per_launch") for k, v in rec.items() if k != "_calibration"}))


def ingest_pmc(d, kind, workload):
    """Per-launch averages of hardware counters for one kernel kind, with the
    MFMA rate and utilisation they imply (MI355X: 1024 SIMDs)."""
    import csv
    import glob
    vals, durs, passes = {}, [], []
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        seen = set()
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if next((k for pat, k in KERNEL_PATTERNS if pat in r["Kernel_Name"]), None) != kind:
                    continue
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                seen.add(r["Counter_Name"])
                if r["Dispatch_Id"] not in {x[0] for x in durs}:
                    durs.append((r["Dispatch_Id"], (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9))
        if seen:
            passes.append(sorted(seen))
    if not vals:
        raise SystemExit(f"no {kind} launches under {d}")
    avg = {k: sum(v) / len(v) for k, v in vals.items()}
    dur = sum(x[1] for x in durs) / len(durs)
    lines = [f"# Hardware counters of {kind}: {workload}", "",
             "Commands (from the repository root, one MI355X; one pass per run):", "", "```"]
    for cs in passes:
        lines.append(f"rocprofv3 --pmc {' '.join(cs)} --kernel-include-regex {kind} -f csv -d <dir>/<pass> -o run "
                     "-- python3 bench.py --steps 3 --warmup 1 --no-cpu-baseline --headline-only")
    lines += [f"python3 bench.py --ingest-pmc <dir> --pmc-kernel {kind}   # writes this file", "```", "",
              f"Averages over the launches of each pass; mean launch duration under counters {dur * 1e6:.1f} µs.",
              "", "| counter | per launch |", "|---|---|"]
    for k in sorted(avg):
        lines.append(f"| {k} | {avg[k]:.6g} |")
    derived = []
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in avg:
        fl = avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        derived.append(f"- bf16 MFMA work: {fl / 1e9:.1f} GFLOP per launch (512 FLOP per counted MOP), "
                       f"{fl / dur / 1e12:.0f} TFLOP/s over the launch = "
                       f"{fl / dur / 1e12 / MFMA_BF16_PEAK_TFLOPS:.1%} of the 2.5 PFLOP/s dense bf16 peak")
    if "MfmaUtil" in avg:
        derived.append(f"- MFMA busy (MfmaUtil: MFMA-busy cycles over GUI-active cycles x 1024 SIMDs): "
                       f"{avg['MfmaUtil']:.1f}%")
    if "SQ_LDS_BANK_CONFLICT" in avg and avg.get("SQ_LDS_IDX_ACTIVE"):
        derived.append(f"- LDS bank-conflict cycles per active LDS cycle: "
                       f"{avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_LDS_IDX_ACTIVE']:.3f}")
    if "SQ_INSTS_VALU" in avg and avg.get("SQ_INSTS_MFMA"):
        derived.append(f"- VALU instructions per MFMA instruction: {avg['SQ_INSTS_VALU'] / avg['SQ_INSTS_MFMA']:.2f}")
    if avg.get("SQ_BUSY_CYCLES"):
        # summed over the 32 shader engines (8 XCDs x 4): cycles of one engine
        cyc = avg["SQ_BUSY_CYCLES"] / 32.0
        derived.append(f"- cycles per launch: {cyc:.4g} (SQ_BUSY_CYCLES over the 32 shader engines), "
                       f"{cyc / dur / 1e9:.2f} GHz over the mean launch duration")
        for k, what in (("SQ_LDS_IDX_ACTIVE", "LDS active"), ("SQ_LDS_BANK_CONFLICT", "LDS bank-conflict")):
            if k in avg:
                derived.append(f"- {what} cycles per CU: {avg[k] / 256:.4g} = {avg[k] / 256 / cyc:.1%} of the launch "
                               f"({avg[k] / 256 / cyc * dur * 1e6:.1f} µs), over 256 CUs")
    if avg.get("SQ_WAVE_CYCLES") and "SQ_WAIT_ANY" in avg:
        derived.append(f"- wave-cycles spent waiting (SQ_WAIT_ANY / SQ_WAVE_CYCLES): "
                       f"{avg['SQ_WAIT_ANY'] / avg['SQ_WAVE_CYCLES']:.1%}")
    if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg:
        h, m = avg["TCC_HIT_sum"], avg["TCC_MISS_sum"]
        derived.append(f"- L2 hit rate: {h / (h + m):.1%} of {h + m:.4g} requests")
    if derived:
        lines += ["", "Derived:", ""] + derived
    path = os.path.join(ROOT, "profiles", f"pmc_{kind}_{workload}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(path)


def ingest_stats(d, cfg):
    """Per-kernel duration statistics of a rocprofv3 --kernel-trace --stats run."""
    import csv
    import glob
    paths = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    if not paths:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    rows = []
    with open(paths[0], newline="") as f:
        for r in csv.DictReader(f):
            rows.append(r)
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# rocprofv3 kernel statistics: {cfg.name} (B={cfg.B}, Hq={cfg.Hq}, Hkv={cfg.Hkv}, N={cfg.N}, "
             f"d={cfg.d}, K={cfg.K}, L={cfg.L}, T={cfg.T}, {cfg.dtype})", "",
             "Commands (from the repository root, one MI355X):", "", "```",
             "rocprofv3 --kernel-trace --stats -f csv -d <dir> -o run -- python3 bench.py --steps 20 --warmup 5 "
             "--no-cpu-baseline --headline-only",
             "python3 bench.py --ingest-stats <dir>   # writes this file", "```", "",
             "The bench runs warmup + 20 graph-replayed steps, then 20 eager steps with per-dispatch events, "
             "then the selection-statistics decodes (one per input copy with the collision counts returned, one "
             "without), so the call counts differ per kernel. `--headline-only` leaves out every other section "
             "(the build timing aside), so every decode launch has the workload's shape.", "",
             "| kernel | calls | avg µs | min µs | max µs | share of GPU time |", "|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        name = r["Name"]
        kind = next((k for pat, k in KERNEL_PATTERNS if pat in name), None)
        if kind is None:
            continue
        short = name.replace("void ", "").replace("lsh::", "").split("(")[0]
        lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{100.0 * float(r['TotalDurationNs']) / total:.2f}% |")
    path = os.path.join(ROOT, "profiles", f"kernel_stats_{cfg.name}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print(path)


def kernel_table(times, alg):
    """Per-kernel averages from a timing window, with achieved rates on the
    algorithmic bytes or flops of one launch."""
    out = {}
    for name, (tot_ms, n) in times.items():
        if n == 0:
            continue
        avg_ms = tot_ms / n
        bound, amount = alg.get(name, ("hbm", 0.0))
        rec = {"avg_us": round(avg_ms * 1e3, 3), "launches": n, "total_ms": round(tot_ms, 4), "bound": bound}
        if bound == "mfma":
            rec["achieved_tflops"] = round(amount / (avg_ms * 1e-3) / 1e12, 2)
        elif amount > 0:
            rec["achieved_gbs"] = round(amount / (avg_ms * 1e-3) / 1e9, 2)
            rec["alg_bytes"] = int(amount)
        out[name] = rec
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by "
              "(sequence, kv head) without exchange, but no multi-GPU run is built here.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.ingest_counters:
        import workloads
        ingest_counters(args.ingest_counters, workloads.CONFIGS[args.config].name)
        return
    if args.ingest_pmc:
        import workloads
        ingest_pmc(args.ingest_pmc, args.pmc_kernel, workloads.CONFIGS[args.config].name)
        return
    if args.ingest_stats:
        import workloads
        ingest_stats(args.ingest_stats, workloads.CONFIGS[args.config])
        return

    import numpy as np
    import torch

    import lsh_sampled_sparse_amd as lsh
    import workloads

    lsh.lib()   # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        raise RuntimeError("bench.py needs a GPU")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = workloads.CONFIGS[args.config]
    B, Hq, Hkv, N, d, K, L, T = cfg.B, cfg.Hq, cfg.Hkv, cfg.N, cfg.d, cfg.K, cfg.L, cfg.T
    G = cfg.G
    R = max(1, args.copies)
    stride = lsh.lsh_default_stride(N, K)
    nch = lsh.lsh_num_chunks(N, stride)
    dt = lsh.LSH_BF16 if cfg.dtype == "bf16" else lsh.LSH_F32
    esz = 2 if cfg.dtype == "bf16" else 4
    qh = B * Hq
    full = not args.headline_only

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ---------------------------------------------------------------- inputs
    copies = []
    for r in range(R):
        seed = cfg.seed + 1000 * r
        data = workloads.generate(cfg.with_(seed=seed), device=dev)
        c = {"keys": data["keys"], "values": data["values"], "W": data["W"], "q": data["q"][0].contiguous()}
        del data
        if full:
            # the same keys, values and W; queries planted on the centred keys
            c["q_centred"] = workloads.generate(cfg.with_(seed=seed, plant="centred"), device=dev)["q"][0].contiguous()
        c["offsets"] = torch.empty(B, Hkv, L, nch, 1 << K, dtype=torch.int16, device=dev)
        c["indices"] = torch.empty(B, Hkv, L, N, dtype=torch.int16, device=dev)
        c["bws"] = torch.empty(max(1, lsh.lsh_build_workspace_size(B, Hkv, N, d, K, L, stride, dt)),
                               dtype=torch.uint8, device=dev)
        c["dws"] = torch.empty(max(1, lsh.lsh_decode_workspace_size(B, Hq, Hkv, N, d, K, L, stride)),
                               dtype=torch.uint8, device=dev)
        for k in ("out", "out_exact"):
            c[k] = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
        c["lse"] = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        c["nsel"] = torch.empty(B, Hq, dtype=torch.int32, device=dev)
        copies.append(c)
        torch.cuda.empty_cache()
    torch.cuda.synchronize()
    log(f"inputs ready: {cfg.name}, {R} copies")

    def build(c):
        lsh.lsh_build_tables(c["keys"], c["W"], K, L, stride, c["offsets"], c["indices"], None, c["bws"])

    def decode(c, q=None, counts=None, out=None):
        lsh.lsh_decode_attention(c["q"] if q is None else q, c["keys"], c["values"], c["W"], c["indices"],
                                 c["offsets"], K, L, T, stride, cfg.scale, c["out"] if out is None else out,
                                 c["lse"], c["nsel"], None, counts, c["dws"])

    def decode_hybrid(c, n_sink, n_window, q=None, out=None):
        lsh.lsh_decode_attention_hybrid(c["q"] if q is None else q, c["keys"], c["values"], c["W"], c["indices"],
                                        c["offsets"], K, L, T, stride, cfg.scale, n_sink, n_window,
                                        c["out"] if out is None else out, c["lse"], c["nsel"], None, None, c["dws"])

    def capture(fn):
        """One HIP graph per input copy of fn(copy); None where capture fails."""
        try:
            gs = []
            for r in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    fn(copies[r])
                gs.append(g)
            for g in gs:
                g.replay()
            torch.cuda.synchronize()
            return gs
        except Exception as exc:  # capture unsupported here: eager only
            log(f"graph capture failed ({exc})")
            return None

    def timed(fn, graphs, steps, warmup, offset=0):
        """Wall ms per step over `steps` steps after `warmup`, rotating copies."""
        run = (lambda i: graphs[i % R].replay()) if graphs else (lambda i: fn(copies[i % R]))
        for i in range(warmup):
            run(offset + i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            run(offset + warmup + i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps

    def kernel_times(fn, steps, offset=0):
        lsh.lsh_timing_begin()
        for i in range(steps):
            fn(copies[(offset + i) % R])
        return lsh.lsh_timing_end()

    # prefill: the tables of every copy (untimed; the build is timed below)
    for c in copies:
        build(c)
        decode(c)      # one eager decode per copy: every kernel's one-time set-up before any capture
    torch.cuda.synchronize()

    # ------------------------------------------------- headline: decode steps
    dec_graphs = capture(decode)
    ms_graph = timed(decode, dec_graphs, args.steps, args.warmup) if dec_graphs else None
    ms_eager = timed(decode, None, args.steps, args.warmup)
    launch_mode = args.launch if dec_graphs else "eager"
    ms_per_step = ms_graph if launch_mode == "graph" else ms_eager
    log(f"decode: graph {ms_graph} ms, eager {ms_eager:.4f} ms per step")
    dtimes = kernel_times(decode, args.steps)

    # ------------------------------------------- measured selection statistics
    # (untimed) one decode per copy with the collision counts returned, and
    # the estimate's error against exact attention: the hybrid decode with
    # every key in the exact set is exact softmax attention on the same kernels
    counts = torch.empty(B, Hq, N, dtype=torch.uint8, device=dev)

    def selection_stats(qkey):
        sel_rows, idx_entries, nsel_tot, errs = [], [], [], []
        for c in copies:
            q = c[qkey]
            decode(c, q=q, counts=counts)
            if full:   # a profiling run (--headline-only) keeps every decode launch at the workload's shape
                decode_hybrid(c, N, 0, q=q, out=c["out_exact"])
            decode(c, q=q)
            torch.cuda.synchronize()
            m = (counts >= T).view(B, Hkv, G, N)
            sel_rows.append(int(m.any(dim=2).sum().item()))
            idx_entries.append(int(counts.sum(dtype=torch.int64).item()))
            nsel_tot.append(int(c["nsel"].sum().item()))
            if full:
                num = (c["out"] - c["out_exact"]).norm(dim=-1)
                den = c["out_exact"].norm(dim=-1).clamp_min(1e-30)
                errs.append((num / den).flatten().cpu().numpy())
        e = np.concatenate(errs) if errs else None
        U_rows, E_idx = float(np.mean(sel_rows)), float(np.mean(idx_entries))
        return {
            "U_rows": U_rows, "E_idx": E_idx,
            "selected_union_rows": U_rows,
            "selected_frac_of_keys": round(U_rows / (B * Hkv * N), 4),
            "nsel_mean_per_head": round(float(np.mean(nsel_tot)) / qh, 1),
            "nsel_frac_per_head": round(float(np.mean(nsel_tot)) / qh / N, 4),
            "probed_index_entries": E_idx,
            "estimate_rel_l2_vs_exact": None if e is None else {
                "mean": round(float(e.mean()), 4), "median": round(float(np.median(e)), 4),
                "max": round(float(e.max()), 4), "heads": int(e.size)},
        }

    sel = selection_stats("q")

    def decode_alg(s):
        """Algorithmic bytes of one decode launch per kernel and in all: probed
        bucket entries (uint16), two uint16 bucket offsets per (head, table,
        chunk), the union of the group's selected K/V rows once per (sequence,
        kv head), q in and fp32 out, W once."""
        kv = s["U_rows"] * 2 * d * esz
        idx = s["E_idx"] * 2
        offs = qh * L * nch * 2 * 2
        qio = qh * d * (esz + 4)
        w = d * L * K * esz
        per = {
            # q in, W, query codes out
            "qhash": ("hbm", qh * d * esz + w + qh * L * 2),
            # query codes, probed entries, bucket offsets, selected K/V rows, q, fp32 out
            "decode": ("hbm", qh * L * 2 + idx + offs + kv + qio),
        }
        return per, kv + idx + offs + qio + w

    dalg, dec_bytes = decode_alg(sel)
    dkernels = kernel_table(dtimes, dalg)
    dec_kernel_us = sum(dkernels[k]["avg_us"] for k in DECODE_KERNELS if k in dkernels)
    dom = max((k for k in DECODE_KERNELS if k in dkernels), key=lambda k: dkernels[k]["total_ms"])
    drec = dkernels[dom]
    roof = {"kernel": dom, "bound": "hbm", "achieved": drec["achieved_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(drec["achieved_gbs"] / HBM_PEAK_GBS, 4), "avg_us": drec["avg_us"],
            "alg_bytes": drec["alg_bytes"], "traffic": measured_traffic(cfg.name, dom),
            "decode": {"kernels": [k for k in DECODE_KERNELS if k in dkernels], "kernel_sum_us": round(dec_kernel_us, 3),
                       "alg_bytes": int(dec_bytes),
                       "achieved": round(dec_bytes / (dec_kernel_us * 1e-6) / 1e9, 2),
                       "frac": round(dec_bytes / (dec_kernel_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                       "wall_frac": round(dec_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}}
    value = qh / (ms_per_step * 1e-3)

    # -------------------------------------------------------------- the build
    tables = B * Hkv * L
    build_bytes = B * Hkv * N * d * esz + tables * (N * 2 + nch * (1 << K) * 2)
    balg = {
        "project_codes": ("mfma", 2.0 * d * K * L * B * Hkv * N),
        # the codes workspace: read once (written by the projection)
        "chunk_sort": ("hbm", tables * N * 2 + tables * (N * 2 + nch * (1 << K) * 2)),
        "transpose_w": ("hbm", 2.0 * d * L * K * esz),
    }
    build_graphs = capture(build)
    ms_build_graph = timed(build, build_graphs, args.steps, 2) if build_graphs else None
    btimes = kernel_times(build, args.steps)
    bkernels = kernel_table(btimes, balg)
    build_kernel_ms = sum(btimes[k][0] for k in BUILD_KERNELS) / args.steps
    build_ms = ms_build_graph if ms_build_graph else build_kernel_ms
    proj = bkernels.get("project_codes")
    peak_mfma = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
    build_rec = {
        "ms": round(build_ms, 5), "launch": "graph" if ms_build_graph else "eager",
        "kernel_sum_ms": round(build_kernel_ms, 5),
        "alg_bytes": int(build_bytes),
        "hbm_frac": round(build_bytes / (build_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "keys_per_s": round(B * Hkv * N / (build_ms * 1e-3), 1),
        "flops": 2.0 * d * K * L * B * Hkv * N,
        "project_mfma_frac": round(proj["achieved_tflops"] / peak_mfma, 4) if proj else None,
        "project_traffic": measured_traffic(cfg.name, "project_codes"),
        "chunk_sort_traffic": measured_traffic(cfg.name, "chunk_sort"),
        "kernels": bkernels,
    }
    log(f"build: {build_ms:.4f} ms")

    # the whole path: build the batch's tables, then decode one step over the
    # tables built one step earlier (another copy)
    def step(i):
        build(copies[i % R])
        decode(copies[(i - 1) % R])

    step_rec = None
    if full:
        step_graphs = []
        try:
            for r in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step(r)
                step_graphs.append(g)
        except Exception as exc:
            log(f"graph capture of the step failed ({exc})")
            step_graphs = None
        for i in range(args.warmup):
            step_graphs[i % R].replay() if step_graphs else step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step_graphs[i % R].replay() if step_graphs else step(i)
        torch.cuda.synchronize()
        step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        step_rec = {"ms": round(step_ms, 5), "qh_per_s": round(qh / (step_ms * 1e-3), 1),
                    "launch": "graph" if step_graphs else "eager"}
        del step_graphs
        for c in copies:
            build(c)
        torch.cuda.synchronize()

    # ---------------------------------------------- centred-plant variant
    centred = None
    if full:
        csel = selection_stats("q_centred")
        cgraphs = capture(lambda c: decode(c, q=c["q_centred"])) if launch_mode == "graph" else None
        cms = timed(lambda c: decode(c, q=c["q_centred"]), cgraphs, args.steps, args.warmup)
        ctimes = kernel_times(lambda c: decode(c, q=c["q_centred"]), args.steps)
        calg, cbytes = decode_alg(csel)
        ck = kernel_table(ctimes, calg)
        c_us = sum(ck[k]["avg_us"] for k in DECODE_KERNELS if k in ck)
        centred = {k: v for k, v in csel.items() if k not in ("U_rows", "E_idx")}
        centred.update({
            "plant": "q planted on k_j - mu (the keys' shared offset removed); same keys, values, W and tables",
            "ms_per_step": round(cms, 5), "launch": "graph" if cgraphs else "eager",
            "qh_per_s": round(qh / (cms * 1e-3), 1),
            "alg_bytes": int(cbytes),
            "hbm_frac": round(cbytes / (c_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "wall_hbm_frac": round(cbytes / (cms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_sum_us": round(c_us, 3),
            "kernels": {k: v["avg_us"] for k, v in ck.items()},
        })
        del cgraphs
        log(f"centred plant: {cms:.4f} ms, selected {centred['selected_frac_of_keys']}")

    decode_hybrid_steady = append_decode = decode_per_head_w = decode_ragged = None
    if full:
        # the hybrid decode: the exact sink + window set runs as extra
        # attention workgroups, the selection leaves those keys out
        htimes = kernel_times(lambda c: decode_hybrid(c, args.hybrid_sink, args.hybrid_window), args.steps)
        hk = kernel_table(htimes, {})
        n_exact = min(N, args.hybrid_sink + args.hybrid_window)
        hyb_ms = sum(htimes[k][0] for k in DECODE_KERNELS) / args.steps
        decode_hybrid_steady = {
            "n_sink": args.hybrid_sink, "n_window": args.hybrid_window,
            "kernel_sum_ms": round(hyb_ms, 5),
            "qh_per_s": round(qh / (hyb_ms * 1e-3), 1),
            # keys and values of the exact set, once per (sequence, kv head)
            "exact_kv_bytes": int(B * Hkv * n_exact * 2 * d * esz),
            "kernels": {k: v["avg_us"] for k, v in hk.items()},
        }

        # one SimHash projection per kv head (W [Hkv, d, L*K]): tables built
        # with kv head g's W[g], query head h hashed with W[h / G]
        c0 = copies[0]
        Wh = workloads.per_head_projections(cfg, seed=cfg.seed + 1000, device=dev).contiguous()
        aux_off, aux_idx = torch.empty_like(c0["offsets"]), torch.empty_like(c0["indices"])
        lsh.lsh_update_tables(c0["keys"], Wh, K, L, stride, 0, N, aux_off, aux_idx, None, c0["bws"])

        def decode_ph(c):
            lsh.lsh_decode_attention_cached(c0["q"], c0["keys"], c0["values"], Wh, aux_idx, aux_off, N, K, L, T,
                                            stride, cfg.scale, 0, 0, c0["out"], c0["lse"], c0["nsel"], None, None,
                                            c0["dws"])
        decode_ph(c0)
        ptimes = kernel_times(decode_ph, args.steps)
        ph_ms = sum(ptimes[k][0] for k in DECODE_KERNELS) / args.steps
        decode_per_head_w = {"kernel_sum_ms": round(ph_ms, 5), "qh_per_s": round(qh / (ph_ms * 1e-3), 1),
                             "kernels": {k: v["avg_us"] for k, v in kernel_table(ptimes, {}).items()}}

        # ragged lengths (batches only): sequence b holds N - (b mod 4) N / 8
        # keys, its tables built over those keys (per-sequence lengths on the
        # device), and the decode attends each sequence's own keys
        if B > 1:
            lens = [N - (b % 4) * (N // 8) for b in range(B)]
            lens_t = torch.tensor(lens, dtype=torch.int32, device=dev)
            zeros_t = torch.zeros_like(lens_t)
            lsh.lsh_update_tables(c0["keys"], c0["W"], K, L, stride, 0, N, aux_off, aux_idx, None, c0["bws"],
                                  old_lens=zeros_t, new_lens=lens_t)

            def decode_rg(c):
                lsh.lsh_decode_attention_cached(c0["q"], c0["keys"], c0["values"], c0["W"], aux_idx, aux_off, N, K,
                                                L, T, stride, cfg.scale, 0, 0, c0["out"], c0["lse"], c0["nsel"],
                                                None, None, c0["dws"], seq_lens=lens_t)
            decode_rg(c0)
            rtimes = kernel_times(decode_rg, args.steps)
            rg_ms = sum(rtimes[k][0] for k in DECODE_KERNELS) / args.steps
            decode_ragged = {"lens": sorted(set(lens), reverse=True), "kernel_sum_ms": round(rg_ms, 5),
                             "qh_per_s": round(qh / (rg_ms * 1e-3), 1),
                             "keys_per_s": round(sum(lens) * Hkv / (rg_ms * 1e-3), 1),
                             "kernels": {k: v["avg_us"] for k, v in kernel_table(rtimes, {}).items()}}
        del aux_off, aux_idx
        torch.cuda.synchronize()

        # multi-step decode over a growing cache: each step appends one key
        # (inserted into the chunk it falls into) and runs the hybrid decode
        # over the keys held.  The cache starts half-way into its last chunk,
        # so an insert moves half a chunk of entries on average.
        c0 = copies[0]
        n_start = max(1, N - stride // 2)
        lsh.lsh_timing_begin()
        ta0 = time.perf_counter()
        for i in range(args.steps):
            n = n_start + i
            lsh.lsh_update_tables(c0["keys"], c0["W"], K, L, stride, n, n + 1, c0["offsets"], c0["indices"], None,
                                  c0["bws"])
            lsh.lsh_decode_attention_cached(c0["q"], c0["keys"], c0["values"], c0["W"], c0["indices"], c0["offsets"],
                                            n + 1, K, L, T, stride, cfg.scale, args.hybrid_sink, args.hybrid_window,
                                            c0["out"], c0["lse"], c0["nsel"], None, None, c0["dws"])
        torch.cuda.synchronize()
        ta1 = time.perf_counter()
        atimes = lsh.lsh_timing_end()
        # back to the tables of all N keys
        lsh.lsh_update_tables(c0["keys"], c0["W"], K, L, stride, n_start, N, c0["offsets"], c0["indices"], None,
                              c0["bws"])
        torch.cuda.synchronize()
        ak = kernel_table(atimes, {})
        append_ms = sum(v[0] for v in atimes.values()) / args.steps
        append_decode = {
            "keys_held": [n_start + 1, n_start + args.steps],
            "kernel_sum_ms": round(append_ms, 5),
            "wall_ms_per_step": round((ta1 - ta0) * 1e3 / args.steps, 5),
            "update_ms": round(sum(atimes[k][0] for k in BUILD_KERNELS) / args.steps, 5),
            "qh_per_s": round(qh / (append_ms * 1e-3), 1),
            "kernels": {k: v["avg_us"] for k, v in ak.items()},
        }

    headline = {k: v for k, v in sel.items() if k not in ("U_rows", "E_idx")}
    line = {
        "metric": "LSH-attn decode queries·heads/s at 32K–128K ctx; % of HBM roofline",
        "value": round(value, 1),
        "unit": "queries·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "Hq": Hq, "Hkv": Hkv, "N": N, "d": d, "K": K, "L": L, "T": T,
                   "kv_dtype": cfg.dtype, "stride": stride,
                   "step": "one decode step of every query head over tables built at prefill",
                   "launch": launch_mode, "input_copies": R},
        "roofline": roof,
        "breakdown": {
            "decode_graph_ms": round(ms_graph, 5) if ms_graph else None,
            "decode_eager_ms": round(ms_eager, 5),
            "decode_eager_qh_per_s": round(qh / (ms_eager * 1e-3), 1),
            "decode_kernel_sum_us": round(dec_kernel_us, 3),
            "decode_alg_bytes": int(dec_bytes),
            "decode_hbm_frac": roof["decode"]["frac"],
            "decode_wall_hbm_frac": roof["decode"]["wall_frac"],
            **headline,
            "kernels": dkernels,
            "build": build_rec,
            "step_build_plus_decode": step_rec,
            "centred_plant": centred,
            "decode_hybrid_steady": decode_hybrid_steady,
            "append_decode_steady": append_decode,
            "decode_per_head_w": decode_per_head_w,
            "decode_ragged": decode_ragged,
        },
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, copies[0], stride)
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, c, stride, budget_s=10.0):
    """The fp64 oracle's decode on (sequence, kv head) units in order: each
    unit's tables are built first (untimed, as prefill), then the decode of
    its G query heads is timed, until about ``budget_s`` seconds of decode or
    the whole step is done; the rate is query heads decoded per second."""
    from threadpoolctl import threadpool_info

    from oracle import lsh_oracle as O

    W = c["W"].float().cpu().numpy()
    units = cfg.B * cfg.Hkv
    done = 0
    spent = 0.0
    while done < units and (done == 0 or spent < budget_s):
        b, g = divmod(done, cfg.Hkv)
        keys = c["keys"][b, g].float().cpu().numpy()
        vals = c["values"][b, g].float().cpu().numpy()
        q = c["q"][b].float().cpu().numpy()
        tb = O.build_tables(keys, W, cfg.K, cfg.L, stride)
        t0 = time.perf_counter()
        for h in range(g * cfg.G, (g + 1) * cfg.G):
            O.decode_head(q[h], keys, vals, W, tb["offsets"], tb["indices"], cfg.K, cfg.L, cfg.T, cfg.scale)
        spent += time.perf_counter() - t0
        done += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(done * cfg.G / spent, 3), "unit": "queries·heads/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of {units} (sequence, kv head) units of one step: fp64 decode of the unit's "
                      f"{cfg.G} query heads over its {cfg.N} keys, {spent:.2f} s of decode in all (each unit's "
                      f"tables built first, untimed); BLAS threads {threads} (matmuls), the rest "
                      f"single-threaded numpy"}


if __name__ == "__main__":
    main()
