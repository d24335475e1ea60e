"""Throughput of LSH-sampled decode attention on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
the table build of the batch's keys (SimHash projection, bucket build) and
one decode step (query hash, probe and count, selection, weighted attention,
log-sum-exp merge).  Steps rotate over ``--copies`` independent input copies;
step i builds the tables of copy i mod R and decodes copy (i - 1) mod R, whose
tables were built one step earlier, so the decode does not read tables that
the build just left in the 256 MB last-level cache.

Prints ONE JSON line.  ``value`` is query-heads per second of whole steps
(build + decode), timed over steps replayed from HIP graphs (``--launch
eager`` launches them one by one instead); the decode alone is reported under
``breakdown``.  The ``roofline`` object is for the kernel with the largest
total time, from the library's per-dispatch timing events in a separate eager
pass over the same steps; ``cpu_baseline`` times the fp64 CPU oracle on a
bounded sample of the same workload.  Two more sections time consecutive
hybrid decodes (exact sinks + recent window) and decode steps that append one
key to a growing cache and update its tables (``--headline-only`` skips them).

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

BUILD_KERNELS = ("transpose_w", "project_codes", "chunk_sort")
DECODE_KERNELS = ("qhash", "count_select", "attend", "merge")
KERNEL_SOURCES = {
    "transpose_w": "build_kernels.hip", "project_codes": "build_kernels.hip",
    "chunk_sort": "build_kernels.hip", "qhash": "decode_kernels.hip",
    "count_select": "decode_kernels.hip", "attend": "attend_bf16.hip",
    "merge": "decode_kernels.hip",
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
                    help="skip the hybrid and growing-cache sections (profiling runs: every launch of a "
                         "kernel then has the headline workload's shape)")
    ap.add_argument("--hybrid-sink", type=int, default=4,
                    help="sink keys of the hybrid decode timed beside the plain one")
    ap.add_argument("--hybrid-window", type=int, default=1024,
                    help="recent-window keys of the hybrid decode timed beside the plain one")
    ap.add_argument("--launch", choices=("graph", "eager"), default="graph",
                    help="replay each step from a HIP graph (default) or launch it eagerly")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def source_digest(kernel):
    h = hashlib.sha256()
    for f in (KERNEL_SOURCES[kernel], "lsh_device.h", "lsh_kernels.h"):
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by "
              "(sequence, kv head) without exchange, but no multi-GPU run is built here.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
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

    # ---------------------------------------------------------------- inputs
    copies = []
    for r in range(R):
        data = workloads.generate(cfg.with_(seed=cfg.seed + 1000 * r), device=dev)
        c = {"keys": data["keys"], "values": data["values"], "W": data["W"],
             "q": data["q"][0].contiguous()}
        c["offsets"] = torch.empty(B, Hkv, L, nch, 1 << K, dtype=torch.int16, device=dev)
        c["indices"] = torch.empty(B, Hkv, L, N, dtype=torch.int16, device=dev)
        c["bws"] = torch.empty(max(1, lsh.lsh_build_workspace_size(B, Hkv, N, d, K, L, stride, dt)),
                               dtype=torch.uint8, device=dev)
        c["dws"] = torch.empty(max(1, lsh.lsh_decode_workspace_size(B, Hq, Hkv, N, d, K, L, stride)),
                               dtype=torch.uint8, device=dev)
        c["out"] = torch.empty(B, Hq, d, dtype=torch.float32, device=dev)
        c["lse"] = torch.empty(B, Hq, dtype=torch.float32, device=dev)
        c["nsel"] = torch.empty(B, Hq, dtype=torch.int32, device=dev)
        copies.append(c)
        del data
    torch.cuda.synchronize()

    def build(c):
        lsh.lsh_build_tables(c["keys"], c["W"], K, L, stride, c["offsets"], c["indices"], None, c["bws"])

    def decode(c, counts=None):
        lsh.lsh_decode_attention(c["q"], c["keys"], c["values"], c["W"], c["indices"], c["offsets"], K, L, T,
                                 stride, cfg.scale, c["out"], c["lse"], c["nsel"], None, counts, c["dws"])

    def decode_hybrid(c):
        lsh.lsh_decode_attention_hybrid(c["q"], c["keys"], c["values"], c["W"], c["indices"], c["offsets"], K, L,
                                        T, stride, cfg.scale, args.hybrid_sink, args.hybrid_window, c["out"],
                                        c["lse"], c["nsel"], None, None, c["dws"])

    def step(i):
        build(copies[i % R])
        decode(copies[(i - 1) % R])

    for c in copies:
        build(c)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- timed
    # Steps are replayed from HIP graphs (one per input copy) unless --launch
    # eager; the kernels and their arguments are those of the eager step.
    launch_mode = args.launch
    graphs = []
    if launch_mode == "graph":
        try:
            for r in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step(r)
                graphs.append(g)
            for i in range(R):
                graphs[i].replay()
            torch.cuda.synchronize()
        except Exception as exc:  # capture unsupported here: time eager launches instead
            print(f"graph capture failed ({exc}); timing eager launches", file=sys.stderr)
            launch_mode, graphs = "eager", []

    def run(i):
        if graphs:
            graphs[i % R].replay()
        else:
            step(i)

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, args.warmup + args.steps):
        run(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # per-dispatch kernel times from a second, eager pass (events ride on the
    # dispatch packets, so they are not part of the timed steps above)
    lsh.lsh_timing_begin()
    for i in range(args.warmup, args.warmup + args.steps):
        step(i)
    ktimes = lsh.lsh_timing_end()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    qh = B * Hq
    value = qh / (ms_per_step * 1e-3)

    # ------------------------------------------- measured selection statistics
    # (untimed) one decode per copy with the collision counts returned
    counts = torch.empty(B, Hq, N, dtype=torch.uint8, device=dev)
    sel_rows = []    # sum over (b, g) of |union of the group's selections|
    idx_entries = []  # sum over heads of probed-bucket entries = sum of counts
    nsel_tot = []
    for c in copies:
        decode(c, counts)
        torch.cuda.synchronize()
        m = (counts >= T).view(B, Hkv, G, N)
        sel_rows.append(int(m.any(dim=2).sum().item()))
        idx_entries.append(int(counts.sum(dtype=torch.int64).item()))
        nsel_tot.append(int(c["nsel"].sum().item()))
    U_rows = float(np.mean(sel_rows))
    E_idx = float(np.mean(idx_entries))

    # algorithmic bytes / flops per launch
    kv_bytes = U_rows * 2 * d * esz
    tables = B * Hkv * L
    csr_out = tables * (N * 2 + nch * (1 << K) * 2)   # uint16 indices + per-chunk bucket offsets
    alg = {
        "project_codes": ("mfma", 2.0 * d * K * L * B * Hkv * N),
        # codes read once, CSR written once
        "chunk_sort": ("hbm", tables * N * 2 + csr_out),
        "transpose_w": ("hbm", 2.0 * d * L * K * esz),
        "qhash": ("hbm", qh * d * esz + d * L * K * esz + qh * L * 2),
        # probed entries, query codes, two bucket offsets per (head, table, chunk), bitmask
        "count_select": ("hbm", E_idx * 2 + qh * L * 2 + qh * L * nch * 4 + qh * N / 8),
        "attend": ("hbm", kv_bytes + qh * d * esz + qh * N / 8),
        "merge": ("hbm", 0.0),
    }
    def kernel_table(times):
        out = {}
        for name, (tot_ms, n) in times.items():
            if n == 0:
                continue
            avg_ms = tot_ms / n
            bound, amount = alg[name]
            rec = {"avg_us": round(avg_ms * 1e3, 3), "launches": n, "total_ms": round(tot_ms, 4), "bound": bound}
            if bound == "mfma":
                rec["achieved_tflops"] = round(amount / (avg_ms * 1e-3) / 1e12, 2)
            elif amount > 0:
                rec["achieved_gbs"] = round(amount / (avg_ms * 1e-3) / 1e9, 2)
            out[name] = rec
        return out

    def roofline_of(name, rec, traffic):
        if rec["bound"] == "mfma":
            peak = MFMA_BF16_PEAK_TFLOPS if cfg.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
            r = {"kernel": name, "bound": "mfma", "achieved": rec["achieved_tflops"], "peak": peak,
                 "unit": "TFLOP/s", "frac": round(rec["achieved_tflops"] / peak, 4)}
        else:
            r = {"kernel": name, "bound": "hbm", "achieved": rec["achieved_gbs"], "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": round(rec["achieved_gbs"] / HBM_PEAK_GBS, 4)}
        r["avg_us"] = rec["avg_us"]
        r["traffic"] = traffic
        return r

    kernels = kernel_table(ktimes)
    dom = max(kernels, key=lambda k: kernels[k]["total_ms"])
    roof = roofline_of(dom, kernels[dom], measured_traffic(cfg.name, dom))

    # decode alone in steady state: consecutive decode steps over the rotating
    # copies with no table build in between (the build's ~0.5 GB of writes
    # otherwise reach HBM while the next decode reads)
    lsh.lsh_timing_begin()
    torch.cuda.synchronize()
    td0 = time.perf_counter()
    for i in range(args.steps):
        decode(copies[i % R])
    torch.cuda.synchronize()
    td1 = time.perf_counter()
    dtimes = lsh.lsh_timing_end()
    dkernels = kernel_table(dtimes)
    dec_ms_steady = sum(dtimes[k][0] for k in DECODE_KERNELS) / args.steps

    decode_hybrid_steady = append_decode = None
    if not args.headline_only:
        # the hybrid decode in steady state: the exact sink + window set runs as
        # extra attention workgroups, the selection leaves those keys out
        lsh.lsh_timing_begin()
        for i in range(args.steps):
            decode_hybrid(copies[i % R])
        htimes = lsh.lsh_timing_end()
        hk = kernel_table(htimes)
        n_exact = min(N, args.hybrid_sink + args.hybrid_window)
        hyb_ms = sum(htimes[k][0] for k in DECODE_KERNELS) / args.steps
        decode_hybrid_steady = {
            "n_sink": args.hybrid_sink, "n_window": args.hybrid_window,
            "ms": round(hyb_ms, 5),
            "qh_per_s": round(qh / (hyb_ms * 1e-3), 1),
            "merge_avg_us": hk["merge"]["avg_us"],
            # keys and values of the exact set, once per (sequence, kv head)
            "exact_kv_bytes": int(B * Hkv * n_exact * 2 * d * esz),
            "kernels": {k: v["avg_us"] for k, v in hk.items()},
        }

        # multi-step decode over a growing cache: each step appends one key (the
        # chunk it falls into is rebuilt) and runs the hybrid decode over the
        # keys held.  The cache starts half-way into its last chunk, the average
        # rebuild size; the tables of the first chunks stay as built.
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
        ak = kernel_table(atimes)
        append_ms = sum(v[0] for v in atimes.values()) / args.steps
        append_decode = {
            "keys_held": [n_start + 1, n_start + args.steps],
            "ms": round(append_ms, 5),
            "wall_ms_per_step": round((ta1 - ta0) * 1e3 / args.steps, 5),
            "update_ms": round(sum(atimes[k][0] for k in BUILD_KERNELS) / args.steps, 5),
            "qh_per_s": round(qh / (append_ms * 1e-3), 1),
            "kernels": {k: v["avg_us"] for k, v in ak.items()},
        }

    build_ms = sum(ktimes[k][0] for k in BUILD_KERNELS) / args.steps
    decode_ms = sum(ktimes[k][0] for k in DECODE_KERNELS) / args.steps
    dec_bytes = E_idx * 2 + qh * L * 8 + kv_bytes + qh * d * (esz + 4) + d * L * K * esz
    decode_steady = {
        "ms": round(dec_ms_steady, 5),
        "wall_ms_per_step": round((td1 - td0) * 1e3 / args.steps, 5),
        "qh_per_s": round(qh / (dec_ms_steady * 1e-3), 1),
        "hbm_frac": round(dec_bytes / (dec_ms_steady * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "attend_roofline": roofline_of("attend", dkernels["attend"], measured_traffic(cfg.name, "attend")),
        "kernels": dkernels,
    }

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
                   "kv_dtype": cfg.dtype, "stride": stride, "step": "table build + 1 decode step", "launch": launch_mode,
                   "input_copies": R},
        "roofline": roof,
        "breakdown": {
            "build_ms": round(build_ms, 5),
            "decode_ms": round(decode_ms, 5),
            "decode_qh_per_s": round(qh / (decode_ms * 1e-3), 1),
            "decode_alg_bytes": int(dec_bytes),
            "decode_hbm_frac": round(dec_bytes / (decode_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "build_keys_per_s": round(B * Hkv * N / (build_ms * 1e-3), 1),
            "selected_union_rows": U_rows,
            "selected_frac_of_keys": round(U_rows / (B * Hkv * N), 4),
            "nsel_mean_per_head": float(np.mean(nsel_tot)) / qh,
            "probed_index_entries": E_idx,
            "kernels": kernels,
            "decode_steady": decode_steady,
            "decode_hybrid_steady": decode_hybrid_steady,
            "append_decode_steady": append_decode,
        },
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, copies[0], stride)
    print(json.dumps(line), flush=True)


def cpu_baseline(cfg, c, stride, budget_s=10.0):
    """The fp64 oracle on (sequence, kv head) units in order, each unit's
    table build plus the decode of its G query heads, until about
    ``budget_s`` seconds of CPU work or the whole step is done; the rate is
    query heads decoded (with their tables built) per second."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import lsh_oracle as O

    W = c["W"].float().cpu().numpy()
    units = cfg.B * cfg.Hkv
    done = 0
    t0 = time.perf_counter()
    while done < units and (done == 0 or time.perf_counter() - t0 < budget_s):
        b, g = divmod(done, cfg.Hkv)
        keys = c["keys"][b, g].float().cpu().numpy()
        vals = c["values"][b, g].float().cpu().numpy()
        q = c["q"][b].float().cpu().numpy()
        tb = O.build_tables(keys, W, cfg.K, cfg.L, stride)
        for h in range(g * cfg.G, (g + 1) * cfg.G):
            O.decode_head(q[h], keys, vals, W, tb["offsets"], tb["indices"], cfg.K, cfg.L, cfg.T, cfg.scale)
        done += 1
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(done * cfg.G / dt, 3), "unit": "queries·heads/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} of {units} (sequence, kv head) units of one step: fp64 table build of {cfg.N} "
                      f"keys + decode of the unit's {cfg.G} query heads each, {dt:.2f} s in all; BLAS threads "
                      f"{threads} (matmuls), the rest single-threaded numpy"}


if __name__ == "__main__":
    main()
