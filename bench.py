"""Benchmark of the paged KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: the Qwen3-1.7B-shaped decode layer -- B=32 sequences, 16 query /
8 KV heads, head_dim 128, 16-token blocks, contexts uniform in [512, 640],
a 1,378-block (22,048-token) pool per layer, bf16.  One step = the step's
append (one new token per sequence) + paged decode attention, on resident
device inputs, run as one pa_decode_append launch (the separate append and
decode launches are timed too, as ``unfused_step_ms``).  The pool holds 28
layers sharing one block table and each step works on the next layer, as a
model's layer loop does, so every step reads its K/V from HBM rather than
from the 256 MB Infinity Cache.

Prints one JSON line.  ``value`` is decode KV-read GB/s over the whole step
(append + decode); ``roofline`` rates the step's one kernel (the fused
append + decode) on its algorithmic bytes; the second half of the metric,
attention tokens/s at B=64, is measured on the 13B-shaped B=64 workload and
reported as ``attention_tok_s_b64``.  ``rows`` gives the other hot-path rows
on the workloads that exercise them.
"""

import argparse
import copy
import dataclasses
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
SHARED_LAYERS = 8  # layers the shared-prefix rows rotate over: 8 x 134 MB, past the 256 MB Infinity Cache

ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "paged_kv_cache_140_amd", "csrc")
# HBM bytes per launch of the counted kernels (rocprofv3 FETCH_SIZE /
# WRITE_SIZE passes over this script, calibrated against a plain copy of
# known size).  A kernel's figure is used only while its sources still hash
# to the value recorded with the counters.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
SRC = {
    "decode": ["pa_decode.hip", "pa_decode_dev.h", "pa_common.h"],
    "shared": ["pa_shared.hip", "pa_decode_dev.h", "pa_prefill_dev.h", "pa_common.h"],
    "cache": ["pa_cache.hip", "pa_common.h"],
    "prefill": ["pa_prefill.hip", "pa_prefill_dev.h", "pa_common.h"],
}
# key: (kernel name as rocprofv3 prints it up to "(", grid size or None,
# sources[, "unsplit": only dispatches not followed by a split's merge])
COUNTED = {
    "decode_b32_gqa16x8_fused": ("pa::decode_kernel<pa::BF16, 128, 2, 16, 1024, true>", None, "decode"),
    "gather_b32_gqa16x8": ("pa::gather_kernel<pa::BF16, 128, 2, 16, 1024>", None, "decode"),
    "decode_b64_mha40_bs16_fused": ("pa::decode_kernel<pa::BF16, 128, 1, 16, 1024, true>", None, "decode"),
    "decode_b64_mha40_bs16": ("pa::decode_kernel<pa::BF16, 128, 1, 16, 1024, false>", None, "decode"),
    "decode_b64_mha40_bs8": ("pa::decode_kernel<pa::BF16, 128, 1, 8, 1024, false>", None, "decode"),
    "decode_b64_mha40_bs32": ("pa::decode_kernel<pa::BF16, 128, 1, 32, 1024, false>", None, "decode"),
    "decode_shared_prefix_plain": ("pa::decode_kernel<pa::BF16, 128, 4, 16, 512, false>", None, "decode"),
    "decode_shared_prefix_shared": ("pa::shared_decode32_kernel<pa::BF16, 128, 4, 16>", None, "shared"),
    "decode_long_ctx": ("pa::decode_kernel<pa::BF16, 128, 8, 16, 512, false>", None, "decode"),
    "append_2048": ("pa::append_kernel", 524288, "cache"),
    "copy_blocks_56": ("pa::copy_blocks_kernel", 1835008, "cache"),  # 56 pairs x 8 layers
    "prefill_chunk_1024": ("pa::prefill_chunk_kernel<pa::BF16, 128, 8, 16>", 131072, "prefill", "unsplit"),
}
HEADLINE = "decode_b32_gqa16x8_fused"
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def sources_sha256(names):
    import hashlib

    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(key):
    """HBM bytes per launch of a counted kernel from the committed counter
    record, or None if there is none or its sources changed since."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f).get("kernels", {}).get(key)
    if not rec or rec.get("source_sha256") != sources_sha256(SRC[COUNTED[key][2]]):
        return None
    return rec.get("traffic_bytes_per_launch")


def traffic_fields(key, algorithmic):
    t = recorded_traffic(key)
    return {"traffic_bytes": t, "traffic_over_algorithmic": round(t / algorithmic, 4) if t else None}


def write_traffic_record(fetch_dir, write_dir, out_path=TRAFFIC_FILE):
    """Turn two rocprofv3 counter runs of this script (``--pmc FETCH_SIZE``,
    then ``--pmc WRITE_SIZE``, each ``-f csv``) into the record the rows'
    ``traffic`` fields come from.  Each counter is summed over its instances
    per dispatch, the median dispatch of each counted kernel is taken, and
    the counter is scaled by what it reads for the 512 MiB plain copy this
    script runs first (true size known)."""
    import csv
    import glob
    import statistics

    def per_dispatch(d, counter):
        path = max(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True), key=os.path.getmtime)
        acc, meta = {}, {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                k = int(r["Dispatch_Id"])
                acc[k] = acc.get(k, 0.0) + float(r["Counter_Value"])
                meta[k] = (r["Kernel_Name"], int(r["Grid_Size"]))
        return acc, meta

    def short(n):
        return n.split("(")[0].replace("void ", "").strip()

    def pick(acc, meta, name, grid, unsplit=False):
        ids = sorted(meta)
        nxt = {a: short(meta[b][0]) for a, b in zip(ids, ids[1:])}
        return [v for k, v in acc.items()
                if short(meta[k][0]) == name and (grid is None or meta[k][1] == grid)
                and not (unsplit and "merge_kernel" in nxt.get(k, ""))]

    fetch, fmeta = per_dispatch(fetch_dir, "FETCH_SIZE")
    write, wmeta = per_dispatch(write_dir, "WRITE_SIZE")
    copy_kib = (512 << 20) / 1024
    f_copy = max(pick(fetch, fmeta, COPY_KERNEL, None))
    w_copy = max(pick(write, wmeta, COPY_KERNEL, None))
    f_scale, w_scale = copy_kib / f_copy, copy_kib / w_copy
    kernels = {}
    for key, (name, grid, src, *flags) in COUNTED.items():
        unsplit = "unsplit" in flags
        fv, wv = pick(fetch, fmeta, name, grid, unsplit), pick(write, wmeta, name, grid, unsplit)
        if not fv or not wv:
            continue
        f_med, w_med = statistics.median(fv), statistics.median(wv)
        kernels[key] = {
            "kernel": name, "grid_size": grid, "dispatches": len(fv),
            "fetch_size_kib_per_dispatch_median": f_med, "write_size_kib_per_dispatch_median": w_med,
            "fetch_bytes_per_launch": int(round(f_med * f_scale * 1024)),
            "write_bytes_per_launch": int(round(w_med * w_scale * 1024)),
            "traffic_bytes_per_launch": int(round((f_med * f_scale + w_med * w_scale) * 1024)),
            "source_sha256": sources_sha256(SRC[src]), "sources": SRC[src]}
    rec = {
        "what": "HBM bytes per launch of each counted kernel on this script's workloads (median dispatch)",
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE -f csv -d {fetch_dir} -o run -- python3 bench.py --steps 20 --warmup 5 "
            "--no-cpu-baseline",
            f"rocprofv3 --pmc WRITE_SIZE -f csv -d {write_dir} -o run -- python3 bench.py --steps 20 --warmup 5 "
            "--no-cpu-baseline",
            f"python bench.py --traffic-record {fetch_dir} {write_dir}",
        ],
        "calibration": {"kernel": COPY_KERNEL + " (torch copy of 512 MiB, run first by bench.py)",
                        "fetch_size_kib": f_copy, "write_size_kib": w_copy, "true_kib": copy_kib,
                        "fetch_scale": f_scale, "write_scale": w_scale},
        "kernels": kernels,
    }
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps({k: v["traffic_bytes_per_launch"] for k, v in kernels.items()}))


def write_trace_summary(trace_dir, out_path=os.path.join(ROOT, "profiles", "bench_kernel_trace_stats.md")):
    """Summarise a ``rocprofv3 --kernel-trace --stats -f csv`` run of this
    script: per kernel (name and grid), dispatches and median / mean / min
    duration from the trace, next to the tool's own stats."""
    import csv
    import glob
    import statistics

    path = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)[0]
    by = {}
    with open(path) as f:
        recs = sorted(csv.DictReader(f), key=lambda r: int(r["Dispatch_Id"]))
    for i, r in enumerate(recs):
        name = r["Kernel_Name"].split("(")[0].replace("void ", "").strip()
        if not name.startswith("pa::"):
            continue
        grid = int(r["Grid_Size"]) if "Grid_Size" in r else \
            int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])
        if name.startswith("pa::prefill_chunk_kernel") and i + 1 < len(recs) and \
                "prefill_merge_kernel" in recs[i + 1]["Kernel_Name"]:
            name += " (split; merge follows)"
        key = (name, grid)
        by.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    lines = ["# rocprofv3 kernel trace of bench.py", "",
             "Command (from the repository root; `cd /tmp && export TMPDIR=/tmp` first):", "",
             f"    rocprofv3 --kernel-trace --stats -f csv -d {trace_dir} -o run -- python3 bench.py --steps 20 "
             "--warmup 5 --no-cpu-baseline",
             f"    python bench.py --trace-summary {trace_dir}", "",
             "Durations in us, per kernel and grid size; eager warm-up dispatches included (the bench's own "
             "figures time graph replays after warm-up).", "",
             "| kernel | grid | dispatches | median | mean | min |", "|---|---|---|---|---|---|"]
    for (name, grid), d in sorted(by.items(), key=lambda x: -sum(x[1])):
        lines.append(f"| `{name}` | {grid} | {len(d)} | {statistics.median(d):.2f} | {statistics.mean(d):.2f} | "
                     f"{min(d):.2f} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(out_path)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=28, help="layers the step rotates over (cache-cold reads)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle sample length")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true", help="skip the other workloads' rows")
    ap.add_argument("--copy-calibration-mib", type=int, default=512,
                    help="size of a plain device copy run once before timing (counter calibration)")
    ap.add_argument("--traffic-record", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic record from two rocprofv3 counter runs, then exit (no GPU)")
    ap.add_argument("--trace-summary", metavar="TRACE_DIR",
                    help="write profiles/bench_kernel_trace_stats.md from a rocprofv3 trace run, then exit (no GPU)")
    return ap.parse_args()


# ------------------------------------------------------------------ bytes/flops

def decode_bytes(lens, H_kv, H_q, d, bs, s):
    """Algorithmic bytes of one decode: every visible K and V once per KV head,
    q and out, and the block-table entries read."""
    lens = [int(x) for x in lens]
    kv = sum(lens) * H_kv * d * 2 * s
    qo = 2 * len(lens) * H_q * d * s
    tables = 4 * sum(-(-n // bs) for n in lens)
    return kv + qo + tables


def append_bytes(T, H_kv, d, s):
    return 2 * (2 * T * H_kv * d * s) + 4 * T


def prefill_flops(T, H_q, d, ctx_before):
    return 4 * H_q * d * (T * ctx_before + T * (T + 1) // 2)


# ------------------------------------------------------------------ timing

def time_replays(torch, fn, iters, warmup, replays):
    """Sorted ms per call of each of ``replays`` timed replays (see time_loop)."""
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(warmup + i)
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / iters)
    del g
    return sorted(times)


def spread(times):
    """median, p10 and p90 of per-replay times (nearest rank)."""
    n = len(times)
    return {"median": round(times[n // 2], 5), "p10": round(times[int(0.1 * (n - 1) + 0.5)], 5),
            "p90": round(times[int(0.9 * (n - 1) + 0.5)], 5), "replays": n}


def time_loop(torch, fn, iters, warmup, replays=5):
    """Average ms per call of fn(i) over ``iters`` consecutive calls.

    ``warmup`` eager calls first; then the ``iters`` calls are captured in one
    HIP graph (the library enqueues plain kernel launches, no memsets), the
    graph is replayed once untimed, and then ``replays`` more times, each
    timed with events on the current stream; the median replay is reported.
    A graph keeps the host's per-call marshalling (tens of microseconds of
    Python) out of kernels that take ~10 us.
    """
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(warmup + i)
    g.replay()
    torch.cuda.synchronize()
    times = []
    for _ in range(replays):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b) / iters)
    del g
    return sorted(times)[len(times) // 2]


def main():
    args = parse()
    if args.traffic_record:
        write_traffic_record(*args.traffic_record)
        return 0
    if args.trace_summary:
        write_trace_summary(args.trace_summary)
        return 0
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU only: the hot path is measured on one GPU's share; "
                                   "run with --gpus 1"}), flush=True)
        return 2

    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        return 2
    import paged_kv_cache_140_amd as pa  # raises if libpa.so is missing
    from paged_kv_cache_140_amd.runner import DeviceRun
    from pa_inputs import build_scenario

    pa.lib()
    dev = "cuda"
    t_start = time.time()

    # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE under rocprofv3
    # calibrate the counters of the kernels below.
    nbytes = args.copy_calibration_mib << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).random_()
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    # ---------------------------------------------------------- headline: config 2
    scn = build_scenario(2, 0)
    cfg = scn.cfg
    L = args.layers
    gpu = DeviceRun(scn, device=dev, num_layers=L, fill="randn")
    gpu.run_setup()
    step = scn.steps[0]
    si = gpu.prepare(step)
    lens = si.lens.cpu().numpy()
    s = 2
    dbytes = decode_bytes(lens, cfg["H_kv"], cfg["H_q"], cfg["d"], cfg["bs"], s)
    abytes = append_bytes(len(step.appends), cfg["H_kv"], cfg["d"], s)

    def full_step(i):
        gpu.layer = i % L
        gpu.launch(si, fused=True)

    def unfused_step(i):
        gpu.layer = i % L
        gpu.launch(si)

    def decode_only(i):
        gpu.layer = i % L
        gpu.launch(si, do_copy=False, do_append=False)

    def append_only(i):
        gpu.layer = i % L
        gpu.launch(si, do_decode=False, do_prefill=False)

    assert si.fusable and si.n_pairs == 0  # the step is exactly one fused launch
    step_times = time_replays(torch, full_step, args.steps, args.warmup, 11)
    ms_step = step_times[len(step_times) // 2]
    ms_unfused = time_loop(torch, unfused_step, args.steps, args.warmup)
    decode_times = time_replays(torch, decode_only, args.steps, args.warmup, 11)
    ms_decode = decode_times[len(decode_times) // 2]
    ms_append = time_loop(torch, append_only, args.steps, args.warmup)

    # Gather ceiling: pa_decode's own grid, tables, unit walk and loads with
    # no arithmetic (pa_gather_checksum), on the same layers; and the same
    # walk over tables that place each sequence's blocks back to back.
    B2 = len(lens)
    cs_buf = torch.empty(max(pa.pa_gather_checksum_size(gpu.pool, B2, cfg["H_q"], si.max_ctx) // 4, 1),
                         dtype=torch.int32, device=dev)

    def gather_scattered(i):
        pa.pa_gather_checksum(gpu.pool, i % L, cfg["H_q"], si.tables, si.lens, si.max_ctx, cs_buf)

    nblk = [-(-int(n) // cfg["bs"]) for n in lens]
    contig = np.zeros(tuple(si.tables.shape), dtype=np.int32)
    off = 0
    for r_, nb in enumerate(nblk):
        contig[r_, :nb] = np.arange(off, off + nb)
        off += nb
    assert off <= cfg["num_blocks"]
    contig_d = torch.from_numpy(contig).to(dev)

    def gather_contiguous(i):
        pa.pa_gather_checksum(gpu.pool, i % L, cfg["H_q"], contig_d, si.lens, si.max_ctx, cs_buf)

    # Fixed cost per launch: the plain decode of the same batch and tables
    # with every context cut to 1/2 and 1/4 of its length; the least-squares
    # line through (bytes, ms) of the three gives the launch's fixed time
    # (intercept) and its marginal streaming rate (1 / slope).
    fit_bytes, fit_ms = [dbytes], [ms_decode]
    for div in (2, 4):
        l_f = np.maximum(lens // div, 1).astype(np.int32)
        si_f = dataclasses.replace(si, lens=torch.from_numpy(l_f).to(dev), max_ctx=int(l_f.max()),
                                   workspace=pa.decode_workspace(gpu.pool, len(l_f), cfg["H_q"], int(l_f.max())))

        def decode_cut(i, si_f=si_f):
            gpu.layer = i % L
            gpu.launch(si_f, do_copy=False, do_append=False)

        fit_ms.append(time_loop(torch, decode_cut, args.steps, args.warmup))
        fit_bytes.append(decode_bytes(l_f, cfg["H_kv"], cfg["H_q"], cfg["d"], cfg["bs"], s))
    slope, icept = np.polyfit(np.array(fit_bytes, dtype=np.float64), np.array(fit_ms), 1)
    fixed_cost = {"what": "pa_decode of the same batch and tables with contexts cut to 1, 1/2 and 1/4 of their "
                          "lengths; least-squares line through (bytes, ms)",
                  "bytes": fit_bytes, "ms": [round(x, 5) for x in fit_ms],
                  "fixed_us": round(icept * 1e3, 2), "marginal_GBps": round(1e-6 / slope, 1),
                  "marginal_hbm_frac": round(1e-6 / slope / HBM_PEAK_GBS, 4)}

    gather_times = time_replays(torch, gather_scattered, args.steps, args.warmup, 11)
    ms_gather = gather_times[len(gather_times) // 2]
    ms_gather_c = time_loop(torch, gather_contiguous, args.steps, args.warmup)
    gbytes = dbytes - 2 * B2 * cfg["H_q"] * cfg["d"] * s  # K/V and tables: what the walk reads
    value = dbytes / (ms_step * 1e-3) / 1e9
    kernel_bytes = dbytes + abytes  # the fused kernel also reads the new rows and writes them into the pool
    achieved = kernel_bytes / (ms_step * 1e-3) / 1e9
    plan_ws = pa.pa_decode_workspace_size(gpu.pool, len(lens), cfg["H_q"], int(lens.max()))
    del gpu, si
    torch.cuda.empty_cache()

    out = {
        "metric": "paged decode KV-read GB/s (% of HBM peak) + attention tokens/s at B=64",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "qwen3-1.7b-shaped paged decode layer: append 32 + decode, B=32, GQA 16/8, head_dim 128, "
                        "block 16, ctx U[512,640] (+1 appended), 1,378-block pool per layer, 28 layers rotated",
            "B": 32, "H_q": 16, "H_kv": 8, "head_dim": 128, "block_size": 16, "pool_blocks": 1378,
            "layers_rotated": L, "seed": 0,
        },
        "timing": "HIP graph of K steps replayed 11 times (the headline, decode and gather figures; 5 times for the "
                  "other rows) after W eager warmup steps and one untimed replay; each replay timed with events, "
                  "the median replay reported",
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "step_ms_spread": spread(step_times),
        "decode_ms_spread": spread(decode_times),
        "gather_ceiling": {
            "what": "pa_gather_checksum: the decode's grid, block tables, unit walk and K/V loads, every loaded dword "
                    "XORed into a checksum, no softmax; same layers rotated, same timing",
            "scattered_ms": round(ms_gather, 5),
            "scattered_GBps": round(gbytes / (ms_gather * 1e-3) / 1e9, 1),
            "scattered_spread": spread(gather_times),
            "contiguous_tables_ms": round(ms_gather_c, 5),
            "contiguous_tables_GBps": round(gbytes / (ms_gather_c * 1e-3) / 1e9, 1),
            "decode_over_ceiling": round(ms_gather / ms_decode, 4),
            "step_over_ceiling": round(ms_gather / ms_step, 4),
            "ceiling_hbm_frac": round(gbytes / (ms_gather * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            **traffic_fields("gather_b32_gqa16x8", gbytes)},
        "unfused_step_ms": round(ms_unfused, 5),
        "decode_ms": round(ms_decode, 5),
        "append_ms": round(ms_append, 5),
        "decode_only_GBps": round(dbytes / (ms_decode * 1e-3) / 1e9, 1),
        "decode_bytes": dbytes,
        "decode_split_workspace_bytes": plan_ws,
        "decode_fixed_cost": fixed_cost,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(HEADLINE),
            "kernel": "pa::decode_kernel<BF16,128,2,16,1024> (pa_decode_append: append + decode)",
            "per_launch_bytes": kernel_bytes,
        },
    }

    # ---------------------------------------------------------- B=64: config 3
    scn3 = build_scenario(3, 0, bs=16)
    g3 = DeviceRun(scn3, device=dev, num_layers=1, fill="randn", pad_pool=True)
    g3.run_setup()
    si3 = g3.prepare(scn3.steps[0], longest_first=True)
    # the same step launched in batch order: the launch rows permuted back
    inv = torch.from_numpy(np.argsort(si3.order)).to(dev)
    si3b = copy.copy(si3)
    for name in ("tables", "lens", "q", "k_new", "v_new", "slots"):
        setattr(si3b, name, getattr(si3, name)[inv].contiguous())
    si3b.out = torch.empty_like(si3.out)
    n3 = max(20, args.steps // 4)
    ms3 = time_loop(torch, lambda i: g3.launch(si3, fused=True), n3, 5)
    ms3d = time_loop(torch, lambda i: g3.launch(si3, do_copy=False, do_append=False), n3, 5)
    ms3_batch = time_loop(torch, lambda i: g3.launch(si3b, fused=True), n3, 5)
    lens3 = si3.lens.cpu().numpy()
    b3 = decode_bytes(lens3, 40, 40, 128, 16, 2)
    out["attention_tok_s_b64"] = round(64 / (ms3 * 1e-3), 1)
    a3 = append_bytes(64, 40, 128, 2)
    out["b64"] = {"workload": "13b-shaped MHA decode layer, B=64, 40 heads, block 16, lognormal ctx, churned pool "
                              "(0x2080000 bytes per KV head); append + decode in one launch, batch submitted "
                              "longest context first",
                  "ms_per_step": round(ms3, 5), "decode_ms": round(ms3d, 5),
                  "decode_GBps": round(b3 / (ms3d * 1e-3) / 1e9, 1),
                  "decode_hbm_frac": round(b3 / (ms3d * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                  "step_GBps": round(b3 / (ms3 * 1e-3) / 1e9, 1),
                  "batch_order_ms_per_step": round(ms3_batch, 5),
                  "step_traffic": traffic_fields("decode_b64_mha40_bs16_fused", b3 + a3),
                  "decode_traffic": traffic_fields("decode_b64_mha40_bs16", b3)}
    del g3, si3, si3b
    torch.cuda.empty_cache()
    # the same workload at the other block sizes it is specified over
    sweep = {"16": {"ms_per_step": round(ms3, 5), "decode_ms": round(ms3d, 5),
                    "decode_GBps": round(b3 / (ms3d * 1e-3) / 1e9, 1)}}
    for bs in (8, 32):
        scn_bs = build_scenario(3, 0, bs=bs)
        g_bs = DeviceRun(scn_bs, device=dev, num_layers=1, fill="randn", pad_pool=True)
        g_bs.run_setup()
        si_bs = g_bs.prepare(scn_bs.steps[0], longest_first=True)
        ms_f = time_loop(torch, lambda i: g_bs.launch(si_bs, fused=True), n3, 5)
        ms_d = time_loop(torch, lambda i: g_bs.launch(si_bs, do_copy=False, do_append=False), n3, 5)
        b_bs = decode_bytes(si_bs.lens.cpu().numpy(), 40, 40, 128, bs, 2)
        sweep[str(bs)] = {"ms_per_step": round(ms_f, 5), "decode_ms": round(ms_d, 5),
                          "decode_GBps": round(b_bs / (ms_d * 1e-3) / 1e9, 1),
                          "decode_traffic": traffic_fields(f"decode_b64_mha40_bs{bs}", b_bs)}
        del g_bs, si_bs
        torch.cuda.empty_cache()
    out["b64"]["block_size_sweep"] = {k: sweep[k] for k in ("8", "16", "32")}
    out["b64"]["block_size_sweep"]["pool"] = ("each KV head's pool allocated at 0x2080000 bytes for every block size "
                                              "(the block manager hands out 64 * (2048 / bs + 1) blocks)")
    # the unpadded block-16 pool (8,256 blocks: a 0x2040000-byte head stride)
    g_u = DeviceRun(scn3, device=dev, num_layers=1, fill="randn")
    g_u.run_setup()
    si_u = g_u.prepare(scn3.steps[0], longest_first=True)
    out["b64"]["block16_unpadded_pool_decode_ms"] = round(
        time_loop(torch, lambda i: g_u.launch(si_u, do_copy=False, do_append=False), n3, 5), 5)
    del g_u, si_u
    torch.cuda.empty_cache()

    # ---------------------------------------------------------- other rows
    if not args.no_rows:
        rows = {}
        # The workload's pool (134 MB per layer) fits the 256 MB Infinity
        # Cache, so, as for the headline, each step works on the next of
        # SHARED_LAYERS layers and reads its K/V cold.
        scn4 = build_scenario(4, 0)
        g4 = DeviceRun(scn4, device=dev, num_layers=SHARED_LAYERS, fill="randn")
        g4.run_setup()
        tail = g4.prepare(scn4.steps[0])
        dec = g4.prepare(scn4.steps[1], shared=True)
        nrep = 50

        def on_layer(fn):
            def f(i):
                g4.layer = i % SHARED_LAYERS
                fn()
            return f
        ms_copy = time_loop(torch, on_layer(lambda: g4.launch(tail, do_append=False)), nrep, 5)
        ms_tail = time_loop(torch, on_layer(lambda: g4.launch(tail, do_copy=False)), nrep, 5)
        ms_d4 = time_loop(torch, on_layer(lambda: g4.launch(dec, do_copy=False, do_append=False)), nrep, 5)
        ms_d4s = time_loop(torch, on_layer(lambda: g4.launch(dec, do_copy=False, do_append=False, shared=True)),
                           nrep, 5)
        L4 = dec.lens.cpu().numpy()
        copy_b = 2 * tail.n_pairs * SHARED_LAYERS * 2 * 8 * 16 * 128 * 2
        uniq = 8 * 3000 * 8 * 128 * 2 * 2 + 64 * (int(L4[0]) - 3000) * 8 * 128 * 2 * 2
        rows["cow_copy_blocks"] = {"workload": f"shared-prefix sampling: 56 copy-on-write block copies, in each of "
                                               f"the pool's {SHARED_LAYERS} layers",
                                   "ms": round(ms_copy, 5), "GBps": round(copy_b / (ms_copy * 1e-3) / 1e9, 1),
                                   **traffic_fields("copy_blocks_56", copy_b)}
        rows["append_2048"] = {"workload": "shared-prefix sampling: 64 x 32-token tails",
                               "ms": round(ms_tail, 5),
                               "GBps": round(append_bytes(2048, 8, 128, 2) / (ms_tail * 1e-3) / 1e9, 1),
                               **traffic_fields("append_2048", append_bytes(2048, 8, 128, 2))}
        rows["decode_shared_prefix"] = {
            "workload": "64 samples sharing 8 x 3,000-token prefixes, ctx 3,034; pa_decode_shared (8 groups of 8 "
                        "rows sharing 187 blocks, read once per group) against pa_decode (read once per sample); "
                        f"{SHARED_LAYERS} layers rotated",
            "ms": round(ms_d4s, 5),
            "unique_GBps": round(uniq / (ms_d4s * 1e-3) / 1e9, 1),
            "unique_hbm_frac": round(uniq / (ms_d4s * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "logical_GBps": round(decode_bytes(L4, 8, 32, 128, 16, 2) / (ms_d4s * 1e-3) / 1e9, 1),
            "groups": [list(g_) for g_ in dec.groups],
            "pa_decode_ms": round(ms_d4, 5),
            "pa_decode_unique_GBps": round(uniq / (ms_d4 * 1e-3) / 1e9, 1),
            "speedup": round(ms_d4 / ms_d4s, 3),
            "unique_bytes": uniq,
            "traffic_over_unique": traffic_fields("decode_shared_prefix_shared", uniq),
            "pa_decode_traffic_over_unique": traffic_fields("decode_shared_prefix_plain", uniq)}
        del g4, tail, dec
        torch.cuda.empty_cache()

        scn5 = build_scenario(5, 0)
        g5 = DeviceRun(scn5, device=dev, fill="randn")
        g5.run_setup()
        s5 = g5.prepare(scn5.steps[0], longest_first=True)
        ms_d5 = time_loop(torch, lambda i: g5.launch(s5, do_copy=False, do_append=False, do_prefill=False), 10, 2)
        ms_p5 = time_loop(torch, lambda i: g5.launch(s5, do_copy=False, do_append=False, do_decode=False), 10, 2)
        L5 = s5.lens.cpu().numpy()
        fl = prefill_flops(1024, 64, 128, 3500)
        rows["decode_long_ctx"] = {"workload": "63 sequences, ctx U[1024, 32768], GQA 64/8, submitted longest first",
                                   "ms": round(ms_d5, 5),
                                   "GBps": round(decode_bytes(L5, 8, 64, 128, 16, 2) / (ms_d5 * 1e-3) / 1e9, 1),
                                   "hbm_frac": round(decode_bytes(L5, 8, 64, 128, 16, 2) / (ms_d5 * 1e-3) / 1e9
                                                     / HBM_PEAK_GBS, 4),
                                   "decode_tok_s": round(63 / (ms_d5 * 1e-3), 1),
                                   **traffic_fields("decode_long_ctx", decode_bytes(L5, 8, 64, 128, 16, 2))}
        rows["prefill_chunk"] = {"workload": "1,024-token causal chunk after 3,500 cached tokens, GQA 64/8",
                                 "ms": round(ms_p5, 5),
                                 "TFLOPs": round(fl / (ms_p5 * 1e-3) / 1e12, 1),
                                 "mfma_frac": round(fl / (ms_p5 * 1e-3) / 1e12 / BF16_MFMA_PEAK_TFLOPS, 4),
                                 "prefill_tok_s": round(1024 / (ms_p5 * 1e-3), 1),
                                 **traffic_fields("prefill_chunk_1024", 1024 * 64 * 128 * 2 * 2 +
                                                  (3500 + 1024) * 8 * 128 * 2 * 2)}
        ms_sep = time_loop(torch, lambda i: g5.launch(s5, do_copy=False, do_append=False), 10, 2)
        ms_mix = time_loop(torch, lambda i: g5.launch(s5, do_copy=False, do_append=False, mixed=True), 10, 2)
        rows["mixed_batch"] = {"workload": "the 63 decodes and the 1,024-token chunk as one pa_mixed_batch launch "
                                           "(+ the partition merge), against pa_decode + pa_prefill_chunk",
                               "ms": round(ms_mix, 5), "separate_ms": round(ms_sep, 5),
                               "speedup": round(ms_sep / ms_mix, 3),
                               "GBps": round(decode_bytes(L5, 8, 64, 128, 16, 2) / (ms_mix * 1e-3) / 1e9, 1),
                               "TFLOPs": round(fl / (ms_mix * 1e-3) / 1e12, 1)}
        rows["mixed_batch_4_chunks"] = four_chunk_row(torch, pa, np, g5, s5, fl)
        rows["chunked_prefill_caps"] = chunked_prefill_row(torch, pa, np, g5, s5, ms_d5)
        del g5, s5
        torch.cuda.empty_cache()
        rows["prefix_cache"] = prefix_cache_row(torch, pa, np)
        rows["capacity"] = capacity_row(pa, np)
        out["rows"] = rows

    # ---------------------------------------------------------- CPU oracle baseline
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.cpu_seconds, dbytes)
    out["wall_s"] = round(time.time() - t_start, 1)
    print(json.dumps(out), flush=True)
    return 0


def four_chunk_row(torch, pa, np, g5, s5, fl_one):
    """The 63 long-context decodes with four 256-row prefill chunks of
    different sequences (after 200, 1,000, 3,500 and 8,000 cached tokens) in
    one pa_mixed_batch, against pa_decode + four pa_prefill_chunk calls."""
    cfg = g5.cfg
    H_q, d = cfg["H_q"], cfg["d"]
    chunks = [(256, 200), (256, 1000), (256, 3500), (256, 8000)]
    tables = []
    for i, (T, cb) in enumerate(chunks):
        seq = 500000 + i
        g5.bm.add_seq(seq)
        g5.bm.append_slots(seq, cb + T)  # the pool already holds N(0,1) K/V everywhere
        tables.append(g5.bm.block_table(seq))
    width = max(len(t) for t in tables)
    pt = torch.tensor([t + [0] * (width - len(t)) for t in tables], dtype=torch.int32, device="cuda")
    pq = torch.randn(sum(T for T, _ in chunks), H_q, d, device="cuda").to(torch.bfloat16)
    pout = torch.empty_like(pq)
    rows0 = np.cumsum([0] + [T for T, _ in chunks])

    # the separate calls get their prefill workspaces, so that short chunks
    # split over their keys as a caller would let them
    wss = [pa.prefill_workspace(g5.pool, T, H_q, cb) for T, cb in chunks]

    def separate(i):
        g5.launch(s5, do_copy=False, do_append=False, do_prefill=False)
        for c, (T, cb) in enumerate(chunks):
            r = slice(int(rows0[c]), int(rows0[c + 1]))
            pa.pa_prefill_chunk(g5.pool, 0, pout[r], pq[r], pt[c], cb, cfg["scale"], wss[c])

    def mixed(i):
        pa.pa_mixed_batch(g5.pool, 0, s5.out, s5.q, s5.tables, s5.lens, s5.max_ctx, pout, pq, chunks, pt,
                          cfg["scale"], 0, s5.workspace)

    ms_sep = time_loop(torch, separate, 10, 2)
    ms_mix = time_loop(torch, mixed, 10, 2)
    flops = sum(prefill_flops(T, H_q, d, cb) for T, cb in chunks)
    return {"workload": "the 63 decodes (longest first) + 4 chunks of 256 rows after 200 / 1,000 / 3,500 / 8,000 "
                        "cached tokens, GQA 64/8, as one pa_mixed_batch; separate: pa_decode + four "
                        "pa_prefill_chunk calls with their key-split workspaces",
            "ms": round(ms_mix, 5), "separate_ms": round(ms_sep, 5), "speedup": round(ms_sep / ms_mix, 3),
            "prefill_GFLOP": round(flops / 1e9, 1)}


def chunked_prefill_row(torch, pa, np, g5, s5, ms_decode):
    """The page's chunked-prefill measurement on this layer: a 3,500-token
    prompt arrives while the 63 long-context sequences decode; pa_plan_step
    cuts it under a per-step cap of 512 / 1,024 / 2,048 / 8,192 tokens (the
    cap counts the 63 decode tokens too), and each step is one
    pa_mixed_batch launch (the decodes + that step's chunk).  Per cap: the
    steps, the slowest step (this layer's share of the longest gap between
    two tokens of a running request) and the time until the prompt is
    prefilled."""
    cfg = g5.cfg
    H_q, d, prompt = cfg["H_q"], cfg["d"], 3500
    seq = 600000
    g5.bm.add_seq(seq)
    g5.bm.append_slots(seq, prompt)  # the pool already holds N(0,1) K/V everywhere
    ptab = torch.tensor([g5.bm.block_table(seq)], dtype=torch.int32, device="cuda")
    pq = torch.randn(prompt, H_q, d, device="cuda").to(torch.bfloat16)
    pout = torch.empty_like(pq)
    n_dec = int(s5.q.shape[0])
    out = {"workload": "63 decodes of 1k-32k tokens (GQA 64/8) running while a 3,500-token prompt is prefilled in "
                       "chunks; per cap: one pa_mixed_batch per step",
           "decode_only_ms": round(ms_decode, 5)}
    for cap in (512, 1024, 2048, 8192):
        done, times, chunks = 0, [], []
        while done < prompt:
            (_, cb, T), = pa.pa_plan_step(cap, n_dec, [(prompt, done)])
            r = slice(cb, cb + T)

            def step(i, r=r, T=T, cb=cb):
                pa.pa_mixed_batch(g5.pool, 0, s5.out, s5.q, s5.tables, s5.lens, s5.max_ctx, pout[r], pq[r],
                                  [(T, cb)], ptab, cfg["scale"], 0, s5.workspace)

            times.append(time_loop(torch, step, 3, 1))
            chunks.append(T)
            done = cb + T
        out[str(cap)] = {"steps": len(times), "chunk_tokens": chunks, "max_step_ms": round(max(times), 5),
                         "mean_step_ms": round(sum(times) / len(times), 5),
                         "prompt_prefilled_ms": round(sum(times), 5)}
    g5.bm.free_seq(seq)
    return out


def capacity_row(pa, np):
    """KV slots that hold tokens: the library's block manager on the
    13B-shaped workload's 64 lognormal lengths, against reserving 2,048
    tokens per request as systems before paging did; and how many 512 + 128
    token requests a 22,048-token KV pool holds either way (host only)."""
    from pa_inputs import build_scenario

    out = {"workload": "64 lognormal context lengths (median 400, clipped to [16, 2048]); 2,048-token reservation"}
    for bs in (8, 16, 32):
        scn = build_scenario(3, 0, bs=bs)
        lens = [int(x) for x in scn.ctx]
        bm = pa.BlockManager(sum(-(-n // bs) for n in lens), bs, np.arange(sum(-(-n // bs) for n in lens)))
        for i, n in enumerate(lens):
            bm.add_seq(i)
            bm.append_slots(i, n)
        slots = sum(len(bm.block_table(i)) for i in range(len(lens))) * bs
        out[f"paged_bs{bs}_token_fraction"] = round(sum(lens) / slots, 4)
        out[f"paged_bs{bs}_mean_waste_tokens"] = round((slots - sum(lens)) / len(lens), 2)
    out["reserved_token_fraction"] = round(sum(lens) / (2048 * len(lens)), 4)
    out["requests_in_22048_tokens_paged"] = 22048 // (-(-640 // 16) * 16)
    out["requests_in_22048_tokens_reserved"] = 22048 // 2048
    return out


def prefix_cache_row(torch, pa, np):
    """The page's prefix-cache workload: a 3,000-token shared prefix plus 32
    unique tokens per request, block 16, 32 query / 8 KV heads, head_dim 128.
    Host: what admitting one request costs in the library's manager (add the
    sequence through the prefix cache, append the uncached rest of the prompt
    with its token ids), through the Python binding, for a request that hits
    2,992 cached tokens and for one that hits none.  GPU: the prefill a hit
    leaves (40 positions after 2,992 cached ones) against the whole prompt."""
    bs, H_kv, H_q, d, N = 16, 8, 32, 128, 8192
    rng = np.random.default_rng(7)
    prefix = [int(x) for x in rng.integers(0, 150000, 3000)]
    bm = pa.BlockManager(N, bs, rng.permutation(N))
    first = prefix + [int(x) for x in rng.integers(0, 150000, 32)]
    bm.add_seq_prefix(0, first)
    bm.append_tokens(0, first)
    reps, seq = 50, 1
    prompts = [prefix + [int(x) for x in rng.integers(0, 150000, 32)] for _ in range(reps)]
    misses = [[int(x) for x in rng.integers(0, 150000, 3032)] for _ in range(reps)]
    t0 = time.perf_counter()
    for pr in prompts:
        hit = bm.add_seq_prefix(seq, pr)
        bm.append_tokens(seq, pr[hit:])
        seq += 1
    t_hit = (time.perf_counter() - t0) / reps
    for s_ in range(1, seq):
        bm.free_seq(s_)
    t0 = time.perf_counter()
    for pr in misses:
        bm.add_seq_prefix(seq, pr)
        bm.append_tokens(seq, pr)
        bm.free_seq(seq)
        seq += 1
    t_miss = (time.perf_counter() - t0) / reps
    assert hit == 2992

    # 28 layers of 13 MB, one per timed call, so that the K/V come from HBM
    layers = 28
    pool = pa.KVPool(layers, H_kv, 200, bs, d, "bf16", device="cuda")
    pool.k.normal_()
    pool.v.normal_()
    table = torch.from_numpy(rng.permutation(200)[:190].astype(np.int32)).cuda()
    scale = float(1 / np.sqrt(d))
    qf = torch.randn(3032, H_q, d, device="cuda").to(torch.bfloat16)
    of = torch.empty_like(qf)
    qh, oh = qf[-40:].contiguous(), torch.empty_like(qf[-40:])
    ms_full = time_loop(torch, lambda i: pa.pa_prefill_chunk(pool, i % layers, of, qf, table, 0, scale), 20, 3)
    ws = pa.prefill_workspace(pool, 40, H_q, 2992)
    ms_hit = time_loop(torch, lambda i: pa.pa_prefill_chunk(pool, i % layers, oh, qh, table, 2992, scale, ws), 20, 3)
    ms_hit_one = time_loop(torch, lambda i: pa.pa_prefill_chunk(pool, i % layers, oh, qh, table, 2992, scale), 20, 3)
    return {"workload": "3,000-token shared prefix + 32-token tail per request, block 16, GQA 32/8, d 128, "
                        f"{layers} layers rotated",
            "hit_tokens": hit, "host_admit_hit_us": round(t_hit * 1e6, 1),
            "host_admit_miss_us": round(t_miss * 1e6, 1),
            "prefill_whole_prompt_ms": round(ms_full, 5), "prefill_after_hit_ms": round(ms_hit, 5),
            "prefill_after_hit_unsplit_ms": round(ms_hit_one, 5),
            "prefill_speedup": round(ms_full / ms_hit, 1)}


def cpu_baseline(seconds, dbytes):
    """The oracle on the same step (append 32 + decode of 32 sequences), timed
    on this host's cores: repeated until ``seconds`` of work are done."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import attention, encoding
    from oracle.run import OracleRun, widen
    from pa_inputs import build_scenario

    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
        scn = build_scenario(2, 0)
        orc = OracleRun(scn)
        orc.run_setup()
        st = scn.steps[0]
        slots, _ = orc.bookkeeping(st)
        cfg = scn.cfg
        kb, vb = encoding.encode(st.k_new, "bf16"), encoding.encode(st.v_new, "bf16")
        q = widen(st.q, "bf16")
        tables = [orc.bm.block_table(s_) for s_ in st.decode_seqs]
        lens = [orc.bm.seq_len(s_) for s_ in st.decode_seqs]
        reps = 0
        t0 = time.perf_counter()
        while True:
            orc.pool.append(0, kb, vb, slots)
            attention.decode(orc.pool, 0, q, tables, lens, cfg["scale"])
            reps += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                break
    one = {}
    with threadpool_limits(limits=1):
        for cid, secs in ((1, 1.0), (2, 3.0)):
            one[f"config{cid}_ms_per_step"] = round(oracle_step_ms(cid, secs), 3)
    return {"value": round(dbytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"the same decode step (append 32 + decode 32 sequences, float64 oracle) repeated {reps} "
                      f"times in {el:.1f} s on {cores} visible host cores",
            "ms_per_step": round(1e3 * el / reps, 3),
            "one_thread": dict(one, sample="the tiny fp32 step (4 sequences) and the same B=32 step, each repeated "
                                           "for ~1 s / ~3 s with BLAS limited to one thread")}


def oracle_step_ms(cid, seconds):
    """ms per append + decode step of workload ``cid`` in the oracle."""
    from oracle import attention, encoding
    from oracle.run import OracleRun, widen
    from pa_inputs import build_scenario

    scn = build_scenario(cid, 0)
    orc = OracleRun(scn)
    orc.run_setup()
    st = scn.steps[0]
    slots, _ = orc.bookkeeping(st)
    cfg = scn.cfg
    kb, vb = encoding.encode(st.k_new, cfg["dtype"]), encoding.encode(st.v_new, cfg["dtype"])
    q = widen(st.q, cfg["dtype"])
    tables = [orc.bm.block_table(s_) for s_ in st.decode_seqs]
    lens = [orc.bm.seq_len(s_) for s_ in st.decode_seqs]
    reps, t0 = 0, time.perf_counter()
    while True:
        orc.pool.append(0, kb, vb, slots)
        attention.decode(orc.pool, 0, q, tables, lens, cfg["scale"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            return 1e3 * el / reps


if __name__ == "__main__":
    sys.exit(main())
