"""Benchmark of unified paged attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--warm-seconds S]
                    [--workload NAME] [--no-cpu-baseline] [--cold N] [--no-configs]
                    [--config-steps K] [--config-warmup W] [--config-warm-seconds S]
                    [--config-cold N] [--force-tile T]
                    [--force-splits S] [--decode-grid G] [--cache-write]
                    [--summarize DIR] [--calibrate-copy]

A step is one call of pa_unified_attention over one synthetic batch (inputs
resident in HBM).  Prints one JSON line: whole-job throughput in the metric's
unit, plus the roofline of one call (algorithmic bytes or flops per call over
the mean GPU time of a call: a pair of HIP events on the launch stream around
the K back-to-back calls of the timed region) and the fp64 CPU oracle timed on
a bounded sample of the same workload.  The default run (the headline decode
workload) also times every other workload of the metric the same way and
reports each in a "configs" map (µs per call from events and cold calls,
algorithmic work, bound, achieved rate, roofline fraction, traffic).

Algorithmic bytes per launch: every valid context token's K and V read once
(sum_s L_s * Hkv * d * e * 2, e = 2 B for bf16 caches and 1 B for fp8) plus q
read and out written (2 * T * Hq * d * 2 B).  Algorithmic flops: 4 * d * Hq * (admissible (query, key) pairs per head).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged varlen attn µs/batch; decode KV-read TB/s & prefill TFLOP/s vs peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
DEFAULT_WORKLOAD = "decode_256seq_ctx1k"


def kv_elem_bytes(b):
    return 1 if b.kv_format == "fp8_e4m3fn" else 2


def algorithmic_work(b):
    d, hq, hkv = b.head_dim, b.num_q_heads, b.num_kv_heads
    kv_bytes = int(b.k_lens.sum()) * hkv * d * 2 * kv_elem_bytes(b)
    qo_bytes = 2 * b.total_q * hq * d * 2
    pairs = 0
    for ql, L in zip(b.q_lens.tolist(), b.k_lens.tolist()):
        if b.causal:
            # query i sees min(L, max(0, L - ql + i + 1)) keys
            i = np.arange(ql)
            pairs += int(np.clip(L - ql + i + 1, 0, L).sum())
        else:
            pairs += ql * L
    flops = 4 * d * hq * pairs
    return kv_bytes + qo_bytes, kv_bytes, flops


def source_hash():
    """Hash of the library's code (line comments and blank lines dropped, so a
    comment edit does not mark the recorded counters stale)."""
    h = hashlib.sha256()
    for f in ("pa_kernels.hip", "pa_api.cpp", "pa_internal.h"):
        with open(os.path.join(ROOT, "paged_kv_cache_unified_amd", "csrc", f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def profile_path(workload, kernel):
    return os.path.join(ROOT, "profiles", f"{kernel}_{workload}.md")


def profile_record(workload):
    """The counter record of the committed rocprofv3 summary for the workload's
    dominant kernel, if its counters were taken on the current kernel sources;
    else None."""
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}.md"))):
        text = open(path).read()
        marker = "<!-- traffic "
        if marker not in text:
            continue
        rec = json.loads(text.split(marker, 1)[1].split(" -->", 1)[0])
        if rec.get("workload") == workload and rec.get("source_hash") == source_hash():
            return rec
    return None


def traffic_record(workload):
    """HBM bytes per launch of the dominant kernel (profile_record), or None."""
    rec = profile_record(workload)
    return rec.get("traffic_bytes_per_launch") if rec else None


PROF_COMMANDS = """cd /tmp && export TMPDIR=/tmp
rocprofv3 --kernel-trace --stats -d $OUT/trace_{w} -o run -- python3 $REPO/bench.py --workload {w} --steps 20 --warmup 5 --warm-seconds 0.3 --no-cpu-baseline --no-configs --cold 0
rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc_FETCH_SIZE_{w} -o run -- python3 $REPO/bench.py --workload {w} --steps 3 --warmup 1 --no-cpu-baseline --no-configs --cold 0
rocprofv3 --pmc WRITE_SIZE -d $OUT/pmc_WRITE_SIZE_{w} -o run -- python3 $REPO/bench.py --workload {w} --steps 3 --warmup 1 --no-cpu-baseline --no-configs --cold 0
rocprofv3 --pmc MfmaUtil MfmaFlopsBF16 LdsBankConflict LdsUtil VALUBusy VmemLatency -d $OUT/pmc_MFMA_{w} -o run -- python3 $REPO/bench.py --workload {w} --steps 3 --warmup 1 --no-cpu-baseline --no-configs --cold 0
rocprofv3 --pmc FETCH_SIZE -d $OUT/pmc_FETCH_SIZE_copy -o run -- python3 $REPO/bench.py --calibrate-copy
rocprofv3 --pmc WRITE_SIZE -d $OUT/pmc_WRITE_SIZE_copy -o run -- python3 $REPO/bench.py --calibrate-copy
python3 $REPO/bench.py --summarize $OUT --workload {w}"""


def summarize_profiles(out_dir, workload):
    """Write profiles/<kernel>_<workload>.md from rocprofv3 output databases,
    for the library kernel with the largest total time in the trace."""
    import sqlite3
    import glob

    def db(sub):
        hits = glob.glob(os.path.join(out_dir, sub, "**", "*.db"), recursive=True)
        if not hits:
            raise SystemExit(f"no rocprofv3 database under {os.path.join(out_dir, sub)}")
        return sqlite3.connect(hits[0])

    con = db(f"trace_{workload}")
    stats = list(con.execute("select name, total_calls, total_duration, average, percentage "
                             "from top_kernels limit 8"))
    ours = [r for r in stats if "pa::" in r[0] and "_kernel" in r[0]]
    if not ours:
        raise SystemExit("no library kernel in the trace")
    top = max(ours, key=lambda r: r[2])
    kernel = top[0].replace("(anonymous namespace)::", "").split("<")[0].split("(")[0]
    kernel = kernel.split("::")[-1]
    like = f"%{kernel}%"

    def counter(sub, name, pattern):
        rows = list(db(sub).execute(
            "select avg(value), count(*) from counters_collection where counter_name = ? "
            "and kernel_name like ?", (name, pattern)))
        return rows[0]

    fetch_k, n_f = counter(f"pmc_FETCH_SIZE_{workload}", "FETCH_SIZE", like)
    write_k, n_w = counter(f"pmc_WRITE_SIZE_{workload}", "WRITE_SIZE", like)
    copy_bytes = 1 << 30
    fetch_c, _ = counter("pmc_FETCH_SIZE_copy", "FETCH_SIZE", "%copyBuffer%")
    write_c, _ = counter("pmc_WRITE_SIZE_copy", "WRITE_SIZE", "%copyBuffer%")
    f_scale = copy_bytes / (fetch_c * 1024.0)
    w_scale = copy_bytes / (write_c * 1024.0)
    fetch_bytes = fetch_k * 1024.0 * f_scale
    write_bytes = write_k * 1024.0 * w_scale

    lines = [f"# {kernel} on workload `{workload}` (MI355X, rocprofv3)", "",
             "Commands (OUT = an output folder, REPO = the repository root):", "", "```",
             PROF_COMMANDS.format(w=workload), "```", "",
             "## Kernel trace (--kernel-trace --stats), top kernels", "",
             "| kernel | calls | total us | average us | % |", "|---|---|---|---|---|"]
    for name, calls, total, avg, pct in stats:
        short = name.replace("(anonymous namespace)::", "").split("(")[0][-70:]
        lines.append(f"| `{short}` | {calls} | {total:.1f} | {avg:.2f} | {pct:.1f} |")
    lines += ["", f"(The run includes "
              f"input generation kernels; `{kernel}` is the kernel whose average is compared "
              f"with the in-benchmark HIP-event timing.)", "",
              f"## HBM traffic of `{kernel}` (--pmc, one counter per run)", "",
              f"- FETCH_SIZE: {fetch_k:.1f} KiB per dispatch (mean of {n_f} dispatches)",
              f"- WRITE_SIZE: {write_k:.1f} KiB per dispatch (mean of {n_w} dispatches)",
              f"- Calibration, 1 GiB device copy (`__amd_rocclr_copyBuffer`, {copy_bytes} B read "
              f"and written): FETCH_SIZE {fetch_c:.1f} KiB, WRITE_SIZE {write_c:.1f} KiB -> scale "
              f"factors {f_scale:.4f} (fetch) and {w_scale:.4f} (write)",
              f"- Scaled: fetched {fetch_bytes / 1e9:.4f} GB, written {write_bytes / 1e9:.4f} GB, "
              f"total {(fetch_bytes + write_bytes) / 1e9:.4f} GB per launch", ""]
    mfma = {}
    if glob.glob(os.path.join(out_dir, f"pmc_MFMA_{workload}", "**", "*.db"), recursive=True):
        for name in ("MfmaUtil", "MfmaFlopsBF16", "LdsBankConflict", "LdsUtil", "VALUBusy",
                     "VmemLatency"):
            mfma[name] = counter(f"pmc_MFMA_{workload}", name, like)[0]
        lines += [f"## Matrix cores and LDS of `{kernel}` (--pmc, derived metrics of the box)", "",
                  f"- MfmaUtil (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs): "
                  f"{mfma['MfmaUtil']:.2f} %",
                  f"- MfmaFlopsBF16 (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512): "
                  f"{mfma['MfmaFlopsBF16'] / 1e9:.3f} GFLOP per dispatch (matrix-core work "
                  f"issued, padding and masked pairs included)",
                  f"- LdsBankConflict (SQ_LDS_BANK_CONFLICT over conflict-free LDS cycles): "
                  f"{mfma['LdsBankConflict']:.4f}"]
        if mfma.get("LdsUtil") is not None:
            lines += [f"- LdsUtil (SQ_LDS_IDX_ACTIVE over busy cycles x CUs): {mfma['LdsUtil']:.2f} %",
                      f"- VALUBusy (SQ_ACTIVE_INST_VALU over busy cycles x CUs): "
                      f"{mfma['VALUBusy']:.2f} %",
                      f"- VmemLatency (in-flight vector memory instructions per issued one, "
                      f"cycles): {mfma['VmemLatency']:.0f}"]
        lines.append("")
    rec = {"workload": workload, "kernel": kernel, "source_hash": source_hash(),
           "kernel_avg_us": top[3],
           "traffic_bytes_per_launch": int(fetch_bytes + write_bytes),
           "fetch_kib": fetch_k, "write_kib": write_k,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "mfma_util_pct": mfma.get("MfmaUtil"), "mfma_flops_bf16": mfma.get("MfmaFlopsBF16"),
           "lds_bank_conflict": mfma.get("LdsBankConflict"), "lds_util_pct": mfma.get("LdsUtil"),
           "valu_busy_pct": mfma.get("VALUBusy"), "vmem_latency_cycles": mfma.get("VmemLatency")}
    lines.append("<!-- traffic " + json.dumps(rec) + " -->")
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    path = profile_path(workload, kernel)
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(path)


def cpu_baseline(b, unit, min_s=10.0, budget_s=20.0):
    """The oracle, as it stands, on a bounded sample of the batch's sequences.

    Sequences are taken longest context first (every 64th first, for a spread
    of lengths) until the oracle has spent budget_s; if the whole batch takes
    less than min_s, it is run again until min_s is reached.  The rate is in
    the metric's unit: algorithmic bytes (TB/s) or flops (TFLOP/s) of the
    sample over oracle time."""
    import threadpoolctl

    import oracle
    cores = len(os.sched_getaffinity(0))
    # the host share may be smaller than the visible cores (OMP_NUM_THREADS)
    threads = min(cores, int(os.environ.get("OMP_NUM_THREADS", cores) or cores), 64)
    order = np.argsort(b.k_lens)[::-1]
    first = list(order[::max(1, len(order) // 64)])
    sequence = first + [s for s in order if s not in set(first)]
    subsets = {}
    picked, t_all, passes = [], 0.0, 0
    with threadpoolctl.threadpool_limits(limits=threads):
        while True:
            for s in sequence:
                s = int(s)
                if s not in subsets:
                    subsets[s] = b.host_subset([s])[0]
                sub = subsets[s]
                t0 = time.perf_counter()
                oracle.paged_attention(sub["q"], sub["k_cache"], sub["v_cache"],
                                       sub["cu_seqlens_q"], sub["seqused_k"], sub["block_table"],
                                       sub["softmax_scale"], sub["causal"], **b.kv_kwargs())
                t_all += time.perf_counter() - t0
                picked.append(s)
                if t_all >= budget_s:
                    break
            passes += 1
            if t_all >= min_s or t_all >= budget_s:
                break
        info = threadpoolctl.threadpool_info()
    blas = ",".join(sorted({i.get("internal_api", "?") for i in info})) or "none"
    sel = np.array(picked)
    kl, ql = b.k_lens[sel], b.q_lens[sel]
    d, hq, hkv = b.head_dim, b.num_q_heads, b.num_kv_heads
    if unit == "TFLOP/s":
        pairs = 0
        for q, L in zip(ql.tolist(), kl.tolist()):
            if b.causal:
                pairs += int(np.clip(L - q + np.arange(q) + 1, 0, L).sum())
            else:
                pairs += q * L
        value = 4 * d * hq * pairs / t_all / 1e12
    else:
        sample_bytes = int(kl.sum()) * hkv * d * 2 * kv_elem_bytes(b) + 2 * int(ql.sum()) * hq * d * 2
        value = sample_bytes / t_all / 1e12
    distinct = len(set(picked))
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{distinct} of {b.num_seqs} sequences ({int(b.k_lens[sorted(set(picked))].sum())} "
                      f"context tokens), {passes} pass(es), {len(picked)} sequence calls, fp64 "
                      f"numpy oracle, {t_all:.1f} s, BLAS {blas}, {cores} host cores visible"}


def bench_cache_write(pa, b, args, dev):
    """pa_cache_write of every sequence's q_s new tokens (context positions
    L_s - q_s .. L_s - 1, slots from the block table) into the batch's caches.
    Algorithmic bytes: the new keys and values read once (bf16) and written
    once in the cache format."""
    import torch
    T, hkv, d = b.total_q, b.num_kv_heads, b.head_dim
    table = b.block_table.cpu().numpy().astype(np.int64)
    slots = np.empty(T, np.int64)
    cu = b.cu_seqlens_q.cpu().numpy()
    for s in range(b.num_seqs):
        L, q = int(b.k_lens[s]), int(b.q_lens[s])
        pos = np.arange(L - q, L)
        slots[cu[s]:cu[s + 1]] = table[s, pos // 16] * 16 + pos % 16
    slot_t = torch.as_tensor(slots.astype(np.int32), device=dev)
    g = torch.Generator(device=dev).manual_seed(5)
    key = torch.randn(T, hkv, d, generator=g, device=dev).to(torch.bfloat16)
    val = torch.randn(T, hkv, d, generator=g, device=dev).to(torch.bfloat16)
    call = lambda: pa.cache_write(key, val, b.k_cache, b.v_cache, slot_t, b.k_scale, b.v_scale)
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    s0.record(stream)
    for _ in range(args.steps):
        call()
    s1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    us = s0.elapsed_time(s1) * 1e3 / args.steps
    nbytes = T * hkv * d * 2 * (2 + kv_elem_bytes(b))
    achieved = nbytes / (us * 1e-6) / 1e9
    print(json.dumps({
        "metric": "KV-cache write GB/s (new tokens into the paged cache)", "value": round(achieved, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": b.kv_format, "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "num_kv_heads": hkv, "head_dim": d},
        "us_per_call_events": round(us, 2), "algorithmic_bytes_per_call": nbytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warm-seconds", type=float, default=0.0,
                    help="keep warming up (untimed) at least this long after the --warmup "
                         "calls (0: exactly --warmup calls)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold", type=int, default=100, help="extra cold-cache timed calls")
    ap.add_argument("--no-configs", action="store_true",
                    help="time the headline workload only (no configs map)")
    ap.add_argument("--config-steps", type=int, default=20,
                    help="back-to-back calls timed per config workload")
    ap.add_argument("--config-warmup", type=int, default=5)
    ap.add_argument("--config-warm-seconds", type=float, default=0.3,
                    help="config workloads: keep warming up (untimed) at least this long; "
                         "five calls right after a workload is generated measured up to 20%% "
                         "slow (the GPU not yet at its steady state)")
    ap.add_argument("--config-cold", type=int, default=20,
                    help="cold-cache calls per config workload")
    ap.add_argument("--force-tile", type=int, default=0,
                    help="pa_options.force_tile (0 = heuristic plan)")
    ap.add_argument("--force-splits", type=int, default=0,
                    help="pa_options.force_num_splits (0 = heuristic plan)")
    ap.add_argument("--decode-grid", type=int, default=0,
                    help="pa_options.decode_grid (0 = resident work-groups)")
    ap.add_argument("--summarize", metavar="DIR",
                    help="write profiles/pa_fwd_<workload>.md from rocprofv3 output in DIR")
    ap.add_argument("--cache-write", action="store_true",
                    help="time pa_cache_write instead: each sequence's new tokens (its "
                         "last q_s positions) written into the workload's caches")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure this GPU's practical matrix ceilings: a library bf16 "
                         "GEMM (random and all-zero operands), the prefill workload with random and all-zero q/k/v, and torch's "
                         "dense attention on the prefill-equivalent shapes")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB device-to-device copy three times (the known-size "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE into bytes)")
    args = ap.parse_args()
    if args.summarize:
        summarize_profiles(args.summarize, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the operation runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": src.numel() * 4}))
        return

    import paged_kv_cache_unified_amd as pa
    from workloads import WORKLOADS, make_workload
    if args.ceilings:
        measure_ceilings(pa, make_workload, args)
        return

    if args.workload not in WORKLOADS:
        sys.exit(f"unknown workload {args.workload}; choose from {sorted(WORKLOADS)}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"bench: generating {args.workload}", file=sys.stderr, flush=True)
    b = make_workload(args.workload, device=dev)
    if args.cache_write:
        bench_cache_write(pa, b, args, dev)
        return
    m = measure(pa, b, args, args.steps, args.warmup, args.cold, args.warm_seconds)

    res = {
        "metric": METRIC,
        "value": m["value"],
        "unit": m["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": m["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m["dtype"],
        "data": "synthetic",
        "config": m["config"],
        "us_per_batch": m["us_per_batch"],
        "us_per_launch_events": m["us_per_launch_events"],
        "us_per_launch_cold_p10_p50_p90": m["us_per_launch_cold_p10_p50_p90"],
        "algorithmic_bytes_per_launch": m["algorithmic_bytes_per_launch"],
        "algorithmic_flops_per_launch": m["algorithmic_flops_per_launch"],
        "plan": m["plan"],
        "roofline": m["roofline"],
        "cpu_baseline": None,
    }
    if m.get("counters"):
        res["counters"] = m["counters"]
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(b, m["unit"])
    del b
    torch.cuda.empty_cache()
    if not args.no_configs and args.workload == DEFAULT_WORKLOAD:
        # every other workload of the metric, timed the same way in this run
        res["configs"] = {}
        for name in CONFIG_WORKLOADS:
            print(f"bench: config {name}", file=sys.stderr, flush=True)
            cb = make_workload(name, device=dev)
            cm = measure(pa, cb, args, args.config_steps, args.config_warmup, args.config_cold,
                         args.config_warm_seconds)
            res["configs"][name] = {k: cm[k] for k in (
                "us_per_launch_events", "us_per_launch_cold_p10_p50_p90", "us_per_batch",
                "algorithmic_bytes_per_launch", "algorithmic_flops_per_launch", "roofline",
                "dtype", "plan", "counters") if k in cm}
            del cb
            torch.cuda.empty_cache()
    print(json.dumps(res), flush=True)


# The workloads timed beside the headline in the default run (the metric's
# other configurations: the mixed batch, its prefill and decode parts, the 70B
# TP=2 share, the two long-context batches, and the headline with an fp8 cache)
CONFIG_WORKLOADS = [
    "mixed_prefill512x8_decode248",
    "prefill512x8_only",
    "prefill512x8_only_d96",
    "prefill512x8_only_d256",
    "decode248_only",
    "decode_gqa8_64seq_ctx2k_4k",
    "long_decode_16seq_ctx32k_128k",
    "long_q16_noncausal_16seq_ctx32k_128k",
    "decode_256seq_ctx1k_fp8",
]


def _event_time(fn, n=20, warm=5):
    """Mean GPU time of fn over n back-to-back calls (s), events on the current stream."""
    import torch
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n * 1e-3


def measure_ceilings(pa, make_workload, args):
    """What this GPU's matrix cores sustain in practice, beside the published
    peak the roofline uses: a library GEMM (operands drawn from N(0, 1), and
    all zeros: the gap is the clock the chip gives up under data-dependent
    power), the prefill
    workload through this library with random and with all-zero q/k/v (same
    code path, no rescale either way after the first key), and torch's dense
    attention on shapes equivalent to that prefill.  One JSON line per item."""
    import torch
    import torch.nn.functional as F
    dev = torch.device("cuda:0")
    out = []
    for kind in ("normal", "zeros"):
        n = 8192
        mk = (lambda: torch.randn(n, n, device=dev, dtype=torch.bfloat16)) if kind == "normal" \
            else (lambda: torch.zeros(n, n, device=dev, dtype=torch.bfloat16))
        a, c = mk(), mk()
        t = _event_time(lambda: a @ c)
        out.append({"ceiling": "bf16 GEMM 8192^3 (torch.matmul)", "operands": kind,
                    "us": round(t * 1e6, 1), "TFLOPs": round(2 * n ** 3 / t / 1e12, 1),
                    "frac_of_2.5PF": round(2 * n ** 3 / t / 2.5e15, 4)})
        del a, c
    name = "prefill512x8_only"
    b = make_workload(name, device=dev)
    res = torch.empty_like(b.q)
    fargs = b.args(res)
    opts = pa.options()
    ws = torch.empty(max(1, pa.workspace_bytes(*fargs[:9], opts)), dtype=torch.uint8, device=dev)
    flops = algorithmic_work(b)[2]
    for kind in ("normal", "zeros"):
        if kind == "zeros":
            b.q.zero_()
            b.k_cache.zero_()
            b.v_cache.zero_()
        t = _event_time(lambda: pa.unified_attention(*fargs, opts=opts, workspace=ws))
        out.append({"ceiling": f"{name} through this library", "qkv": kind,
                    "us": round(t * 1e6, 1), "TFLOPs": round(flops / t / 1e12, 1),
                    "frac_of_2.5PF": round(flops / t / 2.5e15, 4)})
    del b, res, ws
    torch.cuda.empty_cache()
    # dense attention at the prefill's size: 8 sequences x 32 heads, 512 queries
    # over 2048 keys (the longest chunk's context), and a square causal 2048
    for (B, H, Sq, Sk, causal) in ((8, 32, 512, 2048, False), (8, 32, 2048, 2048, True)):
        q = torch.randn(B, H, Sq, 128, device=dev, dtype=torch.bfloat16)
        k = torch.randn(B, H, Sk, 128, device=dev, dtype=torch.bfloat16)
        v = torch.randn(B, H, Sk, 128, device=dev, dtype=torch.bfloat16)
        fl = 4 * B * H * Sq * Sk * 128 * (0.5 if causal else 1.0)
        t = _event_time(lambda: F.scaled_dot_product_attention(q, k, v, is_causal=causal))
        out.append({"ceiling": "torch scaled_dot_product_attention (dense)", "shape": [B, H, Sq, Sk, 128],
                    "causal": causal, "us": round(t * 1e6, 1), "TFLOPs": round(fl / t / 1e12, 1),
                    "frac_of_2.5PF": round(fl / t / 2.5e15, 4)})
        del q, k, v
    for o in out:
        print(json.dumps(o), flush=True)


def measure(pa, b, args, steps, warmup, n_cold, warm_seconds=0.0):
    """Times one workload: `steps` back-to-back calls (wall clock and a pair of
    HIP events on the launch stream), then `n_cold` calls each after a 1 GiB
    read that evicts the Infinity Cache; returns the bench fields of it.
    Untimed warm-up: `warmup` calls, continued until `warm_seconds` have
    passed."""
    import torch
    dev = b.q.device
    out = torch.empty_like(b.q)
    call_args = b.args(out)
    opts, ws = None, None
    if args.force_tile or args.force_splits or args.decode_grid or b.kv_format != "bf16":
        opts = pa.options(force_num_splits=args.force_splits, force_tile=args.force_tile,
                          decode_grid=args.decode_grid, k_scale=b.k_scale, v_scale=b.v_scale)
        ws = torch.empty(max(1, pa.workspace_bytes(*call_args[:9], opts)), dtype=torch.uint8,
                         device=dev)
    plan = pa.plan_describe(*call_args[:9], opts=opts)
    total_bytes, kv_bytes, flops = algorithmic_work(b)

    def call():
        if opts is None:
            pa.unified_attention(*call_args)
        else:
            pa.unified_attention(*call_args, opts=opts, workspace=ws)

    stream = torch.cuda.current_stream(dev)
    t_warm = time.perf_counter() + warm_seconds
    n = 0
    while n < warmup or time.perf_counter() < t_warm:
        call()
        n += 1
        if n % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    # timed region: exactly K steps back to back, bracketed by synchronisation
    # (wall clock: the step rate) and by a pair of HIP events on the launch
    # stream (GPU time: the mean duration of one call's kernels, without the
    # host's per-call overhead, which the queue of calls hides)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        call()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / steps
    launch_ms = ev0.elapsed_time(ev1) / steps

    # cold calls: reading 1 GiB between calls evicts the 256 MB Infinity Cache
    # (a read, so no dirty lines are written back during the timed call)
    cold = []
    if n_cold:
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        for _ in range(n_cold):
            flush.sum()
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record(stream)
            call()
            e.record(stream)
            torch.cuda.synchronize()
            cold.append(s.elapsed_time(e))
        del flush

    bound = "mfma" if flops / (BF16_PEAK_TFLOPS * 1e12) > total_bytes / (HBM_PEAK_GBS * 1e9) else "hbm"
    if bound == "hbm":
        achieved = total_bytes / (launch_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_record(b.name)}
        value = kv_bytes / (ms_per_step * 1e-3) / 1e12
        unit = "TB/s"
    else:
        achieved = flops / (launch_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_record(b.name)}
        value = flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
    res = {
        "value": round(value, 4),
        "unit": unit,
        "ms_per_step": round(ms_per_step, 5),
        "dtype": "bf16" if b.kv_format == "bf16" else "bf16 q/out, fp8 e4m3 KV",
        "config": {
            "workload": b.name,
            "num_seqs": b.num_seqs, "total_q": b.total_q,
            "context_tokens": int(b.k_lens.sum()), "max_seqlen_q": b.max_seqlen_q,
            "max_seqlen_k": b.max_seqlen_k, "num_q_heads": b.num_q_heads,
            "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
            "block_size": b.block_size, "causal": b.causal, "parallelism": "single GPU",
        },
        "us_per_batch": round(ms_per_step * 1e3, 2),
        "us_per_launch_events": round(launch_ms * 1e3, 2),
        "us_per_launch_cold_p10_p50_p90": [round(float(np.percentile(cold, p)) * 1e3, 2)
                                           for p in (10, 50, 90)] if cold else None,
        "algorithmic_bytes_per_launch": total_bytes,
        "algorithmic_flops_per_launch": flops,
        "plan": plan,
        "roofline": roof,
    }
    prof = profile_record(b.name)
    if prof and prof.get("mfma_util_pct") is not None:
        # matrix-core and LDS counters of the same kernel (committed rocprofv3 summary)
        res["counters"] = {"kernel": prof["kernel"], "mfma_util_pct": round(prof["mfma_util_pct"], 2),
                           "mfma_flops_bf16_per_launch": prof["mfma_flops_bf16"],
                           "lds_bank_conflict": prof["lds_bank_conflict"]}
        for key in ("lds_util_pct", "valu_busy_pct", "vmem_latency_cycles"):
            if prof.get(key) is not None:
                res["counters"][key] = round(prof[key], 2)
    return res


if __name__ == "__main__":
    main()
