#!/usr/bin/env python3
"""Decode-attention benchmark: KV-read GB/s (vs MI355X peak HBM bandwidth) and us/step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long]
    python bench.py --probe            # the read-bandwidth ceilings (stream and paged gather)

The default workload is the 32K long-context step (B=4, 64 query / 8 KV heads,
d_h 128, 32768 cached tokens + 1 appended per sequence, block 32, bf16), the
largest configuration that fits one GPU.

One step = one pass of the decode hot path over one batch: the KV append of the
new token (for workloads that append) and paged decode attention, split over
the context with the log-sum-exp merge done by each pair's last workgroup: one
fused kernel launch through the C ABI.  Inputs are seeded
synthetic tensors already resident in HBM when timing starts.  To measure HBM
rather than the 256 MB on-die Infinity Cache, consecutive steps rotate over
copies of the KV pool, enough that a copy is read again only after 1 GiB of
other KV reads when the timed pass has at least as many steps as copies.  A
graph of fewer steps re-reads each of its copies once per pass, after
(K - 1) x the step's bytes (config.reuse_distance_bytes says which; 608 MiB at
the 8K step with K = 20, still more than twice the Infinity Cache).

Workload ``verify4`` is the verification pass of speculative decoding on the
8K grouped-query shape: each step commits 4 new tokens (the pending one and 3
drafts) and attends for all 4 positions, in one fused kernel.  ``verify4_long``
is the same on the 32K long-context shape (G = 8: 32 query rows per sequence
and KV head).

Workload ``mha_fp8_append`` is the fp8 decode step on the 40-head MHA shape:
the quantising append of each sequence's new token (power-of-two scale per
(block, KV head), grown if needed) fused with fp8 attention, one launch.

Workload ``mha_fp8_kivi`` is the 40-head MHA shape with the KIVI scale layout
(keys scaled per channel of each block, values per token); its bytes include
those scales.

Workload ``long_fp8`` is the 32K grouped-query shape (B = 4, 64/8 heads, block
32, 32768 tokens) over an fp8 pool with one scale per (block, KV head), no
append: the matrix path's fp8 variant at G = 8.

Workload ``cow_fork`` measures the copy-on-write block copy instead: 256 prompts
on the 8K grouped-query pool geometry each fork into 8 parallel samples, so each
prompt's partially filled last block is copied to 7 fresh blocks (1792 copies,
one kernel launch per step); its bytes are the unique source blocks read plus
the destination blocks written.

Prints one JSON line (rank 0, N=1).  `value` = algorithmic KV bytes per step /
step time.  `roofline.achieved` = the same bytes / the decode-attention call's
average duration measured with HIP events on the launch stream;
`roofline.sustained_gbs` is what a read probe with the same tiles, table and
bytes per launch reaches on the same box (no compute), and `distribution` the
p10/p50/p90 of the per-step kernel time over further graph replays.  The float64
CPU oracle is timed on a bounded sample as `cpu_baseline`; `context` quotes the
pages' own figures for other hardware.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E peak, 8 TB/s
ROTATE_BYTES = 1 << 30         # distance between reuses of one pool copy
COPY_BYTES = 256 << 20         # read and written by the PMC calibration kernel
METRIC = "decode-attention KV-read HBM GB/s (% of MI355X peak) and µs/step"
MERGE_KERNEL = "merge_splits_kernel"    # the split merge's own launch (16 or more rows)
DEFAULT_WORKLOAD = "long"

# Figures the pages quote for other hardware: context only, neither target nor
# baseline (the metric's denominator is MI355X's own peak).
PAGES_CONTEXT = {
    "note": "the pages' own figures for other hardware; context only",
    "h100_sxm": {"bf16_dense_tflops": 989.0, "hbm_tb_per_s": 3.35,
                 "source": "Module 10: Inference and Deployment Serving, matrix-vector "
                           "section (ridge 989/3.35 = 295 FLOP/byte); The Mathematics of "
                           "Transformer Inference, section 3"},
    "tpu_v5e": {"bf16_tflops": 197.0, "hbm_tb_per_s": 0.82,
                "source": "The Mathematics of Transformer Inference, section 3"},
    "cpu_4_threads": {"effective_gb_per_s": 48.24,
                      "workload": "float32 8192 x 8192 matrix-vector product, B = 1, "
                                  "5.566 ms per product",
                      "source": "Module 10: Inference and Deployment Serving, 'Measure "
                                "the CPU, don't guess from the clock' (Lab 1)"},
}


def pages_context(kv_bytes):
    """PAGES_CONTEXT plus the time each quoted device would need to read this step's KV
    bytes once at its quoted bandwidth (the decode-step lower bound of The Mathematics
    of Transformer Inference, section 6)."""
    ctx = json.loads(json.dumps(PAGES_CONTEXT))
    ctx["kv_read_us_at_quoted_bandwidth"] = {
        "h100_sxm": round(kv_bytes / 3.35e12 * 1e6, 2),
        "tpu_v5e": round(kv_bytes / 0.82e12 * 1e6, 2),
        "cpu_4_threads": round(kv_bytes / 48.24e9 * 1e6, 2),
        "mi355x_peak": round(kv_bytes / (PEAK_HBM_GBS * 1e9) * 1e6, 2),
    }
    return ctx


def kv_bytes_per_step(spec, context_lens):
    """Algorithmic bytes: every attended K and V element at stored width, plus the fp8
    scales of the attended blocks (one K and one V scale per (block, KV head); KIVI:
    d_h key scales and block_size value scales)."""
    import numpy as np
    esz = 1 if spec.kv_dtype.startswith("fp8") else 2
    ctx = context_lens.astype(np.int64)
    total = int(ctx.sum()) * spec.num_kv_heads * spec.head_dim * 2 * esz
    nb = (ctx + spec.block_size - 1) // spec.block_size
    if spec.kv_dtype == "fp8":
        total += int(nb.sum()) * spec.num_kv_heads * 2 * 4
    elif spec.kv_dtype == "fp8_kivi":
        total += int(nb.sum()) * spec.num_kv_heads * (spec.head_dim + spec.block_size) * 4
    return total


FORK_PROMPTS, FORK_SAMPLES = 256, 8     # cow_fork: prompts x parallel samples each


def fork_geometry():
    """(pairs, H_kv, d_h, block_size, blocks per rotation range, algorithmic bytes) of
    the cow_fork step: every prompt's source block is read once and each of its
    FORK_SAMPLES - 1 copies written once, K and V."""
    from workloads import SPECS
    s = SPECS["llama8b"]
    pairs = FORK_PROMPTS * (FORK_SAMPLES - 1)
    block_bytes = s.num_kv_heads * s.block_size * s.head_dim * 2 * 2      # K and V, bf16
    return (pairs, s.num_kv_heads, s.head_dim, s.block_size, FORK_PROMPTS + pairs,
            (FORK_PROMPTS + pairs) * block_bytes)


def fork_pairs(np, seed, first_block):
    """Seeded source/destination lists of one cow_fork range starting at first_block:
    a random permutation of the range gives each prompt its source block and fresh
    destination blocks; copies of one source are adjacent in the list."""
    pairs, _, _, _, nblk, _ = fork_geometry()
    perm = np.random.default_rng([seed, first_block]).permutation(nblk).astype(np.int32)
    perm += first_block
    src = np.repeat(perm[:FORK_PROMPTS], FORK_SAMPLES - 1)
    dst = perm[FORK_PROMPTS:]
    return src, dst


def identity_layout(case):
    """Control-run layout, in place: the same contents with every sequence's blocks
    stored one after another in logical order (then the unused blocks), so the
    block table is the identity over the used blocks."""
    import numpy as np
    tab = case["block_tables"]
    used = [int(x) for x in tab.reshape(-1) if x >= 0]
    used_set = set(used)
    rest = [i for i in range(case["k_pool"].shape[0]) if i not in used_set]
    order = np.array(used + rest, dtype=np.int64)
    for key in ("k_pool", "v_pool", "k_pool_full", "v_pool_full", "k_scale", "v_scale"):
        if case.get(key) is not None:
            case[key] = np.ascontiguousarray(case[key][order])
    ident = np.full_like(tab, -1)
    ident[tab >= 0] = np.arange(len(used), dtype=tab.dtype)
    case["block_tables"] = ident


KERNEL_SOURCES = ("common.h", "decode_kernel.h", "gqa_paged.hip", "kv_cache_ops.h")


def kernel_source_hash():
    """Hash of the sources the decode and block-copy kernels are built from (their
    launch code included); the probes' sources are not part of it."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gqa_decode_attention_paged_amd", "csrc")
    for name in KERNEL_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def profiled_kernel_time(workload):
    """Per-dispatch duration statistics of the workload's kernel from a committed
    rocprofv3 kernel trace (profiles/kernel_time_<workload>.json), if it was taken on
    the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"kernel_time_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t


def write_kernel_time(workload, trace_dir, kv_bytes):
    """Host only: per-dispatch durations of the workload's kernel from a rocprofv3
    `--kernel-trace -f csv` output directory -> profiles/kernel_time_<workload>.json."""
    import csv
    import glob
    import statistics
    kname = "kv_copy_blocks_kernel" if workload == "cow_fork" else "paged_decode_kernel"
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    # A call whose split merge runs in its own launch (merge_splits_kernel) lasts
    # from its decode dispatch's start to the end of the merge dispatch that follows.
    events = []
    for path in files:
        with open(path) as f:
            for row in csv.DictReader(f):
                n = row["Kernel_Name"]
                if kname in n or MERGE_KERNEL in n:
                    events.append((int(row["Start_Timestamp"]), int(row["End_Timestamp"]),
                                   MERGE_KERNEL in n))
    events.sort()
    durs, merged = [], False
    for i, (start, end, is_merge) in enumerate(events):
        if is_merge:
            continue
        if i + 1 < len(events) and events[i + 1][2]:
            end, merged = events[i + 1][1], True
        durs.append((end - start) / 1e3)
    if not durs:
        raise SystemExit(f"no {kname} dispatches in {files}")
    if merged:
        kname = f"{kname} + {MERGE_KERNEL}"
    durs.sort()
    q = lambda f: durs[min(len(durs) - 1, int(f * len(durs)))]
    out = {"workload": workload, "kernel": kname, "kernel_source_sha": kernel_source_hash(),
           "dispatches": len(durs), "avg_us": round(statistics.fmean(durs), 3),
           "p10_us": round(q(0.1), 3), "p50_us": round(statistics.median(durs), 3),
           "p90_us": round(q(0.9), 3), "min_us": round(durs[0], 3), "max_us": round(durs[-1], 3),
           "algorithmic_bytes_per_call": kv_bytes}
    out["achieved_gbs_avg"] = round(kv_bytes / (out["avg_us"] * 1e-6) / 1e9, 2)
    out["frac_avg"] = round(out["achieved_gbs_avg"] / PEAK_HBM_GBS, 4)
    path = os.path.join(ROOT, "profiles", f"kernel_time_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def counted_traffic(workload):
    """HBM bytes per decode call from committed rocprofv3 PMC runs, if they were taken
    on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_call")


def _pmc_per_dispatch(run_dir, counter, name_filter):
    """{dispatch id: counter value} for the dispatches of kernels whose name passes
    name_filter, from a rocprofv3 `--pmc <counter> -f csv` output directory."""
    import csv
    import glob
    vals, names = {}, {}
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    for path in files:
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] != counter or not name_filter(row["Kernel_Name"]):
                    continue
                key = (path, row["Dispatch_Id"])
                vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
                names[key] = row["Kernel_Name"]
    return vals, names


def write_traffic(workload, pmc_dir, kv_bytes):
    """Turn four rocprofv3 PMC runs (decode FETCH_SIZE / WRITE_SIZE, calibration-copy
    FETCH_SIZE / WRITE_SIZE, in <pmc_dir>/{fetch,write,copy_fetch,copy_write}) into
    profiles/traffic_<workload>.json.  Counters are KiB per dispatch; each is scaled
    by (known copy bytes) / (what the same counter reads for the copy kernel)."""
    import statistics
    kname = "kv_copy_blocks_kernel" if workload == "cow_fork" else "paged_decode_kernel"
    is_decode = lambda n: kname in n
    is_merge = lambda n: MERGE_KERNEL in n
    is_copy = lambda n: "elementwise" in n and "Fill" not in n
    out = {"workload": workload, "kernel_source_sha": kernel_source_hash(),
           "algorithmic_bytes_per_call": kv_bytes}
    for counter, sub in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
        cal, _ = _pmc_per_dispatch(os.path.join(pmc_dir, "copy_" + sub), counter, is_copy)
        run, _ = _pmc_per_dispatch(os.path.join(pmc_dir, sub), counter, is_decode)
        mrg, _ = _pmc_per_dispatch(os.path.join(pmc_dir, sub), counter, is_merge)
        if not cal or not run:
            raise SystemExit(f"{counter}: missing dispatches (copy {len(cal)}, decode {len(run)})")
        cal_kib = statistics.median(cal.values())
        scale = COPY_BYTES / (cal_kib * 1024.0)
        kib = statistics.median(run.values())
        out[counter] = {"decode_kib_median": kib, "decode_dispatches": len(run),
                        "copy_kib_median": cal_kib, "copy_dispatches": len(cal), "scale": scale}
        if mrg:                    # the split merge's own launch, one per call
            out[counter]["merge_kib_median"] = statistics.median(mrg.values())
            out[counter]["merge_dispatches"] = len(mrg)
            kib += out[counter]["merge_kib_median"]
        out[counter]["bytes_per_call"] = kib * 1024.0 * scale
    out["hbm_bytes_per_call"] = round(out["FETCH_SIZE"]["bytes_per_call"] +
                                      out["WRITE_SIZE"]["bytes_per_call"])
    out["traffic_over_algorithmic"] = out["hbm_bytes_per_call"] / kv_bytes
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def cpu_baseline(case, kv_bytes, min_seconds, threads=1):
    """Time the float64 oracle (as it stands) on whole steps of the workload with
    `threads` BLAS threads."""
    from threadpoolctl import threadpool_limits
    import oracle
    spec = case["spec"]
    fn = (oracle.paged_multi_query_attention if case.get("num_queries")
          else oracle.paged_decode_attention)
    n, t0 = 0, time.perf_counter()
    with threadpool_limits(limits=threads):
        while True:
            kp, vp, ks, vs = (case["k_pool_full"], case["v_pool_full"], case["k_scale"],
                              case["v_scale"])
            if "fp8_k_new" in case:
                kp, vp, ks, vs = oracle.kv_append_fp8(kp, vp, ks, vs, case["fp8_k_new"],
                                                      case["fp8_v_new"], case["block_tables"],
                                                      case["fp8_start"], spec.block_size)
            fn(case["q"], kp, vp, case["block_tables"],
               case["context_lens"], spec.block_size, case["softmax_scale"], spec.kv_dtype,
               ks, vs)
            n += 1
            el = time.perf_counter() - t0
            if el >= min_seconds:
                break
    per_step = el / n
    return {"value": round(kv_bytes / per_step / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{n} whole step(s) of the {spec.name} workload"
                      f"{' with the fp8 append' if 'fp8_k_new' in case else ''}"
                      f"{' with %d query positions' % case['num_queries'] if case.get('num_queries') else ''}"
                      ", float64 numpy oracle, "
                      f"{threads} BLAS thread(s), {el:.1f} s total ({per_step * 1e3:.1f} ms/step)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    choices=["tiny", "llama8b", "batched", "long", "mha_fp8", "verify4",
                             "verify4_long", "mha_fp8_append", "mha_fp8_kivi", "long_fp8",
                             "cow_fork"])
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--identity-table", action="store_true",
                    help="control run: the same data with each sequence's blocks stored "
                         "contiguously and an identity block table (prices the gather)")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch the timed steps eagerly instead of replaying a HIP graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 256 MiB device copies (for scaling PMC byte counters)")
    ap.add_argument("--traffic-from", metavar="PMC_DIR",
                    help="host only: write profiles/traffic_<workload>.json from rocprofv3 "
                         "PMC runs stored under PMC_DIR/{fetch,write,copy_fetch,copy_write}")
    ap.add_argument("--kernel-stats-from", metavar="TRACE_DIR",
                    help="host only: write profiles/kernel_time_<workload>.json from a "
                         "rocprofv3 --kernel-trace -f csv run of this workload")
    ap.add_argument("--settle-ms", type=float, default=100.0,
                    help="untimed replays of the K-step graph, for at least this long, right "
                         "before the timed pass: the GPU's clocks settle over the first "
                         "10-20 ms of sustained work, and a pass inside that transient runs "
                         "about 3%% slow")
    ap.add_argument("--reps", type=int, default=10,
                    help="further timed replays of the K-step graph for the p10/p50/p90 "
                         "distribution (outside the headline timing)")
    ap.add_argument("--batch-invariant", action="store_true",
                    help="split every sequence by its own length only (GQA_FLAG_BATCH_INVARIANT)")
    ap.add_argument("--split-tokens", type=int, default=0, metavar="T",
                    help="split-length override (gqa_set_split_tokens): the batch-invariant "
                         "plan with about one split per T tokens")
    ap.add_argument("--no-sustained", action="store_true",
                    help="skip the read probe of the workload's tile pattern")
    ap.add_argument("--probe", action="store_true",
                    help="only run the read-bandwidth probes (plain streaming read, paged "
                         "gather at each tile size, a lone workgroup) and print their rates")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this decode-attention path has no "
              "multi-GPU mode (see the sharding notes in the design document).", file=sys.stderr)
        sys.exit(2)

    import numpy as np

    verify = args.workload in ("verify4", "verify4_long")   # 4 query positions
    fp8_append = args.workload == "mha_fp8_append"
    base_name = {"verify4": "llama8b", "verify4_long": "long",
                 "mha_fp8_append": "mha_fp8"}.get(args.workload, args.workload)
    if args.traffic_from and args.workload == "cow_fork":
        write_traffic(args.workload, args.traffic_from, fork_geometry()[5])
        return
    if args.traffic_from:
        from workloads import make_case, SPECS
        spec = SPECS[base_name]
        write_traffic(args.workload, args.traffic_from,
                      kv_bytes_per_step(spec, make_case(spec, seed=args.seed)["context_lens"]))
        return
    if args.kernel_stats_from:
        from workloads import make_case, SPECS
        if args.workload == "cow_fork":
            kvb = fork_geometry()[5]
        else:
            spec = SPECS[base_name]
            kvb = kv_bytes_per_step(spec, make_case(spec, seed=args.seed)["context_lens"])
        write_kernel_time(args.workload, args.kernel_stats_from, kvb)
        return

    import torch

    import gqa_decode_attention_paged_amd as gqa
    from workloads import make_case, make_multi_query_case, new_token_rows, SPECS

    if args.copy_calibration:
        # A plain elementwise kernel that reads and writes COPY_BYTES each: the known
        # size against which the PMC byte counters are scaled.
        src = torch.zeros(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.add(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": COPY_BYTES, "copies": 5}))
        return

    gqa.load()
    if args.probe:
        for line in probe_suite(args, np, torch, gqa):
            print(json.dumps(line), flush=True)
        return
    if args.workload == "cow_fork":
        print(json.dumps(bench_block_copy(args, np, torch, gqa)), flush=True)
        return
    dev = torch.device("cuda:0")
    spec = SPECS[base_name]
    case = (make_multi_query_case(spec, 4, seed=args.seed) if verify
            else make_case(spec, seed=args.seed))
    if fp8_append:
        case["fp8_k_new"] = new_token_rows(spec, 1, seed=args.seed)
        case["fp8_v_new"] = new_token_rows(spec, 1, seed=args.seed + 1)
        case["fp8_start"] = (case["context_lens"] - 1).astype(np.int32)
    nq = case.get("num_queries", 1)
    kv_bytes = kv_bytes_per_step(spec, case["context_lens"])
    if args.identity_table:
        identity_layout(case)

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    def pool(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev) if a.dtype == np.uint8 else bf16(a)

    q = bf16(case["q"])
    bt = torch.from_numpy(case["block_tables"]).to(dev)
    ctx = torch.from_numpy(case["context_lens"]).to(dev)
    pos = torch.from_numpy(case["positions"]).to(dev)
    k_new = bf16(case["k_new"]) if case["k_new"] is not None else None
    v_new = bf16(case["v_new"]) if case["v_new"] is not None else None
    ks = torch.from_numpy(case["k_scale"]).to(dev) if case["k_scale"] is not None else None
    vs = torch.from_numpy(case["v_scale"]).to(dev) if case["v_scale"] is not None else None
    k0, v0 = pool(case["k_pool"]), pool(case["v_pool"])
    copies = min(256, max(1, math.ceil(ROTATE_BYTES / kv_bytes) + 1))
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    if fp8_append:                 # each pool copy has its own scales: the append writes them
        scales = [(ks, vs)] + [(ks.clone(), vs.clone()) for _ in range(copies - 1)]
        k8_new, v8_new = bf16(case["fp8_k_new"][:, 0]), bf16(case["fp8_v_new"][:, 0])
        start8 = torch.from_numpy(case["fp8_start"]).to(dev)
    max_ctx = int(case["context_lens"].max())
    if args.split_tokens:
        gqa.set_split_tokens(args.split_tokens)
    inv = args.batch_invariant or args.split_tokens > 0
    shape = gqa.make_shape(spec.num_seqs, spec.num_q_heads, k0, bt, batch_invariant=inv)
    ws = torch.zeros(max(16, gqa.multi_query_workspace_size(shape, nq, max_ctx)),
                     dtype=torch.uint8, device=dev)
    rows = (spec.num_seqs, nq, spec.num_q_heads) if verify else (spec.num_seqs, spec.num_q_heads)
    out = torch.empty(rows + (spec.head_dim,), dtype=torch.float32, device=dev)
    lse = torch.empty(rows, dtype=torch.float32, device=dev)
    scale = case["softmax_scale"]

    def step(i):
        kc, vc = pools[i % copies]
        if fp8_append:             # fused: quantise and commit the new token, attend
            ksc, vsc = scales[i % copies]
            gqa.paged_decode_append_attention(q, k8_new, v8_new, start8, kc, vc, bt, ctx,
                                              max_ctx, scale, out=out, out_lse=lse,
                                              workspace=ws, k_scale=ksc, v_scale=vsc,
                                              batch_invariant=inv)
        elif verify:               # fused: commit the 4 new tokens, attend for all 4 positions
            gqa.paged_decode_multi_query_append(q, k_new, v_new, kc, vc, bt, ctx, max_ctx, scale,
                                                out=out, out_lse=lse, workspace=ws,
                                                batch_invariant=inv)
        elif k_new is not None:    # fused: commit the new token and attend, one kernel
            gqa.paged_decode_append_attention(q, k_new, v_new, pos, kc, vc, bt, ctx, max_ctx,
                                              scale, out=out, out_lse=lse, workspace=ws,
                                              batch_invariant=inv)
        else:
            gqa.paged_decode_attention(q, kc, vc, bt, ctx, max_ctx, scale, ks, vs, out=out,
                                       out_lse=lse, workspace=ws, batch_invariant=inv)

    ms_per_step, call_ms, graphed, dist = _timed(torch, args, step)
    if gqa.workspace_status(ws) != 0:
        raise SystemExit(f"device status {gqa.workspace_status(ws)}: bad inputs in the bench")
    achieved = kv_bytes / (call_ms * 1e-3) / 1e9
    esz = 1 if spec.kv_dtype.startswith("fp8") else 2
    del pools
    if fp8_append:
        del scales
    torch.cuda.empty_cache()
    sustained = None
    if not args.no_sustained:
        nb = (case["context_lens"].astype(np.int64) + spec.block_size - 1) // spec.block_size
        sustained = sustained_probe(args, np, torch, gqa,
                                    tile_bytes=spec.block_size * spec.head_dim * esz,
                                    num_tiles=int(nb.sum()) * spec.num_kv_heads * 2)
    if fp8_append:
        kernel = ("paged_decode_kernel (fused fp8 KV append with the power-of-two scale "
                  "policy + split attention + log-sum-exp merge)")
    elif verify:
        kernel = ("paged_decode_kernel (fused 4-token KV append + 4 query positions, split "
                  "attention) + merge_splits_kernel (log-sum-exp merge of the splits, its own "
                  "launch at 16 or more rows per KV head)")
    elif k_new is not None:
        kernel = "paged_decode_kernel (fused KV append + split attention + log-sum-exp merge)"
    elif spec.kv_dtype == "fp8_kivi":
        kernel = ("paged_decode_kernel (fp8 with KIVI scales: per-channel keys, per-token "
                  "values; split attention + log-sum-exp merge)")
    else:
        kernel = "paged_decode_kernel (split attention + log-sum-exp merge)"

    prof = profiled_kernel_time(args.workload) if not (args.identity_table or inv) else None
    result = {
        "metric": METRIC,
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.kv_dtype == "bf16" else "fp8",
        # fp8 stores E4M3 codes; the arithmetic is fp32 after dequantisation
        "data": "synthetic (seeded N(0,1) q/k/v, random block placement; no weights)",
        "config": {
            "workload": args.workload, "num_seqs": spec.num_seqs, "num_q_heads": spec.num_q_heads,
            "num_kv_heads": spec.num_kv_heads, "head_dim": spec.head_dim,
            "block_size": spec.block_size, "kv_dtype": spec.kv_dtype,
            "context_lens_total": int(case["context_lens"].sum()), "append": spec.append,
            "query_positions": nq, "fp8_append": fp8_append,
            "block_table": "identity (control run)" if args.identity_table else "random permutation",
            "kv_bytes_per_step": kv_bytes, "pool_copies_rotated": copies,
            "reuse_distance_bytes": (min(copies, args.steps) - 1) * kv_bytes,
            "split_policy": (f"batch-invariant, about one split per {args.split_tokens} tokens"
                             if args.split_tokens else
                             "batch-invariant" if inv else "default (fills the GPU once)"),
        },
        "distribution": dist,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": counted_traffic(args.workload),
            "kernel": kernel,
            "kernel_us_events": round(call_ms * 1e3, 3),
            "timing": ("HIP events on the launch stream around one replay of a graph of the "
                       "K steps (one kernel per step), divided by K" if graphed else
                       "HIP events around K eager steps, divided by K"),
            "sustained_gbs": sustained["gbs"] if sustained else None,
            "frac_of_sustained": (round(achieved / sustained["gbs"], 4) if sustained else None),
            "sustained_probe": sustained["what"] if sustained else None,
            "rocprof": ({k: prof[k] for k in ("dispatches", "avg_us", "p10_us", "p50_us",
                                              "p90_us", "achieved_gbs_avg", "frac_avg")}
                        if prof else None),
        },
        "context": pages_context(kv_bytes),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, kv_bytes, args.cpu_seconds)
        cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
        result["cpu_baseline"]["all_cores"] = {
            k: v for k, v in cpu_baseline(case, kv_bytes, args.cpu_seconds, cores).items()
            if k in ("value", "cores", "sample")}
    print(json.dumps(result), flush=True)


def _timed(torch, args, step):
    """Warm up, record the K timed steps into a HIP graph (unless --no-graph), and
    return (wall ms per step, event ms per step on the launch stream, graph used,
    distribution).  The headline figures come from exactly one timed pass of the K
    steps; the distribution (p10/p50/p90 of the per-step event time) from args.reps
    further passes, each timed alone."""
    dev = torch.device("cuda:0")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    graph = None
    if not args.no_graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(args.steps):
                step(args.warmup + i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
    settle_until = time.perf_counter() + getattr(args, "settle_ms", 0.0) * 1e-3
    while time.perf_counter() < settle_until:       # untimed: lets the clocks settle
        if graph is not None:
            graph.replay()
        else:
            for i in range(args.steps):
                step(args.warmup + i)
        torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(args.warmup + i)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = []
    for r in range(args.reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(args.steps):
                step(args.warmup + (r + 1) * args.steps + i)
        b.record(stream)
        torch.cuda.synchronize()
        per_step.append(a.elapsed_time(b) * 1e3 / args.steps)
    dist = None
    if per_step:
        srt = sorted(per_step)
        pick = lambda f: round(srt[min(len(srt) - 1, int(f * len(srt)))], 3)
        dist = {"reps": len(per_step), "steps_per_rep": args.steps,
                "unit": "µs per step (HIP events per pass of the K steps)",
                "p10": pick(0.1), "p50": round(sorted(per_step)[len(srt) // 2], 3),
                "p90": pick(0.9)}
    return (wall * 1e3 / args.steps, start.elapsed_time(stop) / args.steps, graph is not None,
            dist)


PROBE_PATTERNS = {0: "whole rows (16 B per lane, 1 KiB contiguous per instruction)",
                  1: "operand rows: 16 rows x 64 B of 256-byte rows (bf16 K, MFMA layout)",
                  2: "operand rows: 16 rows x 64 B of 128-byte rows (fp8 K, 16 B per lane)",
                  3: "operand rows: 16 rows x 32 B of 128-byte rows (fp8 K, 8 B per lane)",
                  4: "half operand rows (256-byte rows), half whole rows (K and V tiles)"}


def probe_rate(args, np, torch, gqa, *, total_bytes, tile_bytes, table, non_temporal,
               workgroups=None, steps=None, pattern=0):
    """One read-probe configuration: a graph of `steps` launches, each reading
    total_bytes in tiles of tile_bytes (through a random permutation table, or as a
    plain stream), rotated over copies so each launch reads bytes last touched at
    least 1 GiB of reads ago.  Returns a dict with GB/s (events) and its spread."""
    dev = torch.device("cuda:0")
    if workgroups is None:
        workgroups = torch.cuda.get_device_properties(dev).multi_processor_count
    ntiles = total_bytes // tile_bytes
    copies = max(1, math.ceil(ROTATE_BYTES / (ntiles * tile_bytes)) + 1)
    buf = torch.zeros(copies * ntiles * tile_bytes, dtype=torch.uint8, device=dev)
    ids = None
    if table:
        perm = np.random.default_rng([args.seed, tile_bytes, ntiles]).permutation(ntiles)
        ids = torch.from_numpy(perm.astype(np.int32)).to(dev)
    sink = torch.empty(workgroups * 8, dtype=torch.int32, device=dev)
    base = buf.data_ptr()

    def step(i):
        gqa.probe_read(base + (i % copies) * ntiles * tile_bytes, ntiles, ids, ntiles,
                       tile_bytes, non_temporal, workgroups, sink, pattern=pattern)

    sub = argparse.Namespace(**vars(args))
    sub.steps = steps or max(args.steps, 20)
    sub.warmup = max(args.warmup, 3)
    sub.reps = max(args.reps, 5)
    sub.no_graph = False
    _, call_ms, _, dist = _timed(torch, sub, step)
    del buf
    torch.cuda.empty_cache()
    gbs = lambda us: round(ntiles * tile_bytes / (us * 1e-6) / 1e9, 1)
    return {"gbs": gbs(call_ms * 1e3), "us_per_launch": round(call_ms * 1e3, 3),
            "gbs_p10_p50_p90": [gbs(dist["p90"]), gbs(dist["p50"]), gbs(dist["p10"])],
            "bytes_per_launch": ntiles * tile_bytes, "tile_bytes": tile_bytes,
            "table": "random permutation" if table else "none (contiguous stream)",
            "non_temporal": bool(non_temporal), "workgroups": workgroups,
            "launches": sub.steps, "copies_rotated": copies, "pattern": PROBE_PATTERNS[pattern]}


def sustained_probe(args, np, torch, gqa, tile_bytes, num_tiles):
    """The read probe with the workload's own pattern: its (block, KV head) tile size,
    as many tiles per launch as the step reads (K and V), a random table, and the
    non-temporal hint of the decode kernel's tile loads."""
    r = probe_rate(args, np, torch, gqa, total_bytes=num_tiles * tile_bytes,
                   tile_bytes=tile_bytes, table=True, non_temporal=1)
    r["what"] = (f"gqa_probe_read: {num_tiles} random {tile_bytes}-byte tiles per launch "
                 f"({r['bytes_per_launch']} bytes), non-temporal loads, {r['workgroups']} "
                 f"8-wave workgroups, no compute; HIP events over {r['launches']} launches")
    return r


def probe_suite(args, np, torch, gqa):
    """The read-bandwidth ceilings: a plain streaming read at several sizes, the paged
    gather at each tile size the pools use, and one workgroup gathering alone, each
    with the non-temporal hint and with the default policy; then the paged gather in
    the per-instruction patterns of the decode kernel's K loads."""
    runs = []
    for size in (32 << 20, 128 << 20, 512 << 20):
        for nt in (1, 0):
            runs.append(dict(total_bytes=size, tile_bytes=16384, table=False, non_temporal=nt))
    for tile in (2048, 4096, 8192, 16384):
        for nt in (1, 0):
            runs.append(dict(total_bytes=512 << 20, tile_bytes=tile, table=True, non_temporal=nt))
    for nt in (1, 0):
        runs.append(dict(total_bytes=8 << 20, tile_bytes=4096, table=True, non_temporal=nt,
                         workgroups=1, steps=5))
    # the decode kernel's per-instruction patterns of K loads, with its hint
    for pattern, tile in ((1, 4096), (1, 8192), (4, 8192), (2, 2048), (2, 4096), (3, 2048),
                          (3, 4096)):
        runs.append(dict(total_bytes=512 << 20, tile_bytes=tile, table=True, non_temporal=1,
                         pattern=pattern))
    out = []
    for kw in runs:
        r = probe_rate(args, np, torch, gqa, **kw)
        r["frac_of_peak"] = round(r["gbs"] / PEAK_HBM_GBS, 4)
        out.append(r)
    return out


def bench_block_copy(args, np, torch, gqa):
    """The cow_fork workload: one copy-on-write block-copy launch per step."""
    dev = torch.device("cuda:0")
    pairs, hkv, d, bs, nblk, alg_bytes = fork_geometry()
    copies = min(64, math.ceil(ROTATE_BYTES / alg_bytes) + 1)
    gen = torch.Generator(device=dev)
    gen.manual_seed(args.seed)
    k = torch.randn((copies * nblk, hkv, bs, d), generator=gen, device=dev).to(torch.bfloat16)
    v = torch.randn((copies * nblk, hkv, bs, d), generator=gen, device=dev).to(torch.bfloat16)
    lists = []
    for c in range(copies):
        src, dst = fork_pairs(np, args.seed, c * nblk)
        lists.append((torch.from_numpy(src).to(dev), torch.from_numpy(dst).to(dev)))

    def step(i):
        src, dst = lists[i % copies]
        gqa.kv_copy_blocks(k, v, src, dst)

    ms_per_step, call_ms, graphed, dist = _timed(torch, args, step)
    achieved = alg_bytes / (call_ms * 1e-3) / 1e9
    result = {
        "metric": "copy-on-write block copy HBM GB/s (unique source blocks read + copies "
                  "written, % of MI355X peak) and µs/step",
        "value": round(alg_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "us_per_step": round(ms_per_step * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) pools, random block placement; no weights)",
        "config": {
            "workload": "cow_fork", "prompts": FORK_PROMPTS, "samples_per_prompt": FORK_SAMPLES,
            "copies_per_step": pairs, "num_kv_heads": hkv, "head_dim": d, "block_size": bs,
            "kv_dtype": "bf16", "bytes_per_step": alg_bytes, "pool_ranges_rotated": copies,
        },
        "distribution": dist,
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": counted_traffic("cow_fork"),
            "kernel": "kv_copy_blocks_kernel (copy-on-write block copy)",
            "kernel_us_events": round(call_ms * 1e3, 3),
            "timing": ("HIP events on the launch stream around one replay of a graph of the "
                       "K steps (one kernel per step), divided by K" if graphed else
                       "HIP events around K eager steps, divided by K"),
        },
    }
    if not args.no_cpu_baseline:
        import oracle
        kh = np.random.default_rng(args.seed).integers(0, 1 << 16, (nblk, hkv, bs, d),
                                                       dtype=np.uint16)
        vh = kh[::-1].copy()
        src, dst = fork_pairs(np, args.seed, 0)
        n, t0 = 0, time.perf_counter()
        while True:
            oracle.copy_blocks(kh, vh, src, dst)
            n += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds:
                break
        per = el / n
        result["cpu_baseline"] = {
            "value": round(alg_bytes / per / 1e9, 4), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} whole step(s) of cow_fork (one {nblk}-block range), numpy oracle "
                      f"copy, 1 thread, {el:.1f} s total ({per * 1e3:.1f} ms/step)"}
    return result


if __name__ == "__main__":
    main()
