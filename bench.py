"""Throughput of split-KV MLA decode + LSE combine on one MI355X.

One step = one mla_split_decode call (partial-attention kernel + combine
kernel) over one batch of synthetic inputs resident in HBM.  Default workload:
the 120k-token long-context request (B=1, R=1, H=128, S=8 virtual shards,
interleave 1, bf16 N(0,1), 64-token blocks).

Timing: W warm-up steps, then exactly K steps captured in one HIP graph; the
graph is replayed three times untimed (its first replays run slower) and then
once between two device synchronisations; ms_per_step is that wall time
divided by K.  The K steps cycle through several copies of the KV cache whose
total exceeds the 256 MB Infinity Cache, so KV bytes come from HBM.  The
partial kernel's own duration is measured live with HIP events recorded by the
library on its stream (eager steps), and gives the roofline fraction;
partial_kernel_ms_warm is the same kernel fed the same KV copy every step
(held in the Infinity Cache when it fits), reported beside it.

roofline.traffic comes from a committed counter summary
(profiles/<kernel>_<workload>_counters.json, written by --summarize-counters
from two rocprofv3 --pmc runs) and is reported only while the kernel sources
still hash to what was profiled; otherwise it is null.

Prints one JSON line.
"""

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV tokens/s + HBM GB/s (% of peak) for split-KV MLA decode + LSE combine"
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
ROW_BYTES = 576 * 2
GRAPH_WARM_REPLAYS = 3  # untimed replays of the captured K-step graph before the timed one


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long",
                    choices=["long", "long_b2", "batch", "verify", "padded", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-one-shard", action="store_true",
                    help="skip the one-shard and the warm (same KV copy) partial launches "
                         "(profiled runs, so that every partial-kernel dispatch is a full, "
                         "HBM-fed step's)")
    ap.add_argument("--no-merge", action="store_true",
                    help="skip the timing of the two-way prefix/suffix merge")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the fp8 KV-cache variant of the workload")
    ap.add_argument("--no-gather", action="store_true",
                    help="skip the timing of the chunked-context KV gather")
    ap.add_argument("--no-single-p", action="store_true",
                    help="skip the single-rounding P mode of the workload")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--event-steps", type=int, default=20)
    ap.add_argument("--calibrate-copy-mb", type=float, default=0.0,
                    help="first run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--min-kv-set-mb", type=float, default=640.0,
                    help="cycle KV copies until the cycled set exceeds this many MB")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn the counter CSVs of a FETCH_SIZE run and a WRITE_SIZE run "
                         "(both made with --calibrate-copy-mb) into the JSON summary bench.py reads")
    return ap.parse_args()


KERNEL_SOURCES = ("split_kv_mla_amd/csrc/mla_kernels.h", "split_kv_mla_amd/csrc/mla_plan.h",
                  "split_kv_mla_amd/csrc/mla_split_kv.hip")
PARTIAL_KERNEL = "mla::partial_kernel<false, true>"      # the bf16 cache's instantiation (P as hi + lo)
PARTIAL_KERNEL_FP8 = "mla::partial_kernel<true, true>"   # the fp8 cache's
PARTIAL_KERNEL_SINGLE_P = "mla::partial_kernel<false, false>"  # bf16 cache, P rounded once


def kernel_source_sha():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_path(workload_name):
    return os.path.join(ROOT, "profiles", f"partial_kernel_{workload_name}_counters.json")


def summarize_counters(fetch_dir, write_dir, workload_name, calib_mib):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of every kernel, scaled to bytes by
    what the same counter reads for the plain copy kernels of known size."""
    def per_kernel(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise SystemExit(f"no counter_collection.csv under {d}")
        vals = {}
        for row in csv.DictReader(open(files[0])):
            if row["Counter_Name"] == counter:
                vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
        return vals
    fetch_all = per_kernel(fetch_dir, "FETCH_SIZE")
    write_all = per_kernel(write_dir, "WRITE_SIZE")
    fetch = {k: statistics.mean(v) for k, v in fetch_all.items()}
    write = {k: statistics.mean(v) for k, v in write_all.items()}
    known = calib_mib * 1024.0  # KiB read and written by each calibration copy
    def factor(table_all, name_part):
        # the calibration copy is the largest dispatch of its kernel (the runtime
        # also uses the blit kernel for the small host-to-device uploads)
        hits = [max(v) for k, v in table_all.items() if name_part in k]
        return known / hits[0] if hits and hits[0] > 0 else None
    rec = {
        "workload": workload_name, "source_sha": kernel_source_sha(),
        "calibration_mib": calib_mib,
        "fetch_factor_blit_copy": factor(fetch_all, "copyBuffer"),
        "write_factor_blit_copy": factor(write_all, "copyBuffer"),
        "fetch_factor_elementwise_copy": factor(fetch_all, "neg"),
        "write_factor_elementwise_copy": factor(write_all, "neg"),
        "kernels": {},
    }
    # Scale by the elementwise copy: like the mla kernels it moves whole 128-byte
    # lines with 16-byte lane accesses (the blit copy's factors are kept as a check).
    ff, wf = rec["fetch_factor_elementwise_copy"], rec["write_factor_elementwise_copy"]
    rec["scaled_by"] = "elementwise_copy"
    for k in sorted(set(fetch) | set(write)):
        if "mla::" not in k:
            continue
        short = k.split("(")[0].replace("void ", "")
        r_kib, w_kib = fetch.get(k), write.get(k)
        rec["kernels"][short] = {
            "fetch_kib_raw": r_kib, "write_kib_raw": w_kib,
            "read_bytes": r_kib * ff * 1024 if (r_kib is not None and ff) else None,
            "write_bytes": w_kib * wf * 1024 if (w_kib is not None and wf) else None,
        }
    return rec


def load_traffic(workload_name, kernel=PARTIAL_KERNEL):
    """HBM bytes per launch of the partial kernel from the committed counter
    summary, or None when there is none or the kernel changed since."""
    path = counters_path(workload_name)
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("source_sha") != kernel_source_sha():
        return None
    k = rec.get("kernels", {}).get(kernel)
    if not k or k.get("read_bytes") is None or k.get("write_bytes") is None:
        return None
    return k["read_bytes"] + k["write_bytes"]


def algorithmic_bytes(w):
    """Unique KV rows + q + out + per-shard lse + lse_final, per step."""
    rows = w.B * w.R * w.H
    return (w.unique_kv_tokens * ROW_BYTES + rows * ROW_BYTES + rows * 512 * 2
            + w.num_shards * rows * 4 + rows * 4)


def kernel_bytes(w):
    """What the partial kernel must read: unique KV rows and q."""
    return w.unique_kv_tokens * ROW_BYTES + w.B * w.R * w.H * ROW_BYTES


def host_description():
    """CPU model and the BLAS numpy links against, for the CPU baseline's record."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown BLAS"
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg["Build Dependencies"]["blas"]["name"]
    except Exception:
        pass
    return model, blas


def cpu_baseline(w, budget_s):
    import oracle
    threads = len(os.sched_getaffinity(0))
    model, blas = host_description()
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.mla_decode_oracle(w.q_bits, w.kv_bits, w.block_table, w.seq_lens, w.num_shards,
                                 w.interleave, w.scale, w.causal)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el * (reps + 1) / reps > 3 * budget_s:
            break
    tokens = reps * int(w.seq_lens.astype(np.int64).sum())
    return {"value": tokens / el, "unit": "KV tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} full run(s) of the float64 oracle (unsplit + per-shard attention) "
                      f"on this workload, {el:.1f} s, numpy BLAS ({blas}) threads = {threads}, {model}"}


MERGE_T, MERGE_H, MERGE_D = 131072, 6, 128


def merge_leg(mla, dev, launches):
    """Time the two-way merge in place (out = prefix) on T x 6 heads x 128 bf16
    states: per launch it reads both states and LSEs and writes one state and
    one LSE."""
    import torch
    gen = torch.Generator(device=dev).manual_seed(7)
    shape = (MERGE_T, MERGE_H, MERGE_D)
    p = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
    s = torch.randn(shape, generator=gen, device=dev).to(torch.bfloat16)
    lp = torch.rand((MERGE_H, MERGE_T), generator=gen, device=dev) * 15 - 3
    ls = torch.rand((MERGE_H, MERGE_T), generator=gen, device=dev) * 15 - 3
    for _ in range(2):
        mla.mla_merge_states(p, lp, s, ls, out=p, out_lse=lp)
    torch.cuda.synchronize()
    # back-to-back launches between two events, so that the host's own time
    # per launch is hidden behind the kernels
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(launches):
        mla.mla_merge_states(p, lp, s, ls, out=p, out_lse=lp)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / launches
    rows = MERGE_T * MERGE_H
    nbytes = 3 * rows * MERGE_D * 2 + 3 * rows * 4
    gbps = nbytes / (ms / 1e3) / 1e9
    return {"kernel": "mla::merge_kernel<1>", "workload": f"T={MERGE_T} H={MERGE_H} D={MERGE_D} bf16, in place",
            "ms": ms, "launches_timed": launches, "bytes_per_launch": nbytes, "achieved_gbps": gbps,
            "frac": gbps / HBM_PEAK_GBPS}


def variant_leg(mla, dev, launches, min_set_mb, counters_workload, fp8=False, single_p=False):
    """A variant of the long-context workload: its cache stored as fp8 E4M3
    codes plus one float32 scale per token (580 bytes per token instead of
    1152), or P rounded once to bf16 (half the value products): the partial
    kernel's own duration (HIP events the library records on its stream,
    cycling cache copies past the Infinity Cache), and the whole step
    (back-to-back steps between two events)."""
    import torch
    import workloads
    w = workloads.long_context(1)
    if fp8:
        w = workloads.to_fp8(w)
    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    if fp8:
        kv_mb = (w.kv_bits.nbytes + w.kv_scale.nbytes) / 1e6
    else:
        kv_mb = w.kv_bits.nbytes / 1e6
    copies = max(1, math.ceil(min_set_mb / kv_mb))
    if fp8:
        kvs = [(torch.from_numpy(w.kv_bits).to(dev), torch.from_numpy(w.kv_scale).to(dev)) for _ in range(copies)]
    else:
        host = torch.from_numpy(w.kv_bits.view(np.int16)).view(torch.bfloat16)
        kvs = [(host.to(dev), None) for _ in range(copies)]
    S, I = w.num_shards, w.interleave
    a = mla.decode_args(q, kvs[0][0], bt, sl, S, I, w.scale, w.causal, kv_scale=kvs[0][1], single_p=single_p)
    ws = mla.new_workspace(a, dev)
    out = torch.empty((w.B, w.R, w.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((S, w.B, w.R, w.H), dtype=torch.float32, device=dev)
    lf = torch.empty((w.B, w.R, w.H), dtype=torch.float32, device=dev)

    def step(i, events=None):
        kv, ks = kvs[i % copies]
        mla.mla_split_decode(q, kv, bt, sl, S, I, w.scale, w.causal, out=out, lse=lse, lse_final=lf,
                             workspace=ws, events=events, kv_scale=ks, single_p=single_p)

    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(launches)]
    for e in evs:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    for i, e in enumerate(evs):
        step(i, events=e)
    torch.cuda.synchronize()
    part = statistics.mean(e[0].elapsed_time(e[1]) for e in evs)
    comb = statistics.mean(e[1].elapsed_time(e[2]) for e in evs)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(launches):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    step_ms = e0.elapsed_time(e1) / launches
    tokens = int(w.seq_lens.astype(np.int64).sum())
    row = 576 + 4 if fp8 else ROW_BYTES
    kb = tokens * row + w.B * w.R * w.H * ROW_BYTES  # what the partial kernel must read: the cache rows and q
    gbps = kb / (part / 1e3) / 1e9
    kernel = PARTIAL_KERNEL_FP8 if fp8 else (PARTIAL_KERNEL_SINGLE_P if single_p else PARTIAL_KERNEL)
    rec = {"workload": w.name, "kv_bytes_per_token": row, "kv_copies_cycled": copies,
           "partial_kernel_ms": part, "combine_kernel_ms": comb, "ms_per_step": step_ms,
           "value": tokens / (step_ms / 1e3), "unit": "KV tokens/s",
           "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": gbps / HBM_PEAK_GBPS, "kernel": kernel, "bytes_per_launch": kb,
                        "traffic": load_traffic(counters_workload, kernel)}}
    if single_p:
        rec["p_precision"] = "bf16 (one rounding)"
    return rec


def gather_leg(mla, dev, steps):
    """Time the chunked-context KV gather of the 120k-token run's cached
    context: one step gathers every chunk of the plan (each request's whole
    context once); per row it reads 1152 bytes of KV and writes 1152."""
    import torch
    import workloads
    w = workloads.long_context_gather()
    kv = torch.from_numpy(w.kv_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    tables = torch.from_numpy(w.local_tables).to(dev)
    align = mla.mla_chunked_context_alignment(w.block_size, w.num_shards, w.interleave)
    ws_rows = mla.mla_align_chunked_context_workspace(w.workspace_rows, w.block_size, w.num_shards,
                                                      w.interleave, len(w.context_lens))
    C, K, _, _ = mla.mla_context_chunk_plan(w.context_lens, ws_rows, align)
    chunks = []
    for k in range(K):
        _, _, st, cu = mla.mla_context_chunk_plan(w.context_lens, ws_rows, align, chunk_index=k)
        chunks.append((torch.from_numpy(st).to(dev), torch.from_numpy(cu).to(dev), int(cu[-1])))
    out = torch.empty((ws_rows, 576), dtype=torch.bfloat16, device=dev)
    rows = sum(c[2] for c in chunks)
    views = [(st, cu, out[:n]) for st, cu, n in chunks]

    def one_step():
        for st, cu, o in views:
            mla.mla_gather_context_chunk(kv, tables, st, cu, w.interleave, out=o)

    for _ in range(2):
        one_step()
    torch.cuda.synchronize()
    # back-to-back steps between two events (the host's time per launch hidden)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        one_step()
    e1.record()
    torch.cuda.synchronize()
    med = e0.elapsed_time(e1) / steps
    nbytes = 2 * rows * ROW_BYTES
    gbps = nbytes / (med / 1e3) / 1e9
    return {"kernel": "mla::gather_kernel", "workload": w.name, "chunks": K, "chunk_rows": C,
            "alignment": align, "workspace_rows": ws_rows, "rows_per_step": rows, "steps_timed": steps,
            "ms_per_step": med,
            "bytes_per_step": nbytes, "achieved_gbps": gbps, "frac": gbps / HBM_PEAK_GBPS,
            "rows_per_s": rows / (med / 1e3)}


def pct(xs, q):
    xs = sorted(xs)
    return xs[min(len(xs) - 1, max(0, int(round(q * (len(xs) - 1)))))]


def main():
    args = parse()
    if args.summarize_counters:
        import workloads
        name = workloads.STANDARD[args.workload]().name
        calib = args.calibrate_copy_mb if args.calibrate_copy_mb > 0 else 256.0
        print(json.dumps(summarize_counters(*args.summarize_counters, name, calib), indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU; --gpus {args.gpus} is not supported "
              f"(the S shards are virtual, all on one device)", file=sys.stderr)
        sys.exit(2)
    import torch
    import split_kv_mla_amd as mla
    import workloads

    mla.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy_mb > 0:
        # counter calibration: a blit copy and an elementwise (negating) copy,
        # each reading and writing exactly calibrate_copy_mb MiB
        n = int(args.calibrate_copy_mb * (1 << 20)) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    w = workloads.STANDARD[args.workload]()
    q = torch.from_numpy(w.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    kv_host = torch.from_numpy(w.kv_bits.view(np.int16)).view(torch.bfloat16)
    kv_mb = kv_host.numel() * 2 / 1e6
    copies = max(1, math.ceil(args.min_kv_set_mb / kv_mb))
    kvs = [kv_host.to(dev) for _ in range(copies)]
    S, I = w.num_shards, w.interleave
    a = mla.decode_args(q, kvs[0], bt, sl, S, I, w.scale, w.causal)
    ws = mla.new_workspace(a, dev)
    out = torch.empty((w.B, w.R, w.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((S, w.B, w.R, w.H), dtype=torch.float32, device=dev)
    lf = torch.empty((w.B, w.R, w.H), dtype=torch.float32, device=dev)

    def step(i, events=None):
        mla.mla_split_decode(q, kvs[i % copies], bt, sl, S, I, w.scale, w.causal, out=out, lse=lse,
                             lse_final=lf, workspace=ws, events=events)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # per-kernel durations from events the library records on its stream
    part_ms, comb_ms = [], []
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.event_steps)]
    for e in evs:
        for x in e:
            x.record()
    torch.cuda.synchronize()
    for i, e in enumerate(evs):
        step(i, events=e)
    torch.cuda.synchronize()
    for e in evs:
        part_ms.append(e[0].elapsed_time(e[1]))
        comb_ms.append(e[1].elapsed_time(e[2]))

    # warm: the same KV copy every step, so it sits in the 256 MB Infinity
    # Cache when it fits (reported beside the cycled, HBM-fed figures)
    warm_ms = []
    for i in range(0 if args.no_one_shard else args.event_steps + 2):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        for x in e:
            x.record()
        torch.cuda.synchronize()
        mla.mla_split_decode(q, kvs[0], bt, sl, S, I, w.scale, w.causal, out=out, lse=lse, lse_final=lf,
                             workspace=ws, events=e)
        torch.cuda.synchronize()
        if i >= 2:
            warm_ms.append(e[0].elapsed_time(e[1]))

    # one DCP rank's share: mla_shard_decode_partial over shard 0 alone (its
    # partial kernel and the per-shard merge of its items), back-to-back calls
    # between two events so that the host's time per call stays hidden
    rank_ms = []
    if not args.no_one_shard:
        sh_o = torch.empty((1, w.B, w.R, w.H, 512), dtype=torch.float32, device=dev)
        sh_l = torch.empty((1, w.B, w.R, w.H), dtype=torch.float32, device=dev)

        def one_shard(i):
            mla.mla_shard_decode_partial(q, kvs[i % copies], bt, sl, S, I, w.scale, w.causal, shard_begin=0,
                                         shard_count=1, out_partial=sh_o, lse=sh_l, workspace=ws)

        for i in range(2):
            one_shard(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(args.event_steps):
            one_shard(i)
        e1.record()
        torch.cuda.synchronize()
        rank_ms.append(e0.elapsed_time(e1) / args.event_steps)

    # the two-way prefix/suffix merge, in place, on a chunked-context shape
    merge = None if args.no_merge else merge_leg(mla, dev, args.event_steps + 2)
    # the chunked-context KV gather (the prefill side of the same shards)
    gather = None if args.no_gather else gather_leg(mla, dev, args.event_steps)
    # the same decode over an fp8 cache
    fp8 = None if args.no_fp8 else variant_leg(mla, dev, args.event_steps, args.min_kv_set_mb, w.name, fp8=True)
    single = None if args.no_single_p else variant_leg(mla, dev, args.event_steps, args.min_kv_set_mb, w.name,
                                                       single_p=True)

    # K steps in one graph, replayed between synchronisations
    K = args.steps
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(0)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(K):
            step(i)
    # Untimed replays first: the first replays of a freshly captured graph run
    # slower (measured: 82-85 µs per step against 74-75 once settled, for both
    # graph and eager launches), so the timed replay is the fourth.
    for _ in range(GRAPH_WARM_REPLAYS):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / K

    tokens = int(w.seq_lens.astype(np.int64).sum())
    value = tokens / (ms_per_step / 1e3)
    alg = algorithmic_bytes(w)
    part_avg = statistics.mean(part_ms)
    kb = kernel_bytes(w)
    achieved = kb / (part_avg / 1e3) / 1e9
    step_gbps = alg / (ms_per_step / 1e3) / 1e9
    flops = 2176.0 * w.B * w.R * w.H * (w.seq_lens.astype(np.int64).sum() / w.B)
    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "graph_warm_replays": GRAPH_WARM_REPLAYS,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, **{k: v for k, v in w.describe().items() if k != "workload"},
                   "parallelism": "S virtual KV shards on one GPU"},
        "hbm_gbps": step_gbps,
        "hbm_frac_of_peak": step_gbps / HBM_PEAK_GBPS,
        "partial_kernel_ms": part_avg,
        "partial_kernel_ms_p10_p50_p90": [pct(part_ms, 0.1), pct(part_ms, 0.5), pct(part_ms, 0.9)],
        "combine_kernel_ms": statistics.mean(comb_ms),
        "combine_kernel_ms_p10_p50_p90": [pct(comb_ms, 0.1), pct(comb_ms, 0.5), pct(comb_ms, 0.9)],
        "partial_kernel_ms_warm": statistics.median(warm_ms) if warm_ms else None,
        "one_shard_partial_ms": rank_ms[0] if rank_ms else None,
        "mfma_tflops_partial": flops / (part_avg / 1e3) / 1e12,
        "mfma_frac_of_bf16_peak": flops / (part_avg / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
        "kv_copies_cycled": copies,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBPS, "traffic": load_traffic(w.name),
                     "kernel": PARTIAL_KERNEL, "bytes_per_launch": kb},
    }
    if merge is not None:
        rec["merge_states"] = merge
    if gather is not None:
        rec["context_gather"] = gather
    if fp8 is not None:
        rec["fp8_kv"] = fp8
    if single is not None:
        rec["single_p"] = single
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
