"""Benchmark: one paged-attention step (KV append + decode) on one MI355X.

A step is one pass of the hot path over one batch: the KV append of the new
tokens and decode attention over every sequence -- by default in one launch,
pa_decode_append (append fused into the decode kernel); with --unfused as
pa_reshape_and_cache then pa_decode.  For the mixed workload the prefill
chunks' tokens go through pa_reshape_and_cache and pa_prefill_chunk first.  Inputs are the
seeded synthetic workloads of paged_kv_cache_275_amd.workloads, resident in
HBM before timing starts.  To time HBM rather than the 256 MB Infinity Cache,
the step rotates over R independent copies of the KV pool, so each step's K/V
was last touched R-1 steps (GBs of traffic) earlier.

Prints ONE JSON line.  value = effective KV bandwidth of the whole step
(decode KV bytes / step wall time, GB/s); us_per_step sits next to it.
roofline = the kernel with the largest average duration, timed with HIP
events on the stream it runs on; its traffic comes from a committed
rocprofv3 counter summary (profiles/) when that summary was taken on the
kernel's current source, else null.

Other modes (for the profiling summaries under profiles/):
  --copy-calibration   a plain 512 MiB device copy, to scale HBM counters
  --summarize-pmc ...  turn rocprofv3 counter CSVs into a traffic summary
  --summarize-stats ...  turn a rocprofv3 --stats CSV and the profiled bench
                       log into a kernel-time summary
  --summarize-counters ...  per-dispatch medians and ratios of SQ/GRBM counters
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged-attn decode \u00b5s/step + effective KV GB/s (% HBM peak), Llama-3-8B shape"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA
CALIB_BYTES = 512 << 20      # size of the plain copy used to scale HBM counters

# Sources the streaming decode kernel is compiled from: a traffic summary is
# valid only for the exact bytes it was measured on.
KERNEL_SOURCES = {
    "decode_stream_kernel": ["pa_decode.hip", "pa_device.h", "pa_launch.h"],
    "decode_stream_kernel_fp8": ["pa_decode.hip", "pa_device.h", "pa_launch.h"],
    "prefill_kernel": ["pa_prefill.hip", "pa_device.h", "pa_launch.h"],
}


def kernel_matches(kernel: str, name: str) -> bool:
    """Whether a profiler's (demangled) kernel name is an instance of `kernel`:
    decode_stream_kernel's last template argument tells the fp8-cache
    instances (true) from the others (false)."""
    if kernel == "decode_stream_kernel":
        return "decode_stream_kernel<" in name and name.split("(")[0].rstrip().endswith("false>")
    if kernel == "decode_stream_kernel_fp8":
        return "decode_stream_kernel<" in name and name.split("(")[0].rstrip().endswith("true>")
    return kernel in name
CSRC = os.path.join(ROOT, "paged_kv_cache_275_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_summary_path(kernel: str, workload: str) -> str:
    return os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")


def read_traffic(kernel: str, workload: str):
    """HBM bytes per dispatch from the committed counter summary, or None when
    there is none or it was taken on other kernel sources."""
    path = traffic_summary_path(kernel, workload)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != source_hash(kernel):
        return None
    return float(kv["hbm_bytes_per_dispatch"])


def _to_dev(a, dev):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(wl, budget_s: float):
    """Time the fp64 oracle (as it stands) on the host over a bounded sample.

    The sample is the KV append of all new tokens plus decode of the first k
    sequences, k chosen so that one thread takes about half the budget.  The
    same sample then runs on all host threads (one sequence per task; the
    oracle releases the GIL), capped at 16, the CPU share of one GPU.  value
    is the all-thread KV bytes per second of wall time; the single-thread
    rate, the thread counts and the CPU model sit beside it.
    """
    import concurrent.futures as cf

    import numpy as np

    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    q = np.ascontiguousarray(wl.q)
    bt = np.ascontiguousarray(wl.block_tables)
    cl = np.ascontiguousarray(wl.context_lens)
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    t0 = time.perf_counter()
    oracle.reshape_and_cache(wl.k_new, wl.v_new, kc, vc, wl.slot_mapping)
    t_append = time.perf_counter() - t0
    out = np.zeros(wl.q.shape, dtype=np.float64)

    # single thread: sequences in order until half the budget is spent
    t0 = time.perf_counter()
    k = 0
    while k < wl.num_seqs and time.perf_counter() - t0 < budget_s / 2:
        oracle.decode_rows_into(out, q, kc, vc, bt, cl, wl.scale, k, k + 1)
        k += 1
    t_one = time.perf_counter() - t0 + t_append
    # all threads, the same k sequences
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda s: oracle.decode_rows_into(out, q, kc, vc, bt, cl, wl.scale, s, s + 1), range(k)))
    t_all = time.perf_counter() - t0 + t_append
    kv_bytes = int(cl[:k].astype(np.int64).sum()) * wl.num_kv_heads * wl.head_dim * 2 * wl.elem_bytes
    return {
        "value": round(kv_bytes / t_all / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "single_thread_value": round(kv_bytes / t_one / 1e9, 4),
        "single_thread_s": round(t_one, 3), "all_threads_s": round(t_all, 3),
        "os_cpu_count": os.cpu_count(), "cpu_model": _cpu_model(),
        "sample": f"KV append of {len(wl.slot_mapping)} tokens + fp64 decode of the first {k}/{wl.num_seqs} "
                  f"sequences ({kv_bytes / 1e6:.1f} MB of KV), timed on 1 thread ({t_one:.2f} s) and on "
                  f"{threads} threads ({t_all:.2f} s)",
    }


def extras(wl, kc, vc, stream):
    """Measurements of the block-management row, after (outside) the timed region:
    the host manager's per-step work for this batch (one append per sequence,
    then the batch's tables), and pa_copy_blocks bandwidth on 1024 blocks."""
    import numpy as np
    import torch

    from paged_kv_cache_275_amd.blocks import BlockManager, copy_blocks
    out = {}
    nb, s = wl.num_blocks, wl.num_seqs
    mb = wl.max_blocks_per_seq
    m = BlockManager(nb)
    ids = list(range(s))
    for i, n in enumerate(wl.context_lens.tolist()):
        m.add_sequence(i, max(0, n - 64))          # leave room to append 64 tokens each
    steps = 64
    t0 = time.perf_counter()
    for _ in range(steps):
        m.append_batch(ids)
        m.batch_tables(ids, mb)
    host_us = (time.perf_counter() - t0) / steps * 1e6
    m.close()
    out["block_manager_step_us"] = round(host_us, 2)
    out["block_manager_step_note"] = (f"pa_bm_append_batch + pa_bm_batch_tables for {s} sequences "
                                      "(host C++, through ctypes), mean of 64 steps")
    npairs = min(1024, nb // 2)
    perm = np.random.default_rng(0).permutation(nb)
    pairs = torch.from_numpy(np.stack([perm[:npairs], perm[npairs:2 * npairs]], 1).astype(np.int32)).to(kc.device)
    for _ in range(3):
        copy_blocks(kc, vc, pairs)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    reps = 20
    for _ in range(reps):
        copy_blocks(kc, vc, pairs)
    ev[1].record(stream)
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
    block_bytes = kc[0].numel() * kc.element_size()
    moved = 2 * 2 * npairs * block_bytes                      # K and V, read + write
    out["copy_blocks_us"] = round(us, 2)
    out["copy_blocks_gbs"] = round(moved / (us * 1e-6) / 1e9, 1)
    out["copy_blocks_note"] = f"{npairs} block pairs of K and V ({block_bytes} B each), read + write bytes"
    return out


def graph_step(wl, pools, pre, out, q, kn, vn, bt, cl, ws, stream):
    """The decode step replayed as HIP graphs (pa_decode_append_graph, one per
    pool copy), outside the timed region: launch gaps shrink, kernels are the
    same.  Decode-only workloads."""
    import torch

    from paged_kv_cache_275_amd import ops
    if pre is not None:
        return {}
    graphs = [ops.DecodeStepGraph(out, q, kn, vn, kc, vc, bt, cl, wl.scale, workspace=ws) for kc, vc in pools]
    for i in range(8):
        graphs[i % len(graphs)].launch(stream)
    torch.cuda.synchronize()
    reps = 200
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    # replays already queued when the clock starts, so that the host's cost of
    # the first launch is not inside the timed region
    for i in range(4):
        graphs[i % len(graphs)].launch(stream)
    ev[0].record(stream)
    t0 = time.perf_counter()
    for i in range(reps):
        graphs[i % len(graphs)].launch(stream)
    host_us = (time.perf_counter() - t0) * 1e6 / reps
    ev[1].record(stream)
    torch.cuda.synchronize()
    us = ev[0].elapsed_time(ev[1]) * 1e3 / reps
    for g in graphs:
        g.close()
    return {"graph_step_us": round(us, 2),
            "graph_step_kv_gbs": round(wl.decode_kv_bytes() / (us * 1e-6) / 1e9, 1),
            "graph_host_launch_us": round(host_us, 2),
            "graph_step_note": f"pa_decode_append_graph replays over {len(pools)} pool copies, mean of {reps}; "
                               "graph_host_launch_us is the host's time per pa_graph_launch call"}


def fp8_prefill(wl, pools, pre, stream):
    """The chunked prefill over an fp8 copy of the first pool
    (pa_prefill_chunk_fp8), outside the timed region; mixed workloads only."""
    import numpy as np
    import torch

    from paged_kv_cache_275_amd import ops
    if pre is None:
        return {}
    ks, vs = 0.02, 0.015
    kc, vc = pools[0]
    nb, bs, hkv, d = kc.shape
    slots = torch.arange(nb * bs, dtype=torch.int32, device=kc.device)
    k8 = torch.empty(kc.shape, dtype=torch.uint8, device=kc.device)
    v8 = torch.empty_like(k8)
    ops.reshape_and_cache_fp8(kc.view(-1, hkv, d), vc.view(-1, hkv, d), k8, v8, slots, ks, vs)
    out8 = torch.empty_like(pre["out"])

    def call():
        ops.prefill_chunk_fp8(out8, pre["q"], k8, v8, pre["bt"], pre["qsl"], pre["cl"], wl.scale, ks, vs)
    for _ in range(3):
        call()
    reps = 20
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for e0, e1 in evs:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3
    flops = prefill_flops(wl)
    return {"fp8_prefill_us": round(us, 2),
            "fp8_prefill_tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "fp8_prefill_note": f"pa_prefill_chunk_fp8 on the workload's chunks over an fp8 pool copy, mean of {reps}"}


def fp8_decode(wl, pools, q, kn, vn, bt, cl, ws, stream):
    """Decode over fp8 E4M3 copies of the pools (pa_decode_fp8), outside the
    timed region.  The copies are quantized on the GPU by
    pa_reshape_and_cache_fp8 over every slot of each pool; decode reads one
    byte per K/V element, so its KV bytes are half the bf16 step's.  Also the
    whole fp8 decode step, pa_decode_append_fp8 (quantized append of the new
    rows, then decode), back to back over the same copies."""
    import numpy as np
    import torch

    from paged_kv_cache_275_amd import ops
    if wl.dtype != "bf16":
        return {}
    ks, vs = 0.02, 0.015
    nb, bs, hkv, d = pools[0][0].shape
    slots = torch.arange(nb * bs, dtype=torch.int32, device=q.device)
    calls = []
    out8 = torch.empty_like(q)
    for kc, vc in pools:
        k8 = torch.empty(kc.shape, dtype=torch.uint8, device=q.device)
        v8 = torch.empty(vc.shape, dtype=torch.uint8, device=q.device)
        ops.reshape_and_cache_fp8(kc.view(-1, hkv, d), vc.view(-1, hkv, d), k8, v8, slots, ks, vs)
        calls.append((ops.bind_decode_fp8(out8, q, k8, v8, bt, cl, wl.scale, ks, vs, workspace=ws), k8, v8,
                      ops.bind_decode_append_fp8(out8, q, kn, vn, k8, v8, bt, cl, wl.scale, ks, vs, workspace=ws)))
    for i in range(200):
        calls[i % len(calls)][0]()
    # as in the main loop, the kernel is bracketed by dispatch events on every
    # eighth call only (a bracketed call runs slower)
    reps, every = 320, 8
    evs = []
    for _ in range(reps // every):
        pair = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        for e in pair:
            e.record(stream)
        evs.append(pair)
    call_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    call_ev[0].record(stream)
    for i in range(reps):
        ev = evs[i // every] if i % every == 0 else None
        calls[i % len(calls)][0](None if ev is None else (ev[0].cuda_event, ev[1].cuda_event))
    call_ev[1].record(stream)
    torch.cuda.synchronize()
    k_us = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3
    call_us = call_ev[0].elapsed_time(call_ev[1]) * 1e3 / reps
    for i in range(40):
        calls[i % len(calls)][3]()
    torch.cuda.synchronize()
    call_ev[0].record(stream)
    for i in range(reps):
        calls[i % len(calls)][3]()
    call_ev[1].record(stream)
    torch.cuda.synchronize()
    step_us = call_ev[0].elapsed_time(call_ev[1]) * 1e3 / reps
    fp8_bytes = wl.decode_kv_bytes() // wl.elem_bytes      # one byte per element
    gbs = fp8_bytes / (k_us * 1e-6) / 1e9
    return {"fp8_decode_stream_kernel_us": round(k_us, 2),
            "fp8_decode_call_us": round(call_us, 2),
            "fp8_decode_kv_bytes": fp8_bytes,
            "fp8_decode_kernel_gbs": round(gbs, 1),
            "fp8_decode_kernel_frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "fp8_step_us": round(step_us, 2),
            "fp8_step_kv_gbs": round(fp8_bytes / (step_us * 1e-6) / 1e9, 1),
            "fp8_decode_note": f"pa_decode_fp8 over {len(calls)} fp8 pool copies, {reps} back-to-back calls; "
                               "kernel time from HIP events set at its dispatch, on every eighth call; "
                               "fp8_step_us: pa_decode_append_fp8 "
                               "(quantized append + decode), mean of the same number of back-to-back calls"}


def prefill_flops(wl) -> int:
    """Algorithmic flops of the prefill chunks: 4*D per (query head, causal pair)."""
    p = wl.prefill
    pairs = 0
    for s in range(len(p.context_lens)):
        c = int(p.query_start_loc[s + 1] - p.query_start_loc[s])
        n = int(p.context_lens[s])
        pairs += sum(n - c + i + 1 for i in range(c))
    return 4 * wl.head_dim * wl.num_q_heads * pairs


def stream_reference(stream, nbytes=4 << 30, reps=10):
    """Reference streaming rates measured on the same GPU in the same run, over
    nbytes (16 times the MALL; long enough that the kernel's start and end
    cost little), outside the timed region:
    a plain read (pa_stream_read_probe: every 16-byte vector loaded once, as
    the decode kernel loads K and V, without the gather) and a device-to-device
    copy (read + write bytes).  Returns (read GB/s, copy GB/s)."""
    import numpy as np
    import torch

    from paged_kv_cache_275_amd import ops
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    xor_out = torch.zeros(1, dtype=torch.int32, device=dev)

    def timed(fn):
        for _ in range(2):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return float(np.median([e0.elapsed_time(e1) for e0, e1 in evs])) * 1e3
    read_us = timed(lambda: ops.stream_read_probe(src, xor_out, stream))
    copy_us = timed(lambda: dst.copy_(src))
    del src, dst
    return nbytes / (read_us * 1e-6) / 1e9, 2 * nbytes / (copy_us * 1e-6) / 1e9


def copy_calibration():
    """A plain device-to-device copy of CALIB_BYTES, three times, for counter scaling."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(CALIB_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": CALIB_BYTES, "copies": 3}), flush=True)


def _pmc_rows(path, counter, kernel):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and kernel_matches(kernel, r["Kernel_Name"]):
                rows.append(float(r["Counter_Value"]))
    return rows


def summarize_pmc(args):
    """Write profiles/<kernel>_<workload>_traffic.txt from four rocprofv3 --pmc CSVs."""
    import statistics
    fetch = _pmc_rows(args.pmc_fetch, "FETCH_SIZE", args.kernel)
    write = _pmc_rows(args.pmc_write, "WRITE_SIZE", args.kernel)
    cfetch = max(_pmc_rows(args.calib_fetch, "FETCH_SIZE", "copyBuffer"))
    cwrite = max(_pmc_rows(args.calib_write, "WRITE_SIZE", "copyBuffer"))
    if not fetch or not write:
        raise SystemExit(f"no {args.kernel} dispatches in the counter files")
    ff = CALIB_BYTES / (cfetch * 1024.0)
    wf = CALIB_BYTES / (cwrite * 1024.0)
    f_kib, w_kib = statistics.median(fetch), statistics.median(write)
    total = f_kib * 1024.0 * ff + w_kib * 1024.0 * wf
    lines = [
        f"# HBM traffic of {args.kernel} on the {args.workload} workload (rocprofv3 --pmc)",
        "# Counters are KiB per dispatch, median over the dispatches of the run.  Each is",
        f"# scaled by (bytes / counter) of a plain {CALIB_BYTES >> 20} MiB device copy, which reads",
        "# and writes exactly that many bytes.",
        "# Commands, from the repository root:",
        *[f"#   {c}" for c in args.commands.split(";;")],
        f"kernel = {args.kernel}",
        f"workload = {args.workload}",
        f"kernel_source_sha256 = {source_hash(args.kernel)}",
        f"dispatches_fetch = {len(fetch)}",
        f"dispatches_write = {len(write)}",
        f"fetch_size_kib_per_dispatch = {f_kib:.1f}",
        f"write_size_kib_per_dispatch = {w_kib:.1f}",
        f"copy_fetch_size_kib = {cfetch:.1f}",
        f"copy_write_size_kib = {cwrite:.1f}",
        f"copy_fetch_factor = {ff:.4f}",
        f"copy_write_factor = {wf:.4f}",
        f"hbm_bytes_per_dispatch = {total:.0f}",
    ]
    if args.algorithmic_bytes:
        lines.append(f"algorithmic_bytes_per_dispatch = {args.algorithmic_bytes}")
        lines.append(f"traffic_over_algorithmic = {total / float(args.algorithmic_bytes):.4f}")
    with open(args.out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_stats(args):
    """Write profiles/<kernel>_<workload>_kernel_stats.md from a rocprofv3
    --kernel-trace --stats CSV and the log of the bench run it profiled."""
    with open(args.stats_csv) as f:
        rows = list(csv.DictReader(f))
    with open(args.bench_log) as f:
        bench = [line.strip() for line in f if line.startswith("{")][-1]
    b = json.loads(bench)
    rf = b["roofline"]
    lines = [f"# {args.kernel} on {args.workload}: rocprofv3 kernel trace", "",
             "Commands, from the repository root (on one MI355X):", "", "```",
             *args.commands.split(";;"), "```", "",
             "Per-kernel summary (rocprofv3 --stats, durations in ns; the calls include the warm-up, "
             "breakdown and extra passes of bench.py):", "",
             "| kernel | calls | average ns | min ns | max ns | share |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("void ", "").split("(")[0]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']):.0f} | {r['MinNs']} | {r['MaxNs']} | "
                     f"{float(r['Percentage']):.1f}% |")
    # the instance the bench line timed: the bf16-cache (non-fp8) one
    inst = [r for r in rows if kernel_matches(rf["kernel"], r["Name"]) and "true>" not in r["Name"]]
    lines.append("")
    if inst:
        avg = float(inst[0]["AverageNs"]) / 1e3
        lines.append(f"The bench line timed `{rf['kernel']}` with HIP events at {rf['avg_us']} us per launch on "
                     f"average; rocprofv3 gives {avg:.2f} us for `{inst[0]['Name'].replace('void ', '').split('(')[0]}`.")
        if args.plain_bench_log:
            with open(args.plain_bench_log) as f:
                plain = json.loads([line.strip() for line in f if line.startswith("{")][-1])
            pr = plain["roofline"]
            lines.append(f"The same bench command without the profiler (`{args.plain_bench_log}`) timed it at "
                         f"{pr['avg_us']} us; the rocprofv3 average is {avg / pr['avg_us']:.3f} of that.  Kernel "
                         "tracing lengthens the event-bracketed launches of the profiled run.")
    lines += [f"roofline of that line: achieved {rf['achieved']} {rf['unit']} of {rf['peak']} "
              f"({rf['frac'] * 100:.1f}%).", "", "Bench line of the profiled run:", "", "```", bench, "```", ""]
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


# Ratios derived from SQ / GRBM counters: (name, numerator, denominator, scale, meaning)
COUNTER_RATIOS = [
    ("mfma_busy", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES", 0.25,
     "matrix-core busy cycles per SIMD over CU-busy cycles (4 SIMDs per CU)"),
    ("lds_bank_conflict", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", 1.0,
     "LDS cycles stalled by bank conflicts over LDS active cycles"),
    ("lds_wait_per_lds_inst", "SQ_WAIT_INST_LDS", "SQ_INSTS_LDS", 1.0,
     "wave cycles waiting to issue an LDS instruction, per LDS instruction"),
    ("mfma_flops_per_mops", None, None, 512.0, "one MFMA MOP is 512 flops (bf16)"),
]


def summarize_counters(args):
    """Write profiles/<kernel>_<workload>_counters.md: per-dispatch medians of
    rocprofv3 --pmc counters for one kernel (several CSVs, one per pass)."""
    import statistics
    med = {}
    n_disp = {}
    for path in args.counter_csvs.split(","):
        vals = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if kernel_matches(args.kernel, r["Kernel_Name"]) and "true>" not in r["Kernel_Name"]:
                    vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        for k, v in vals.items():
            med[k] = statistics.median(v)
            n_disp[k] = len(v)
    if not med:
        raise SystemExit(f"no {args.kernel} dispatches in the counter files")
    lines = [f"# {args.kernel} on {args.workload}: hardware counters (rocprofv3 --pmc)", "",
             "Commands, from the repository root (on one MI355X; one counter pass per command):", "", "```",
             *args.commands.split(";;"), "```", "",
             "Median per dispatch of the bf16-cache instance (counters summed over the device):", "",
             "| counter | dispatches | median |", "|---|---|---|"]
    for k in sorted(med):
        lines.append(f"| {k} | {n_disp[k]} | {med[k]:.0f} |")
    lines += ["", "| ratio | value | definition |", "|---|---|---|"]
    for name, num, den, scale, meaning in COUNTER_RATIOS:
        if num and num in med and den in med and med[den] > 0:
            lines.append(f"| {name} | {med[num] / med[den] * scale:.3f} | {num} / {den}"
                         f"{'' if scale == 1.0 else f' x {scale:g}'}: {meaning} |")
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in med:
        fl = med["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
        extra = f"; algorithmic {args.algorithmic_flops:.4g}, ratio {fl / args.algorithmic_flops:.3f}" \
            if args.algorithmic_flops else ""
        lines.append(f"| mfma_flops | {fl:.4g} | SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512{extra} |")
    lines.append("")
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # 3000 untimed steps (about 0.3 s of decode): the GPU's clocks settle
    # within that; after 10 warm-up steps the timed decode step measured
    # 1.5 us slower (87.3 against 85.9 us on llama3_8b)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=3000)
    ap.add_argument("--config", default="llama3_8b")
    ap.add_argument("--rotate", type=int, default=4, help="independent KV pool copies")
    ap.add_argument("--event-every", type=int, default=8,
                    help="bracket the dominant kernel with timing events on every N-th timed step")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unfused", action="store_true",
                    help="append decode tokens with pa_reshape_and_cache, then pa_decode (default: pa_decode_append)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-pmc", action="store_true")
    ap.add_argument("--pmc-fetch")
    ap.add_argument("--pmc-write")
    ap.add_argument("--calib-fetch")
    ap.add_argument("--calib-write")
    ap.add_argument("--kernel", default="decode_stream_kernel")
    ap.add_argument("--workload", default="llama3_8b")
    ap.add_argument("--algorithmic-bytes", type=int, default=0)
    ap.add_argument("--commands", default="")
    ap.add_argument("--plain-bench-log", default="",
                    help="--summarize-stats: log of the same bench command run without the profiler")
    ap.add_argument("--out")
    ap.add_argument("--summarize-stats", action="store_true")
    ap.add_argument("--stats-csv")
    ap.add_argument("--bench-log")
    ap.add_argument("--summarize-counters", action="store_true")
    ap.add_argument("--counter-csvs", default="")
    ap.add_argument("--algorithmic-flops", type=float, default=0.0)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this paged-attention path has no multi-GPU "
              "mode (how it would shard is described in DESIGN.md); use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.summarize_pmc:
        summarize_pmc(args)
        return
    if args.summarize_stats:
        summarize_stats(args)
        return
    if args.summarize_counters:
        summarize_counters(args)
        return
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch

    from paged_kv_cache_275_amd import ops
    from paged_kv_cache_275_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ops.load_library()
    seed = W.CONFIG_NAMES.index(args.config)
    wl = W.make_workload(args.config, seed=seed)
    kv_bytes = wl.decode_kv_bytes()

    q = _to_dev(wl.q, dev)
    out = torch.empty_like(q)
    k_new, v_new = _to_dev(wl.k_new, dev), _to_dev(wl.v_new, dev)
    slots = _to_dev(wl.slot_mapping, dev)
    bt = _to_dev(wl.block_tables, dev)
    cl = _to_dev(wl.context_lens, dev)
    ws = ops.decode_workspace(q, _to_dev(wl.k_cache[:1], dev), bt)
    kc0, vc0 = _to_dev(wl.k_cache, dev), _to_dev(wl.v_cache, dev)
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(args.rotate - 1)]
    pre = None
    if wl.prefill is not None:
        p = wl.prefill
        pre = dict(q=_to_dev(p.q, dev), bt=_to_dev(p.block_tables, dev),
                   cl=_to_dev(p.context_lens, dev), qsl=_to_dev(p.query_start_loc, dev))
        pre["out"] = torch.empty_like(pre["q"])
    stream = torch.cuda.current_stream(dev)

    # arguments are checked once per pool copy; the loop only crosses the C ABI.
    # Default step: prefill tokens (if any) through pa_reshape_and_cache, then
    # pa_decode_append, which appends each sequence's new token and attends in
    # one kernel.  --unfused: every token through pa_reshape_and_cache, then
    # pa_decode.
    t_new, s_dec = k_new.shape[0], wl.num_seqs
    n_sep = t_new if args.unfused else t_new - s_dec   # tokens appended by pa_reshape_and_cache
    calls = []
    for kc, vc in pools:
        calls.append({
            "append": None if n_sep == 0 else ops.bind_reshape_and_cache(
                k_new[:n_sep], v_new[:n_sep], kc, vc, slots[:n_sep]),
            "prefill": None if pre is None else ops.bind_prefill_chunk(
                pre["out"], pre["q"], kc, vc, pre["bt"], pre["qsl"], pre["cl"], wl.scale),
            "decode": ops.bind_decode(out, q, kc, vc, bt, cl, wl.scale, workspace=ws) if args.unfused else
            ops.bind_decode_append(out, q, k_new[t_new - s_dec:], v_new[t_new - s_dec:], kc, vc, bt, cl,
                                   wl.scale, workspace=ws),
        })

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)   # creates the HIP event, so its handle can go to the library
        return evs

    # ev: call boundaries (append | prefill | decode) or None; kev: the decode
    # streaming kernel's start / stop, set by the library from its dispatch
    def step(i, ev=None, kev=None):
        c = calls[i % len(calls)]
        if ev is not None and ev[0] is not None:
            ev[0].record(stream)
        if c["append"] is not None:
            c["append"]()
        if ev is not None and ev[1] is not None:
            ev[1].record(stream)
        if c["prefill"] is not None:
            c["prefill"]()
        if ev is not None and ev[2] is not None:
            ev[2].record(stream)
        c["decode"](None if kev is None else (kev[0].cuda_event, kev[1].cuda_event))
        if ev is not None and ev[3] is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)

    # breakdown pass (not the timed region): every call bracketed, and the
    # dominant kernel picked from it
    n_prof = max(5, min(args.steps, 20))
    prof = [(new_events(4), new_events(2)) for _ in range(n_prof)]
    torch.cuda.synchronize()
    for i, (ev, kev) in enumerate(prof):
        step(args.warmup + i, ev, kev)
    torch.cuda.synchronize()

    def span(evs, a, b):
        return np.array([e[a].elapsed_time(e[b]) for e in evs]) * 1e3   # us

    pev, pkev = [p[0] for p in prof], [p[1] for p in prof]
    append_us, prefill_us, decode_us = span(pev, 0, 1), span(pev, 1, 2), span(pev, 2, 3)
    stream_us = span(pkev, 0, 1)
    kernels = {"decode_stream_kernel": float(stream_us.mean())}
    if n_sep > 0:
        kernels["reshape_and_cache_kernel"] = float(append_us.mean())
    if pre is not None:
        kernels["prefill_kernel"] = float(prefill_us.mean())
    dom = max(kernels, key=kernels.get)

    # timed region: exactly K steps.  The dominant kernel is bracketed by
    # events on every event_every-th step only: timing events cost the GPU a
    # few microseconds per bracketed launch (measured 3-4 us per decode call),
    # which would otherwise be counted in every step.
    every = max(1, args.event_every)
    tev = [new_events(2) for _ in range((args.steps + every - 1) // every)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        e = tev[i // every] if i % every == 0 else None
        if e is None:
            step(i)
        elif dom == "decode_stream_kernel":
            step(i, None, e)
        elif dom == "prefill_kernel":
            step(i, (None, e[0], e[1], None))
        else:
            step(i, (e[0], e[1], None, None))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_us = span(tev, 0, 1)
    step_ms = wall * 1e3 / args.steps
    value = kv_bytes / (step_ms * 1e-3) / 1e9

    if dom == "prefill_kernel":
        work = prefill_flops(wl)
        achieved = work / (float(dom_us.mean()) * 1e-6) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": MFMA_BF16_PEAK_TFS, "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4),
                "traffic": None if read_traffic(dom, args.config) is None else round(read_traffic(dom, args.config)),
                "work_per_launch": work, "avg_us": round(float(dom_us.mean()), 2)}
    else:
        # decode bytes: K and V of every context token read once
        achieved = kv_bytes / (float(dom_us.mean()) * 1e-6) / 1e9
        tr = read_traffic(dom, args.config) if dom in KERNEL_SOURCES else None
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if tr is None else round(tr), "work_per_launch": kv_bytes,
                "avg_us": round(float(dom_us.mean()), 2)}

    def pct(a):
        return {"avg": round(float(a.mean()), 2), "p10": round(float(np.percentile(a, 10)), 2),
                "p50": round(float(np.percentile(a, 50)), 2), "p90": round(float(np.percentile(a, 90)), 2)}

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 5),
        "us_per_step": round(step_ms * 1e3, 2),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic",
        "config": {
            "workload": args.config, "num_seqs": wl.num_seqs, "num_q_heads": wl.num_q_heads,
            "num_kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim, "block_size": 16,
            "context_tokens": int(wl.context_lens.sum()), "pool_blocks": wl.num_blocks,
            "seed": seed, "kv_bytes_per_step": kv_bytes, "pool_copies": len(pools),
            "prefill_rows": None if pre is None else int(wl.prefill.query_start_loc[-1]),
            "decode_append": "separate pa_reshape_and_cache + pa_decode" if args.unfused else
                             "fused (pa_decode_append)",
        },
        "timing_us": {
            "dominant_kernel_timed": pct(dom_us),
            "dominant_kernel_samples": f"{len(tev)} of {args.steps} timed steps (every {every}-th)",
            "breakdown_steps": n_prof,
            "append_call": pct(append_us) if n_sep > 0 else None,
            "prefill_call": pct(prefill_us) if pre is not None else None,
            "decode_call": pct(decode_us),
            "decode_stream_kernel": pct(stream_us),
            "decode_kv_gbs_call": round(kv_bytes / (float(decode_us.mean()) * 1e-6) / 1e9, 2),
        },
        "roofline": roof,
    }
    if pre is not None:
        pf = prefill_flops(wl)
        res["timing_us"]["prefill_tflops"] = round(pf / (float(prefill_us.mean()) * 1e-6) / 1e12, 2)
    res["extras"] = extras(wl, pools[0][0], pools[0][1], stream)
    read_gbs, copy_gbs = stream_reference(stream)
    res["extras"]["stream_read_gbs"] = round(read_gbs, 1)
    res["extras"]["stream_copy_gbs"] = round(copy_gbs, 1)
    res["extras"]["dominant_kernel_frac_of_stream_read"] = (
        round(res["roofline"]["achieved"] / read_gbs, 4) if res["roofline"]["unit"] == "GB/s" else None)
    res["extras"]["stream_reference_note"] = ("plain streaming over 4 GiB on the same GPU in the same run, median of "
                                              "10: pa_stream_read_probe (read bytes; the same 16-byte non-temporal "
                                              "loads as the decode kernel, without the gather) and a torch "
                                              "device-to-device copy (read + write bytes), for context beside the "
                                              "8 TB/s peak")
    if not args.unfused:
        res["extras"].update(graph_step(wl, pools, pre, out, q, k_new[t_new - s_dec:], v_new[t_new - s_dec:], bt, cl,
                                        ws, stream))
    res["extras"].update(fp8_decode(wl, pools, q, k_new[t_new - s_dec:], v_new[t_new - s_dec:], bt, cl, ws, stream))
    res["extras"].update(fp8_prefill(wl, pools, pre, stream))
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
