"""Benchmark: one paged-attention decode step (KV append + decode) on one MI355X.

A step is one pass of the hot path over one batch: pa_reshape_and_cache of
the new tokens, then pa_decode over every sequence (and, for the mixed
workload, pa_prefill_chunk over the prefill chunks).  Inputs are the seeded
synthetic workloads of paged_kv_cache_275_amd.workloads, resident in HBM before
timing starts.  To time HBM rather than the 256 MB Infinity Cache, the step
rotates over R independent copies of the KV pool, so each step's K/V was last
touched R-1 steps (GBs of traffic) earlier.

Prints ONE JSON line.  value = effective KV bandwidth of the step (decode KV
bytes / step time, GB/s); us_per_step is reported next to it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16


def _to_dev(a, dev):
    import numpy as np
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def cpu_baseline(wl, budget_s: float):
    """Time the fp64 oracle (as it stands) on the host over a bounded sample.

    The sample is the KV append of all new tokens plus decode of the first
    sequences whose oracle time fits the budget; value is their KV bytes per
    second of wall time, threads = one sequence each.
    """
    import concurrent.futures as cf

    import numpy as np

    import oracle
    threads = max(1, min(16, os.cpu_count() or 1))
    t0 = time.perf_counter()
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    oracle.reshape_and_cache(wl.k_new, wl.v_new, kc, vc, wl.slot_mapping)
    out = np.zeros(wl.q.shape, dtype=np.float64)
    q = np.ascontiguousarray(wl.q)
    bt = np.ascontiguousarray(wl.block_tables)
    cl = np.ascontiguousarray(wl.context_lens)

    def work(s):
        if time.perf_counter() - t0 > budget_s:
            return None
        oracle.decode_rows_into(out, q, kc, vc, bt, cl, wl.scale, s, s + 1)
        return s

    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        done = [s for s in ex.map(work, range(wl.num_seqs)) if s is not None]
    el = time.perf_counter() - t0
    seqs = sorted(done)
    kv_bytes = int(wl.context_lens[seqs].astype(np.int64).sum()) * wl.num_kv_heads * \
        wl.head_dim * 2 * wl.elem_bytes
    return {
        "value": round(kv_bytes / el / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
        "sample": f"KV append of {len(wl.slot_mapping)} tokens + fp64 decode of {len(seqs)}/"
                  f"{wl.num_seqs} sequences ({kv_bytes / 1e6:.1f} MB of KV) in {el:.2f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="llama3_8b")
    ap.add_argument("--rotate", type=int, default=4, help="independent KV pool copies")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the paged-attention path here has no "
              "multi-GPU mode (see the sharding note in DESIGN.md); use --gpus 1.", file=sys.stderr)
        sys.exit(2)

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

    def step(i, ev=None):
        kc, vc = pools[i % len(pools)]
        if ev is not None:
            ev[0].record(stream)
        ops.reshape_and_cache(k_new, v_new, kc, vc, slots)
        if ev is not None:
            ev[1].record(stream)
        if pre is not None:
            ops.prefill_chunk(pre["out"], pre["q"], kc, vc, pre["bt"], pre["qsl"], pre["cl"], wl.scale)
        if ev is not None:
            ev[2].record(stream)
        ops.decode(out, q, kc, vc, bt, cl, wl.scale, workspace=ws)
        if ev is not None:
            ev[3].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    append_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    prefill_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
    decode_ms = np.array([e[2].elapsed_time(e[3]) for e in events])
    step_ms = wall * 1e3 / args.steps
    dec_avg = float(decode_ms.mean())
    achieved = kv_bytes / (dec_avg * 1e-3) / 1e9
    value = kv_bytes / (step_ms * 1e-3) / 1e9

    res = {
        "metric": "paged-attn decode us/step + effective KV GB/s (% HBM peak), Llama-3-8B shape",
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
        },
        "timing_us": {
            "append_avg": round(float(append_ms.mean()) * 1e3, 2),
            "prefill_avg": round(float(prefill_ms.mean()) * 1e3, 2) if pre is not None else None,
            "decode_avg": round(dec_avg * 1e3, 2),
            "decode_p10": round(float(np.percentile(decode_ms, 10)) * 1e3, 2),
            "decode_p50": round(float(np.percentile(decode_ms, 50)) * 1e3, 2),
            "decode_p90": round(float(np.percentile(decode_ms, 90)) * 1e3, 2),
        },
        "roofline": {
            "kernel": "pa_decode",
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
        },
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
