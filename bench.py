"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole hot path for one layer of the Llama-3-8B-shaped workload
(batch 64, 32 query / 8 KV heads, head dim 128, bf16, context lengths uniform
in [512, 4096], 16-token blocks from a 20,000-block pool): slot mapping of
each sequence's newest position, the cache write of the new K/V token, and
paged attention (partition kernel + log-sum-exp combine).  The library's
decode-step entry runs the first three in the attention launch itself.

Inputs are resident in HBM before timing.  To keep the 256 MB Infinity Cache
from serving a step out of the previous one, the step cycles over R
independent copies of the inputs (R * 1.3 GB of pools), so the copy a step
reads was last touched R-1 steps (>= 1.8 GB of other traffic) earlier.

Prints one JSON line.  `value` is KV GB/s of the whole step (algorithmic
bytes / wall time per step); the roofline object reports the attention call
(its kernels timed with HIP events on the stream they run on) against the
8 TB/s HBM peak.  The CPU baseline is the oracle on the host, timed on the
same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def algorithmic_bytes(wl, part_blocks_unused=None):
    """Bytes the method must move for one step (see module docstring)."""
    import numpy as np

    e_kv = {"f32": 4, "bf16": 2, "i8": 1, "fp8": 1}[wl.quant or wl.kv_dtype]
    e_q = {"f32": 4, "bf16": 2}[wl.q_dtype]
    L = wl.lens.astype(np.int64)
    nblk = (L + 15) // 16
    kv = int(L.sum()) * wl.Hkv * wl.D * 2 * e_kv
    tables = int(nblk.sum()) * 4
    scales = int(nblk.sum()) * wl.Hkv * 2 * 4 if wl.quant else 0
    q_out = wl.B * wl.Hq * wl.D * 2 * e_q
    lens = wl.B * 4
    attention = kv + tables + scales + q_out + lens
    write = (wl.B * wl.Hkv * wl.D * 2 * e_kv * 2 + wl.B * 4) if wl.write else 0
    slots = (wl.B * 4 * 2 + wl.B * 4) if wl.write else 0   # lens + one table entry in, slot out
    return dict(attention=attention, kv=kv, write=write, slots=slots,
                step=attention + write + slots)


class Replica:
    def __init__(self, wl, part, layout):
        import torch
        import paged_kv_cache_434_amd as pkv
        from paged_kv_cache_434_amd import workloads as W

        d = W.to_device(wl, layout=layout)
        self.d = d
        self.cache = pkv.PagedCache(d["k_pool"], d["v_pool"], wl.kv_dtype)
        self.slots = torch.empty(wl.B, dtype=torch.int32, device="cuda")
        self.out = torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.bfloat16, device="cuda")
        self.ws = pkv.alloc_workspace(wl.B, wl.Hq, wl.D, wl.max_blocks, part)
        self.part = part
        self.scale = float(wl.scale)


def run_step(pkv, rep, ev=None):
    """One decode step: append of the new token fused into the attention
    launch (slot of position L-1 + cache write + attention), then the
    cross-partition combine when the context is split."""
    d = rep.d
    if ev is not None:
        ev[0].record()
    pkv.decode_step(rep.cache, d["q"], d["k_new"], d["v_new"], d["tables"], d["lens"],
                    rep.scale, partition_tokens=rep.part, workspace=rep.ws, out=rep.out)
    if ev is not None:
        ev[1].record()


def cpu_baseline(wl, budget_s=10.0):
    """The oracle (as it stands) timed on the host: cache write + decode of the
    whole workload, repeated until about budget_s seconds have passed."""
    import numpy as np
    import oracle

    k, v = wl.k_pool.copy(), wl.v_pool.copy()
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        slots = oracle.slot_mapping(wl.tables, wl.lens)
        oracle.cache_write(k, v, wl.kv_dtype, wl.k_new, wl.v_new, slots)
        oracle.decode(wl.q, wl.q_dtype, k, v, wl.kv_dtype, wl.tables, wl.lens, wl.scale)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 50:
            break
    return statistics.median(times), len(times), oracle.max_threads()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--partition", type=int, default=None,
                    help="split: tokens per partition, 0 for none, -1 for the balanced split "
                         "(default: the library's recommendation)")
    ap.add_argument("--layout", choices=("blocks", "split"), default="blocks",
                    help="pool layout: one [NB][2][Hkv][16][D] tensor (blocks) or two dense "
                         "[NB][Hkv][16][D] pools (split)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU; runs on more than one GPU are not part of this "
              "library (the design notes describe how the path would shard)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_434_amd as pkv
    from paged_kv_cache_434_amd import workloads as W

    torch.cuda.set_device(0)
    wl = W.make(2)
    part = args.partition if args.partition is not None else pkv.default_partition(
        wl.B, wl.Hkv, wl.max_blocks)
    reps = [Replica(wl, part, args.layout) for _ in range(max(1, args.replicas))]
    print(f"# workload {wl.name}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} "
          f"sum(L)={int(wl.lens.sum())} pool={wl.num_blocks} partition={part} "
          f"replicas={len(reps)}", file=sys.stderr, flush=True)

    for i in range(args.warmup):
        run_step(pkv, reps[i % len(reps)])
    torch.cuda.synchronize()

    K = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        run_step(pkv, reps[i % len(reps)], evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_s = (t1 - t0) / K
    step_ms = [a.elapsed_time(b) for a, b in evs]
    attn_s = statistics.mean(step_ms) / 1e3

    ab = algorithmic_bytes(wl)
    value = ab["step"] / step_s / 1e9
    achieved = ab["step"] / attn_s / 1e9
    line = {
        "metric": "paged decode KV HBM GB/s (% of peak) + seq-steps/s, Llama-3-8B shape",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "num_q_heads": wl.Hq,
                   "num_kv_heads": wl.Hkv, "head_dim": wl.D, "block_size": 16,
                   "context_lens": "uniform[512,4096]", "sum_context": int(wl.lens.sum()),
                   "pool_blocks": wl.num_blocks, "partition_tokens": part,
                   "split": "balanced" if part == pkv.SPLIT_BALANCED else "fixed",
                   "layout": args.layout,
                   "step": "decode step: slot of position L-1 + cache write + paged "
                           "attention (one launch) + partition combine",
                   "replicas": len(reps)},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(wl.B / step_s, 1),
        "gpu_step_ms": round(attn_s * 1e3, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "kernel": "decode step call (fused append + attention, combine)",
                     "bytes_per_launch": ab["step"]},
    }
    if not args.no_cpu_baseline:
        med, reps_done, threads = cpu_baseline(wl)
        line["cpu_baseline"] = {"value": round(ab["step"] / med / 1e9, 3), "unit": "GB/s",
                                "cores": threads, "kind": "oracle",
                                "sample": f"whole workload (slot mapping + cache write + decode "
                                          f"of all {wl.B} sequences), median of {reps_done} "
                                          f"runs, {med:.2f} s each"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
