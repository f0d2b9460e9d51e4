"""Benchmark: one decode step of paged attention on one MI355X.

A step is the whole hot path for one layer of a workload (default: the
Llama-3-8B layer shape -- batch 64, 32 query / 8 KV heads, head dim 128, bf16,
context lengths uniform in [512, 4096], 16-token blocks from a 20,000-block
pool): the slot of each sequence's newest position, the cache write of the new
K/V token and paged attention, which the library's decode-step entry runs in
one launch, then the log-sum-exp combine of split contexts.  The
quantized-prefix workload has no new token: its step is attention over a pool
quantized once before timing.

Inputs are resident in HBM before timing.  To keep the 256 MB Infinity Cache
from serving a step out of the previous one, the step cycles over R
independent copies of the inputs, so the copy a step reads was last touched
R-1 steps (>= 1.3 GB of other traffic for the default workload) earlier.

Prints one JSON line.  `value` is the algorithmic bytes of a step divided by
the wall time per step (GB/s); `roofline` divides the same bytes by the
average duration of the step's kernels, measured with HIP events recorded on
the stream they run on, against the 8 TB/s HBM peak; `traffic` is the HBM
bytes per step that rocprofv3 counters measured for the current kernel source
(recorded under profiles/), or null.  The CPU baseline is the oracle on the
host, timed on the same workload.

    python bench.py                     # headline: Llama-3-8B shape
    python bench.py --workload 3        # other workloads (1..5; 5 takes --quant)
    python bench.py --copy-calibration  # plain 1 GiB device copy, for counter scaling
    python bench.py --op quantize       # pkv_quantize / pkv_copy_blocks bandwidth
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import re
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
METRIC = "paged decode KV HBM GB/s (% of peak) + seq-steps/s, Llama-3-8B shape"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ("paged_kv_cache_434_amd/csrc/decode.hip", "paged_kv_cache_434_amd/csrc/common.hpp")


def algorithmic_bytes(wl, ntok=1, window=0):
    """Bytes the method must move for one step: K/V of every context token,
    the used block-table entries, 8-bit scales, q in and out, lengths, and for
    workloads with a new token its K/V row read and written plus its slot."""
    import numpy as np

    e_kv = {"f32": 4, "bf16": 2, "i8": 1, "fp8": 1, "u8z": 1, "fp4": 0.5}[wl.quant or wl.kv_dtype]
    e_q = {"f32": 4, "bf16": 2}[wl.q_dtype]
    L = wl.lens.astype(np.int64)
    nblk = (L + 15) // 16
    if window > 0:
        # only the positions some query's window covers: the last W + k - 1
        L = np.minimum(L, window + ntok - 1)
        nblk = (L + 15) // 16
    kv = int(int(L.sum()) * wl.Hkv * wl.D * 2 * e_kv)
    tables = int(nblk.sum()) * 4
    if wl.quant == "u8z":       # a binary32 scale and a uint8 zero point per K and V row
        scales = int(L.sum()) * wl.Hkv * 2 * 5
    else:                       # a binary32 scale per (block, head) of K and of V
        scales = int(nblk.sum()) * wl.Hkv * 2 * 4 if wl.quant else 0
    q_out = wl.B * ntok * wl.Hq * wl.D * 2 * e_q
    lens = wl.B * 4
    attention = kv + tables + scales + q_out + lens
    q_out_tables_lens = tables + q_out + lens
    write = 0
    if wl.write and ntok == 1 and window == 0:
        # new K/V rows read (in the pool's type, or q's for a quantizing
        # append) and written into the pool, with their row parameters
        e_new = e_q if wl.quant else e_kv
        write = int(wl.B * wl.Hkv * wl.D * 2 * (e_new + e_kv))
        if wl.quant == "u8z":
            write += wl.B * wl.Hkv * 2 * 5
        elif wl.quant:          # the tile's scale read and written
            write += wl.B * wl.Hkv * 2 * 8
    return dict(attention=attention, kv=kv, write=write, step=attention + write,
                q_out_tables_lens=q_out_tables_lens)


def unique_bytes(wl, ntok=1, window=0):
    """Bytes of the distinct K/V rows (and their scales) a step reads: a
    physical row that several sequences share (a common prefix) counts once.
    With no sharing this equals the K/V part of algorithmic_bytes."""
    import numpy as np

    e_kv = {"f32": 4, "bf16": 2, "i8": 1, "fp8": 1, "u8z": 1, "fp4": 0.5}[wl.quant or wl.kv_dtype]
    rows = {}
    for s in range(wl.B):
        L = int(wl.lens[s])
        first = 0
        if window > 0:
            first = max(0, L - ntok + 1 - window)
        for j in range(first // 16, -(-L // 16)):
            b = int(wl.tables[s, j])
            rows[b] = max(rows.get(b, 0), min(16, L - 16 * j))
    n_rows = int(sum(rows.values()))
    kv = int(n_rows * wl.Hkv * wl.D * 2 * e_kv)
    if wl.quant == "u8z":
        scales = n_rows * wl.Hkv * 2 * 5
    else:
        scales = len(rows) * wl.Hkv * 2 * 4 if wl.quant else 0
    return dict(kv=kv, scales=scales, rows=n_rows, blocks=len(rows))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def code_only(text: str) -> str:
    """C++ source without comments and blank lines: what the compiler sees."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(l.rstrip() for l in text.splitlines() if l.strip())


def kernel_source_hash(read=None) -> str:
    """Hash of the attention kernels' code (comments left out, so counters
    recorded on a source stay valid across edits of its comments)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        if read is None:
            with open(os.path.join(ROOT, rel)) as f:
                text = f.read()
        else:
            text = read(rel)
        h.update(code_only(text).encode())
    return h.hexdigest()[:16]


def recorded_traffic(key: str):
    """HBM bytes per step recorded from rocprofv3 counters for this workload,
    if they were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("bytes_per_step")


class Replica:
    """One independent copy of the workload's device inputs plus a prepared
    step call."""

    def __init__(self, wl, part, layout, ntok=1, window=0, prefix_blocks=0):
        import numpy as np
        import torch
        import paged_kv_cache_434_amd as pkv
        from paged_kv_cache_434_amd import workloads as W

        d = W.to_device(wl, layout=layout)
        cache = pkv.PagedCache(d["k_pool"], d["v_pool"], wl.kv_dtype)
        if wl.quant:
            # quantized once, before timing
            NB, Hkv, bs, D = d["k_pool"].shape
            qt = torch.int8 if wl.quant == "i8" else torch.uint8
            pshape = (NB, Hkv, bs) if wl.quant == "u8z" else (NB, Hkv)
            Ds = D // 2 if wl.quant == "fp4" else D
            ks = torch.empty(pshape, dtype=torch.float32, device="cuda")
            vs = torch.empty_like(ks)
            kz = vz = None
            if wl.quant == "u8z":
                kz = torch.empty(pshape, dtype=torch.uint8, device="cuda")
                vz = torch.empty_like(kz)
            if layout == "blocks":
                qcache = pkv.PagedCache.from_blocks(
                    torch.empty((NB, 2, Hkv, bs, Ds), dtype=qt, device="cuda"), wl.quant, ks, vs,
                    kz, vz)
            else:
                kq = torch.empty((NB, Hkv, bs, Ds), dtype=qt, device="cuda")
                qcache = pkv.PagedCache(kq, torch.empty_like(kq), wl.quant, ks, vs, kz, vz)
            pkv.quantize(cache, qcache)
            for k in ("kv", "k_pool", "v_pool"):
                d.pop(k, None)
            cache = qcache
        out_dtype = torch.float32 if wl.q_dtype == "f32" else torch.bfloat16
        ws = pkv.alloc_workspace(wl.B, wl.Hq, wl.D, wl.max_blocks, part)
        if ntok > 1 or window > 0:
            # several query tokens per sequence (their K/V already in the pool)
            rng = np.random.default_rng(1)
            q = torch.from_numpy(W.to_bf16_bits(rng.standard_normal(
                (wl.B, ntok, wl.Hq, wl.D)).astype(np.float32)).view(np.int16)).view(
                torch.bfloat16).cuda()
            ws = pkv.alloc_workspace(wl.B * ntok, wl.Hq, wl.D, wl.max_blocks, part)
            tables, lens, scale = d["tables"], d["lens"], float(wl.scale)
            self.out = torch.empty((wl.B, ntok, wl.Hq, wl.D), dtype=out_dtype, device="cuda")
            self.call = lambda: pkv.attention_multi(cache, q, tables, lens, scale,
                                                    partition_tokens=part, workspace=ws,
                                                    out=self.out,
                                                    window=window if window > 0 else None)
        elif wl.write:
            self.call, self.out = pkv.prepare_decode_step(
                cache, d["q"], d["k_new"], d["v_new"], d["tables"], d["lens"], float(wl.scale),
                partition_tokens=part, workspace=ws, out_dtype=out_dtype)
            # the same step without the append: attention and the combine only
            self.attention_only, _ = pkv.prepare_attention_decode(
                cache, d["q"], d["tables"], d["lens"], float(wl.scale), partition_tokens=part,
                workspace=ws, out=self.out)
        elif prefix_blocks > 0:
            # the tables share their first prefix_blocks entries (a common prompt)
            ws = pkv.alloc_workspace(wl.B, wl.Hq, wl.D, wl.max_blocks, pkv.SPLIT_BALANCED)
            self.call, self.out = pkv.prepare_attention_prefix(
                cache, d["q"], d["tables"], d["lens"], float(wl.scale), prefix_blocks,
                workspace=ws, out_dtype=out_dtype)
        else:
            self.call, self.out = pkv.prepare_attention_decode(
                cache, d["q"], d["tables"], d["lens"], float(wl.scale), partition_tokens=part,
                workspace=ws, out_dtype=out_dtype)
        self.d, self.cache = d, cache
        if not hasattr(self, "attention_only"):
            self.attention_only = None


def cpu_baseline(wl, budget_s=10.0):
    """The oracle (as it stands) timed on the host over the whole workload:
    slot mapping + cache write + decode (or quantize once + decode for the
    quantized workload), repeated until about budget_s seconds have passed."""
    import oracle

    k, v = wl.k_pool.copy(), wl.v_pool.copy()
    ks = vs = kz = vz = None
    kvd = wl.kv_dtype
    if wl.quant == "u8z":
        k, ks, kz = oracle.quantize_asym(k, wl.kv_dtype)
        v, vs, vz = oracle.quantize_asym(v, wl.kv_dtype)
        kvd = wl.quant
    elif wl.quant:
        k, ks = oracle.quantize(k, wl.kv_dtype, wl.quant)
        v, vs = oracle.quantize(v, wl.kv_dtype, wl.quant)
        kvd = wl.quant
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        if wl.write:
            slots = oracle.slot_mapping(wl.tables, wl.lens)
            if wl.quant == "u8z":
                oracle.cache_write_quant(k, v, ks, vs, kz, vz, wl.k_new, wl.v_new,
                                         wl.kv_dtype, slots)
            elif wl.quant:
                oracle.cache_write_sym(k, v, ks, vs, wl.quant, wl.k_new, wl.v_new,
                                       wl.kv_dtype, slots)
            else:
                oracle.cache_write(k, v, wl.kv_dtype, wl.k_new, wl.v_new, slots)
        oracle.decode(wl.q, wl.q_dtype, k, v, kvd, wl.tables, wl.lens, wl.scale,
                      k_scale=ks, v_scale=vs, k_zero=kz, v_zero=vz)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 50:
            break
    return statistics.median(times), len(times), oracle.max_threads()


def achievable_context():
    """What plain torch device ops reach on this GPU in the same process, as
    context for the roofline fraction (the peak stays the published 8 TB/s):
    a 1 GiB device copy (bytes read + written per second) and a sum over
    1 GiB of bfloat16 (bytes read per second); best of five each."""
    import torch

    n = 1 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)

    def best(fn):
        t = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b) / 1e3)
        return min(t)

    copy_s = best(lambda: dst.copy_(src))
    sum_s = best(lambda: src.sum(dtype=torch.float32))
    del src, dst
    return {"device_copy_GBps": round(2 * n / copy_s / 1e9, 1),
            "device_sum_read_GBps": round(n / sum_s / 1e9, 1),
            "note": "torch ops on 1 GiB in this process; context only"}


def copy_calibration():
    """A plain device-to-device copy of 1 GiB, five times: under rocprofv3
    --pmc FETCH_SIZE / WRITE_SIZE it gives the counters' reading for a known
    number of bytes (1 GiB read and 1 GiB written per dispatch)."""
    import torch

    torch.cuda.set_device(0)
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        t.append(a.elapsed_time(b) / 1e3)
    print(json.dumps({"calibration": "device copy", "bytes_read": n, "bytes_written": n,
                      "ms": round(min(t) * 1e3, 4),
                      "GBps_read_plus_write": round(2 * n / min(t) / 1e9, 1)}), flush=True)


def op_bench(args):
    """Bandwidth of the operations outside the decode step, on the workload's
    pool: pkv_quantize of the whole pool (bf16 source -> 8-bit codes + scales)
    and pkv_copy_blocks of half the pool's blocks into the other half.  One
    JSON line; bytes are what the operation must read and write."""
    import numpy as np
    import torch
    import paged_kv_cache_434_amd as pkv
    from paged_kv_cache_434_amd import workloads as W

    torch.cuda.set_device(0)
    wl = W.make(args.workload)
    d = W.to_device(wl, layout=args.layout)
    cache = pkv.PagedCache(d["k_pool"], d["v_pool"], wl.kv_dtype)
    NB, Hkv, bs, D = d["k_pool"].shape
    e = {"f32": 4, "bf16": 2}[wl.kv_dtype]
    if args.op == "quantize":
        quant = args.quant or "i8"
        qt = torch.int8 if quant == "i8" else torch.uint8
        rows = quant == "u8z"
        Ds = D // 2 if quant == "fp4" else D
        e_q = 0.5 if quant == "fp4" else 1
        pshape = (NB, Hkv, bs) if rows else (NB, Hkv)
        ks = torch.empty(pshape, dtype=torch.float32, device="cuda")
        vs = torch.empty_like(ks)
        kz = torch.empty(pshape, dtype=torch.uint8, device="cuda") if rows else None
        vz = torch.empty_like(kz) if rows else None
        dst = pkv.PagedCache.from_blocks(
            torch.empty((NB, 2, Hkv, bs, Ds), dtype=qt, device="cuda"), quant, ks, vs, kz, vz)
        fn = lambda: pkv.quantize(cache, dst)
        nbytes = int(2 * NB * Hkv * bs * D * (e + e_q)) + (2 * NB * Hkv * bs * 5 if rows
                                                           else 2 * NB * Hkv * 4)
        what = f"pkv_quantize {wl.kv_dtype}->{quant}, all {NB} blocks"
    else:
        rng = np.random.default_rng(0)
        ids = rng.permutation(NB).astype(np.int32)
        n = NB // 2
        pairs = torch.from_numpy(np.stack([ids[:n], ids[n:2 * n]], 1)).cuda()
        fn = lambda: pkv.copy_blocks(cache, pairs)
        nbytes = 2 * 2 * n * Hkv * bs * D * e
        what = f"pkv_copy_blocks, {n} block pairs"
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = statistics.mean(a.elapsed_time(b) for a, b in evs) / 1e3
    gbs = nbytes / t / 1e9
    print(json.dumps({"metric": f"{args.op} HBM GB/s", "value": round(gbs, 1), "unit": "GB/s",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "ms_per_step": round(t * 1e3, 4), "higher_is_better": True,
                      "dtype": wl.kv_dtype, "data": "synthetic",
                      "config": {"workload": wl.name, "op": what, "layout": args.layout},
                      "bytes_per_launch": nbytes,
                      "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None}}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=2, choices=(1, 2, 3, 4, 5))
    ap.add_argument("--quant", choices=("i8", "fp8", "u8z", "fp4"), default=None,
                    help="quantized pool format: i8, fp8 (E4M3), fp4 (E2M1), each with a "
                         "scale per (block, KV head), or u8z (asymmetric per-row uint8); the "
                         "quantized-prefix workload (5) defaults to i8, and on the decode-step "
                         "workloads (2-4) the pool is quantized once and the step appends the "
                         "new token quantized")
    ap.add_argument("--replicas", type=int, default=0,
                    help="input copies cycled through (0: enough for 1.3 GB of pools)")
    ap.add_argument("--partition", type=int, default=None,
                    help="split: tokens per partition, 0 for none, -1 for the balanced split "
                         "(default: the library's recommendation)")
    ap.add_argument("--layout", choices=("blocks", "split"), default="blocks",
                    help="pool layout: one [NB][2][Hkv][16][D] tensor (blocks) or two dense "
                         "[NB][Hkv][16][D] pools (split)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--tokens", type=int, default=1,
                    help="query tokens per sequence (>1: multi-token attention, e.g. verifying "
                         "drafted tokens; their K/V are taken as already written)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window in tokens (>0: attention over each query's most recent "
                         "window only; no append)")
    ap.add_argument("--append", action="store_true",
                    help="workload 5: a decode step whose new tokens are appended into the "
                         "quantized pool before attention")
    ap.add_argument("--prefix-blocks", type=int, default=-1,
                    help="shared-prefix attention over that many common table entries "
                         "(-1: the workload's shared prefix for workload 5, none otherwise; "
                         "0: the general attention path)")
    ap.add_argument("--op", choices=("step", "quantize", "copy_blocks"), default="step",
                    help="what to time: the decode step (default) or another operation")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU; runs on more than one GPU are not part of this "
              "library (the design notes describe how the path would shard)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.op != "step":
        op_bench(args)
        return

    import torch
    import paged_kv_cache_434_amd as pkv
    from paged_kv_cache_434_amd import workloads as W

    torch.cuda.set_device(0)
    if args.workload == 5:
        # --append: a decode step, each sequence's new token appended into its
        # own blocks (quantized) before attention
        extra = dict(write=True, suffix_lo=1) if args.append else {}
        wl = W.make(5, quant=args.quant or "i8", **extra)
    else:
        wl = W.make(args.workload)
        if args.quant:
            if wl.kv_dtype != "bf16":
                sys.exit("--quant needs a bf16 workload (2-4)")
            wl = dataclasses.replace(wl, quant=args.quant)
    part = args.partition if args.partition is not None else pkv.default_partition(
        wl.B, wl.Hkv, wl.max_blocks)
    e_kv = {"f32": 4, "bf16": 2, "i8": 1, "fp8": 1, "u8z": 1, "fp4": 0.5}[wl.quant or wl.kv_dtype]
    pool_bytes = int(wl.num_blocks * wl.Hkv * 16 * wl.D * 2 * e_kv)
    n_rep = args.replicas or max(2, min(8, math.ceil(1.3e9 / pool_bytes) + 1))
    prefix_blocks = args.prefix_blocks
    if prefix_blocks < 0:
        prefix_blocks = W.SPECS[5]["prefix"] // 16 if args.workload == 5 and not wl.write else 0
    if prefix_blocks > 0 and (wl.write or args.tokens > 1 or args.window > 0):
        sys.exit("--prefix-blocks applies to attention over the shared-prefix workload (5)")
    if prefix_blocks > 0:
        part = pkv.SPLIT_BALANCED
    reps = [Replica(wl, part, args.layout, args.tokens, args.window, prefix_blocks)
            for _ in range(n_rep)]
    print(f"# workload {wl.name}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} "
          f"sum(L)={int(wl.lens.sum())} pool={wl.num_blocks} quant={wl.quant} "
          f"partition={part} layout={args.layout} replicas={len(reps)}",
          file=sys.stderr, flush=True)

    for i in range(args.warmup):
        reps[i % len(reps)].call()
    torch.cuda.synchronize()

    # wall time of K back-to-back steps
    K = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        reps[i % len(reps)].call()
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - t0) / K

    # kernel time of each step: HIP events on the stream the kernels run on
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for i in range(K):
        evs[i][0].record(stream)
        reps[i % len(reps)].call()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    kern_s = statistics.mean(a.elapsed_time(b) for a, b in evs) / 1e3

    def event_time(fn_of):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(K)]
        for i in range(K):
            evs[i][0].record(stream)
            fn_of(reps[i % len(reps)])()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        return statistics.mean(a.elapsed_time(b) for a, b in evs) / 1e3

    attn_s = None
    if reps[0].attention_only is not None:
        attn_s = event_time(lambda r: r.attention_only)

    ab = algorithmic_bytes(wl, args.tokens, args.window)
    value = ab["step"] / step_s / 1e9
    achieved = ab["step"] / kern_s / 1e9
    key = (f"{wl.name}{'_' + wl.quant if wl.quant else ''}/{args.layout}/"
           + (f"prefix{prefix_blocks}" if prefix_blocks > 0 else f"{part}")
           + (f"/tokens{args.tokens}" if args.tokens > 1 else "")
           + (f"/window{args.window}" if args.window > 0 else "")
           + ("/append" if wl.write and args.workload == 5 else ""))
    traffic = recorded_traffic(key)
    e_q = {"f32": "f32", "bf16": "bf16"}[wl.q_dtype]
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(step_s * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": e_q if not wl.quant else f"{e_q}/{wl.quant}",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "num_q_heads": wl.Hq,
                   "num_kv_heads": wl.Hkv, "head_dim": wl.D, "block_size": 16,
                   "kv_dtype": wl.quant or wl.kv_dtype, "sum_context": int(wl.lens.sum()),
                   "pool_blocks": wl.num_blocks, "partition_tokens": part,
                   "split": ("shared prefix" if prefix_blocks > 0 else
                             "balanced" if part == pkv.SPLIT_BALANCED else "fixed"),
                   "prefix_blocks": prefix_blocks,
                   "layout": args.layout, "replicas": len(reps),
                   "query_tokens_per_seq": args.tokens,
                   "window": args.window,
                   "step": (f"sliding-window paged attention ({args.window} tokens) of "
                            f"{args.tokens} query token(s) per sequence + partition combine")
                           if args.window > 0 else
                           (f"paged attention of {args.tokens} query tokens per sequence + "
                            "partition combine") if args.tokens > 1 else
                           ("decode step: quantized append of position L-1 (own launch) + "
                            "paged attention + partition combine") if wl.write and wl.quant else
                           ("decode step: slot of position L-1 + cache write + paged attention "
                            "(one launch) + partition combine") if wl.write else
                           (f"shared-prefix paged attention ({prefix_blocks} common blocks run "
                            "once per group of sequences) + partition combine")
                           if prefix_blocks > 0 else
                           "paged attention over a quantized pool + partition combine"},
        "pct_of_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(wl.B / step_s, 1),
        "kernel_ms_per_step": round(kern_s * 1e3, 4),
        "attention_only_ms": None if attn_s is None else round(attn_s * 1e3, 4),
        "bytes_per_step": ab["step"],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "traffic_key": key,
                     "kernel": "the step's kernels (decode attention, then the combine)",
                     "bytes_per_launch": ab["step"]},
    }
    if wl.quant or args.workload == 5:
        # blocks shared between sequences are read once from HBM at best: the
        # distinct rows' bytes beside the logical ones
        ub = unique_bytes(wl, args.tokens, args.window)
        ubytes = ub["kv"] + ub["scales"] + ab["q_out_tables_lens"] + ab["write"]
        line["unique_bytes_per_step"] = ubytes
        line["unique_GBps"] = round(ubytes / kern_s / 1e9, 1)
        line["unique_frac_of_peak"] = round(ubytes / kern_s / 1e9 / HBM_PEAK_GBS, 4)
        if ubytes < ab["step"]:
            # the HBM roofline is priced on the bytes HBM must deliver: a
            # shared block's bytes once; the logical figure stays in `value`
            line["roofline"].update(
                achieved=round(ubytes / kern_s / 1e9, 1),
                frac=round(ubytes / kern_s / 1e9 / HBM_PEAK_GBS, 4), bytes_per_launch=ubytes,
                note="unique bytes (each shared block once); value counts them per sequence")
    if not args.no_cpu_baseline and args.tokens == 1 and args.window == 0:
        med, runs, threads = cpu_baseline(wl)
        line["cpu_baseline"] = {
            "value": round(ab["step"] / med / 1e9, 3), "unit": "GB/s", "cores": threads,
            "cpu": cpu_model(), "kind": "oracle",
            "sample": (f"the whole workload ({wl.B} sequences, {int(wl.lens.sum())} context "
                       f"tokens) per run, median of {runs} runs of {med:.3f} s; "
                       f"{wl.B / med:.1f} seq-steps/s")}
    if args.tokens == 1 and args.window == 0:
        line["achievable"] = achievable_context()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
