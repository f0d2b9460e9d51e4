"""Seeded synthetic inputs for paged-KV decode (host numpy arrays).

This module only draws random inputs; it holds none of the attention, cache
write, slot or quantization arithmetic, so both the GPU path and the CPU
oracle can take their inputs from it.

Five workloads, in the shapes the KV-cache pages discuss (16-token blocks, GQA
groups of 32 query / 8 KV heads, head dim 128; a Llama-3-70B-like 64/8 group;
a long context; shared-prefix and quantized KV):

  1 tiny_fp32        B=4, lens {17,33,64,100}, Hq=4, Hkv=2, D=64, pool 64, fp32
  2 llama3_8b_bf16   B=64, lens U{512..4096}, Hq=32, Hkv=8, D=128, pool 20000
  3 llama3_70b_bf16  B=256, lens clip(rint(exp N(ln 1500, 1)), 64, 8192), Hq=64,
                     Hkv=8, pool ceil(1.1 x blocks needed)
  4 long_split_bf16  B=8, lens 32768, Hq=32, Hkv=8, 512-token partitions; every
                     64th key (positions t with (t+1) % 64 == 0) scaled by 8 in
                     fp32 before the bf16 cast
  5 quant_prefix     B=128, 2048-token prefix shared by every table (the same
                     128 physical blocks) + U{0..1024} private tokens; bf16
                     source pool that the caller quantizes to INT8 or FP8
                     (tests shrink it; a sequence shorter than the prefix
                     still has the prefix ids as its first table entries;
                     with write=True and suffix_lo=1 each sequence also
                     gets a new token in a private block)

Recipe: ``numpy.random.default_rng(seed)`` (seed = workload number unless
given); draw order lens -> block permutation -> pool K -> pool V -> new K ->
new V -> q -> padding of unused table entries.  Values are N(0,1) in float32,
rounded to bf16 (round-to-nearest-even) where the dtype is bf16.  Physical
blocks are handed out from a random permutation of the pool: sequence 0 takes
the first ceil(L_0/16) ids, sequence 1 the next, and so on (workload 5: the 128
shared prefix ids first).  Table entries past a sequence's last block hold
random valid block ids; every slot of every pool block holds N(0,1) data.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BLOCK_SIZE = 16

NP_STORAGE = {"f32": np.float32, "bf16": np.uint16, "i8": np.int8, "fp8": np.uint8}


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    kv_dtype: str            # dtype of the stored pool handed to attention ("f32"/"bf16")
    q_dtype: str             # "f32" or "bf16"
    num_blocks: int
    max_blocks: int          # block-table width
    lens: np.ndarray         # int32 [B]
    tables: np.ndarray       # int32 [B][max_blocks]
    k_pool: np.ndarray       # storage dtype [NB][Hkv][16][D]
    v_pool: np.ndarray
    k_new: Optional[np.ndarray]  # storage dtype [B][Hkv][D] (None: attention only)
    v_new: Optional[np.ndarray]
    q: np.ndarray            # storage dtype [B][Hq][D]
    scale: np.float32        # 1/sqrt(D) as binary32
    partition_tokens: int    # 0: caller's choice; otherwise the workload's split size
    quant: Optional[str] = None   # "i8"/"fp8": the pool is a quantization source
    block_size: int = BLOCK_SIZE

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def write(self) -> bool:
        return self.k_new is not None


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (via torch's cast)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal(rng, shape, dtype: str, chunk_rows: int = 4096) -> np.ndarray:
    """N(0,1) values of the given shape in storage dtype, drawn in chunks."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=NP_STORAGE[dtype])
    flat = out.reshape(shape[0], -1)
    for i in range(0, shape[0], chunk_rows):
        x = rng.standard_normal((min(chunk_rows, shape[0] - i), flat.shape[1]), dtype=np.float32)
        flat[i:i + x.shape[0]] = to_bf16_bits(x) if dtype == "bf16" else x
    return out


def _pool_normal(rng, shape, dtype, boost=None):
    """Pool values; ``boost`` = (slot mask [NB*16] bool, factor) scales those rows in fp32."""
    NB, Hkv, bs, D = shape
    out = np.empty(shape, dtype=NP_STORAGE[dtype])
    chunk = 2048
    for b0 in range(0, NB, chunk):
        n = min(chunk, NB - b0)
        x = rng.standard_normal((n, Hkv, bs, D), dtype=np.float32)
        if boost is not None:
            mask, factor = boost
            m = mask[b0 * bs:(b0 + n) * bs].reshape(n, 1, bs, 1)
            x = np.where(m, x * np.float32(factor), x)
        out[b0:b0 + n] = to_bf16_bits(x) if dtype == "bf16" else x
    return out


SPECS = {
    1: dict(name="tiny_fp32", B=4, Hq=4, Hkv=2, D=64, kv="f32", q="f32", pool=64, write=True,
            part=0),
    2: dict(name="llama3_8b_bf16", B=64, Hq=32, Hkv=8, D=128, kv="bf16", q="bf16", pool=20000,
            write=True, part=0, lo=512, hi=4096),
    3: dict(name="llama3_70b_bf16", B=256, Hq=64, Hkv=8, D=128, kv="bf16", q="bf16", pool=None,
            write=True, part=0, median=1500.0, sigma=1.0, lo=64, hi=8192),
    4: dict(name="long_split_bf16", B=8, Hq=32, Hkv=8, D=128, kv="bf16", q="bf16", pool=None,
            write=True, part=512, L=32768, boost_every=64, boost=8.0),
    5: dict(name="quant_prefix", B=128, Hq=32, Hkv=8, D=128, kv="bf16", q="bf16", pool=None,
            write=False, part=0, prefix=2048, suffix_hi=1024),
}


def make(cfg: int, seed: Optional[int] = None, quant: Optional[str] = None, **over) -> Workload:
    """Build workload ``cfg`` (1..5).  Keyword overrides shrink it for tests:
    B, lo, hi (length range), L, prefix, suffix_hi, pool (block count or None
    for 1.1 x needed), lens (explicit list), Hq, Hkv, D, kv, q."""
    spec = dict(SPECS[cfg])
    spec.update(over)
    rng = np.random.default_rng(cfg if seed is None else seed)
    B, Hq, Hkv, D = spec["B"], spec["Hq"], spec["Hkv"], spec["D"]
    bs = BLOCK_SIZE

    # -- lens
    if "lens" in spec and spec["lens"] is not None:
        lens = np.asarray(spec["lens"], dtype=np.int64)
        hi_len = int(lens.max(initial=0))
    elif cfg == 1:
        lens = np.array([17, 33, 64, 100], dtype=np.int64)
        hi_len = 100
    elif cfg == 2:
        lens = rng.integers(spec["lo"], spec["hi"], size=B, endpoint=True)
        hi_len = spec["hi"]
    elif cfg == 3:
        x = rng.normal(math.log(spec["median"]), spec["sigma"], size=B)
        lens = np.clip(np.rint(np.exp(x)), spec["lo"], spec["hi"]).astype(np.int64)
        hi_len = spec["hi"]
    elif cfg == 4:
        lens = np.full(B, spec["L"], dtype=np.int64)
        hi_len = spec["L"]
    else:
        suffix = rng.integers(spec.get("suffix_lo", 0), spec["suffix_hi"], size=B, endpoint=True)
        lens = spec["prefix"] + suffix
        hi_len = spec["prefix"] + spec["suffix_hi"]
    lens = lens.astype(np.int32)
    max_blocks = max(1, -(-hi_len // bs))
    if cfg == 5:   # every table holds the shared prefix, however short its sequence
        max_blocks = max(max_blocks, spec["prefix"] // bs)
    nblk = [-(-int(L) // bs) for L in lens]

    # -- pool size and block permutation
    if cfg == 5:
        n_prefix = spec["prefix"] // bs
        needed = n_prefix + sum(max(n - n_prefix, 0) for n in nblk)
    else:
        needed = sum(nblk)
    NB = spec["pool"] if spec.get("pool") else max(1, math.ceil(1.1 * needed))
    assert NB >= needed, "pool smaller than the blocks needed"
    perm = rng.permutation(NB).astype(np.int32)
    tables = np.zeros((B, max_blocks), dtype=np.int32)
    used = np.zeros((B, max_blocks), dtype=bool)
    if cfg == 5:
        prefix_ids = perm[:n_prefix]
        cur = n_prefix
        for s in range(B):
            tables[s, :n_prefix] = prefix_ids
            k = max(nblk[s] - n_prefix, 0)
            tables[s, n_prefix:n_prefix + k] = perm[cur:cur + k]
            cur += k
            used[s, :max(nblk[s], n_prefix)] = True
    else:
        cur = 0
        for s in range(B):
            tables[s, :nblk[s]] = perm[cur:cur + nblk[s]]
            cur += nblk[s]
            used[s, :nblk[s]] = True

    # -- pool values (workload 4: every 64th key boosted before the cast)
    kv = spec["kv"]
    boost = None
    if cfg == 4 and spec.get("boost_every"):
        every = spec["boost_every"]
        mask = np.zeros(NB * bs, dtype=bool)
        for s in range(B):
            t = np.arange(every - 1, int(lens[s]), every)
            mask[tables[s, t // bs].astype(np.int64) * bs + t % bs] = True
        boost = (mask, spec["boost"])
    k_pool = _pool_normal(rng, (NB, Hkv, bs, D), kv, boost)
    v_pool = _pool_normal(rng, (NB, Hkv, bs, D), kv)

    # -- new tokens (position L-1 of each sequence)
    k_new = v_new = None
    if spec["write"]:
        if boost is not None:
            x = rng.standard_normal((B, Hkv, D), dtype=np.float32)
            hit = (lens % spec["boost_every"] == 0).reshape(B, 1, 1)
            x = np.where(hit, x * np.float32(spec["boost"]), x)
            k_new = to_bf16_bits(x) if kv == "bf16" else x
        else:
            k_new = _normal(rng, (B, Hkv, D), kv)
        v_new = _normal(rng, (B, Hkv, D), kv)

    q = _normal(rng, (B, Hq, D), spec["q"])

    # -- unused table entries: random valid ids
    pad = rng.integers(0, NB, size=(B, max_blocks)).astype(np.int32)
    tables = np.where(used, tables, pad).astype(np.int32)

    return Workload(name=spec["name"], B=B, Hq=Hq, Hkv=Hkv, D=D, kv_dtype=kv, q_dtype=spec["q"],
                    num_blocks=NB, max_blocks=max_blocks, lens=lens, tables=tables,
                    k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new, q=q,
                    scale=np.float32(1.0 / math.sqrt(D)), partition_tokens=spec["part"],
                    quant=quant if cfg == 5 else None)


def to_device(wl: Workload, device="cuda", layout: str = "split") -> dict:
    """Copy a workload's arrays to the GPU as torch tensors (bf16 bit patterns
    become torch.bfloat16).  layout "split": K and V pools are two dense
    [NB][Hkv][16][D] tensors; "blocks": one [NB][2][Hkv][16][D] tensor ``kv``
    whose halves are returned as the (block-strided) ``k_pool`` / ``v_pool``."""
    import torch

    def dev(a, kind):
        if a is None:
            return None
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
                torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)

    out = dict(q=dev(wl.q, wl.q_dtype), k_new=dev(wl.k_new, wl.kv_dtype),
               v_new=dev(wl.v_new, wl.kv_dtype), tables=dev(wl.tables, "i32"),
               lens=dev(wl.lens, "i32"))
    if layout == "split":
        out["k_pool"] = dev(wl.k_pool, wl.kv_dtype)
        out["v_pool"] = dev(wl.v_pool, wl.kv_dtype)
    elif layout == "blocks":
        k = dev(wl.k_pool, wl.kv_dtype)
        kv = torch.empty((k.shape[0], 2) + tuple(k.shape[1:]), dtype=k.dtype, device=device)
        kv[:, 0].copy_(k)
        del k
        kv[:, 1].copy_(dev(wl.v_pool, wl.kv_dtype))
        out["kv"] = kv
        out["k_pool"], out["v_pool"] = kv[:, 0], kv[:, 1]
    else:
        raise ValueError(f"unknown layout {layout!r}")
    return out


def from_device(t) -> np.ndarray:
    """torch tensor -> numpy in storage dtype (bf16 as uint16 bit patterns)."""
    import torch

    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy()
    return t.numpy()
