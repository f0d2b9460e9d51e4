"""Small test-side helpers: tiny random paged inputs and an independent
contiguous (un-paged) view of them built with numpy fancy indexing."""
from __future__ import annotations

import numpy as np

from paged_kv_cache_434_amd import workloads as W

BS = 16


def tiny_paged(rng, lens, Hq, Hkv, D, NB=None, dtype="f32", q_dtype=None, extra_cols=2):
    """Random pool + tables for explicit context lengths; tables drawn from a
    random permutation; padding entries hold random valid ids."""
    q_dtype = q_dtype or dtype
    lens = np.asarray(lens, dtype=np.int32)
    nblk = [-(-int(L) // BS) for L in lens]
    need = sum(nblk)
    NB = NB or need + 5
    maxb = max(max(nblk, default=0), 1) + extra_cols
    perm = rng.permutation(NB).astype(np.int32)
    tables = rng.integers(0, NB, size=(len(lens), maxb)).astype(np.int32)
    cur = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = perm[cur:cur + n]
        cur += n
    k = rng.standard_normal((NB, Hkv, BS, D)).astype(np.float32)
    v = rng.standard_normal((NB, Hkv, BS, D)).astype(np.float32)
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
    if dtype == "bf16":
        k, v = W.to_bf16_bits(k), W.to_bf16_bits(v)
    if q_dtype == "bf16":
        q = W.to_bf16_bits(q)
    return dict(q=q, k=k, v=v, tables=tables, lens=lens, NB=NB)


def as_f64(a, dtype):
    if dtype == "bf16":
        return W.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def contiguous(pool, tables, s, L):
    """[L][Hkv][D] rows of sequence s in logical order (numpy fancy index)."""
    t = np.arange(L)
    return pool[tables[s, t // BS], :, t % BS, :]


def brute_attention(q64, k64, v64, scale):
    """softmax(scale * q k^T) v for one sequence; q [Hq][D], k/v [L][Hkv][D]
    float64; GQA by repeating each KV head over its contiguous query group."""
    Hq = q64.shape[0]
    L, Hkv, D = k64.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D))
    if L == 0:
        return out
    for h in range(Hq):
        g = h // G
        s = scale * (k64[:, g, :] @ q64[h])
        w = np.exp(s - s.max())
        out[h] = (w[:, None] * v64[:, g, :]).sum(0) / w.sum()
    return out
