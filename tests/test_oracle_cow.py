"""Oracle pins for the copy-on-write block copy (page on KV cache and
PagedAttention, section 二 "写时复制"; vLLM deep-dive page, "意外的收获：prefix
sharing"): the copy against numpy indexing, and a beam-search branch that
writes into a shared block against brute-force contiguous attention."""
import numpy as np

import oracle
from helpers import BS, as_f64, brute_attention, contiguous


def test_copy_blocks_matches_fancy_index_and_leaves_others():
    rng = np.random.default_rng(5)
    NB, Hkv, D = 20, 3, 64
    k = rng.standard_normal((NB, Hkv, BS, D)).astype(np.float32)
    v = rng.standard_normal((NB, Hkv, BS, D)).astype(np.float32)
    ks = rng.random((NB, Hkv)).astype(np.float32)
    vs = rng.random((NB, Hkv)).astype(np.float32)
    src = np.array([3, 3, 7, 0], dtype=np.int32)
    dst = np.array([11, 12, 19, 5], dtype=np.int32)
    want_k, want_v, want_ks, want_vs = k.copy(), v.copy(), ks.copy(), vs.copy()
    want_k[dst], want_v[dst] = k[src], v[src]
    want_ks[dst], want_vs[dst] = ks[src], vs[src]
    pairs = np.stack([src, dst], axis=1)
    oracle.copy_blocks(k, v, "f32", pairs, ks, vs)
    assert np.array_equal(k, want_k) and np.array_equal(v, want_v)
    assert np.array_equal(ks, want_ks) and np.array_equal(vs, want_vs)


def test_copy_blocks_skips_out_of_range_ids():
    rng = np.random.default_rng(6)
    k = rng.standard_normal((4, 1, BS, 64)).astype(np.float32)
    v = k.copy()
    before = k.copy()
    oracle.copy_blocks(k, v, "f32", np.array([[0, 4], [-1, 2], [1, 1 << 20]], np.int32))
    assert np.array_equal(k, before) and np.array_equal(v, before)


def test_branch_write_after_copy_on_write():
    """Two beam branches share every block of a 37-token history (the last
    block half full).  Branch B appends its next token: its last block is
    shared, so it is copied to a free block first, B's table is pointed at the
    copy and the token is written there.  Branch A must see exactly the same
    result as before, and B attention over the history plus its token."""
    rng = np.random.default_rng(7)
    Hq, Hkv, D, L = 4, 2, 64, 37
    NB = 10
    k = rng.standard_normal((NB, Hkv, BS, D)).astype(np.float32)
    v = rng.standard_normal((NB, Hkv, BS, D)).astype(np.float32)
    shared = np.array([4, 1, 6], dtype=np.int32)           # ceil(37 / 16) = 3 blocks
    q = rng.standard_normal((2, Hq, D)).astype(np.float32)
    tables = np.stack([shared, shared])
    lens = np.array([L, L], dtype=np.int32)
    scale = np.float32(1 / 8)
    before = oracle.decode(q, "f32", k, v, "f32", tables, lens, scale)
    hist_k, hist_v = contiguous(k, tables, 0, L), contiguous(v, tables, 0, L)

    # copy on write: B gets a private copy of the shared last block
    free = 8
    oracle.copy_blocks(k, v, "f32", np.array([[shared[-1], free]], np.int32))
    tables[1, -1] = free
    lens[1] = L + 1
    k_new = rng.standard_normal((1, Hkv, D)).astype(np.float32)
    v_new = rng.standard_normal((1, Hkv, D)).astype(np.float32)
    slot = oracle.slot_mapping(tables[1:], lens[1:])
    assert slot[0] == free * BS + L % BS
    oracle.cache_write(k, v, "f32", k_new, v_new, slot)

    after = oracle.decode(q, "f32", k, v, "f32", tables, lens, scale)
    assert np.array_equal(after[0], before[0])              # branch A untouched, bit for bit
    kb = np.concatenate([hist_k, k_new], axis=0)
    vb = np.concatenate([hist_v, v_new], axis=0)
    ref_b = brute_attention(as_f64(q[1], "f32"), as_f64(kb, "f32"), as_f64(vb, "f32"),
                            float(scale))
    assert np.max(np.abs(after[1] - ref_b)) < 1e-12
    # the shared block itself still holds A's history (the write went to the copy)
    assert np.array_equal(contiguous(k, tables, 0, L), hist_k)
