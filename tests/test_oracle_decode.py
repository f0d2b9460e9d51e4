"""Pins for the oracle's decode attention (CPU only).

The oracle is checked against things other than itself: brute-force
attention on a contiguous copy (numpy and torch's scaled_dot_product_attention
in float64), closed forms, invariants, the split-context identity and the
pages' worked KV-size example.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import BS, as_f64, brute_attention, contiguous, tiny_paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dec(d, Hkv, scale, dtype="f32", q_dtype=None, **kw):
    return oracle.decode(d["q"], q_dtype or dtype, d["k"], d["v"], dtype, d["tables"], d["lens"],
                         scale, **kw)


def test_kv_size_formula_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "kv_size_llama2_7b.json")))
    got = oracle.kv_cache_bytes(g["layers"], g["kv_heads"], g["head_dim"], g["seq_len"],
                                g["bytes_per_elem"], g["batch"])
    assert got == g["expected_bytes"] == 2 ** 31
    got16 = oracle.kv_cache_bytes(g["layers"], g["kv_heads"], g["head_dim"], g["seq_len"],
                                  g["bytes_per_elem"], g["batch16"])
    assert got16 == g["batch16_expected_gib"] * 2 ** 30


def test_kv_size_matches_paged_pool_layout():
    # 4096 tokens in 16-token blocks, 32 layers, K and V pools of
    # [blocks][32 heads][16][128] fp16 each: the pool bytes equal the formula.
    blocks = 4096 // BS
    pool_bytes = 32 * 2 * blocks * 32 * BS * 128 * 2
    assert pool_bytes == oracle.kv_cache_bytes(32, 32, 128, 4096, 2, 1)


@pytest.mark.parametrize("lens,Hq,Hkv,D", [
    ([1, 16, 17, 40], 4, 2, 64),
    ([100, 33, 5], 8, 8, 32),      # MHA
    ([64, 80], 8, 1, 16),          # MQA
    ([31, 48, 1, 97], 8, 2, 128),
])
def test_decode_matches_contiguous_bruteforce(lens, Hq, Hkv, D):
    rng = np.random.default_rng(sum(lens) + Hq)
    d = tiny_paged(rng, lens, Hq, Hkv, D)
    scale = np.float32(1 / math.sqrt(D))
    got = _dec(d, Hkv, scale)
    for s, L in enumerate(d["lens"]):
        k = contiguous(d["k"], d["tables"], s, L).astype(np.float64)
        v = contiguous(d["v"], d["tables"], s, L).astype(np.float64)
        ref = brute_attention(d["q"][s].astype(np.float64), k, v, float(scale))
        np.testing.assert_allclose(got[s], ref, rtol=0, atol=1e-12)
        # library routine: torch SDPA in float64 with grouped-query heads
        qt = torch.from_numpy(d["q"][s].astype(np.float64))[None, :, None, :]
        kt = torch.from_numpy(k.transpose(1, 0, 2).copy())[None]
        vt = torch.from_numpy(v.transpose(1, 0, 2).copy())[None]
        sd = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, scale=float(scale), enable_gqa=True)[0, :, 0, :].numpy()
        np.testing.assert_allclose(got[s], sd, rtol=0, atol=1e-12)


def test_decode_bf16_inputs_widen_exactly():
    rng = np.random.default_rng(7)
    d = tiny_paged(rng, [23, 50], 4, 2, 32, dtype="bf16")
    scale = np.float32(0.25)
    got = _dec(d, 2, scale, dtype="bf16")
    k64, v64, q64 = as_f64(d["k"], "bf16"), as_f64(d["v"], "bf16"), as_f64(d["q"], "bf16")
    for s, L in enumerate(d["lens"]):
        ref = brute_attention(q64[s], contiguous(k64, d["tables"], s, L),
                              contiguous(v64, d["tables"], s, L), float(scale))
        np.testing.assert_allclose(got[s], ref, rtol=0, atol=1e-12)


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(1)
    d = tiny_paged(rng, [1, 1], 4, 2, 16)
    got = _dec(d, 2, np.float32(0.3))
    for s in range(2):
        b = d["tables"][s, 0]
        for h in range(4):
            assert np.array_equal(got[s, h], d["v"][b, h // 2, 0].astype(np.float64))


def test_equal_keys_give_mean_of_values_and_zero_query_uniform():
    rng = np.random.default_rng(2)
    d = tiny_paged(rng, [37], 2, 1, 16)
    # zero query: every logit is 0, weights uniform
    d0 = dict(d, q=np.zeros_like(d["q"]))
    got = _dec(d0, 1, np.float32(1.0))
    v = contiguous(d["v"], d["tables"], 0, 37).astype(np.float64)
    np.testing.assert_allclose(got[0, 0], v[:, 0].mean(0), rtol=0, atol=1e-14)
    # identical keys at every position: same uniform average
    k = d["k"].copy()
    k[:] = d["k"][0, 0, 0]
    got = _dec(dict(d, k=k), 1, np.float32(0.7))
    np.testing.assert_allclose(got[0, 1], v[:, 0].mean(0), rtol=0, atol=1e-14)


def test_dominant_logit_selects_that_token():
    rng = np.random.default_rng(3)
    d = tiny_paged(rng, [45], 1, 1, 8)
    q = np.zeros_like(d["q"])
    q[0, 0, 0] = 1.0
    k = np.zeros_like(d["k"])
    t = 29
    b = d["tables"][0, t // BS]
    k[b, 0, t % BS, 0] = 1000.0
    got = _dec(dict(d, q=q, k=k), 1, np.float32(1.0))
    assert np.array_equal(got[0, 0], d["v"][b, 0, t % BS].astype(np.float64))


def test_gqa_equals_mha_with_replicated_kv_heads():
    rng = np.random.default_rng(4)
    Hq, Hkv = 8, 2
    G = Hq // Hkv
    d = tiny_paged(rng, [20, 70, 3], Hq, Hkv, 32)
    scale = np.float32(0.2)
    gqa = _dec(d, Hkv, scale)
    krep = np.repeat(d["k"], G, axis=1)
    vrep = np.repeat(d["v"], G, axis=1)
    mha = _dec(dict(d, k=krep, v=vrep), Hq, scale)
    assert np.array_equal(gqa, mha)
    # the other head-to-group map (h % Hkv) gives a different answer
    kalt = np.tile(d["k"], (1, G, 1, 1))
    valt = np.tile(d["v"], (1, G, 1, 1))
    alt = _dec(dict(d, k=kalt, v=valt), Hq, scale)
    assert not np.allclose(gqa, alt)


def test_block_permutation_invariance_bit_exact():
    rng = np.random.default_rng(5)
    d = tiny_paged(rng, [18, 64, 77, 5], 4, 2, 32, extra_cols=0)
    scale = np.float32(0.17)
    base = _dec(d, 2, scale)
    NB = d["NB"]
    pi = rng.permutation(NB)           # physical block b moves to pi[b]
    k2 = np.empty_like(d["k"])
    v2 = np.empty_like(d["v"])
    k2[pi] = d["k"]
    v2[pi] = d["v"]
    t2 = pi[d["tables"]].astype(np.int32)
    got = _dec(dict(d, k=k2, v=v2, tables=t2), 2, scale)
    assert np.array_equal(base, got)


def test_unused_slots_and_table_entries_are_ignored():
    rng = np.random.default_rng(6)
    d = tiny_paged(rng, [18, 35, 64], 4, 2, 32, extra_cols=3)
    scale = np.float32(0.17)
    base = _dec(d, 2, scale)
    k, v, tables = d["k"].copy(), d["v"].copy(), d["tables"].copy()
    used = np.zeros(d["NB"], dtype=bool)
    for s, L in enumerate(d["lens"]):
        n = -(-int(L) // BS)
        used[tables[s, :n]] = True
        last = tables[s, n - 1]
        off = int(L) - (n - 1) * BS
        k[last, :, off:, :] = np.nan
        v[last, :, off:, :] = np.nan
    free = np.flatnonzero(~used)
    k[free] = np.nan
    v[free] = np.nan
    for s, L in enumerate(d["lens"]):
        n = -(-int(L) // BS)
        tables[s, n:] = rng.choice(free, size=tables.shape[1] - n)
    got = _dec(dict(d, k=k, v=v, tables=tables), 2, scale)
    assert np.array_equal(base, got)


def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(8)
    d = tiny_paged(rng, [300, 17], 4, 2, 16)
    ones = np.ones_like(d["v"])
    got = _dec(dict(d, v=ones), 2, np.float32(3.0))
    np.testing.assert_allclose(got, 1.0, rtol=0, atol=1e-15)


def test_zero_length_gives_zero_row():
    rng = np.random.default_rng(9)
    d = tiny_paged(rng, [0, 5], 2, 1, 8)
    got = _dec(d, 1, np.float32(1.0))
    assert np.array_equal(got[0], np.zeros((2, 8)))
    assert np.isfinite(got[1]).all()


@pytest.mark.parametrize("part", [16, 32, 48, 512])
def test_split_context_identity(part):
    rng = np.random.default_rng(10 + part)
    d = tiny_paged(rng, [1, 15, 16, 17, 100, 300, 0], 8, 2, 32)
    # stress the softmax range: every 64th key x8, as in the long-context workload
    for s, L in enumerate(d["lens"]):
        for t in range(63, int(L), 64):
            d["k"][d["tables"][s, t // BS], :, t % BS, :] *= 8
    scale = np.float32(1 / math.sqrt(32))
    full = _dec(d, 2, scale)
    m, l, o = oracle.decode_partials(d["q"], "f32", d["k"], d["v"], "f32", d["tables"], d["lens"],
                                     scale, part)
    comb = oracle.combine_partials(m, l, o)
    np.testing.assert_allclose(comb, full, rtol=0, atol=1e-12)


def test_shared_prefix_partials_identical():
    # two sequences share the first 4 physical blocks and have equal queries
    rng = np.random.default_rng(11)
    d = tiny_paged(rng, [64 + 20, 64 + 33, 64], 4, 2, 16, NB=40)
    t = d["tables"]
    t[1, :4] = t[0, :4]
    t[2, :4] = t[0, :4]
    d["q"][1] = d["q"][0]
    d["q"][2] = d["q"][0]
    scale = np.float32(0.25)
    m, l, o = oracle.decode_partials(d["q"], "f32", d["k"], d["v"], "f32", t, d["lens"], scale, 64)
    assert np.array_equal(m[0, :, 0], m[1, :, 0]) and np.array_equal(m[0, :, 0], m[2, :, 0])
    assert np.array_equal(l[0, :, 0], l[1, :, 0]) and np.array_equal(o[0, :, 0], o[1, :, 0])
    # the prefix-only sequence equals the prefix partition's output
    full = _dec(dict(d, tables=t), 2, scale)
    assert np.array_equal(full[2], o[2, :, 0])


def test_quantized_decode_is_attention_over_dequantized_values():
    rng = np.random.default_rng(12)
    d = tiny_paged(rng, [40, 19], 8, 2, 32, dtype="bf16", q_dtype="bf16")
    scale = np.float32(1 / math.sqrt(32))
    for qd in ("i8", "fp8"):
        kc, ks = oracle.quantize(d["k"], "bf16", qd)
        vc, vs = oracle.quantize(d["v"], "bf16", qd)
        got = oracle.decode(d["q"], "bf16", kc, vc, qd, d["tables"], d["lens"], scale,
                            k_scale=ks, v_scale=vs)
        if qd == "i8":
            kf, vf = kc.astype(np.float64), vc.astype(np.float64)
        else:
            kf = torch.from_numpy(kc).view(torch.float8_e4m3fn).double().numpy()
            vf = torch.from_numpy(vc).view(torch.float8_e4m3fn).double().numpy()
        kf = kf * ks.astype(np.float64)[:, :, None, None]
        vf = vf * vs.astype(np.float64)[:, :, None, None]
        q64 = as_f64(d["q"], "bf16")
        for s, L in enumerate(d["lens"]):
            ref = brute_attention(q64[s], contiguous(kf, d["tables"], s, L),
                                  contiguous(vf, d["tables"], s, L), float(scale))
            np.testing.assert_allclose(got[s], ref, rtol=0, atol=1e-12)


def test_decode_rows_matches_full():
    rng = np.random.default_rng(13)
    d = tiny_paged(rng, [30, 70], 4, 2, 16)
    full = _dec(d, 2, np.float32(0.5))
    rows = np.array([0, 3, 5, 7])
    got = oracle.decode_rows(d["q"], "f32", d["k"], d["v"], "f32", d["tables"], d["lens"],
                             np.float32(0.5), rows)
    assert np.array_equal(got, full.reshape(-1, 16)[rows])
