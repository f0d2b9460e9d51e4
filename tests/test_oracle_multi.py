"""Oracle pins for several query tokens per sequence (vLLM deep-dive page,
"投机解码": the target model verifies k drafted tokens in one pass; each query
token sees the context up to and including its own position)."""
import numpy as np
import pytest
import torch

import oracle
from helpers import BS, as_f64, contiguous, tiny_paged


def _causal_ref(q64, k64, v64, scale, L, ntok):
    """numpy: the last ntok positions of a contiguous sequence, causal mask."""
    Hq = q64.shape[1]
    _, Hkv, D = k64.shape
    G = Hq // Hkv
    out = np.zeros((ntok, Hq, D))
    for i in range(ntok):
        p = L - ntok + i
        if p < 0:
            continue
        for h in range(Hq):
            s = scale * (k64[:p + 1, h // G, :] @ q64[i, h])
            w = np.exp(s - s.max())
            out[i, h] = (w[:, None] * v64[:p + 1, h // G, :]).sum(0) / w.sum()
    return out


@pytest.mark.parametrize("ntok,Hq,Hkv,D", [(1, 4, 2, 64), (3, 4, 2, 64), (4, 8, 2, 64),
                                          (2, 8, 8, 128), (7, 6, 3, 64)])
def test_multi_matches_contiguous_causal_bruteforce(ntok, Hq, Hkv, D):
    rng = np.random.default_rng(ntok * 10 + Hq)
    lens = [ntok, 5, 16, 17, 40, 2]
    t = tiny_paged(rng, lens, Hq, Hkv, D)
    q = rng.standard_normal((len(lens), ntok, Hq, D)).astype(np.float32)
    scale = np.float32(1 / np.sqrt(D))
    got = oracle.decode_multi(q, "f32", t["k"], t["v"], "f32", t["tables"], t["lens"], scale)
    for s, L in enumerate(lens):
        ref = _causal_ref(as_f64(q[s], "f32"), as_f64(contiguous(t["k"], t["tables"], s, L), "f32"),
                          as_f64(contiguous(t["v"], t["tables"], s, L), "f32"), float(scale),
                          L, ntok)
        assert np.max(np.abs(got[s] - ref)) < 1e-12


def test_multi_matches_torch_sdpa_with_causal_mask():
    rng = np.random.default_rng(3)
    ntok, Hq, Hkv, D, L = 5, 8, 2, 64, 70
    t = tiny_paged(rng, [L], Hq, Hkv, D)
    q = rng.standard_normal((1, ntok, Hq, D)).astype(np.float32)
    got = oracle.decode_multi(q, "f32", t["k"], t["v"], "f32", t["tables"], t["lens"], 0.125)
    K = torch.from_numpy(as_f64(contiguous(t["k"], t["tables"], 0, L), "f32")).permute(1, 0, 2)
    V = torch.from_numpy(as_f64(contiguous(t["v"], t["tables"], 0, L), "f32")).permute(1, 0, 2)
    Q = torch.from_numpy(q[0].astype(np.float64)).permute(1, 0, 2)          # [Hq][ntok][D]
    pos = torch.arange(L - ntok, L)[:, None]
    mask = torch.arange(L)[None, :] <= pos                                    # [ntok][L]
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q[None], K[None], V[None], attn_mask=mask, scale=0.125, enable_gqa=True)[0]
    assert np.max(np.abs(got[0] - ref.permute(1, 0, 2).numpy())) < 1e-12


def test_multi_with_one_token_is_decode():
    rng = np.random.default_rng(4)
    t = tiny_paged(rng, [1, 30, 64, 0], 4, 2, 64)
    q = rng.standard_normal((4, 4, 64)).astype(np.float32)
    dec = oracle.decode(q, "f32", t["k"], t["v"], "f32", t["tables"], t["lens"], 0.125)
    mul = oracle.decode_multi(q[:, None], "f32", t["k"], t["v"], "f32", t["tables"], t["lens"],
                              0.125)
    assert np.array_equal(mul[:, 0], dec)


def test_query_token_i_is_decode_of_the_prefix_ending_at_it():
    """Query token i of a sequence of length L is exactly single-token decode
    over the first L - ntok + i + 1 tokens."""
    rng = np.random.default_rng(8)
    ntok, lens = 4, [9, 33, 50]
    t = tiny_paged(rng, lens, 4, 2, 64)
    q = rng.standard_normal((3, ntok, 4, 64)).astype(np.float32)
    mul = oracle.decode_multi(q, "f32", t["k"], t["v"], "f32", t["tables"], t["lens"], 0.125)
    for i in range(ntok):
        li = np.array(lens, np.int32) - ntok + i + 1
        dec = oracle.decode(q[:, i], "f32", t["k"], t["v"], "f32", t["tables"], li, 0.125)
        assert np.array_equal(mul[:, i], dec)


def test_query_tokens_before_the_start_get_zero_rows():
    rng = np.random.default_rng(9)
    t = tiny_paged(rng, [2, 0], 2, 1, 64)
    q = rng.standard_normal((2, 4, 2, 64)).astype(np.float32)
    mul = oracle.decode_multi(q, "f32", t["k"], t["v"], "f32", t["tables"], t["lens"], 0.125)
    assert np.all(mul[0, :2] == 0) and np.all(mul[1] == 0)
    assert np.all(np.abs(mul[0, 2:]).sum(-1) > 0)


def test_slot_mapping_tokens():
    rng = np.random.default_rng(10)
    t = tiny_paged(rng, [3, 17, 40, 0], 2, 1, 64)
    slots = oracle.slot_mapping_tokens(t["tables"], t["lens"], 4)
    for s, L in enumerate(t["lens"]):
        for i in range(4):
            p = int(L) - 4 + i
            want = -1 if p < 0 else int(t["tables"][s, p // BS]) * BS + p % BS
            assert slots[s, i] == want
    assert np.array_equal(oracle.slot_mapping_tokens(t["tables"], t["lens"], 1)[:, 0],
                          oracle.slot_mapping(t["tables"], t["lens"]))
