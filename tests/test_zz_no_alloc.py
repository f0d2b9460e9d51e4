"""The allocation-free decode step (pkv_decode_step_noalloc, through the C
ABI) against pkv_decode_step with a caller workspace: identical outputs and
pool bytes, and the oracle's tolerance, on two calls in a row, the second
with a smaller input (the scratch array keeps the first call's partials)."""
import sys

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_434_amd as pkv
from paged_kv_cache_434_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2, "u8z": 2e-2}


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _qcache_u8z(NB, Hkv, D):
    mk = lambda shape, dt: torch.empty(shape, dtype=dt, device="cuda")
    return pkv.PagedCache.from_blocks(mk((NB, 2, Hkv, 16, D), torch.uint8), "u8z",
                                      mk((NB, Hkv, 16), torch.float32),
                                      mk((NB, Hkv, 16), torch.float32),
                                      mk((NB, Hkv, 16), torch.uint8), mk((NB, Hkv, 16), torch.uint8))


def _one(wl, part, u8z=False):
    """(noalloc output, decode_step output, noalloc pool, decode_step pool)."""
    outs, pools = [], []
    for noalloc in (True, False):
        d = W.to_device(wl, layout="blocks")
        cache = pkv.PagedCache(d["k_pool"], d["v_pool"], wl.kv_dtype)
        if u8z:
            qc = _qcache_u8z(wl.num_blocks, wl.Hkv, wl.D)
            pkv.quantize(cache, qc)
            cache = qc
        out = torch.empty((wl.B, wl.Hq, wl.D), dtype=torch.float32, device="cuda")
        fn = pkv.decode_step_noalloc if noalloc else pkv.decode_step
        fn(cache, d["q"], d["k_new"], d["v_new"], d["tables"], d["lens"], float(wl.scale),
           partition_tokens=part, out=out)
        torch.cuda.synchronize()
        outs.append(out.cpu())
        pools.append(W.from_device(cache.k_cache).copy())
        pools.append(W.from_device(cache.v_cache).copy())
    return outs, pools


def _ref(wl, u8z=False):
    k, v = wl.k_pool.copy(), wl.v_pool.copy()
    slots = oracle.slot_mapping(wl.tables, wl.lens)
    if u8z:
        kc, ks, kz = oracle.quantize_asym(k, wl.kv_dtype)
        vc, vs, vz = oracle.quantize_asym(v, wl.kv_dtype)
        oracle.cache_write_quant(kc, vc, ks, vs, kz, vz, wl.k_new, wl.v_new, wl.kv_dtype, slots)
        return oracle.decode(wl.q, wl.q_dtype, kc, vc, "u8z", wl.tables, wl.lens, wl.scale,
                             k_scale=ks, v_scale=vs, k_zero=kz, v_zero=vz)
    oracle.cache_write(k, v, wl.kv_dtype, wl.k_new, wl.v_new, slots)
    return oracle.decode(wl.q, wl.q_dtype, k, v, wl.kv_dtype, wl.tables, wl.lens, wl.scale)


@pytest.mark.parametrize("part", [-1, 256])
def test_noalloc_step_equals_workspace_step_twice(part):
    """The Llama-3-8B step (20.2 MB of partials with the balanced split), then
    a smaller step on the same scratch array."""
    for i, wl in enumerate((W.make(2), W.make(2, B=9, lo=1, hi=700, pool=600))):
        _say(f"noalloc call {i}: {wl.name} B={wl.B} part={part}")
        (a, b), pools = _one(wl, part)
        assert torch.equal(a, b), f"call {i}: outputs differ from pkv_decode_step"
        assert np.array_equal(pools[0], pools[2]) and np.array_equal(pools[1], pools[3])
        err = float(np.max(np.abs(a.numpy().astype(np.float64) - _ref(wl))))
        _say(f"  max abs err vs oracle {err:.3e}")
        assert err <= TOL["bf16"]


def test_noalloc_step_per_row_uint8_pool():
    """A per-row uint8 pool (its append is a launch of its own), two calls."""
    for i, wl in enumerate((W.make(2, B=20, lo=1, hi=2000, pool=3000),
                            W.make(2, B=5, lo=1, hi=300, pool=200))):
        _say(f"noalloc u8z call {i}: B={wl.B}")
        (a, b), pools = _one(wl, -1, u8z=True)
        assert torch.equal(a, b)
        assert np.array_equal(pools[0], pools[2]) and np.array_equal(pools[1], pools[3])
        err = float(np.max(np.abs(a.numpy().astype(np.float64) - _ref(wl, u8z=True))))
        _say(f"  max abs err vs oracle {err:.3e}")
        assert err <= TOL["u8z"]


def test_noalloc_rejects_a_split_beyond_the_scratch_array():
    """The 70B shape with the balanced split needs ~277 MB of partials: the
    call returns PKV_ERR_WORKSPACE and launches nothing (out stays as it was)."""
    B, Hq, Hkv, D, maxb = 256, 64, 8, 128, 512
    assert pkv.decode_workspace_bytes(B, Hq, D, maxb, -1) > pkv.NOALLOC_MAX_WORKSPACE
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    kn = torch.zeros((B, Hkv, D), dtype=torch.bfloat16, device="cuda")
    pool = torch.zeros((4, 2, Hkv, 16, D), dtype=torch.bfloat16, device="cuda")
    cache = pkv.PagedCache.from_blocks(pool, "bf16")
    tables = torch.zeros((B, maxb), dtype=torch.int32, device="cuda")
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    out = torch.full((B, Hq, D), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(pkv.PkvError) as e:
        pkv.decode_step_noalloc(cache, q, kn, kn, tables, lens, 0.1, partition_tokens=-1,
                                out=out)
    assert e.value.status == 5
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
