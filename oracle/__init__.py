"""CPU oracle for paged-KV decode attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports it and
the two share no code: this wrapper drives ``oracle.c`` (plain C, double
precision, built with gcc) through ctypes on numpy arrays in host memory.

Storage dtypes (numpy): ``f32`` float32, ``bf16`` uint16 bit patterns,
``i8`` int8, ``fp8`` uint8 bit patterns of OCP E4M3, ``u8z`` uint8 codes of the
asymmetric per-row format (with float32 scales and uint8 zero points
[NB][Hkv][16]), ``fp4`` OCP E2M1 codes packed two per uint8 (element 2i in the
low nibble), so an fp4 pool is [NB][Hkv][16][D/2].

Every function states the passage it follows in ``oracle.c``; the pins that
tie each one to the pages or to mathematics are in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DTYPES = {"f32": 0, "bf16": 1, "i8": 2, "fp8": 3, "u8z": 4, "fp4": 5}
NP_STORAGE = {"f32": np.float32, "bf16": np.uint16, "i8": np.int8, "fp8": np.uint8,
              "u8z": np.uint8, "fp4": np.uint8}

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
               "-shared", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        F = ctypes.c_float
        lib.orc_kv_cache_bytes.restype = ctypes.c_uint64
        lib.orc_kv_cache_bytes.argtypes = [ctypes.c_uint64] * 6
        lib.orc_bf16_to_double.restype = ctypes.c_double
        lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.orc_e4m3_to_double.restype = ctypes.c_double
        lib.orc_e4m3_to_double.argtypes = [ctypes.c_uint8]
        lib.orc_e4m3_from_float.restype = ctypes.c_uint8
        lib.orc_e4m3_from_float.argtypes = [F]
        lib.orc_e2m1_to_double.restype = ctypes.c_double
        lib.orc_e2m1_to_double.argtypes = [ctypes.c_uint8]
        lib.orc_e2m1_from_float.restype = ctypes.c_uint8
        lib.orc_e2m1_from_float.argtypes = [F]
        lib.orc_slot_of.restype = ctypes.c_int32
        lib.orc_slot_of.argtypes = [P, I, I, I, I]
        lib.orc_slot_mapping.restype = None
        lib.orc_slot_mapping.argtypes = [P, I, P, I, I, P]
        lib.orc_cache_write.restype = None
        lib.orc_cache_write.argtypes = [P, P, I, I, I, I, I, P, P, P, I]
        lib.orc_copy_blocks.restype = None
        lib.orc_copy_blocks.argtypes = [P, P, P, P, P, P, I, I, I, I, I, P, I]
        lib.orc_gather.restype = None
        lib.orc_gather.argtypes = [P, P, I, I, I, I, P, I, P, P, I, P, P]
        lib.orc_decode.restype = I
        lib.orc_decode.argtypes = [P, I, P, P, I, P, P, P, P, P, I, P, I, I, I, I, I, F, P]
        lib.orc_decode_rows.restype = I
        lib.orc_decode_rows.argtypes = [P, I, P, P, I, P, P, P, P, P, I, P, I, I, I, I, I, F, P,
                                        I, P]
        lib.orc_decode_multi.restype = I
        lib.orc_decode_multi.argtypes = [P, I, P, P, I, P, P, P, P, P, I, P, I, I, I, I, I, I, F,
                                         P]
        lib.orc_decode_window.restype = I
        lib.orc_decode_window.argtypes = [P, I, P, P, I, P, P, P, P, P, I, P, I, I, I, I, I, I,
                                          I, F, P]
        lib.orc_slot_mapping_tokens.restype = None
        lib.orc_slot_mapping_tokens.argtypes = [P, I, P, I, I, I, P]
        lib.orc_decode_partials.restype = I
        lib.orc_decode_partials.argtypes = [P, I, P, P, I, P, P, P, P, P, I, P, I, I, I, I, I, F,
                                            I, I, P, P, P]
        lib.orc_combine_partials.restype = None
        lib.orc_combine_partials.argtypes = [P, P, P, I, I, I, P]
        lib.orc_quantize.restype = I
        lib.orc_quantize.argtypes = [P, I, P, I, P, I, I, I, I, P, I]
        lib.orc_quantize_row_asym.restype = None
        lib.orc_quantize_row_asym.argtypes = [P, I, P, P, P]
        lib.orc_quantize_asym.restype = I
        lib.orc_quantize_asym.argtypes = [P, I, P, P, P, I, I, I, I, P, I]
        lib.orc_cache_write_quant.restype = I
        lib.orc_cache_write_quant.argtypes = [P, P, P, P, P, P, I, I, I, P, P, I, P, I]
        lib.orc_cache_write_sym.restype = I
        lib.orc_cache_write_sym.argtypes = [P, P, P, P, I, I, I, I, P, P, I, P, I]
        lib.orc_max_threads.restype = I
        lib.orc_max_threads.argtypes = []
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def max_threads() -> int:
    return _load().orc_max_threads()


def kv_cache_bytes(layers, kv_heads, head_dim, seq_len, bytes_per_elem, batch=1) -> int:
    """KV size formula of the page on KV Cache / vLLM (section "KV Cache 的本质")."""
    return int(_load().orc_kv_cache_bytes(layers, kv_heads, head_dim, seq_len, bytes_per_elem,
                                          batch))


def bf16_to_f64(bits) -> np.ndarray:
    f = np.vectorize(lambda b: _load().orc_bf16_to_double(int(b)), otypes=[np.float64])
    return f(np.asarray(bits, dtype=np.uint16))


def e4m3_to_f64(codes) -> np.ndarray:
    f = np.vectorize(lambda c: _load().orc_e4m3_to_double(int(c)), otypes=[np.float64])
    return f(np.asarray(codes, dtype=np.uint8))


def e4m3_from_f32(x) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.orc_e4m3_from_float(float(flat_in[i]))
    return out


def e2m1_to_f64(codes) -> np.ndarray:
    f = np.vectorize(lambda c: _load().orc_e2m1_to_double(int(c)), otypes=[np.float64])
    return f(np.asarray(codes, dtype=np.uint8))


def e2m1_from_f32(x) -> np.ndarray:
    lib = _load()
    x = np.asarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    flat_in, flat_out = x.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.orc_e2m1_from_float(float(flat_in[i]))
    return out


def pool_dims(pool, kv_dtype):
    """(num_blocks, Hkv, block_size, head_dim) of a stored pool (fp4 pools hold
    head_dim / 2 bytes per row)."""
    NB, Hkv, bs, last = pool.shape
    return NB, Hkv, bs, last * 2 if kv_dtype == "fp4" else last


def slot_mapping(block_tables, context_lens, block_size=16) -> np.ndarray:
    """Slot of each sequence's newest token (page on KV-cache management, section 二)."""
    bt = _c(block_tables, np.int32)
    lens = _c(context_lens, np.int32)
    out = np.empty(lens.shape[0], dtype=np.int32)
    _load().orc_slot_mapping(_ptr(bt), bt.shape[1], _ptr(lens), lens.shape[0], block_size,
                             _ptr(out))
    return out


def cache_write(k_cache, v_cache, dtype, k_new, v_new, slot_mapping):
    """In-place byte copy of new tokens into their slots."""
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    NB, Hkv, bs, D = k_cache.shape
    kn = _c(k_new, NP_STORAGE[dtype])
    vn = _c(v_new, NP_STORAGE[dtype])
    sm = _c(slot_mapping, np.int32)
    _load().orc_cache_write(_ptr(k_cache), _ptr(v_cache), DTYPES[dtype], NB, Hkv, bs, D,
                            _ptr(kn), _ptr(vn), _ptr(sm), sm.shape[0])


def copy_blocks(k_cache, v_cache, dtype, pairs, k_scale=None, v_scale=None, k_zero=None,
                v_zero=None):
    """In-place copy-on-write block copies (page on KV cache / PagedAttention,
    section 二, and the vLLM deep-dive page, "prefix sharing"): pairs [n][2] of
    (src, dst) physical block ids, applied in order; scales (and, for the
    asymmetric format, zero points) travel with their block."""
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    NB, Hkv, bs, D = pool_dims(k_cache, dtype)
    pr = _c(pairs, np.int32).reshape(-1, 2)
    for sc in (k_scale, v_scale):
        assert sc is None or (sc.dtype == np.float32 and sc.flags.c_contiguous)
    for zp in (k_zero, v_zero):
        assert zp is None or (zp.dtype == np.uint8 and zp.flags.c_contiguous)
    _load().orc_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                            _ptr(k_zero), _ptr(v_zero), DTYPES[dtype], NB, Hkv, bs, D, _ptr(pr),
                            pr.shape[0])


def gather(k_cache, v_cache, dtype, block_tables, context_lens):
    """Contiguous [sum L][Hkv][D] copies of each sequence's K and V."""
    NB, Hkv, bs, D = pool_dims(k_cache, dtype)
    bt = _c(block_tables, np.int32)
    lens = _c(context_lens, np.int32)
    cu = np.zeros(lens.shape[0] + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    total = int(cu[-1])
    row = k_cache.shape[3]          # stored elements (bytes for fp4) per row
    ko = np.zeros((total, Hkv, row), dtype=NP_STORAGE[dtype])
    vo = np.zeros((total, Hkv, row), dtype=NP_STORAGE[dtype])
    _load().orc_gather(_ptr(_c(k_cache, NP_STORAGE[dtype])), _ptr(_c(v_cache, NP_STORAGE[dtype])),
                       DTYPES[dtype], Hkv, bs, D, _ptr(bt), bt.shape[1], _ptr(lens), _ptr(cu),
                       lens.shape[0], _ptr(ko), _ptr(vo))
    return ko, vo, cu


def _decode_args(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, block_tables,
                 context_lens, k_zero=None, v_zero=None):
    qa = _c(q, NP_STORAGE[q_dtype])
    kc = _c(k_cache, NP_STORAGE[kv_dtype])
    vc = _c(v_cache, NP_STORAGE[kv_dtype])
    ks = None if k_scale is None else _c(k_scale, np.float32)
    vs = None if v_scale is None else _c(v_scale, np.float32)
    if kv_dtype == "u8z":
        NB, Hkv, bs, _ = kc.shape
        assert ks is not None and vs is not None and k_zero is not None and v_zero is not None
        assert ks.shape == (NB, Hkv, bs) and vs.shape == (NB, Hkv, bs)
    kz = None if k_zero is None else _c(k_zero, np.uint8)
    vz = None if v_zero is None else _c(v_zero, np.uint8)
    bt = _c(block_tables, np.int32)
    lens = _c(context_lens, np.int32)
    return qa, kc, vc, ks, vs, kz, vz, bt, lens


def decode(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens, scale,
           k_scale=None, v_scale=None, k_zero=None, v_zero=None) -> np.ndarray:
    """Plain-definition paged decode attention; float64 [B][Hq][D]."""
    qa, kc, vc, ks, vs, kz, vz, bt, lens = _decode_args(q, q_dtype, k_cache, v_cache, kv_dtype,
                                                        k_scale, v_scale, block_tables,
                                                        context_lens, k_zero, v_zero)
    B, Hq, D = qa.shape
    NB, Hkv, bs, D2 = pool_dims(kc, kv_dtype)
    assert D == D2 and Hq % Hkv == 0
    out = np.zeros((B, Hq, D), dtype=np.float64)
    rc = _load().orc_decode(_ptr(qa), DTYPES[q_dtype], _ptr(kc), _ptr(vc), DTYPES[kv_dtype],
                            _ptr(ks), _ptr(vs), _ptr(kz), _ptr(vz), _ptr(bt), bt.shape[1], _ptr(lens), B, Hq, Hkv, D,
                            bs, float(np.float32(scale)), _ptr(out))
    if rc != 0:
        raise MemoryError("oracle decode: allocation failed")
    return out


def decode_multi(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens, scale,
                 k_scale=None, v_scale=None, k_zero=None, v_zero=None) -> np.ndarray:
    """Several query tokens per sequence, each attending to the context up to
    and including its own position (vLLM deep-dive page, "投机解码"); q is
    [B][ntok][Hq][D]; float64 output of the same shape."""
    qa = _c(q, NP_STORAGE[q_dtype])
    B, ntok, Hq, D = qa.shape
    _, kc, vc, ks, vs, kz, vz, bt, lens = _decode_args(qa.reshape(B * ntok, Hq, D), q_dtype,
                                                       k_cache, v_cache, kv_dtype, k_scale,
                                                       v_scale, block_tables, context_lens,
                                                       k_zero, v_zero)
    NB, Hkv, bs, D2 = pool_dims(kc, kv_dtype)
    assert D == D2 and Hq % Hkv == 0 and lens.shape[0] == B
    out = np.zeros((B, ntok, Hq, D), dtype=np.float64)
    rc = _load().orc_decode_multi(_ptr(qa), DTYPES[q_dtype], _ptr(kc), _ptr(vc), DTYPES[kv_dtype],
                                  _ptr(ks), _ptr(vs), _ptr(kz), _ptr(vz), _ptr(bt), bt.shape[1], _ptr(lens), B, ntok,
                                  Hq, Hkv, D, bs, float(np.float32(scale)), _ptr(out))
    if rc != 0:
        raise MemoryError("oracle decode_multi: allocation failed")
    return out


def decode_window(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens, scale,
                  window, k_scale=None, v_scale=None, k_zero=None, v_zero=None) -> np.ndarray:
    """Sliding-window attention (page on KV cache and PagedAttention, "三个直接推论"):
    q [B][ntok][Hq][D]; query token i at position p = L - ntok + i attends to
    the window most recent positions up to p; window <= 0: no window.
    float64 output of q's shape."""
    qa = _c(q, NP_STORAGE[q_dtype])
    B, ntok, Hq, D = qa.shape
    _, kc, vc, ks, vs, kz, vz, bt, lens = _decode_args(qa.reshape(B * ntok, Hq, D), q_dtype,
                                                       k_cache, v_cache, kv_dtype, k_scale,
                                                       v_scale, block_tables, context_lens,
                                                       k_zero, v_zero)
    NB, Hkv, bs, D2 = pool_dims(kc, kv_dtype)
    assert D == D2 and Hq % Hkv == 0 and lens.shape[0] == B
    out = np.zeros((B, ntok, Hq, D), dtype=np.float64)
    rc = _load().orc_decode_window(_ptr(qa), DTYPES[q_dtype], _ptr(kc), _ptr(vc),
                                   DTYPES[kv_dtype], _ptr(ks), _ptr(vs), _ptr(kz), _ptr(vz),
                                   _ptr(bt), bt.shape[1], _ptr(lens), B, ntok, int(window), Hq,
                                   Hkv, D, bs, float(np.float32(scale)), _ptr(out))
    if rc != 0:
        raise MemoryError("oracle decode_window: allocation failed")
    return out


def slot_mapping_tokens(block_tables, context_lens, ntok, block_size=16) -> np.ndarray:
    """Slots of the last ntok positions of every sequence ([B][ntok], -1 for
    negative positions)."""
    bt = _c(block_tables, np.int32)
    lens = _c(context_lens, np.int32)
    out = np.empty((lens.shape[0], ntok), dtype=np.int32)
    _load().orc_slot_mapping_tokens(_ptr(bt), bt.shape[1], _ptr(lens), lens.shape[0], ntok,
                                    block_size, _ptr(out))
    return out


def decode_rows(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens, scale, rows,
                k_scale=None, v_scale=None, k_zero=None, v_zero=None) -> np.ndarray:
    """Decode only the listed rows (row = s * Hq + h); float64 [n][D]."""
    qa, kc, vc, ks, vs, kz, vz, bt, lens = _decode_args(q, q_dtype, k_cache, v_cache, kv_dtype,
                                                        k_scale, v_scale, block_tables,
                                                        context_lens, k_zero, v_zero)
    B, Hq, D = qa.shape
    NB, Hkv, bs, _ = pool_dims(kc, kv_dtype)
    r = _c(rows, np.int64)
    out = np.zeros((r.shape[0], D), dtype=np.float64)
    rc = _load().orc_decode_rows(_ptr(qa), DTYPES[q_dtype], _ptr(kc), _ptr(vc), DTYPES[kv_dtype],
                                 _ptr(ks), _ptr(vs), _ptr(kz), _ptr(vz), _ptr(bt), bt.shape[1], _ptr(lens), B, Hq,
                                 Hkv, D, bs, float(np.float32(scale)), _ptr(r), r.shape[0],
                                 _ptr(out))
    if rc != 0:
        raise MemoryError("oracle decode_rows: allocation failed")
    return out


def decode_partials(q, q_dtype, k_cache, v_cache, kv_dtype, block_tables, context_lens, scale,
                    partition_tokens, k_scale=None, v_scale=None, k_zero=None, v_zero=None):
    """Per-partition (m, l, o) of the split-context form; shapes [B][Hq][P](,D)."""
    qa, kc, vc, ks, vs, kz, vz, bt, lens = _decode_args(q, q_dtype, k_cache, v_cache, kv_dtype,
                                                        k_scale, v_scale, block_tables,
                                                        context_lens, k_zero, v_zero)
    B, Hq, D = qa.shape
    NB, Hkv, bs, _ = pool_dims(kc, kv_dtype)
    n_parts = max(1, -(-int(lens.max(initial=0)) // partition_tokens))
    m = np.zeros((B, Hq, n_parts), dtype=np.float64)
    l = np.zeros((B, Hq, n_parts), dtype=np.float64)
    o = np.zeros((B, Hq, n_parts, D), dtype=np.float64)
    rc = _load().orc_decode_partials(_ptr(qa), DTYPES[q_dtype], _ptr(kc), _ptr(vc),
                                     DTYPES[kv_dtype], _ptr(ks), _ptr(vs), _ptr(kz), _ptr(vz),
                                     _ptr(bt), bt.shape[1],
                                     _ptr(lens), B, Hq, Hkv, D, bs, float(np.float32(scale)),
                                     partition_tokens, n_parts, _ptr(m), _ptr(l), _ptr(o))
    if rc != 0:
        raise MemoryError("oracle decode_partials: allocation failed")
    return m, l, o


def combine_partials(m, l, o) -> np.ndarray:
    """Log-sum-exp combination of partition results; float64 [B][Hq][D]."""
    m = _c(m, np.float64)
    l = _c(l, np.float64)
    o = _c(o, np.float64)
    B, Hq, P, D = o.shape
    out = np.zeros((B, Hq, D), dtype=np.float64)
    _load().orc_combine_partials(_ptr(m), _ptr(l), _ptr(o), B * Hq, P, D, _ptr(out))
    return out


def quantize(src, src_dtype, dst_dtype, block_ids=None):
    """Symmetric per-(block, head) quantization of one pool; returns (codes, scales)
    (fp4 codes packed two per byte, [NB][Hkv][16][D/2])."""
    s = _c(src, NP_STORAGE[src_dtype])
    NB, Hkv, bs, D = s.shape
    codes = np.zeros((NB, Hkv, bs, D // 2 if dst_dtype == "fp4" else D),
                     dtype=NP_STORAGE[dst_dtype])
    scales = np.zeros((NB, Hkv), dtype=np.float32)
    ids = None if block_ids is None else _c(block_ids, np.int32)
    rc = _load().orc_quantize(_ptr(s), DTYPES[src_dtype], _ptr(codes), DTYPES[dst_dtype],
                              _ptr(scales), NB, Hkv, bs, D, _ptr(ids),
                              0 if ids is None else ids.shape[0])
    if rc != 0:
        raise ValueError("oracle quantize: unsupported dtype pair")
    return codes, scales


def quantize_row_asym(x):
    """One row through the asymmetric per-row quantizer of the KV-management
    page (section 四, quantize_key with per-channel parameters), in binary32;
    returns (codes uint8 [n], scale float32, zero_point uint8)."""
    xa = _c(x, np.float32).reshape(-1)
    codes = np.zeros(xa.shape[0], dtype=np.uint8)
    sc = np.zeros(1, dtype=np.float32)
    zp = np.zeros(1, dtype=np.uint8)
    _load().orc_quantize_row_asym(_ptr(xa), xa.shape[0], _ptr(codes), _ptr(sc), _ptr(zp))
    return codes, sc[0], zp[0]


def quantize_asym(src, src_dtype, block_ids=None):
    """Per-row asymmetric quantization of one pool [NB][Hkv][16][D]; returns
    (codes uint8, scales float32 [NB][Hkv][16], zero points uint8 [NB][Hkv][16]).
    Blocks not listed in block_ids keep zero codes and parameters."""
    s = _c(src, NP_STORAGE[src_dtype])
    NB, Hkv, bs, D = s.shape
    codes = np.zeros(s.shape, dtype=np.uint8)
    scales = np.zeros((NB, Hkv, bs), dtype=np.float32)
    zeros = np.zeros((NB, Hkv, bs), dtype=np.uint8)
    ids = None if block_ids is None else _c(block_ids, np.int32)
    rc = _load().orc_quantize_asym(_ptr(s), DTYPES[src_dtype], _ptr(codes), _ptr(scales),
                                   _ptr(zeros), NB, Hkv, bs, D, _ptr(ids),
                                   0 if ids is None else ids.shape[0])
    if rc != 0:
        raise ValueError("oracle quantize_asym: unsupported source dtype or allocation failure")
    return codes, scales, zeros


def cache_write_sym(k_cache, v_cache, k_scale, v_scale, dtype, k_new, v_new, src_dtype,
                    slot_mapping):
    """In-place quantized append into a pool with one symmetric scale per
    (block, KV head) tile (``i8``, ``fp8``, ``fp4``): a new row that needs a
    larger scale grows its tile's scale and re-expresses the earlier rows; a
    row at offset 0 starts a fresh tile (negative slot: skipped).  Pools are
    [NB][Hkv][16][D] codes ([NB][Hkv][16][D/2] bytes for fp4), scales [NB][Hkv]."""
    for a in (k_cache, v_cache):
        assert a.dtype == NP_STORAGE[dtype] and a.flags.c_contiguous
    for a in (k_scale, v_scale):
        assert a.dtype == np.float32 and a.flags.c_contiguous
    NB, Hkv, bs, Ds = k_cache.shape
    D = Ds * 2 if dtype == "fp4" else Ds
    kn = _c(k_new, NP_STORAGE[src_dtype])
    vn = _c(v_new, NP_STORAGE[src_dtype])
    sm = _c(slot_mapping, np.int32)
    rc = _load().orc_cache_write_sym(_ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                                     DTYPES[dtype], Hkv, bs, D, _ptr(kn), _ptr(vn),
                                     DTYPES[src_dtype], _ptr(sm), sm.shape[0])
    if rc != 0:
        raise ValueError("oracle cache_write_sym: unsupported dtype")


def cache_write_quant(k_cache, v_cache, k_scale, v_scale, k_zero, v_zero, k_new, v_new,
                      src_dtype, slot_mapping):
    """In-place quantized append into an asymmetric per-row pool: each new
    (token, head) row is quantized on its own and stored with its scale and
    zero point at its slot (negative slot: skipped)."""
    for a, dt in ((k_cache, np.uint8), (v_cache, np.uint8), (k_scale, np.float32),
                  (v_scale, np.float32), (k_zero, np.uint8), (v_zero, np.uint8)):
        assert a.dtype == dt and a.flags.c_contiguous
    NB, Hkv, bs, D = k_cache.shape
    kn = _c(k_new, NP_STORAGE[src_dtype])
    vn = _c(v_new, NP_STORAGE[src_dtype])
    sm = _c(slot_mapping, np.int32)
    rc = _load().orc_cache_write_quant(_ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                       _ptr(v_scale), _ptr(k_zero), _ptr(v_zero), Hkv, bs, D,
                                       _ptr(kn), _ptr(vn), DTYPES[src_dtype], _ptr(sm),
                                       sm.shape[0])
    if rc != 0:
        raise ValueError("oracle cache_write_quant: unsupported source dtype")
