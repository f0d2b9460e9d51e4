"""pkv: paged KV-cache decode attention for AMD MI355X (gfx950).

Thin Python binding over the C ABI in ``include/pkv.h`` (``libpkv.so``, built
in-tree by ``paged_kv_cache_434_amd.build``).  Functions take torch tensors
that already live on the GPU and only marshal pointers, sizes and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing or a call fails, an exception
is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY names another build of the same library (e.g. one whose host
# code is compiled with sanitizers)
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(_HERE, "libpkv.so")

PKV_OK = 0
SPLIT_BALANCED = -1     # partition_tokens value: balanced split (PKV_SPLIT_BALANCED)
DTYPE_CODES = {"f32": 0, "bf16": 1, "i8": 2, "fp8": 3, "u8z": 4, "fp4": 5}
BLOCK_SIZE = 16
QUANTIZED = ("i8", "fp8", "u8z", "fp4")

_lib = None


class PkvError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _load().pkv_strerror(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed with status {status}: {msg}")


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("block_stride", ctypes.c_int64),
        ("k_zero", ctypes.c_void_p),
        ("v_zero", ctypes.c_void_p),
    ]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run "
                              "`python -m paged_kv_cache_434_amd.build` first")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        C = ctypes.POINTER(CacheDesc)
        sig = {
            "pkv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
            "pkv_version": (ctypes.c_int, []),
            "pkv_pool_bytes": (ctypes.c_uint64, [I32, I32, I32, I32, I32]),
            "pkv_slot_mapping": (ctypes.c_int, [P, I32, P, I32, P, P]),
            "pkv_slot_mapping_tokens": (ctypes.c_int, [P, I32, P, I32, I32, P, P]),
            "pkv_cache_write": (ctypes.c_int, [C, P, P, P, I32, P]),
            "pkv_cache_write_quant": (ctypes.c_int, [C, P, P, I32, P, I32, P]),
            "pkv_decode_workspace_bytes": (ctypes.c_size_t, [I32, I32, I32, I32, I32]),
            "pkv_decode_default_partition": (I32, [I32, I32, I32]),
            "pkv_attention_decode": (ctypes.c_int, [C, P, I32, P, I32, P, I32, I32, F, I32, P,
                                                    ctypes.c_size_t, P, I32, P]),
            "pkv_decode_step": (ctypes.c_int, [C, P, I32, P, P, P, I32, P, I32, I32, F, I32, P,
                                               ctypes.c_size_t, P, I32, P]),
            "pkv_attention_prefix": (ctypes.c_int, [C, P, I32, P, I32, P, I32, I32, F, I32, P,
                                                    ctypes.c_size_t, P, I32, P]),
            "pkv_decode_step_noalloc": (ctypes.c_int, [C, P, I32, P, P, P, I32, P, I32, I32, F,
                                                       I32, P, I32, P]),
            "pkv_attention_multi": (ctypes.c_int, [C, P, I32, I32, P, I32, P, I32, I32, F, I32, P,
                                                   ctypes.c_size_t, P, I32, P]),
            "pkv_attention_window": (ctypes.c_int, [C, P, I32, I32, I32, P, I32, P, I32, I32, F,
                                                    I32, P, ctypes.c_size_t, P, I32, P]),
            "pkv_quantize": (ctypes.c_int, [C, C, P, I32, P]),
            "pkv_gather": (ctypes.c_int, [C, P, I32, P, P, I32, P, P, P]),
            "pkv_copy_blocks": (ctypes.c_int, [C, P, I32, P]),
            "pkv_validate_tables": (ctypes.c_int, [P, I32, P, I32, I32,
                                                   ctypes.POINTER(I32), P]),
            "pkv_validate_slots": (ctypes.c_int, [P, I32, I32, I32, ctypes.POINTER(I32), P]),
            "pkv_validate_slots_host": (ctypes.c_int, [P, I32, I32, I32, ctypes.POINTER(I32)]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def lib():
    """The loaded ctypes library (raises ImportError if it is not built)."""
    return _load()


EXPORTED_SYMBOLS = ("pkv_strerror", "pkv_version", "pkv_pool_bytes", "pkv_slot_mapping",
                    "pkv_slot_mapping_tokens", "pkv_attention_multi", "pkv_attention_window",
                    "pkv_cache_write", "pkv_cache_write_quant", "pkv_decode_workspace_bytes",
                    "pkv_decode_default_partition", "pkv_attention_decode", "pkv_decode_step",
                    "pkv_decode_step_noalloc", "pkv_attention_prefix",
                    "pkv_quantize", "pkv_copy_blocks",
                    "pkv_gather", "pkv_validate_tables", "pkv_validate_slots",
                    "pkv_validate_slots_host")


def _check(fn: str, status: int):
    if status != PKV_OK:
        raise PkvError(fn, status)


def _torch():
    import torch
    return torch


def _storage_dtype(name: str):
    torch = _torch()
    return {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8,
            "fp8": torch.uint8, "u8z": torch.uint8, "fp4": torch.uint8}[name]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t, name, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims")


class PagedCache:
    """One layer's K and V pools and, for quantized pools, their binary32 scales:
    [num_blocks][Hkv] for ``i8`` / ``fp8`` / ``fp4``, [num_blocks][Hkv][16] plus
    uint8 zero points of the same shape for ``u8z`` (the asymmetric per-row
    format).  ``k_cache`` / ``v_cache`` are [num_blocks][Hkv][16][D] tensors
    ([num_blocks][Hkv][16][D/2] uint8 for ``fp4``, two codes per byte) whose
    last three dimensions are dense; the block dimension may be strided, so both
    separate dense pools and the two halves of one [num_blocks][2][Hkv][16][D]
    allocation (see ``from_blocks``) are accepted.  Holds references so the
    tensors outlive the descriptor."""

    def __init__(self, k_cache, v_cache, kv_dtype: str, k_scale=None, v_scale=None,
                 k_zero=None, v_zero=None):
        torch = _torch()
        sd = _storage_dtype(kv_dtype)
        if kv_dtype == "fp8" and k_cache.dtype == torch.float8_e4m3fn:
            k_cache, v_cache = k_cache.view(torch.uint8), v_cache.view(torch.uint8)
        for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
            if not isinstance(t, torch.Tensor) or not t.is_cuda:
                raise TypeError(f"{name} must be a CUDA (HIP) tensor")
            if t.dtype != sd:
                raise TypeError(f"{name} has dtype {t.dtype}, expected {sd}")
            if t.dim() != 4:
                raise ValueError(f"{name} must have 4 dims")
            _, H, bs, D = t.shape
            if tuple(t.stride()[1:]) != (bs * D, D, 1):
                raise ValueError(f"{name}: the last three dimensions must be dense")
        if k_cache.shape != v_cache.shape or k_cache.stride() != v_cache.stride():
            raise ValueError("k_cache and v_cache shapes or strides differ")
        NB, Hkv, bs, D = k_cache.shape
        if kv_dtype == "fp4":
            D *= 2
        if kv_dtype in ("i8", "fp8", "fp4"):
            _need(k_scale, "k_scale", torch.float32, 2)
            _need(v_scale, "v_scale", torch.float32, 2)
            if tuple(k_scale.shape) != (NB, Hkv) or k_scale.shape != v_scale.shape:
                raise ValueError("k_scale/v_scale must be [num_blocks][num_kv_heads]")
        if kv_dtype == "u8z":
            for name, t, dt in (("k_scale", k_scale, torch.float32),
                                ("v_scale", v_scale, torch.float32),
                                ("k_zero", k_zero, torch.uint8), ("v_zero", v_zero, torch.uint8)):
                _need(t, name, dt, 3)
                if tuple(t.shape) != (NB, Hkv, bs):
                    raise ValueError(f"{name} must be [num_blocks][num_kv_heads][block_size]")
        else:
            k_zero = v_zero = None
        stride = int(k_cache.stride(0)) * (2 if kv_dtype == "fp4" else 1)   # in elements
        self.block_stride = 0 if stride == Hkv * bs * D else stride
        self.k_cache, self.v_cache, self.k_scale, self.v_scale = k_cache, v_cache, k_scale, v_scale
        self.k_zero, self.v_zero = k_zero, v_zero
        self.kv_dtype = kv_dtype
        self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim = NB, Hkv, bs, D
        self.desc = CacheDesc(NB, Hkv, bs, D, DTYPE_CODES[kv_dtype], k_cache.data_ptr(),
                              v_cache.data_ptr(), _ptr(k_scale), _ptr(v_scale), self.block_stride,
                              _ptr(k_zero), _ptr(v_zero))

    @classmethod
    def from_blocks(cls, kv, kv_dtype: str, k_scale=None, v_scale=None, k_zero=None,
                    v_zero=None):
        """A pool held as one [num_blocks][2][Hkv][16][D] tensor: each block
        holds every head's K, then every head's V."""
        torch = _torch()
        if kv_dtype == "fp8" and kv.dtype == torch.float8_e4m3fn:
            kv = kv.view(torch.uint8)
        _need(kv, "kv", _storage_dtype(kv_dtype), 5)
        if kv.shape[1] != 2:
            raise ValueError("kv must be [num_blocks][2][num_kv_heads][block_size][head_dim]")
        return cls(kv[:, 0], kv[:, 1], kv_dtype, k_scale, v_scale, k_zero, v_zero)


def pool_bytes(num_blocks, num_kv_heads, head_dim, dtype, block_size=BLOCK_SIZE) -> int:
    return int(_load().pkv_pool_bytes(num_blocks, num_kv_heads, block_size, head_dim,
                                      DTYPE_CODES[dtype]))


def slot_mapping(block_tables, context_lens, out=None, stream=None):
    torch = _torch()
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    B = context_lens.shape[0]
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=context_lens.device)
    _need(out, "slot_mapping", torch.int32, 1)
    _check("pkv_slot_mapping",
           _load().pkv_slot_mapping(_ptr(block_tables), block_tables.shape[1],
                                    _ptr(context_lens), B, _ptr(out), _stream(stream)))
    return out


def slot_mapping_tokens(block_tables, context_lens, tokens_per_seq: int, out=None, stream=None):
    """Slots of the last tokens_per_seq positions of every sequence, [B][k]."""
    torch = _torch()
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    B = context_lens.shape[0]
    if out is None:
        out = torch.empty((B, tokens_per_seq), dtype=torch.int32, device=context_lens.device)
    _need(out, "slot_mapping", torch.int32, 2)
    _check("pkv_slot_mapping_tokens",
           _load().pkv_slot_mapping_tokens(_ptr(block_tables), block_tables.shape[1],
                                           _ptr(context_lens), B, tokens_per_seq, _ptr(out),
                                           _stream(stream)))
    return out


def cache_write(cache: PagedCache, k, v, slot_mapping, stream=None):
    torch = _torch()
    sd = _storage_dtype(cache.kv_dtype)
    _need(k, "k", sd, 3)
    _need(v, "v", sd, 3)
    _need(slot_mapping, "slot_mapping", torch.int32, 1)
    n = slot_mapping.shape[0]
    if tuple(k.shape) != (n, cache.num_kv_heads, cache.head_dim) or k.shape != v.shape:
        raise ValueError("k/v must be [n][num_kv_heads][head_dim]")
    _same_device(k, (("v", v), ("slot_mapping", slot_mapping)) + _cache_tensors(cache))
    _check("pkv_cache_write",
           _load().pkv_cache_write(ctypes.byref(cache.desc), _ptr(k), _ptr(v),
                                   _ptr(slot_mapping), n, _stream(stream)))


def cache_write_quant(cache: PagedCache, k, v, slot_mapping, stream=None):
    """Quantized append into a quantized pool: the new (token, head) rows of k
    and v (float32 or bfloat16 [n][Hkv][D]) are quantized and stored at their
    slots.  ``u8z``: each row gets its own scale and zero point.  ``i8`` /
    ``fp8`` / ``fp4``: the row joins its tile, whose scale grows (and whose
    earlier rows are re-encoded) when the row needs it; the slots of one call
    must lie in distinct blocks."""
    torch = _torch()
    sd = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(k.dtype)
    if sd is None:
        raise TypeError("k must be float32 or bfloat16")
    _need(k, "k", k.dtype, 3)
    _need(v, "v", k.dtype, 3)
    _need(slot_mapping, "slot_mapping", torch.int32, 1)
    n = slot_mapping.shape[0]
    if tuple(k.shape) != (n, cache.num_kv_heads, cache.head_dim) or k.shape != v.shape:
        raise ValueError("k/v must be [n][num_kv_heads][head_dim]")
    _same_device(k, (("v", v), ("slot_mapping", slot_mapping)) + _cache_tensors(cache))
    _check("pkv_cache_write_quant",
           _load().pkv_cache_write_quant(ctypes.byref(cache.desc), _ptr(k), _ptr(v),
                                         DTYPE_CODES[sd], _ptr(slot_mapping), n,
                                         _stream(stream)))


def decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                           partition_tokens) -> int:
    return int(_load().pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim,
                                                  max_blocks_per_seq, partition_tokens))


def default_partition(num_seqs, num_kv_heads, max_blocks_per_seq) -> int:
    return int(_load().pkv_decode_default_partition(num_seqs, num_kv_heads, max_blocks_per_seq))


def alloc_workspace(num_seqs, num_q_heads, head_dim, max_blocks_per_seq, partition_tokens,
                    device="cuda"):
    torch = _torch()
    nbytes = decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_blocks_per_seq,
                                    partition_tokens)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def _check_query_out(cache, q, out, tensors, lead):
    """Shape and device checks of a decode-family call, made before any
    pointer is taken: q is [*lead][Hq][head_dim] with the pool's head_dim and
    Hq a multiple of its KV heads, out (if given) has q's shape, and every
    other tensor lives on q's device.  The kernels index q, out and the
    workspace with the pool's head_dim, so a mismatch here would otherwise
    read or write out of bounds."""
    if q.dim() != len(lead) + 2:
        raise ValueError(f"q must have {len(lead) + 2} dims")
    Hq, D = q.shape[-2], q.shape[-1]
    if D != cache.head_dim:
        raise ValueError(f"q has head_dim {D}, the pool {cache.head_dim}")
    if Hq % cache.num_kv_heads != 0:
        raise ValueError(f"{Hq} query heads are not a multiple of {cache.num_kv_heads} KV heads")
    if tuple(q.shape[:-2]) != tuple(lead):
        raise ValueError(f"q's leading dims {tuple(q.shape[:-2])} differ from {tuple(lead)}")
    if out is not None and tuple(out.shape) != tuple(q.shape):
        raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(q.shape)}")
    for name, t in tuple(tensors) + _cache_tensors(cache):
        if t is not None and t.device != q.device:
            raise ValueError(f"{name} is on {t.device}, q on {q.device}")


def _cache_tensors(cache):
    names = ("k_cache", "v_cache", "k_scale", "v_scale", "k_zero", "v_zero")
    return tuple((n, getattr(cache, n, None)) for n in names)


def _same_device(ref, tensors):
    for name, t in tensors:
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


def _decode_call(cache: PagedCache, q, block_tables, context_lens, scale: float,
                 partition_tokens: int, workspace, out, out_dtype, stream, append):
    """Checks and marshals one decode call; returns (name, function, args, out,
    workspace) so the call can be made now or kept and repeated."""
    torch = _torch()
    qd = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(q.dtype)
    if qd is None:
        raise TypeError("q must be float32 or bfloat16")
    if q.dim() != 3:
        raise ValueError("q must be [num_seqs][num_q_heads][head_dim]")
    B, Hq, D = q.shape
    _check_query_out(cache, q, out, (("block_tables", block_tables),
                                     ("context_lens", context_lens), ("out", out),
                                     ("workspace", workspace),
                                     ("k_new", None if append is None else append[0]),
                                     ("v_new", None if append is None else append[1])), (B,))
    _need(q, "q", None, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    if context_lens.shape[0] != B or block_tables.shape[0] != B:
        raise ValueError("q, block_tables and context_lens disagree on the batch size")
    if append is not None:
        # new rows for a quantized pool come in q's dtype and are quantized on append
        sd = q.dtype if cache.kv_dtype in QUANTIZED else _storage_dtype(cache.kv_dtype)
        k_new, v_new = append
        _need(k_new, "k_new", sd, 3)
        _need(v_new, "v_new", sd, 3)
        if (tuple(k_new.shape) != (B, cache.num_kv_heads, cache.head_dim)
                or k_new.shape != v_new.shape):
            raise ValueError("k_new/v_new must be [num_seqs][num_kv_heads][head_dim]")
    od = out_dtype or (out.dtype if out is not None else q.dtype)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=od, device=q.device)
    _need(out, "out", od, 3)
    odn = {torch.float32: "f32", torch.bfloat16: "bf16"}[od]
    maxb = block_tables.shape[1]
    ws_need = decode_workspace_bytes(B, Hq, D, maxb, partition_tokens)
    if ws_need and workspace is None:
        workspace = alloc_workspace(B, Hq, D, maxb, partition_tokens, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    common = (_ptr(block_tables), maxb, _ptr(context_lens), B, Hq, ctypes.c_float(scale),
              partition_tokens, _ptr(workspace), ws_bytes, _ptr(out), DTYPE_CODES[odn],
              _stream(stream))
    lib = _load()
    if append is None:
        return ("pkv_attention_decode", lib.pkv_attention_decode,
                (ctypes.byref(cache.desc), _ptr(q), DTYPE_CODES[qd]) + common, out, workspace)
    return ("pkv_decode_step", lib.pkv_decode_step,
            (ctypes.byref(cache.desc), _ptr(q), DTYPE_CODES[qd], _ptr(append[0]),
             _ptr(append[1])) + common, out, workspace)


def attention_decode(cache: PagedCache, q, block_tables, context_lens, scale: float,
                     partition_tokens: int = 0, workspace=None, out=None, out_dtype=None,
                     stream=None):
    """out[s][h] = softmax(scale q k^T) v over each sequence's paged context."""
    name, fn, args, out, _ = _decode_call(cache, q, block_tables, context_lens, scale,
                                          partition_tokens, workspace, out, out_dtype, stream,
                                          None)
    _check(name, fn(*args))
    return out


def decode_step(cache: PagedCache, q, k_new, v_new, block_tables, context_lens, scale: float,
                partition_tokens: int = 0, workspace=None, out=None, out_dtype=None,
                stream=None):
    """Append each sequence's new token at position context_lens - 1, then
    attention over the whole context.  For bf16 pools the append is part of
    the attention launch; quantized pools append in a launch of their own
    first (k_new / v_new then come in q's dtype)."""
    name, fn, args, out, _ = _decode_call(cache, q, block_tables, context_lens, scale,
                                          partition_tokens, workspace, out, out_dtype, stream,
                                          (k_new, v_new))
    _check(name, fn(*args))
    return out


def prepare_attention_prefix(cache: PagedCache, q, block_tables, context_lens, scale: float,
                             prefix_blocks: int, workspace=None, out=None, out_dtype=None,
                             stream=None):
    """attention_prefix, prepared: returns (PreparedCall, out)."""
    name, fn, args, out, ws = _decode_call(cache, q, block_tables, context_lens, scale,
                                           SPLIT_BALANCED, workspace, out, out_dtype, stream,
                                           None)
    if int(prefix_blocks) < 0 or int(prefix_blocks) > block_tables.shape[1]:
        raise ValueError("prefix_blocks must lie in [0, max_blocks_per_seq]")
    # pkv_attention_decode's arguments with prefix_blocks in place of the split
    assert len(args) == 15
    args = args[:9] + (int(prefix_blocks),) + args[10:]
    keep = (cache, q, block_tables, context_lens, ws, out)
    return PreparedCall("pkv_attention_prefix", _load().pkv_attention_prefix, args, keep), out


def attention_prefix(cache: PagedCache, q, block_tables, context_lens, scale: float,
                     prefix_blocks: int, workspace=None, out=None, out_dtype=None, stream=None):
    """Decode attention whose sequences share their first ``prefix_blocks``
    table entries (a common prompt): the shared blocks run once per group of
    16 / G sequences.  Same result as attention_decode."""
    call, out = prepare_attention_prefix(cache, q, block_tables, context_lens, scale,
                                         prefix_blocks, workspace, out, out_dtype, stream)
    call()
    return out


NOALLOC_MAX_WORKSPACE = 32 << 20   # bytes of the library's fixed scratch array


def decode_step_noalloc(cache: PagedCache, q, k_new, v_new, block_tables, context_lens,
                        scale: float, partition_tokens: int = 0, out=None, out_dtype=None,
                        stream=None):
    """decode_step through pkv_decode_step_noalloc: the split partials go to the
    library's fixed per-GPU scratch array instead of a workspace, so nothing
    is allocated beyond ``out`` (pass ``out`` to allocate nothing at all).
    Calls that overlap in time on one GPU race on that array."""
    name, fn, args, out, _ = _decode_call(cache, q, block_tables, context_lens, scale, 0,
                                          None, out, out_dtype, stream, (k_new, v_new))
    # pkv_decode_step's arguments (desc, q, q dtype, k, v, tables, max blocks,
    # lens, B, Hq, scale | partition, workspace, bytes | out, out dtype,
    # stream) without the workspace and its size
    assert len(args) == 17
    args = args[:11] + (partition_tokens,) + args[14:]
    _check("pkv_decode_step_noalloc", _load().pkv_decode_step_noalloc(*args))
    return out


def attention_multi(cache: PagedCache, q, block_tables, context_lens, scale: float,
                    partition_tokens: int = 0, workspace=None, out=None, out_dtype=None,
                    stream=None, window: Optional[int] = None):
    """Several query tokens per sequence (q [B][k][Hq][D]); query token i of a
    sequence of length L attends to the tokens up to position L - k + i (with
    ``window``, only to the window most recent of them)."""
    torch = _torch()
    qd = {torch.float32: "f32", torch.bfloat16: "bf16"}.get(q.dtype)
    if qd is None:
        raise TypeError("q must be float32 or bfloat16")
    if q.dim() != 4:
        raise ValueError("q must be [num_seqs][tokens_per_seq][num_q_heads][head_dim]")
    B, k, Hq, D = q.shape
    _check_query_out(cache, q, out, (("block_tables", block_tables),
                                     ("context_lens", context_lens), ("out", out),
                                     ("workspace", workspace)), (B, k))
    _need(q, "q", None, 4)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    if context_lens.shape[0] != B or block_tables.shape[0] != B:
        raise ValueError("q, block_tables and context_lens disagree on the batch size")
    od = out_dtype or (out.dtype if out is not None else q.dtype)
    if out is None:
        out = torch.empty((B, k, Hq, D), dtype=od, device=q.device)
    _need(out, "out", od, 4)
    odn = {torch.float32: "f32", torch.bfloat16: "bf16"}[od]
    maxb = block_tables.shape[1]
    if decode_workspace_bytes(B * k, Hq, D, maxb, partition_tokens) and workspace is None:
        workspace = alloc_workspace(B * k, Hq, D, maxb, partition_tokens, q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rest = (_ptr(block_tables), maxb, _ptr(context_lens), B, Hq, ctypes.c_float(scale),
            partition_tokens, _ptr(workspace), ws_bytes, _ptr(out), DTYPE_CODES[odn],
            _stream(stream))
    if window is None:
        _check("pkv_attention_multi",
               _load().pkv_attention_multi(ctypes.byref(cache.desc), _ptr(q), DTYPE_CODES[qd], k,
                                           *rest))
    else:
        _check("pkv_attention_window",
               _load().pkv_attention_window(ctypes.byref(cache.desc), _ptr(q), DTYPE_CODES[qd], k,
                                            int(window), *rest))
    return out


def attention_window(cache: PagedCache, q, block_tables, context_lens, scale: float,
                     window: int, partition_tokens: int = 0, workspace=None, out=None,
                     out_dtype=None, stream=None):
    """Sliding-window attention: q [B][k][Hq][D] (k = 1 for decode); query
    token i at position p = L - k + i sees positions p - window < t <= p;
    window 0: no window."""
    return attention_multi(cache, q, block_tables, context_lens, scale, partition_tokens,
                           workspace, out, out_dtype, stream, window=window)


class PreparedCall:
    """A decode call whose arguments were checked and marshalled once; calling
    it launches the same work again on the same stream with the tensors given
    at preparation (which it keeps alive).  For loops that repeat one call
    shape: the per-call host cost is one foreign-function call."""

    def __init__(self, name, fn, args, keep):
        self.name, self._fn, self._args, self._keep = name, fn, args, keep

    def __call__(self):
        status = self._fn(*self._args)
        if status != PKV_OK:
            raise PkvError(self.name, status)


def prepare_decode_step(cache: PagedCache, q, k_new, v_new, block_tables, context_lens,
                        scale: float, partition_tokens: int = 0, workspace=None, out=None,
                        out_dtype=None, stream=None):
    """decode_step, prepared: returns (PreparedCall, out)."""
    name, fn, args, out, ws = _decode_call(cache, q, block_tables, context_lens, scale,
                                           partition_tokens, workspace, out, out_dtype, stream,
                                           (k_new, v_new))
    keep = (cache, q, k_new, v_new, block_tables, context_lens, ws, out)
    return PreparedCall(name, fn, args, keep), out


def prepare_attention_decode(cache: PagedCache, q, block_tables, context_lens, scale: float,
                             partition_tokens: int = 0, workspace=None, out=None,
                             out_dtype=None, stream=None):
    """attention_decode, prepared: returns (PreparedCall, out)."""
    name, fn, args, out, ws = _decode_call(cache, q, block_tables, context_lens, scale,
                                           partition_tokens, workspace, out, out_dtype, stream,
                                           None)
    keep = (cache, q, block_tables, context_lens, ws, out)
    return PreparedCall(name, fn, args, keep), out


def quantize(src: PagedCache, dst: PagedCache, block_ids=None, stream=None):
    torch = _torch()
    n = 0
    if block_ids is not None:
        _need(block_ids, "block_ids", torch.int32, 1)
        n = block_ids.shape[0]
    _same_device(src.k_cache, _cache_tensors(src) + _cache_tensors(dst) +
                 (("block_ids", block_ids),))
    _check("pkv_quantize",
           _load().pkv_quantize(ctypes.byref(src.desc), ctypes.byref(dst.desc), _ptr(block_ids),
                                n, _stream(stream)))


def copy_blocks(cache: PagedCache, pairs, stream=None):
    """Copy-on-write block copies: pairs is int32 [n][2] of (src, dst) block ids."""
    torch = _torch()
    _need(pairs, "pairs", torch.int32, 2)
    if pairs.shape[1] != 2:
        raise ValueError("pairs must be [n][2]")
    _same_device(cache.k_cache, _cache_tensors(cache) + (("pairs", pairs),))
    _check("pkv_copy_blocks",
           _load().pkv_copy_blocks(ctypes.byref(cache.desc), _ptr(pairs), pairs.shape[0],
                                   _stream(stream)))


def gather(cache: PagedCache, block_tables, context_lens, cu_seqlens, total_tokens: int,
           stream=None):
    """Each sequence's K and V in logical order into contiguous rows (codes
    for quantized pools): returns (k_out, v_out) of total_tokens rows, where
    total_tokens must be cu_seqlens[num_seqs], the prefix sum of the lengths
    (the kernel writes row cu_seqlens[s] + t)."""
    torch = _torch()
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1)
    B = context_lens.shape[0]
    if block_tables.shape[0] != B or cu_seqlens.shape[0] != B + 1:
        raise ValueError("block_tables must have num_seqs rows and cu_seqlens num_seqs + 1 entries")
    _same_device(cache.k_cache, _cache_tensors(cache) + (
        ("block_tables", block_tables), ("context_lens", context_lens),
        ("cu_seqlens", cu_seqlens)))
    shape = (total_tokens, cache.num_kv_heads, cache.k_cache.shape[3])
    ko = torch.empty(shape, dtype=cache.k_cache.dtype, device=cache.k_cache.device)
    vo = torch.empty(shape, dtype=cache.k_cache.dtype, device=cache.k_cache.device)
    _check("pkv_gather",
           _load().pkv_gather(ctypes.byref(cache.desc), _ptr(block_tables), block_tables.shape[1],
                              _ptr(context_lens), _ptr(cu_seqlens), B, _ptr(ko), _ptr(vo),
                              _stream(stream)))
    return ko, vo


def validate_tables(block_tables, context_lens, num_blocks, stream=None):
    """Debug check (synchronises): returns (status, first bad sequence or -1)."""
    bad = ctypes.c_int32(-1)
    rc = _load().pkv_validate_tables(_ptr(block_tables), block_tables.shape[1],
                                     _ptr(context_lens), context_lens.shape[0], num_blocks,
                                     ctypes.byref(bad), _stream(stream))
    return rc, bad.value


def validate_slots(slot_mapping, num_blocks, one_per_block=False, stream=None):
    """Debug check of a slot list (device tensor: synchronises; numpy array
    or list: checked on the host): returns (status, first bad index or -1)."""
    bad = ctypes.c_int32(-1)
    torch = _torch()
    if isinstance(slot_mapping, torch.Tensor) and slot_mapping.is_cuda:
        _need(slot_mapping, "slot_mapping", torch.int32, 1)
        rc = _load().pkv_validate_slots(_ptr(slot_mapping), slot_mapping.shape[0], num_blocks,
                                        int(one_per_block), ctypes.byref(bad), _stream(stream))
    else:
        import numpy as np
        a = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int32))
        rc = _load().pkv_validate_slots_host(a.ctypes.data_as(ctypes.c_void_p), a.shape[0],
                                             num_blocks, int(one_per_block), ctypes.byref(bad))
    return rc, bad.value
