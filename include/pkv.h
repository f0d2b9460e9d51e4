/*
 * pkv -- paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes; no C++ or framework types.  Device
 * pointers are HIP device memory owned by the caller; the library never
 * allocates, frees or retains memory between calls.  `stream` is a
 * hipStream_t passed as void* (NULL = the default stream); every call only
 * enqueues work on it and returns without synchronising.  Calls on one
 * stream run in order, so a cache write followed by attention on the same
 * stream sees the written token.
 *
 * Errors.  Every entry point checks its arguments on the host before it
 * touches the GPU and returns a status; it never aborts or throws.  Values
 * that live in device memory (block ids in tables, slot numbers, context
 * lengths) are not read by the host: kernels skip a block id outside
 * [0, num_blocks), a slot outside [0, num_blocks*block_size) and a length
 * outside [0, max_blocks_per_seq*block_size] instead of touching memory out
 * of range, so bad table contents give unspecified numbers, never a fault.
 * pkv_validate_tables() copies tables to the host and reports such values.
 *
 * Sources (web pages on the KV cache, cited by title and section):
 *   [KVC]  "LLM 推理优化深度解析：KV Cache、Continuous Batching、PagedAttention
 *          与量化，从原理到 vLLM 实战": "KV Cache 的本质" (each decode step
 *          appends the new token's K/V; size formula), "MQA 与 GQA" (query
 *          heads share KV heads), "PagedAttention：vLLM 的显存碎片治理"
 *          (16-token blocks; block table maps logical to physical blocks;
 *          shared blocks for common prefixes).
 *   [CSDN] the ascendai.csdn.net article on PagedAttention and KV quantization
 *          (its text carries no title): section 二 "核心突破：PagedAttention与
 *          虚拟内存" (copy-on-write of shared blocks), section 三 "进阶优化：KV
 *          Cache量化与压缩" (INT8, FP8 and FP4 KV).
 *   [WIKI] "KV Cache 与 PagedAttention": "三个直接推论" (GQA, KV quantization,
 *          sliding windows and paging as the ways to save KV bytes).
 *   [MGMT] "大模型推理的KV Cache管理从内存碎片到前缀缓存的优化实战": section
 *          二 (KVCacheBlock stores [heads][block_size][head_dim]; append_slot
 *          takes logical block token_idx // block_size; allocation failure is
 *          a return value), section 四 (KV stored as 8-bit codes, restored as
 *          code * scale; KVQuantizationCache: asymmetric uint8 codes with a
 *          scale and a zero point per (head, token) row).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL                        */
  PKV_ERR_SHAPE = 2,       /* a size is negative, zero where it must not be, or
                              inconsistent (Hq % Hkv, block_size != 16, ...)   */
  PKV_ERR_DTYPE = 3,       /* unknown dtype code or unsupported dtype pairing   */
  PKV_ERR_RANGE = 4,       /* a value read by pkv_validate_tables is out of range */
  PKV_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required        */
  PKV_ERR_UNSUPPORTED = 6, /* valid request outside what this build implements  */
  PKV_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed        */
};

/* Element types. */
enum {
  PKV_F32 = 0,      /* IEEE binary32                                            */
  PKV_BF16 = 1,     /* bfloat16 (upper half of binary32)                        */
  PKV_I8 = 2,       /* int8 code, value = code * scale                          */
  PKV_FP8_E4M3 = 3, /* OCP E4M3 "fn" code (bias 7, max 448, no inf), value = decoded * scale */
  PKV_U8_ZP = 4,    /* uint8 code with a binary32 scale and a uint8 zero point per
                       (block, KV head, row): value = (code - zero) * scale */
  PKV_FP4_E2M1 = 5  /* OCP E2M1 4-bit code (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and
                       negatives), two per byte, element 2i in the low nibble of
                       byte i of its row: value = decoded * scale */
};

#define PKV_BLOCK_SIZE 16

/* partition_tokens value selecting the balanced split (see
 * pkv_attention_decode). */
#define PKV_SPLIT_BALANCED (-1)

/* A paged KV pool for one layer.
 *   K of block b, KV head g, row t, element d is
 *     k_cache[b * block_stride + (g * block_size + t) * head_dim + d]
 *   and V the same from v_cache: within a block, one KV head's
 *   [block_size][head_dim] tile is contiguous (4 KiB for bf16 x 16 x 128) and the
 *   heads follow one another, the per-block layout of [MGMT] section 二
 *   (KVCacheBlock: [heads][block_size][head_dim]).
 *   block_stride: elements from one block to the next; 0 means
 *     num_kv_heads * block_size * head_dim, i.e. K and V in two separate
 *     dense pools [num_blocks][num_kv_heads][block_size][head_dim].  With one
 *     allocation [num_blocks][2][num_kv_heads][block_size][head_dim] (a block
 *     holds every head's K, then every head's V, as KVCacheBlock does), pass
 *     k_cache = base, v_cache = base + num_kv_heads * block_size * head_dim
 *     and block_stride = 2 * num_kv_heads * block_size * head_dim; that
 *     layout reads fastest on MI355X (the eight heads' K and V of one block
 *     are one contiguous run).  Must be 0 or at least num_kv_heads *
 *     block_size * head_dim, even, with its size in bytes a multiple of 16;
 *     the K and V regions of all blocks must not overlap.  Element offsets
 *     of PKV_FP4_E2M1 pools are halved to give byte offsets (and k_cache /
 *     v_cache point at bytes).
 *   k_scale, v_scale: [num_blocks][num_kv_heads] binary32 scales, required for
 *     PKV_I8 / PKV_FP8_E4M3 / PKV_FP4_E2M1; for PKV_U8_ZP
 *     [num_blocks][num_kv_heads][block_size]
 *     (one per row); ignored for float pools.
 *   k_zero, v_zero: [num_blocks][num_kv_heads][block_size] uint8 zero points,
 *     required for PKV_U8_ZP and ignored otherwise.  Scales and zero points are
 *     dense arrays whatever block_stride is.
 * block_size must be 16 ([KVC] "PagedAttention"); head_dim must be 64 or 128;
 * num_blocks at most INT32_MAX / 16, since slots (block * 16 + row) are
 * int32 (PKV_ERR_SHAPE otherwise). */
typedef struct pkv_cache_t {
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t head_dim;
  int32_t kv_dtype;
  void* k_cache;
  void* v_cache;
  float* k_scale;
  float* v_scale;
  int64_t block_stride;
  uint8_t* k_zero;
  uint8_t* v_zero;
} pkv_cache_t;

/* Human-readable text for a status code (static storage). */
const char* pkv_strerror(int status);

/* Library version as major*10000 + minor*100 + patch. */
int pkv_version(void);

/* Bytes of one of the two pools (K or V) for the given geometry and dtype:
 * num_blocks * num_kv_heads * block_size * head_dim * element size.  Returns
 * 0 for an unknown dtype or a negative size. */
uint64_t pkv_pool_bytes(int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                        int32_t head_dim, int32_t dtype);

/* Slot mapping ([MGMT] section 二, append_slot): for each sequence s with
 * context_lens[s] > 0, slot_mapping[s] = block_tables[s][t / 16] * 16 + t % 16
 * for its newest position t = context_lens[s] - 1; sequences with length 0
 * (or a length past the table) get -1.
 *   block_tables: device int32 [num_seqs][max_blocks_per_seq]
 *   context_lens: device int32 [num_seqs]
 *   slot_mapping: device int32 [num_seqs], written. */
int pkv_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t num_seqs, int32_t* slot_mapping,
                     void* stream);

/* Slot mapping for several new tokens per sequence: slot_mapping[s][i] is
 * the slot of position t = context_lens[s] - tokens_per_seq + i (i <
 * tokens_per_seq), or -1 when t < 0 or the length is past the table.  With
 * tokens_per_seq = 1 this is pkv_slot_mapping.
 *   slot_mapping: device int32 [num_seqs][tokens_per_seq], written. */
int pkv_slot_mapping_tokens(const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t tokens_per_seq,
                            int32_t* slot_mapping, void* stream);

/* Cache write ([KVC] "KV Cache 的本质": each decode step appends the new
 * token's K and V): for i < n with slot = slot_mapping[i] >= 0, copies the
 * bytes of k[i][g][:] and v[i][g][:] into row slot % 16 of block slot / 16,
 * KV head g, for every g.  Bit-exact copy.
 *   k, v: device [n][num_kv_heads][head_dim] of cache->kv_dtype
 *   slot_mapping: device int32 [n]; negative = skip; slots must be distinct.
 * kv_dtype must be PKV_F32 or PKV_BF16 (quantized pools take
 * pkv_cache_write_quant, which quantizes the new rows). */
int pkv_cache_write(const pkv_cache_t* cache, const void* k, const void* v,
                    const int32_t* slot_mapping, int32_t n, void* stream);

/* Quantized append ([KVC] "KV Cache 的本质": each step appends the new token's
 * K and V) into a quantized pool.  For i < n with slot = slot_mapping[i] in
 * range, each KV head's row k[i][g][:] (and v[i][g][:]) goes to row
 * r = slot % 16 of block slot / 16:
 *   PKV_U8_ZP ([MGMT] section 四, KVQuantizationCache with per-channel
 *     parameters, restored as (code - zero) * scale): the row is quantized on
 *     its own over its range widened to hold 0,
 *       lo = min(min x, 0), hi = max(max x, 0), scale = (hi - lo) / 255,
 *       zero = clamp(rint(-lo / scale), 0, 255),
 *       code = clamp(rint(x / scale) + zero, 0, 255),
 *     so every value restores within half a step; an all-zero row is stored
 *     as scale 0, zero 0, codes 0.  Its scale and zero point go to the same
 *     row of k_scale / k_zero (v_scale / v_zero); no other row changes.
 *     Bit-exact with pkv_quantize of the same values.
 *   PKV_I8, PKV_FP8_E4M3, PKV_FP4_E2M1 ([MGMT] section 四, codes restored as
 *     code * scale with one scale per (block, KV head) tile): the tile's
 *     scale covers the rows written so far.  With a = max |x| of the new row
 *     and c = a / Q (Q = 127, 448, 6): at r == 0 the tile starts afresh,
 *     scale = c (its old contents are ignored); at r > 0, if c exceeds the
 *     tile's scale s_old the scale grows to c and every earlier row's code
 *     becomes encode(decode(code) * s_old / c), otherwise it stays; the new
 *     row's codes are encode(x / scale) (zero codes when the scale is 0).
 *     encode is clamp(rint(.), -127, 127) for INT8 and the nearest code
 *     (ties to even, saturating) for E4M3 and E2M1.  Rows after r are left
 *     alone.  Filling a tile in position order ends with the scale
 *     pkv_quantize gives the whole tile.  The slots of one call must lie in
 *     distinct blocks (rows of one tile share its scale): append several
 *     rows of one block in successive calls, in position order.
 * Every step is a binary32 operation rounding to nearest even.
 *   cache: kv_dtype PKV_U8_ZP, PKV_I8, PKV_FP8_E4M3 or PKV_FP4_E2M1
 *   k, v: device [n][num_kv_heads][head_dim] of src_dtype (PKV_F32 or PKV_BF16)
 *   slot_mapping: device int32 [n]; negative = skip; slots must be distinct. */
int pkv_cache_write_quant(const pkv_cache_t* cache, const void* k, const void* v,
                          int32_t src_dtype, const int32_t* slot_mapping, int32_t n,
                          void* stream);

/* Workspace bytes pkv_attention_decode / pkv_decode_step need for the given
 * split.  The pages describe no split of a context; this is the standard
 * partition-and-reduce of softmax attention (each partition of a long context
 * leaves a partial maximum, sum and output, and a second pass combines them
 * with the log-sum-exp rule, which equals the unsplit softmax up to
 * rounding).  Per (sequence, query head) and partial slot
 * a running maximum, a sum and a head_dim output row, all binary32, plus one
 * int32 per sequence, each part 256-byte aligned.  Fixed split
 * (partition_tokens > 0, a multiple of 16): one slot per partition; returns 0
 * when one partition covers max_blocks_per_seq * 16 tokens or
 * partition_tokens == 0 (no workspace needed).  Balanced split
 * (PKV_SPLIT_BALANCED, also for pkv_attention_prefix): ceil(max_blocks_per_seq
 * / 16) + 3 slots (a range holds at least 16 blocks, so a run of n blocks
 * meets at most ceil((n - 1) / 16) + 1 ranges, and a shared prefix cuts a
 * sequence's blocks into two runs).
 * Returns 0 for invalid sizes. */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t partition_tokens);

/* The split this library recommends for the given geometry: always
 * PKV_SPLIT_BALANCED (one generation of wavefronts with even shares of the
 * blocks), or 0 for invalid sizes. */
int32_t pkv_decode_default_partition(int32_t num_seqs, int32_t num_kv_heads,
                                     int32_t max_blocks_per_seq);

/* Paged decode attention ([KVC] "PagedAttention", "MQA 与 GQA"):
 *   out[s][h] = sum_{t < L} softmax_t(scale * q[s][h] . k_t) v_t,
 *   L = context_lens[s], k_t / v_t at (block_tables[s][t / 16], h / G, t % 16),
 *   G = num_q_heads / num_kv_heads; L == 0 gives a zero row.
 *   q: device [num_seqs][num_q_heads][head_dim] of q_dtype
 *   block_tables: device int32 [num_seqs][max_blocks_per_seq]; entries past
 *     ceil(L / 16) are never read
 *   context_lens: device int32 [num_seqs], 0 <= L <= max_blocks_per_seq * 16
 *   partition_tokens: how the context is split over wavefronts.
 *     0: one pass per (sequence, KV head), no split.
 *     a positive multiple of 16 (fixed split): the context is cut into
 *       partitions of that many tokens, each gives a partial (max, sum,
 *       output) and a second kernel combines them with the log-sum-exp rule.
 *     PKV_SPLIT_BALANCED: for each KV head the blocks of all sequences, laid
 *       end to end, are cut into equal ranges, one per wavefront of a grid
 *       that fills the GPU once (at least 16 blocks per range; each
 *       sequence start counts as 4 more blocks when ranges stay above 16;
 *       for bf16 pools, pairs of ranges one sixteenth larger and smaller,
 *       the larger on the even XCDs, which run faster); pieces of a sequence
 *       are combined as above.  With the fixed split, results are
 *       reproducible for given inputs; with the balanced split they are
 *       reproducible for given inputs and GPU model (the ranges depend on the
 *       compute-unit count).
 *   workspace: device memory of at least pkv_decode_workspace_bytes(...) when
 *     that is nonzero (contents need not be initialised), else may be NULL
 *   out: device [num_seqs][num_q_heads][head_dim] of out_dtype.
 * Supported (q_dtype, kv_dtype): (F32, F32), (BF16, BF16), (BF16, I8),
 * (BF16, FP8_E4M3), (BF16, U8_ZP), (BF16, FP4_E2M1); out_dtype F32 or BF16
 * (bf16 rounded to nearest even).  Quantized pools are restored as
 * code * scale (I8, FP8_E4M3, FP4_E2M1) or (code - zero) * scale (U8_ZP) on the
 * fly; rows past L are never used, so
 * their codes and parameters may hold anything. */
int pkv_attention_decode(const pkv_cache_t* cache, const void* q, int32_t q_dtype,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                         float scale, int32_t partition_tokens, void* workspace,
                         size_t workspace_bytes, void* out, int32_t out_dtype, void* stream);

/* One decode step for one layer, in a single attention launch: appends each
 * sequence's new token at position t = context_lens[s] - 1 (slot
 * block_tables[s][t / 16] * 16 + t % 16, [MGMT] section 二 append_slot) and
 * then computes the same attention as pkv_attention_decode, with the new
 * token included.  Equivalent to pkv_slot_mapping + pkv_cache_write +
 * pkv_attention_decode, and leaves the pool in the same state.
 *   k, v: device [num_seqs][num_kv_heads][head_dim] of cache->kv_dtype (the
 *     new token of each sequence; ignored for sequences with length 0)
 * For quantized pools (PKV_U8_ZP, PKV_I8, PKV_FP8_E4M3, PKV_FP4_E2M1), k and
 * v are of q_dtype and are quantized as pkv_cache_write_quant does, by a
 * launch of its own before the attention.  Other arguments as for
 * pkv_attention_decode.  Tables must not map the new token's slot of two
 * sequences to the same physical row (for the per-tile formats, to the same
 * block). */
int pkv_decode_step(const pkv_cache_t* cache, const void* q, int32_t q_dtype, const void* k,
                    const void* v, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    float scale, int32_t partition_tokens, void* workspace,
                    size_t workspace_bytes, void* out, int32_t out_dtype, void* stream);

/* Paged decode attention over a shared prefix ([KVC] "意外的收获：prefix
 * sharing": requests that start with the same prompt share its KV blocks;
 * [MGMT] section 二, copy_prefix: a new request's table takes the prefix's
 * physical blocks).  The first prefix_blocks entries of every sequence's
 * block table must be the same physical blocks; the caller knows this from
 * the prefix it shared.  The result is that of pkv_attention_decode with the
 * balanced split (the same definition, up to rounding): each group of
 * 16 / G sequences (G = num_q_heads / num_kv_heads) runs the shared blocks
 * once for all its query heads, every sequence's remaining blocks run as
 * usual, and the pieces are combined.  A sequence may be shorter than the
 * prefix (positions past its length are masked) or empty.
 *   prefix_blocks: 0 <= prefix_blocks <= max_blocks_per_seq (0: no sharing)
 *   workspace: at least pkv_decode_workspace_bytes(num_seqs, num_q_heads,
 *     head_dim, max_blocks_per_seq, PKV_SPLIT_BALANCED) bytes.
 * Other arguments and dtypes as for pkv_attention_decode, except that fp32
 * pools are PKV_ERR_UNSUPPORTED here.  Tables that do not share their first
 * prefix_blocks entries give unspecified output (never a memory fault). */
int pkv_attention_prefix(const pkv_cache_t* cache, const void* q, int32_t q_dtype,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                         float scale, int32_t prefix_blocks, void* workspace,
                         size_t workspace_bytes, void* out, int32_t out_dtype, void* stream);

/* pkv_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and pool update
 * as pkv_decode_step; the split partials go to a fixed array of 32 MiB
 * (33554432 bytes) in device memory that the library holds on every GPU it
 * runs on until the process ends.  Requests whose
 * pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim,
 * max_blocks_per_seq, partition_tokens) exceeds 32 MiB return
 * PKV_ERR_WORKSPACE (the Llama-3-8B shape with 64 sequences of up to 4096
 * tokens and the balanced split needs 20.2 MB).  The call allocates nothing:
 * no hipMalloc, hipFree or allocating library routine.  All calls on one GPU
 * share that GPU's array and nothing in it needs clearing between calls;
 * calls that overlap in time on one GPU (on different streams, or from
 * different threads without ordering) race on it and give unspecified
 * results. */
int pkv_decode_step_noalloc(const pkv_cache_t* cache, const void* q, int32_t q_dtype,
                            const void* k, const void* v, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, float scale,
                            int32_t partition_tokens, void* out, int32_t out_dtype,
                            void* stream);

/* Paged attention for several query tokens per sequence ([KVC] "投机解码":
 * the large model checks k drafted tokens in one forward pass; "Continuous
 * Batching": a long prompt is fed in chunks).  The last k = tokens_per_seq of
 * the L = context_lens[s] cached tokens are the queries: query token i sits at
 * position L - k + i and attends to the tokens t <= L - k + i (causal within
 * the chunk; tokens before it and itself):
 *   out[s][i][h] = sum_{t <= L-k+i} softmax_t(scale * q[s][i][h] . k_t) v_t;
 * a query token with L - k + i < 0 gets a zero row.  Their K/V must already be
 * in the pool (pkv_slot_mapping_tokens + pkv_cache_write).
 *   q, out: device [num_seqs][tokens_per_seq][num_q_heads][head_dim]
 *   workspace: at least pkv_decode_workspace_bytes(num_seqs * tokens_per_seq,
 *     num_q_heads, head_dim, max_blocks_per_seq, partition_tokens) bytes when
 *     that is nonzero.
 * A wavefront takes the query heads of one KV head for 16 / G query tokens
 * (16 columns of the matrix cores), or with the balanced split up to 32 / G
 * tokens in two column groups over one staging of each block; more tokens run
 * in passes of 16 / G whose wavefronts read each block at the same time, so
 * its K/V comes from HBM once.  Other arguments, splits and dtypes as for
 * pkv_attention_decode, except that fp32 pools are PKV_ERR_UNSUPPORTED
 * here. */
int pkv_attention_multi(const pkv_cache_t* cache, const void* q, int32_t q_dtype,
                        int32_t tokens_per_seq, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                        int32_t num_q_heads, float scale, int32_t partition_tokens,
                        void* workspace, size_t workspace_bytes, void* out, int32_t out_dtype,
                        void* stream);

/* Sliding-window paged attention ([WIKI] "三个直接推论": attending to, and
 * keeping, only a window of the most recent tokens is one of the ways to cut
 * KV bytes).  As pkv_attention_multi, except that query token i at position
 * p = L - k + i (k = tokens_per_seq) attends only to max(0, p - window + 1)
 * <= t <= p:
 *   out[s][i][h] = sum_{p-window < t <= p} softmax_t(scale q[s][i][h] . k_t) v_t.
 * window == 0 means no window (then the call equals pkv_attention_multi);
 * negative is PKV_ERR_SHAPE.  Table entries before block
 * (L - k + 1 - window) / 16 (when that is positive) are never read, so a
 * caller may recycle the blocks that left every window; K/V rows outside
 * every query's window may hold anything (NaN included).
 *   q, out: device [num_seqs][tokens_per_seq][num_q_heads][head_dim]
 *   workspace: as for pkv_attention_multi.
 * Splits and dtypes as for pkv_attention_multi (fp32 pools are
 * PKV_ERR_UNSUPPORTED). */
int pkv_attention_window(const pkv_cache_t* cache, const void* q, int32_t q_dtype,
                         int32_t tokens_per_seq, int32_t window, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_q_heads, float scale,
                         int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                         void* out, int32_t out_dtype, void* stream);

/* KV quantization ([MGMT] section 四, with one symmetric binary32 scale per
 * (block, KV head) tile): for each listed block b and KV head g, with
 * a = max |x| over the whole 16 x head_dim tile of src (every row),
 *   PKV_I8:       scale = a / 127, code = clamp(rint(x / scale), -127, 127)
 *   PKV_FP8_E4M3: scale = a / 448, code = nearest E4M3 (ties to even), values
 *                 beyond 448 in magnitude saturate to +-448
 *   PKV_FP4_E2M1: scale = a / 6, code = nearest E2M1 (ties to the even
 *                 mantissa bit), magnitudes beyond 6 saturate to +-6 ([CSDN]
 *                 section 三: FP4 KV)
 * a == 0 gives scale 0 and zero codes; src values must be finite (the codes
 * of a tile holding NaN or infinity are unspecified).  With dst PKV_U8_ZP
 * ([MGMT] section 四,
 * KVQuantizationCache with per-channel parameters) every (block, head, row) of
 * head_dim values is quantized on its own, as pkv_cache_write_quant states,
 * and its scale and zero point go to that row of the parameter arrays.
 * Divisions and rounding are binary32, round-to-nearest-even.  Quantizes
 * src->k_cache into dst->k_cache (scales to dst->k_scale, zero points to
 * dst->k_zero) and src->v_cache into dst->v_cache (dst->v_scale, v_zero).
 *   src: kv_dtype F32 or BF16; dst: kv_dtype I8, FP8_E4M3, U8_ZP or FP4_E2M1,
 *   same geometry
 *   block_ids: device int32 [n_ids], or NULL for every block (n_ids ignored). */
int pkv_quantize(const pkv_cache_t* src, const pkv_cache_t* dst, const int32_t* block_ids,
                 int32_t n_ids, void* stream);

/* Block copy for copy-on-write ([CSDN] section 二 "写时复制": branches of a
 * beam search or of parallel sampling share their history blocks and a block
 * is copied only when a new token is written into it; [KVC] "意外的收获：prefix
 * sharing": shared blocks are reference-counted and copied on write).  For
 * each i < n with (src, dst) = (pairs[2i], pairs[2i+1]): every KV head's K and
 * V tile of block dst becomes a bit-exact copy of block src's, and for 8-bit
 * pools the block's scales (and zero points) too.
 *   pairs: device int32 [n][2]; a pair with an id outside [0, num_blocks) is
 *     skipped.  Destinations must be distinct and no destination may also be
 *     a source (the result would depend on the order of the copies).
 * The caller updates its block tables; the library keeps no reference counts. */
int pkv_copy_blocks(const pkv_cache_t* cache, const int32_t* pairs, int32_t n, void* stream);

/* Gather (diagnostic): copies each sequence's K and V, in logical order, into
 * contiguous rows k_out[cu_seqlens[s] + t][g][:] for t < context_lens[s]:
 * the logical-to-physical translation of [KVC] "PagedAttention：vLLM 的显存碎片
 * 治理" (a sequence's block table maps its logical blocks to physical ones,
 * which need not be contiguous) undone into one contiguous copy, so that a
 * test can compare a sequence's cached K/V byte for byte.  Bit-exact copy of
 * the stored elements (codes for 8- and 4-bit pools).
 *   cu_seqlens: device int32 [num_seqs + 1], cu_seqlens[s+1] = cu_seqlens[s] + L_s
 *   k_out, v_out: device [cu_seqlens[num_seqs]][num_kv_heads][head_dim]. */
int pkv_gather(const pkv_cache_t* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
               const int32_t* context_lens, const int32_t* cu_seqlens, int32_t num_seqs,
               void* k_out, void* v_out, void* stream);

/* Debug check of device tables (synchronises `stream`, copies to the host):
 * every context length in [0, max_blocks_per_seq * 16] and every used table
 * entry (index < ceil(L / 16)) in [0, num_blocks).  Returns PKV_OK or
 * PKV_ERR_RANGE; *bad_seq (if not NULL) receives the first offending
 * sequence or -1. */
int pkv_validate_tables(const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_blocks,
                        int32_t* bad_seq, void* stream);

/* Debug check of a slot list before a cache write ([MGMT] section 二: a
 * failed append is reported as a return value, not a crash).  Writes skip a
 * negative slot and one outside [0, num_blocks * 16); two entries with the
 * same slot would race (the result depends on their order), and for the
 * per-tile formats (PKV_I8, PKV_FP8_E4M3, PKV_FP4_E2M1) two entries in the
 * same block would race on the tile's scale.  Returns PKV_ERR_RANGE if an
 * entry is at or past num_blocks * 16, or repeats the slot (with
 * one_per_block != 0: the block, slot / 16) of an earlier entry; negative
 * entries are padding and pass.  *bad_index (if not NULL) receives the first
 * offending index, or -1.
 *   pkv_validate_slots: slot_mapping is device memory; the call copies it to
 *     the host and synchronises `stream`.
 *   pkv_validate_slots_host: slot_mapping is host memory (a scheduler's own
 *     copy); no HIP call. */
int pkv_validate_slots(const int32_t* slot_mapping, int32_t n, int32_t num_blocks,
                       int32_t one_per_block, int32_t* bad_index, void* stream);
int pkv_validate_slots_host(const int32_t* slot_mapping, int32_t n, int32_t num_blocks,
                            int32_t one_per_block, int32_t* bad_index);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
