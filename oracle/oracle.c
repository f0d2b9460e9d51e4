/*
 * CPU oracle for paged-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It is plain C, runs on
 * the host, accumulates in double precision and follows the written
 * definitions step by step, with no blocking, fusion or reordering beyond
 * what those definitions state.  It shares no code, header, table or constant
 * generator with the GPU library.
 *
 * Sources (web pages on the KV cache; cited by title and section):
 *   [KVC]  "LLM 推理优化深度解析：KV Cache、Continuous Batching、PagedAttention
 *          与量化，从原理到 vLLM 实战" -- sections "KV Cache 的本质" (the size
 *          formula and its Llama-2-7B example), "MQA 与 GQA" (query heads
 *          sharing KV heads), "PagedAttention：vLLM 的显存碎片治理" (16-token
 *          blocks, a block table mapping logical to physical blocks).
 *   [MGMT] "大模型推理的KV Cache管理从内存碎片到前缀缓存的优化实战" -- section
 *          二 (classes KVCacheBlock: one block holds [heads][block_size][dim];
 *          PagedKVCache.append_slot: logical block = token_idx // block_size),
 *          section 四 (INT8 quantization of cached K/V, dequantize = code*scale).
 *   [CSDN] the ascendai.csdn.net article on PagedAttention and KV quantization
 *          (its text carries no title): section 二 "核心突破：PagedAttention与
 *          虚拟内存" (copy-on-write of shared blocks), section 三 "进阶优化：KV
 *          Cache量化与压缩" (INT8, FP8 and FP4 KV).
 *   [WIKI] "KV Cache 与 PagedAttention" -- "KV cache 有多大" (per-token size),
 *          "三个直接推论" (GQA, KV quantization and sliding windows as byte
 *          savers).
 *
 * Readings where the pages leave a step open (each is listed in the design
 * notes): pool layout [num_blocks][num_kv_heads][block_size][head_dim]; slot =
 * physical_block*block_size + offset, negative slot = padding; query head h
 * uses KV head h / (Hq/Hkv); context_len counts the newly written token;
 * context_len 0 gives a zero output row; symmetric per-(block, head) scales
 * with fp32 arithmetic; FP8 is OCP E4M3 ("fn": no infinities, 0x7F/0xFF NaN,
 * max finite 448), round-to-nearest-even with saturation.  The asymmetric
 * per-row format (uint8 code, binary32 scale, uint8 zero point per (block,
 * head, row)) follows [MGMT] section 四's KVQuantizationCache in binary32,
 * with each row's range widened to hold 0 (so the zero point never clamps)
 * and an all-zero row stored as scale 0, zero point 0, codes 0.
 *
 * Parity pins for every function live in tests/test_oracle_*.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Element type codes understood by the oracle (its own numbering). */
enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_I8 = 2, ORC_FP8 = 3, ORC_U8Z = 4, ORC_FP4 = 5 };

/* Number of threads the parallel loops below use (1 without OpenMP).       */
int orc_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Bits of one stored element; FP4 codes are packed two to a byte, element
 * 2i in the low nibble and element 2i + 1 in the high nibble.               */
static size_t orc_elem_bits(int dtype) {
  switch (dtype) {
    case ORC_F32: return 32;
    case ORC_BF16: return 16;
    case ORC_I8: return 8;
    case ORC_FP8: return 8;
    case ORC_U8Z: return 8;
    case ORC_FP4: return 4;
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* KV-cache size.  [KVC] "KV Cache 的本质": bytes = 2 (K and V) x layers x
 * KV heads x head dim x sequence length x bytes per element x batch.        */
uint64_t orc_kv_cache_bytes(uint64_t layers, uint64_t kv_heads, uint64_t head_dim,
                            uint64_t seq_len, uint64_t bytes_per_elem, uint64_t batch) {
  return 2ull * layers * kv_heads * head_dim * seq_len * bytes_per_elem * batch;
}

/* ------------------------------------------------------------------------ */
/* Scalar conversions to double.                                             */

/* bfloat16 is the upper half of an IEEE binary32: widening appends 16 zero
 * bits, which is exact.                                                     */
double orc_bf16_to_double(uint16_t bits) {
  uint32_t w = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &w, 4);
  return (double)f;
}

/* OCP 8-bit float E4M3 ("fn" variant): 1 sign bit, 4 exponent bits with bias
 * 7, 3 mantissa bits.  Exponent field 0 encodes subnormals m/8 * 2^-6;
 * exponent field 15 with mantissa 7 encodes NaN (no infinities); every other
 * pattern is (1 + m/8) * 2^(e-7).                                           */
double orc_e4m3_to_double(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 15;
  int m = code & 7;
  double mag;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    mag = ldexp((double)m / 8.0, -6);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Encode a binary32 value as E4M3 by choosing the nearest finite value,
 * ties to the code with an even mantissa (its lowest bit clear), values above
 * the largest finite magnitude (448) clamped to it.  The positive finite codes
 * 0x00..0x7E are in increasing order of value, so the search is a binary
 * search over that ordered set.  The sign bit copies the sign of the input
 * (so small negative values become negative zero).  NaN input is outside the
 * oracle's domain and is not handled.                                       */
uint8_t orc_e4m3_from_float(float x) {
  double a = fabs((double)x);
  int sign = signbit(x) ? 1 : 0;
  int lo = 0, hi = 0x7E; /* decode(lo) <= a is kept invariant below */
  uint8_t mag;
  if (a >= orc_e4m3_to_double(0x7E)) {
    mag = 0x7E;
  } else {
    /* find the largest code c with decode(c) <= a */
    while (lo < hi) {
      int mid = (lo + hi + 1) / 2;
      if (orc_e4m3_to_double((uint8_t)mid) <= a)
        lo = mid;
      else
        hi = mid - 1;
    }
    {
      double below = orc_e4m3_to_double((uint8_t)lo);
      double above = orc_e4m3_to_double((uint8_t)(lo + 1));
      double d_below = a - below, d_above = above - a;
      if (d_below < d_above)
        mag = (uint8_t)lo;
      else if (d_above < d_below)
        mag = (uint8_t)(lo + 1);
      else
        mag = (lo & 1) ? (uint8_t)(lo + 1) : (uint8_t)lo;
    }
  }
  return (uint8_t)((sign << 7) | mag);
}

/* OCP 4-bit float E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa
 * bit; exponent field 0 encodes the subnormals m/2 (0 and 0.5), every other
 * pattern (1 + m/2) * 2^(e-1); no infinities, no NaN.  So the eight
 * magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6.                                */
double orc_e2m1_to_double(uint8_t code) {
  int sign = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return sign ? -mag : mag;
}

/* Nearest E2M1 code of x, ties to the code with an even mantissa bit,
 * magnitudes above 6 clamped to 6; the sign bit copies the sign of x.  The
 * positive codes 0..7 are in increasing order of value, so the nearest one
 * is found by scanning them.  NaN input is outside the oracle's domain.     */
uint8_t orc_e2m1_from_float(float x) {
  double a = fabs((double)x);
  int sign = signbit(x) ? 1 : 0;
  int best = 0;
  if (a >= 6.0) return (uint8_t)((sign << 3) | 7);   /* saturate */
  for (int c = 1; c < 8; ++c) {
    double dc = fabs(orc_e2m1_to_double((uint8_t)c) - a);
    double db = fabs(orc_e2m1_to_double((uint8_t)best) - a);
    if (dc < db || (dc == db && (c & 1) == 0)) best = c;
  }
  return (uint8_t)((sign << 3) | best);
}

/* Widen one stored KV element to double.  Quantized codes are multiplied by
 * their (block, head) scale, as in [MGMT] section 四 (dequantize: code times
 * scale); the product of an 8-bit code and a binary32 scale is exact in
 * double.  Asymmetric codes first lose their row's zero point ([MGMT] 四,
 * dequantize_key: (code - zero_point) * scale); the difference is an integer
 * in [-255, 255], so that product is exact in double too.                   */
static double orc_load_elem(const void* base, size_t idx, int dtype, double scale, double zero) {
  switch (dtype) {
    case ORC_F32: return (double)((const float*)base)[idx];
    case ORC_BF16: return orc_bf16_to_double(((const uint16_t*)base)[idx]);
    case ORC_I8: return (double)((const int8_t*)base)[idx] * scale;
    case ORC_FP8: return orc_e4m3_to_double(((const uint8_t*)base)[idx]) * scale;
    case ORC_U8Z: return ((double)((const uint8_t*)base)[idx] - zero) * scale;
    case ORC_FP4: {
      uint8_t byte = ((const uint8_t*)base)[idx / 2];
      return orc_e2m1_to_double((uint8_t)((idx & 1) ? byte >> 4 : byte & 15)) * scale;
    }
  }
  return NAN;
}

/* Scale and zero point of the stored row (block b, KV head g, row o): one
 * pair per (block, head) for the symmetric formats, one per row for the
 * asymmetric one, none (1, 0) for float pools.                              */
static void orc_row_params(int dtype, const float* scale, const uint8_t* zero, size_t b,
                           size_t g, size_t o, int Hkv, int bs, double* sc, double* zp) {
  *sc = 1.0;
  *zp = 0.0;
  if (dtype == ORC_U8Z) {
    size_t r = (b * (size_t)Hkv + g) * (size_t)bs + o;
    *sc = (double)scale[r];
    *zp = (double)zero[r];
  } else if (scale) {
    *sc = (double)scale[b * (size_t)Hkv + g];
  }
}

static double orc_load_q(const void* q, size_t idx, int dtype) {
  if (dtype == ORC_F32) return (double)((const float*)q)[idx];
  return orc_bf16_to_double(((const uint16_t*)q)[idx]);
}

/* Offset (in elements) of (block b, KV head g, row o, dim 0) in a pool laid
 * out as [num_blocks][num_kv_heads][block_size][head_dim]: one block holds
 * every head's [block_size][head_dim] tile, as [MGMT] section 二 stores it. */
static size_t orc_pool_offset(size_t b, size_t g, size_t o, int Hkv, int bs, int D) {
  return ((b * (size_t)Hkv + g) * (size_t)bs + o) * (size_t)D;
}

/* ------------------------------------------------------------------------ */
/* Slot of the token at logical position t of sequence s.  [MGMT] section 二,
 * PagedKVCache.append_slot: the logical block is t // block_size; the block
 * table maps it to a physical block; the row inside the block is
 * t % block_size.                                                           */
int32_t orc_slot_of(const int32_t* block_tables, int max_blocks, int s, int t, int bs) {
  int32_t phys = block_tables[(size_t)s * max_blocks + t / bs];
  return phys * bs + t % bs;
}

/* Slots for the newest token of every sequence (position context_len - 1);
 * sequences with context_len 0 get slot -1 (nothing to write).              */
void orc_slot_mapping(const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                      int num_seqs, int bs, int32_t* slots) {
  for (int s = 0; s < num_seqs; ++s)
    slots[s] = context_lens[s] > 0
                   ? orc_slot_of(block_tables, max_blocks, s, context_lens[s] - 1, bs)
                   : -1;
}

/* ------------------------------------------------------------------------ */
/* Cache write.  [KVC] "KV Cache 的本质": each decode step appends the new
 * token's K and V to the cache.  Token i goes to slot slot_mapping[i]; its
 * bytes for KV head g are copied unchanged into (slot / bs, g, slot % bs).
 * A negative slot means "no token" and is skipped.                          */
void orc_cache_write(void* k_cache, void* v_cache, int dtype, int num_blocks, int Hkv, int bs,
                     int D, const void* k_new, const void* v_new, const int32_t* slot_mapping,
                     int n) {
  size_t bits = orc_elem_bits(dtype);
  size_t row = (size_t)D * bits / 8;
  (void)num_blocks;
  for (int i = 0; i < n; ++i) {
    int32_t slot = slot_mapping[i];
    if (slot < 0) continue;
    for (int g = 0; g < Hkv; ++g) {
      size_t dst = orc_pool_offset((size_t)(slot / bs), (size_t)g, (size_t)(slot % bs), Hkv, bs, D);
      size_t src = ((size_t)i * Hkv + g) * (size_t)D;
      memcpy((char*)k_cache + dst * bits / 8, (const char*)k_new + src * bits / 8, row);
      memcpy((char*)v_cache + dst * bits / 8, (const char*)v_new + src * bits / 8, row);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Block copy for copy-on-write ([CSDN] section 二 "写时复制"; [KVC]
 * "意外的收获：prefix sharing"): a branch that shares a block with another and
 * is about to write into it first gets its own copy.  Pair i copies every
 * element of physical block src = pairs[2i] (all KV heads, K and V) into
 * block dst = pairs[2i+1], and the per-(block, head) scales when given.
 * Pairs are applied in order; ids outside [0, num_blocks) are skipped.       */
void orc_copy_blocks(void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                     uint8_t* k_zero, uint8_t* v_zero, int dtype, int num_blocks, int Hkv, int bs,
                     int D, const int32_t* pairs, int n) {
  size_t blk = (size_t)Hkv * bs * D * orc_elem_bits(dtype) / 8;
  /* parameters per block: one scale per head, or (asymmetric) one scale and
   * one zero point per (head, row)                                           */
  size_t np = dtype == ORC_U8Z ? (size_t)Hkv * bs : (size_t)Hkv;
  for (int i = 0; i < n; ++i) {
    int32_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
    memmove((char*)k_cache + (size_t)dst * blk, (const char*)k_cache + (size_t)src * blk, blk);
    memmove((char*)v_cache + (size_t)dst * blk, (const char*)v_cache + (size_t)src * blk, blk);
    for (size_t j = 0; j < np; ++j) {
      if (k_scale) k_scale[(size_t)dst * np + j] = k_scale[(size_t)src * np + j];
      if (v_scale) v_scale[(size_t)dst * np + j] = v_scale[(size_t)src * np + j];
      if (k_zero) k_zero[(size_t)dst * np + j] = k_zero[(size_t)src * np + j];
      if (v_zero) v_zero[(size_t)dst * np + j] = v_zero[(size_t)src * np + j];
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Gather: copy each sequence's K and V into logical order, giving the
 * contiguous layout the paging replaces ([KVC] "预分配的困境").  Output rows
 * are [cu_seqlens[s] + t][g][:].                                            */
void orc_gather(const void* k_cache, const void* v_cache, int dtype, int Hkv, int bs, int D,
                const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                const int32_t* cu_seqlens, int num_seqs, void* k_out, void* v_out) {
  size_t bits = orc_elem_bits(dtype);
  size_t row = (size_t)D * bits / 8;
  for (int s = 0; s < num_seqs; ++s) {
    for (int t = 0; t < context_lens[s]; ++t) {
      int32_t b = block_tables[(size_t)s * max_blocks + t / bs];
      for (int g = 0; g < Hkv; ++g) {
        size_t src = orc_pool_offset((size_t)b, (size_t)g, (size_t)(t % bs), Hkv, bs, D);
        size_t dst = ((size_t)(cu_seqlens[s] + t) * Hkv + g) * (size_t)D;
        memcpy((char*)k_out + dst * bits / 8, (const char*)k_cache + src * bits / 8, row);
        memcpy((char*)v_out + dst * bits / 8, (const char*)v_cache + src * bits / 8, row);
      }
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Attention of one query row over tokens [t0, t1) of sequence s, head h.
 * Writes the logits' maximum m, the sum l of exp(logit - m) and, into o, the
 * weighted sum of V rows divided by l.  An empty range gives m = -inf, l = 0,
 * o = 0.  Tokens are visited in logical order through the block table.      */
static void orc_attend_range(const void* q, int q_dtype, const void* k_cache,
                             const void* v_cache, int kv_dtype, const float* k_scale,
                             const float* v_scale, const uint8_t* k_zero, const uint8_t* v_zero,
                             const int32_t* block_tables, int max_blocks,
                             int s, int h, int Hq, int Hkv, int D, int bs, double scale, int t0,
                             int t1, size_t qrow, double* logits, double* m_out, double* l_out,
                             double* o_out) {
  /* [KVC] "MQA 与 GQA": Hq/Hkv query heads share one KV head; head h reads
   * KV head h / (Hq/Hkv) (contiguous groups).  qrow: element offset of the
   * query row in q.                                                          */
  int G = Hq / Hkv;
  int g = h / G;
  double m = -INFINITY, l = 0.0;
  for (int d = 0; d < D; ++d) o_out[d] = 0.0;
  if (t1 <= t0) {
    *m_out = m;
    *l_out = 0.0;
    return;
  }
  /* logits: scale * q . k_t  */
  for (int t = t0; t < t1; ++t) {
    int32_t b = block_tables[(size_t)s * max_blocks + t / bs];
    size_t base = orc_pool_offset((size_t)b, (size_t)g, (size_t)(t % bs), Hkv, bs, D);
    double ks, kz, dot = 0.0;
    orc_row_params(kv_dtype, k_scale, k_zero, (size_t)b, (size_t)g, (size_t)(t % bs), Hkv, bs,
                   &ks, &kz);
    for (int d = 0; d < D; ++d)
      dot += orc_load_q(q, qrow + d, q_dtype) *
             orc_load_elem(k_cache, base + d, kv_dtype, ks, kz);
    logits[t - t0] = scale * dot;
  }
  /* softmax with the maximum subtracted, then the weighted sum of V rows    */
  for (int t = t0; t < t1; ++t)
    if (logits[t - t0] > m) m = logits[t - t0];
  for (int t = t0; t < t1; ++t) {
    int32_t b = block_tables[(size_t)s * max_blocks + t / bs];
    size_t base = orc_pool_offset((size_t)b, (size_t)g, (size_t)(t % bs), Hkv, bs, D);
    double vs, vz, w = exp(logits[t - t0] - m);
    orc_row_params(kv_dtype, v_scale, v_zero, (size_t)b, (size_t)g, (size_t)(t % bs), Hkv, bs,
                   &vs, &vz);
    l += w;
    for (int d = 0; d < D; ++d)
      o_out[d] += w * orc_load_elem(v_cache, base + d, kv_dtype, vs, vz);
  }
  for (int d = 0; d < D; ++d) o_out[d] /= l;
  *m_out = m;
  *l_out = l;
}

/* ------------------------------------------------------------------------ */
/* Paged decode attention, the plain definition:
 *   out[s][h] = sum_{t < L_s} softmax_t(scale * q[s][h] . k_t) * v_t
 * with k_t, v_t read at (block_tables[s][t / bs], h / G, t % bs).  Paging
 * changes where the bytes live, not the result ([KVC] "PagedAttention：vLLM
 * 的显存碎片治理"; [MGMT] section 二).  context_len 0 gives a zero row.
 * out is double [num_seqs][Hq][D].  Rows (s, h) are independent; OpenMP
 * spreads them over threads without changing any row's arithmetic.         */
int orc_decode(const void* q, int q_dtype, const void* k_cache, const void* v_cache, int kv_dtype,
               const float* k_scale, const float* v_scale, const uint8_t* k_zero,
               const uint8_t* v_zero, const int32_t* block_tables, int max_blocks,
               const int32_t* context_lens, int num_seqs, int Hq, int Hkv, int D, int bs,
               float scale, double* out) {
  int max_len = 0;
  int fail = 0;
  for (int s = 0; s < num_seqs; ++s)
    if (context_lens[s] > max_len) max_len = context_lens[s];
#pragma omp parallel reduction(| : fail)
  {
    double* logits = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    if (!logits) {
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long r = 0; r < (long)num_seqs * Hq; ++r) {
        int s = (int)(r / Hq), h = (int)(r % Hq);
        double m, l;
        orc_attend_range(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, k_zero,
                         v_zero, block_tables,
                         max_blocks, s, h, Hq, Hkv, D, bs, (double)scale, 0, context_lens[s],
                         ((size_t)s * Hq + h) * (size_t)D, logits, &m, &l, out + (size_t)r * D);
      }
      free(logits);
    }
  }
  return fail ? -1 : 0;
}

/* Decode for a subset of rows: rows[i] = s * Hq + h.  out is [n_rows][D].   */
int orc_decode_rows(const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                    int kv_dtype, const float* k_scale, const float* v_scale,
                    const uint8_t* k_zero, const uint8_t* v_zero, const int32_t* block_tables,
                    int max_blocks, const int32_t* context_lens, int num_seqs, int Hq, int Hkv,
                    int D, int bs, float scale, const int64_t* rows, int n_rows, double* out) {
  int max_len = 0, fail = 0;
  for (int s = 0; s < num_seqs; ++s)
    if (context_lens[s] > max_len) max_len = context_lens[s];
#pragma omp parallel reduction(| : fail)
  {
    double* logits = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    if (!logits) {
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int i = 0; i < n_rows; ++i) {
        int s = (int)(rows[i] / Hq), h = (int)(rows[i] % Hq);
        double m, l;
        orc_attend_range(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, k_zero,
                         v_zero, block_tables,
                         max_blocks, s, h, Hq, Hkv, D, bs, (double)scale, 0, context_lens[s],
                         ((size_t)s * Hq + h) * (size_t)D, logits, &m, &l, out + (size_t)i * D);
      }
      free(logits);
    }
  }
  return fail ? -1 : 0;
}

/* ------------------------------------------------------------------------ */
/* Several query tokens per sequence ([KVC] "投机解码": the large model checks
 * k drafted tokens in one forward pass; "Continuous Batching": long prompts
 * are fed in chunks).  Sequence s has L = context_lens[s] tokens, the last
 * ntok of which are its query tokens: query token i (0 <= i < ntok) sits at
 * position p = L - ntok + i and attends to the tokens t <= p, so each query
 * sees the context before it and itself, never a later token.  q and out are
 * [num_seqs][ntok][Hq][D]; a query token with p < 0 gets a zero row.         */
int orc_decode_multi(const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                     int kv_dtype, const float* k_scale, const float* v_scale,
                     const uint8_t* k_zero, const uint8_t* v_zero, const int32_t* block_tables,
                     int max_blocks, const int32_t* context_lens, int num_seqs, int ntok, int Hq,
                     int Hkv, int D, int bs, float scale, double* out) {
  int max_len = 0, fail = 0;
  for (int s = 0; s < num_seqs; ++s)
    if (context_lens[s] > max_len) max_len = context_lens[s];
#pragma omp parallel reduction(| : fail)
  {
    double* logits = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    if (!logits) {
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long r = 0; r < (long)num_seqs * ntok * Hq; ++r) {
        int s = (int)(r / ((long)ntok * Hq));
        int i = (int)((r / Hq) % ntok), h = (int)(r % Hq);
        int p = context_lens[s] - ntok + i;
        double m, l;
        orc_attend_range(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, k_zero,
                         v_zero, block_tables,
                         max_blocks, s, h, Hq, Hkv, D, bs, (double)scale, 0, p + 1 > 0 ? p + 1 : 0,
                         (size_t)r * D, logits, &m, &l, out + (size_t)r * D);
      }
      free(logits);
    }
  }
  return fail ? -1 : 0;
}

/* Slots of the last ntok positions of every sequence: slots[s][i] is the slot
 * of position L - ntok + i ([MGMT] 二, append_slot), or -1 when that position
 * is negative.                                                               */
void orc_slot_mapping_tokens(const int32_t* block_tables, int max_blocks,
                             const int32_t* context_lens, int num_seqs, int ntok, int bs,
                             int32_t* slots) {
  for (int s = 0; s < num_seqs; ++s)
    for (int i = 0; i < ntok; ++i) {
      int p = context_lens[s] - ntok + i;
      slots[(size_t)s * ntok + i] = p >= 0 ? orc_slot_of(block_tables, max_blocks, s, p, bs) : -1;
    }
}

/* ------------------------------------------------------------------------ */
/* Split-context form.  The context of sequence s is cut into partitions of
 * `part` tokens; partition p covers [p*part, min((p+1)*part, L)).  For each
 * (s, h, p) this writes the partition's maximum m, sum l and normalised
 * output o (empty partitions: -inf, 0, 0).  m, l are [num_seqs][Hq][P], o is
 * [num_seqs][Hq][P][D] with P = n_parts.                                    */
int orc_decode_partials(const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                        int kv_dtype, const float* k_scale, const float* v_scale,
                        const uint8_t* k_zero, const uint8_t* v_zero,
                        const int32_t* block_tables, int max_blocks, const int32_t* context_lens,
                        int num_seqs, int Hq, int Hkv, int D, int bs, float scale, int part,
                        int n_parts, double* m_out, double* l_out, double* o_out) {
  int fail = 0;
#pragma omp parallel reduction(| : fail)
  {
    double* logits = (double*)malloc(sizeof(double) * (size_t)part);
    if (!logits) {
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long r = 0; r < (long)num_seqs * Hq; ++r) {
        int s = (int)(r / Hq), h = (int)(r % Hq);
        int L = context_lens[s];
        for (int p = 0; p < n_parts; ++p) {
          int t0 = p * part;
          int t1 = (p + 1) * part < L ? (p + 1) * part : L;
          size_t i = (size_t)r * n_parts + p;
          orc_attend_range(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                           k_zero, v_zero, block_tables, max_blocks, s, h, Hq, Hkv, D, bs, (double)scale, t0,
                           t1, ((size_t)s * Hq + h) * (size_t)D, logits, &m_out[i], &l_out[i],
                           o_out + i * D);
        }
      }
      free(logits);
    }
  }
  return fail ? -1 : 0;
}

/* Combine partition results with the log-sum-exp rule:
 *   M = max_p m_p,  w_p = exp(m_p - M) * l_p,  out = sum_p w_p o_p / sum_p w_p
 * skipping empty partitions; a row with no tokens gives zeros.              */
void orc_combine_partials(const double* m, const double* l, const double* o, int rows,
                          int n_parts, int D, double* out) {
  for (int r = 0; r < rows; ++r) {
    double M = -INFINITY, den = 0.0;
    for (int p = 0; p < n_parts; ++p)
      if (l[(size_t)r * n_parts + p] > 0.0 && m[(size_t)r * n_parts + p] > M)
        M = m[(size_t)r * n_parts + p];
    for (int d = 0; d < D; ++d) out[(size_t)r * D + d] = 0.0;
    for (int p = 0; p < n_parts; ++p) {
      size_t i = (size_t)r * n_parts + p;
      if (!(l[i] > 0.0)) continue;
      double w = exp(m[i] - M) * l[i];
      den += w;
      for (int d = 0; d < D; ++d) out[(size_t)r * D + d] += w * o[i * D + d];
    }
    if (den > 0.0)
      for (int d = 0; d < D; ++d) out[(size_t)r * D + d] /= den;
  }
}

/* ------------------------------------------------------------------------ */
/* KV quantization, symmetric with one binary32 scale per (block, KV head)
 * tile of block_size x head_dim values ([MGMT] section 四 quantizes cached
 * K/V to 8 bits and restores them as code * scale; [CSDN] section 三 adds
 * FP4; the per-(block, head) symmetric grouping is this build's reading).
 * With a = max |x| over the whole tile (every row, used or not):
 *   INT8:  scale = a / 127,  code = clamp(rint(x / scale), -127, 127)
 *   FP8:   scale = a / 448,  code = E4M3(x / scale), nearest-even, saturating
 *   FP4:   scale = a / 6,    code = E2M1(x / scale), nearest-even, saturating
 * a == 0 gives scale 0 and all codes 0.  Divisions and rint are binary32
 * operations with round-to-nearest-even, matching the stored scale format.
 * block_ids == NULL means every block.                                      */
int orc_quantize(const void* src, int src_dtype, void* dst_k, int dst_dtype, float* scales,
                 int num_blocks, int Hkv, int bs, int D, const int32_t* block_ids, int n_ids) {
  int n = block_ids ? n_ids : num_blocks;
  if (dst_dtype != ORC_I8 && dst_dtype != ORC_FP8 && dst_dtype != ORC_FP4) return -1;
  if (src_dtype != ORC_F32 && src_dtype != ORC_BF16) return -1;
#pragma omp parallel for schedule(static)
  for (long it = 0; it < (long)n * Hkv; ++it) {
    int b = block_ids ? block_ids[it / Hkv] : (int)(it / Hkv);
    int g = (int)(it % Hkv);
    size_t base = orc_pool_offset((size_t)b, (size_t)g, 0, Hkv, bs, D);
    size_t cnt = (size_t)bs * D;
    float a = 0.0f, sc;
    for (size_t i = 0; i < cnt; ++i) {
      float x = (float)orc_load_elem(src, base + i, src_dtype, 1.0, 0.0);
      float ax = fabsf(x);
      if (ax > a) a = ax;
    }
    sc = (dst_dtype == ORC_I8) ? a / 127.0f : (dst_dtype == ORC_FP8) ? a / 448.0f : a / 6.0f;
    scales[(size_t)b * Hkv + g] = sc;
    for (size_t i = 0; i < cnt; ++i) {
      float x = (float)orc_load_elem(src, base + i, src_dtype, 1.0, 0.0);
      if (dst_dtype == ORC_I8) {
        float r = (a == 0.0f) ? 0.0f : rintf(x / sc);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        ((int8_t*)dst_k)[base + i] = (int8_t)r;
      } else if (dst_dtype == ORC_FP8) {
        ((uint8_t*)dst_k)[base + i] = (a == 0.0f) ? 0 : orc_e4m3_from_float(x / sc);
      } else {
        /* element base + i goes to nibble (base + i) & 1 of byte (base + i) / 2 */
        uint8_t c = (a == 0.0f) ? 0 : orc_e2m1_from_float(x / sc);
        uint8_t* byte = (uint8_t*)dst_k + (base + i) / 2;
        if ((base + i) & 1)
          *byte = (uint8_t)((*byte & 0x0F) | (c << 4));
        else
          *byte = (uint8_t)((*byte & 0xF0) | c);
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Asymmetric uint8 quantization of one row of n values, [MGMT] section 四,
 * KVQuantizationCache with per_channel on: the parameters come from the
 * minimum and maximum along the last (head_dim) axis, so every (head, token)
 * row gets its own scale and zero point, and dequantize_key restores
 * (code - zero_point) * scale.  The page's quantize_key takes the code
 * relative to the row minimum and clamps the zero point to [0, 255]; for a
 * row without negative values (or without positive ones) the zero point then
 * clamps and the restore formula returns about x - min (x - max).  The
 * reading taken here is the affine quantizer that the restore formula
 * inverts: the range is widened to hold 0, so the zero point is the code of
 * 0 and never clamps, and each value takes the code whose restored value is
 * nearest:
 *   lo = min(min x, 0), hi = max(max x, 0)
 *   scale      = (hi - lo) / 255
 *   zero_point = clamp(round(-lo / scale), 0, 255)
 *   code       = clamp(round(x / scale) + zero_point, 0, 255)
 * so (code - zero_point) * scale is within scale / 2 of x.  Every step is a
 * binary32 operation (the stored scale's type; the page computes in the
 * tensor's 16-bit type) and round is to nearest, ties to even, as
 * torch.round does.  An all-zero row has scale 0 (the divisions are then
 * undefined) and is stored as scale 0, zero point 0 and codes 0.            */
void orc_quantize_row_asym(const float* x, int n, uint8_t* codes, float* scale_out,
                           uint8_t* zero_out) {
  float lo = 0.0f, hi = 0.0f, sc, z;
  for (int i = 0; i < n; ++i) {
    if (x[i] < lo) lo = x[i];
    if (x[i] > hi) hi = x[i];
  }
  sc = (hi - lo) / 255.0f;
  if (sc == 0.0f) {
    *scale_out = 0.0f;
    *zero_out = 0;
    for (int i = 0; i < n; ++i) codes[i] = 0;
    return;
  }
  z = rintf(-lo / sc);
  if (z < 0.0f) z = 0.0f;
  if (z > 255.0f) z = 255.0f;
  *scale_out = sc;
  *zero_out = (uint8_t)z;
  for (int i = 0; i < n; ++i) {
    float c = rintf(x[i] / sc) + z;
    if (c < 0.0f) c = 0.0f;
    if (c > 255.0f) c = 255.0f;
    codes[i] = (uint8_t)c;
  }
}

/* Per-row asymmetric quantization of a pool (F32 or BF16 source) into codes
 * [num_blocks][Hkv][bs][D] and parameters scales, zeros [num_blocks][Hkv][bs].
 * block_ids == NULL means every block.                                      */
int orc_quantize_asym(const void* src, int src_dtype, uint8_t* codes, float* scales,
                      uint8_t* zeros, int num_blocks, int Hkv, int bs, int D,
                      const int32_t* block_ids, int n_ids) {
  int n = block_ids ? n_ids : num_blocks;
  int fail = 0;
  if (src_dtype != ORC_F32 && src_dtype != ORC_BF16) return -1;
#pragma omp parallel reduction(| : fail)
  {
    float* row = (float*)malloc(sizeof(float) * (size_t)D);
    if (!row) {
      fail = 1;
    } else {
#pragma omp for schedule(static)
      for (long it = 0; it < (long)n * Hkv * bs; ++it) {
        int b = block_ids ? block_ids[it / ((long)Hkv * bs)] : (int)(it / ((long)Hkv * bs));
        int g = (int)((it / bs) % Hkv), o = (int)(it % bs);
        size_t base = orc_pool_offset((size_t)b, (size_t)g, (size_t)o, Hkv, bs, D);
        size_t r = ((size_t)b * Hkv + g) * (size_t)bs + (size_t)o;
        for (int d = 0; d < D; ++d) row[d] = (float)orc_load_elem(src, base + d, src_dtype, 1.0, 0.0);
        orc_quantize_row_asym(row, D, codes + base, scales + r, zeros + r);
      }
      free(row);
    }
  }
  return fail ? -1 : 0;
}

/* Quantized append: the cache write of [KVC] "KV Cache 的本质" into an
 * asymmetric per-row pool.  Token i's K and V rows of head g (F32 or BF16
 * values in k_new, v_new [n][Hkv][D]) are quantized row by row as above and
 * stored at slot slot_mapping[i] (negative = skip) with their parameters;
 * because every row has its own scale and zero point, no other row of the
 * block changes.                                                            */
int orc_cache_write_quant(uint8_t* k_cache, uint8_t* v_cache, float* k_scale, float* v_scale,
                          uint8_t* k_zero, uint8_t* v_zero, int Hkv, int bs, int D,
                          const void* k_new, const void* v_new, int src_dtype,
                          const int32_t* slot_mapping, int n) {
  float* row = (float*)malloc(sizeof(float) * (size_t)D);
  if (!row) return -1;
  if (src_dtype != ORC_F32 && src_dtype != ORC_BF16) {
    free(row);
    return -1;
  }
  for (int i = 0; i < n; ++i) {
    int32_t slot = slot_mapping[i];
    if (slot < 0) continue;
    for (int g = 0; g < Hkv; ++g) {
      size_t b = (size_t)(slot / bs), o = (size_t)(slot % bs);
      size_t dst = orc_pool_offset(b, (size_t)g, o, Hkv, bs, D);
      size_t r = (b * Hkv + g) * (size_t)bs + o;
      size_t src = ((size_t)i * Hkv + g) * (size_t)D;
      for (int d = 0; d < D; ++d) row[d] = (float)orc_load_elem(k_new, src + d, src_dtype, 1.0, 0.0);
      orc_quantize_row_asym(row, D, k_cache + dst, k_scale + r, k_zero + r);
      for (int d = 0; d < D; ++d) row[d] = (float)orc_load_elem(v_new, src + d, src_dtype, 1.0, 0.0);
      orc_quantize_row_asym(row, D, v_cache + dst, v_scale + r, v_zero + r);
    }
  }
  free(row);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Quantized append into a pool with one symmetric scale per (block, KV head)
 * tile (INT8, E4M3, E2M1: the quantizer above).  Each decode step appends
 * one token's K and V ([KVC] "KV Cache 的本质"), but the pages quantize whole
 * token groups and say nothing of a row joining a tile that already has a
 * scale.  The reading taken: the tile's scale always covers the rows written
 * so far, so a row that needs a larger scale grows it and the earlier rows
 * are re-expressed in the new scale; a row at offset 0 starts a fresh tile
 * (no earlier row of its sequence lives there, so the tile's old contents are
 * ignored).  Per token i with slot = slot_mapping[i] >= 0 (block b, offset
 * r), KV head g, K and V separately, every step a binary32 operation with
 * round-to-nearest-even:
 *   a = max |x| over the new row,  c = a / Q  (Q = 127, 448 or 6)
 *   r == 0:      s = c
 *   r > 0:       s_old = the tile's scale; if c > s_old the scale grows to
 *                s = c and each earlier row's code becomes
 *                encode(decode(code) * s_old / s) (the product rounded to
 *                binary32, then divided); otherwise s = s_old
 *   new row:     code = encode(x / s); s == 0 gives zero codes
 * where encode is clamp(rint(.), -127, 127) for INT8 and the nearest code,
 * ties to even, saturating, for E4M3 and E2M1.  Rows after r are untouched.
 * Filling a tile in order ends with the scale that quantizing it whole gives
 * (the maximum of the rows' a / Q).                                         */
static uint8_t orc_sym_encode(int dtype, float v) {
  if (dtype == ORC_I8) {
    float r = rintf(v);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (uint8_t)(int8_t)r;
  }
  return dtype == ORC_FP8 ? orc_e4m3_from_float(v) : orc_e2m1_from_float(v);
}

static float orc_sym_decode(int dtype, uint8_t code) {
  if (dtype == ORC_I8) return (float)(int8_t)code;
  return (float)(dtype == ORC_FP8 ? orc_e4m3_to_double(code) : orc_e2m1_to_double(code));
}

/* code at element index idx of a pool, and its store (E2M1: two per byte,
 * element 2i in the low nibble of byte i)                                   */
static uint8_t orc_sym_get(const uint8_t* pool, int dtype, size_t idx) {
  if (dtype != ORC_FP4) return pool[idx];
  return (uint8_t)((idx & 1) ? pool[idx / 2] >> 4 : pool[idx / 2] & 15);
}

static void orc_sym_put(uint8_t* pool, int dtype, size_t idx, uint8_t c) {
  if (dtype != ORC_FP4) {
    pool[idx] = c;
  } else if (idx & 1) {
    pool[idx / 2] = (uint8_t)((pool[idx / 2] & 0x0F) | (c << 4));
  } else {
    pool[idx / 2] = (uint8_t)((pool[idx / 2] & 0xF0) | c);
  }
}

static void orc_sym_append_row(uint8_t* pool, float* scales, int dtype, int Hkv, int bs, int D,
                               size_t b, size_t g, size_t r, const float* x) {
  const float Q = dtype == ORC_I8 ? 127.0f : dtype == ORC_FP8 ? 448.0f : 6.0f;
  float a = 0.0f, c, s;
  size_t tile = orc_pool_offset(b, g, 0, Hkv, bs, D);
  for (int d = 0; d < D; ++d)
    if (fabsf(x[d]) > a) a = fabsf(x[d]);
  c = a / Q;
  if (r == 0) {
    s = c;
  } else {
    float s_old = scales[b * Hkv + g];
    s = s_old;
    if (c > s_old) {
      s = c;
      for (size_t e = 0; e < r * (size_t)D; ++e) {
        float v = orc_sym_decode(dtype, orc_sym_get(pool, dtype, tile + e)) * s_old;
        orc_sym_put(pool, dtype, tile + e, orc_sym_encode(dtype, v / s));
      }
    }
  }
  scales[b * Hkv + g] = s;
  for (int d = 0; d < D; ++d)
    orc_sym_put(pool, dtype, tile + r * (size_t)D + (size_t)d,
                s == 0.0f ? 0 : orc_sym_encode(dtype, x[d] / s));
}

int orc_cache_write_sym(uint8_t* k_cache, uint8_t* v_cache, float* k_scale, float* v_scale,
                        int dtype, int Hkv, int bs, int D, const void* k_new, const void* v_new,
                        int src_dtype, const int32_t* slot_mapping, int n) {
  float* row;
  if (dtype != ORC_I8 && dtype != ORC_FP8 && dtype != ORC_FP4) return -1;
  if (src_dtype != ORC_F32 && src_dtype != ORC_BF16) return -1;
  row = (float*)malloc(sizeof(float) * (size_t)D);
  if (!row) return -1;
  for (int i = 0; i < n; ++i) {
    int32_t slot = slot_mapping[i];
    if (slot < 0) continue;
    for (int g = 0; g < Hkv; ++g) {
      size_t b = (size_t)(slot / bs), r = (size_t)(slot % bs);
      size_t src = ((size_t)i * Hkv + g) * (size_t)D;
      for (int d = 0; d < D; ++d) row[d] = (float)orc_load_elem(k_new, src + d, src_dtype, 1.0, 0.0);
      orc_sym_append_row(k_cache, k_scale, dtype, Hkv, bs, D, b, (size_t)g, r, row);
      for (int d = 0; d < D; ++d) row[d] = (float)orc_load_elem(v_new, src + d, src_dtype, 1.0, 0.0);
      orc_sym_append_row(v_cache, v_scale, dtype, Hkv, bs, D, b, (size_t)g, r, row);
    }
  }
  free(row);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Sliding-window attention ([WIKI] "三个直接推论": keeping only a window of
 * the most recent tokens is one of the ways to cut KV bytes).  As in
 * orc_decode_multi, query token i of sequence s sits at position
 * p = L - ntok + i, but it attends only to the `window` most recent tokens up
 * to itself: max(0, p - window + 1) <= t <= p.  window <= 0 means no window
 * (the whole prefix, orc_decode_multi).  Tokens before every query's window
 * are never read.  q and out are [num_seqs][ntok][Hq][D].                   */
int orc_decode_window(const void* q, int q_dtype, const void* k_cache, const void* v_cache,
                      int kv_dtype, const float* k_scale, const float* v_scale,
                      const uint8_t* k_zero, const uint8_t* v_zero, const int32_t* block_tables,
                      int max_blocks, const int32_t* context_lens, int num_seqs, int ntok,
                      int window, int Hq, int Hkv, int D, int bs, float scale, double* out) {
  int max_len = 0, fail = 0;
  for (int s = 0; s < num_seqs; ++s)
    if (context_lens[s] > max_len) max_len = context_lens[s];
#pragma omp parallel reduction(| : fail)
  {
    double* logits = (double*)malloc(sizeof(double) * (size_t)(max_len > 0 ? max_len : 1));
    if (!logits) {
      fail = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long r = 0; r < (long)num_seqs * ntok * Hq; ++r) {
        int s = (int)(r / ((long)ntok * Hq));
        int i = (int)((r / Hq) % ntok), h = (int)(r % Hq);
        int p = context_lens[s] - ntok + i;
        int t1 = p + 1 > 0 ? p + 1 : 0;
        int t0 = (window > 0 && p - window + 1 > 0) ? p - window + 1 : 0;
        double m, l;
        orc_attend_range(q, q_dtype, k_cache, v_cache, kv_dtype, k_scale, v_scale, k_zero,
                         v_zero, block_tables, max_blocks, s, h, Hq, Hkv, D, bs, (double)scale,
                         t0 < t1 ? t0 : t1, t1, (size_t)r * D, logits, &m, &l,
                         out + (size_t)r * D);
      }
      free(logits);
    }
  }
  return fail ? -1 : 0;
}

