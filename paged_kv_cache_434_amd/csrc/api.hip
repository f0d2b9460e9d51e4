// C ABI entry points (include/pkv.h): argument checks on the host, then one
// or two kernel launches on the caller's stream.  Nothing here allocates
// device memory or synchronises, except pkv_validate_tables (a debug check).
#include <limits.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <utility>
#include <vector>

#include "common.hpp"

using namespace pkv;

namespace {

// ---- fixed scratch of pkv_decode_step_noalloc ------------------------------
// The split partials of the allocation-free decode step live in this array,
// one copy on every GPU the library runs on, held until the process ends.  In
// host code `scratch` only names the symbol: its device address is looked up
// once per device with hipGetSymbolAddress and only that address is passed
// to kernels.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
std::atomic<void*> scratch_addr[kScratchDevices];
std::mutex scratch_mu;

// Device address of the current device's scratch array (looked up on the
// first call on that device), or null if the lookup fails.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) return nullptr;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(scratch_mu);
  p = scratch_addr[dev].load(std::memory_order_relaxed);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  scratch_addr[dev].store(q, std::memory_order_release);
  return q;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_cache(const pkv_cache_t* c) {
  if (!c) return PKV_ERR_NULL;
  if (elem_bits(c->kv_dtype) == 0) return PKV_ERR_DTYPE;
  // slots (block * 16 + row) are 32-bit, so a pool holds at most INT_MAX / 16 blocks
  if (c->block_size != PKV_BLOCK_SIZE || c->num_blocks < 0 ||
      c->num_blocks > INT_MAX / PKV_BLOCK_SIZE || c->num_kv_heads <= 0 || c->head_dim <= 0)
    return PKV_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return PKV_ERR_UNSUPPORTED;
  if (!c->k_cache || !c->v_cache) return PKV_ERR_NULL;
  if (is_quantized(c->kv_dtype) && (!c->k_scale || !c->v_scale)) return PKV_ERR_NULL;
  if (c->kv_dtype == PKV_U8_ZP) {
    if (!c->k_zero || !c->v_zero) return PKV_ERR_NULL;
    // zero points are read four rows per 32-bit load
    if ((reinterpret_cast<uintptr_t>(c->k_zero) & 3u) || (reinterpret_cast<uintptr_t>(c->v_zero) & 3u))
      return PKV_ERR_UNSUPPORTED;
  }
  if (!aligned16(c->k_cache) || !aligned16(c->v_cache)) return PKV_ERR_UNSUPPORTED;
  if (c->block_stride != 0) {
    if (c->block_stride < block_elems(*c)) return PKV_ERR_SHAPE;
    if (c->block_stride % 2 != 0 || elems_to_bytes(c->block_stride, c->kv_dtype) % 16 != 0)
      return PKV_ERR_UNSUPPORTED;
  }
  return PKV_OK;
}

// First offending index of a slot list held on the host (see
// pkv_validate_slots), or -1: an entry outside [0, num_slots), or one whose
// slot (block, with one_per_block) an earlier entry already holds.
int first_bad_slot(const int32_t* sl, int32_t n, int64_t num_slots, bool one_per_block) {
  int best = INT_MAX;
  std::vector<std::pair<int64_t, int>> keys;
  keys.reserve((size_t)n);
  for (int i = 0; i < n; ++i) {
    const int32_t v = sl[i];
    if (v < 0) continue;   // padding, skipped by the writes
    if ((int64_t)v >= num_slots) {
      best = std::min(best, i);
      continue;
    }
    keys.emplace_back(one_per_block ? v / PKV_BLOCK_SIZE : v, i);
  }
  std::sort(keys.begin(), keys.end());
  for (size_t k = 1; k < keys.size(); ++k)
    if (keys[k].first == keys[k - 1].first) best = std::min(best, keys[k].second);
  return best == INT_MAX ? -1 : best;
}

bool split_ok(int32_t partition_tokens) {
  return partition_tokens == PKV_SPLIT_BALANCED ||
         (partition_tokens >= 0 && partition_tokens % PKV_BLOCK_SIZE == 0);
}

}  // namespace

extern "C" {

const char* pkv_strerror(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "invalid or inconsistent size";
    case PKV_ERR_DTYPE: return "unknown or unsupported dtype combination";
    case PKV_ERR_RANGE: return "table or length value out of range";
    case PKV_ERR_WORKSPACE: return "workspace missing or too small";
    case PKV_ERR_UNSUPPORTED: return "request outside what this build implements";
    case PKV_ERR_HIP: return "HIP runtime call or kernel launch failed";
    default: return "unknown status";
  }
}

int pkv_version(void) { return 100; }

uint64_t pkv_pool_bytes(int32_t num_blocks, int32_t num_kv_heads, int32_t block_size,
                        int32_t head_dim, int32_t dtype) {
  const int bits = elem_bits(dtype);
  if (bits == 0 || num_blocks < 0 || num_kv_heads < 0 || block_size < 0 || head_dim < 0) return 0;
  return (uint64_t)num_blocks * num_kv_heads * block_size * head_dim * bits / 8;
}

int pkv_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t num_seqs, int32_t* slot_mapping,
                     void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_blocks_per_seq > INT_MAX / PKV_BLOCK_SIZE)
    return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!block_tables || !context_lens || !slot_mapping) return PKV_ERR_NULL;
  return launch_slot_mapping(block_tables, max_blocks_per_seq, context_lens, num_seqs, 1,
                             slot_mapping, static_cast<hipStream_t>(stream));
}

int pkv_slot_mapping_tokens(const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs, int32_t tokens_per_seq,
                            int32_t* slot_mapping, void* stream) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_blocks_per_seq > INT_MAX / PKV_BLOCK_SIZE ||
      tokens_per_seq <= 0 || (int64_t)num_seqs * tokens_per_seq > (int64_t)INT_MAX)
    return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!block_tables || !context_lens || !slot_mapping) return PKV_ERR_NULL;
  return launch_slot_mapping(block_tables, max_blocks_per_seq, context_lens, num_seqs,
                             tokens_per_seq, slot_mapping, static_cast<hipStream_t>(stream));
}

int pkv_cache_write(const pkv_cache_t* cache, const void* k, const void* v,
                    const int32_t* slot_mapping, int32_t n, void* stream) {
  int rc = check_cache(cache);
  if (rc != PKV_OK) return rc;
  if (cache->kv_dtype != PKV_F32 && cache->kv_dtype != PKV_BF16) return PKV_ERR_UNSUPPORTED;
  if (n < 0) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!k || !v || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned16(k) || !aligned16(v)) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)n * cache->num_kv_heads * cache->head_dim > (int64_t)UINT_MAX) return PKV_ERR_SHAPE;
  return launch_cache_write(*cache, k, v, slot_mapping, n, static_cast<hipStream_t>(stream));
}

int pkv_cache_write_quant(const pkv_cache_t* cache, const void* k, const void* v,
                          int32_t src_dtype, const int32_t* slot_mapping, int32_t n,
                          void* stream) {
  int rc = check_cache(cache);
  if (rc != PKV_OK) return rc;
  if (!is_quantized(cache->kv_dtype) || (src_dtype != PKV_F32 && src_dtype != PKV_BF16))
    return PKV_ERR_DTYPE;
  if (n < 0) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!k || !v || !slot_mapping) return PKV_ERR_NULL;
  if (!aligned16(k) || !aligned16(v)) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)n * cache->num_kv_heads > (int64_t)INT_MAX) return PKV_ERR_SHAPE;
  return launch_cache_write_quant(*cache, k, v, src_dtype, slot_mapping, nullptr, 0, nullptr, n,
                                  static_cast<hipStream_t>(stream));
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_blocks_per_seq, int32_t partition_tokens) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_blocks_per_seq <= 0 ||
      max_blocks_per_seq > INT_MAX / PKV_BLOCK_SIZE || !split_ok(partition_tokens))
    return 0;
  const int k = decode_slots(max_blocks_per_seq, partition_tokens);
  if (k <= 1) return 0;
  return decode_workspace_layout((int64_t)num_seqs * num_q_heads, k, head_dim, num_seqs, nullptr,
                                 nullptr, nullptr);
}

int32_t pkv_decode_default_partition(int32_t num_seqs, int32_t num_kv_heads,
                                     int32_t max_blocks_per_seq) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_blocks_per_seq <= 0) return 0;
  return PKV_SPLIT_BALANCED;
}

static int decode_common(const pkv_cache_t* cache, const void* q, int32_t q_dtype,
                         const void* k_new, const void* v_new, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_q_heads, float scale,
                         int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                         void* out, int32_t out_dtype, void* stream, bool append,
                         int32_t ntok = 1, int32_t window = 0, bool use_scratch = false,
                         int32_t prefix_blocks = -1) {
  int rc = check_cache(cache);
  if (rc != PKV_OK) return rc;
  if ((q_dtype != PKV_F32 && q_dtype != PKV_BF16) || (out_dtype != PKV_F32 && out_dtype != PKV_BF16))
    return PKV_ERR_DTYPE;
  const int kv = cache->kv_dtype;
  const bool pair_ok = (q_dtype == PKV_F32 && kv == PKV_F32) ||
                       (q_dtype == PKV_BF16 && (kv == PKV_BF16 || is_quantized(kv)));
  if (!pair_ok) return PKV_ERR_DTYPE;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq <= 0 || !split_ok(partition_tokens) ||
      max_blocks_per_seq > INT_MAX / PKV_BLOCK_SIZE)
    return PKV_ERR_SHAPE;
  if (num_q_heads % cache->num_kv_heads != 0) return PKV_ERR_SHAPE;
  if (num_q_heads / cache->num_kv_heads > 16) return PKV_ERR_UNSUPPORTED;
  if (ntok <= 0 || ntok > 1024) return PKV_ERR_SHAPE;
  if (window < 0) return PKV_ERR_SHAPE;
  if ((ntok > 1 || window > 0) && kv == PKV_F32) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)num_seqs * ntok * num_q_heads > (int64_t)INT_MAX) return PKV_ERR_SHAPE;
  if (prefix_blocks >= 0) {
    if (prefix_blocks > max_blocks_per_seq) return PKV_ERR_SHAPE;
    if (kv == PKV_F32) return PKV_ERR_UNSUPPORTED;
    partition_tokens = PKV_SPLIT_BALANCED;
  }
  if (num_seqs == 0) return PKV_OK;
  if (append) {
    if (!k_new || !v_new) return PKV_ERR_NULL;
    if (!aligned16(k_new) || !aligned16(v_new)) return PKV_ERR_UNSUPPORTED;
  }
  if (!q || !block_tables || !context_lens || !out) return PKV_ERR_NULL;
  if (!aligned16(q) || !aligned16(out)) return PKV_ERR_UNSUPPORTED;
  const int np = decode_slots(max_blocks_per_seq, partition_tokens);
  if ((int64_t)num_seqs * cache->num_kv_heads * np > (int64_t)INT_MAX) return PKV_ERR_SHAPE;
  // balanced split: flat block positions (and a range past the last) fit in int
  if ((int64_t)num_seqs * max_blocks_per_seq > (int64_t)(INT_MAX / 2)) return PKV_ERR_SHAPE;
  if (np > 1) {
    size_t need = decode_workspace_layout((int64_t)num_seqs * ntok * num_q_heads, np,
                                          cache->head_dim, num_seqs, nullptr, nullptr, nullptr);
    if (use_scratch) {
      if (need > kScratchBytes) return PKV_ERR_WORKSPACE;
      workspace = scratch_on_current_device();
      if (!workspace) return PKV_ERR_HIP;
      workspace_bytes = kScratchBytes;
    }
    if (!workspace || workspace_bytes < need) return PKV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return PKV_ERR_WORKSPACE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  // quantized pools: the new rows are quantized and stored by a launch of
  // their own, then the attention reads them from the pool
  const bool fused = append && !is_quantized(kv);
  if (append && !fused) {
    rc = launch_cache_write_quant(*cache, k_new, v_new, q_dtype, nullptr, block_tables,
                                  max_blocks_per_seq, context_lens, num_seqs, st);
    if (rc != PKV_OK) return rc;
  }
  DecodeArgs a{cache,     q,          q_dtype,   block_tables,     max_blocks_per_seq,
               context_lens, num_seqs, num_q_heads, scale,          partition_tokens,
               workspace, out,        out_dtype, fused ? k_new : nullptr,
               fused ? v_new : nullptr, ntok, window, prefix_blocks};
  return launch_decode(a, st);
}

int pkv_attention_decode(const pkv_cache_t* cache, const void* q, int32_t q_dtype,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                         float scale, int32_t partition_tokens, void* workspace,
                         size_t workspace_bytes, void* out, int32_t out_dtype, void* stream) {
  return decode_common(cache, q, q_dtype, nullptr, nullptr, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, partition_tokens, workspace,
                       workspace_bytes, out, out_dtype, stream, false);
}

int pkv_decode_step(const pkv_cache_t* cache, const void* q, int32_t q_dtype, const void* k,
                    const void* v, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                    float scale, int32_t partition_tokens, void* workspace,
                    size_t workspace_bytes, void* out, int32_t out_dtype, void* stream) {
  return decode_common(cache, q, q_dtype, k, v, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, scale, partition_tokens, workspace, workspace_bytes,
                       out, out_dtype, stream, true);
}

int pkv_decode_step_noalloc(const pkv_cache_t* cache, const void* q, int32_t q_dtype,
                            const void* k, const void* v, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, float scale,
                            int32_t partition_tokens, void* out, int32_t out_dtype,
                            void* stream) {
  return decode_common(cache, q, q_dtype, k, v, block_tables, max_blocks_per_seq, context_lens,
                       num_seqs, num_q_heads, scale, partition_tokens, nullptr, 0, out,
                       out_dtype, stream, true, 1, 0, true);
}

int pkv_attention_prefix(const pkv_cache_t* cache, const void* q, int32_t q_dtype,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                         float scale, int32_t prefix_blocks, void* workspace,
                         size_t workspace_bytes, void* out, int32_t out_dtype, void* stream) {
  if (prefix_blocks < 0) return PKV_ERR_SHAPE;
  return decode_common(cache, q, q_dtype, nullptr, nullptr, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, PKV_SPLIT_BALANCED, workspace,
                       workspace_bytes, out, out_dtype, stream, false, 1, 0, false,
                       prefix_blocks);
}

int pkv_attention_multi(const pkv_cache_t* cache, const void* q, int32_t q_dtype,
                        int32_t tokens_per_seq, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                        int32_t num_q_heads, float scale, int32_t partition_tokens,
                        void* workspace, size_t workspace_bytes, void* out, int32_t out_dtype,
                        void* stream) {
  return decode_common(cache, q, q_dtype, nullptr, nullptr, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, partition_tokens, workspace,
                       workspace_bytes, out, out_dtype, stream, false, tokens_per_seq);
}

int pkv_attention_window(const pkv_cache_t* cache, const void* q, int32_t q_dtype,
                         int32_t tokens_per_seq, int32_t window, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* context_lens,
                         int32_t num_seqs, int32_t num_q_heads, float scale,
                         int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                         void* out, int32_t out_dtype, void* stream) {
  return decode_common(cache, q, q_dtype, nullptr, nullptr, block_tables, max_blocks_per_seq,
                       context_lens, num_seqs, num_q_heads, scale, partition_tokens, workspace,
                       workspace_bytes, out, out_dtype, stream, false, tokens_per_seq, window);
}

int pkv_quantize(const pkv_cache_t* src, const pkv_cache_t* dst, const int32_t* block_ids,
                 int32_t n_ids, void* stream) {
  int rc = check_cache(src);
  if (rc != PKV_OK) return rc;
  rc = check_cache(dst);
  if (rc != PKV_OK) return rc;
  if ((src->kv_dtype != PKV_F32 && src->kv_dtype != PKV_BF16) || !is_quantized(dst->kv_dtype))
    return PKV_ERR_DTYPE;
  if (src->num_blocks != dst->num_blocks || src->num_kv_heads != dst->num_kv_heads ||
      src->head_dim != dst->head_dim)
    return PKV_ERR_SHAPE;
  if (block_ids && n_ids < 0) return PKV_ERR_SHAPE;
  const int64_t n = block_ids ? n_ids : src->num_blocks;
  if (n * src->num_kv_heads > (int64_t)INT_MAX) return PKV_ERR_SHAPE;
  return launch_quantize(*src, *dst, block_ids, n_ids, static_cast<hipStream_t>(stream));
}

int pkv_copy_blocks(const pkv_cache_t* cache, const int32_t* pairs, int32_t n, void* stream) {
  int rc = check_cache(cache);
  if (rc != PKV_OK) return rc;
  if (n < 0 || n > 65535 * 1024) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!pairs) return PKV_ERR_NULL;
  if (elems_to_bytes(block_elems(*cache), cache->kv_dtype) / 16 > (int64_t)INT_MAX)
    return PKV_ERR_SHAPE;
  return launch_copy_blocks(*cache, pairs, n, static_cast<hipStream_t>(stream));
}

int pkv_gather(const pkv_cache_t* cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
               const int32_t* context_lens, const int32_t* cu_seqlens, int32_t num_seqs,
               void* k_out, void* v_out, void* stream) {
  int rc = check_cache(cache);
  if (rc != PKV_OK) return rc;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || max_blocks_per_seq > INT_MAX / PKV_BLOCK_SIZE)
    return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!block_tables || !context_lens || !cu_seqlens || !k_out || !v_out) return PKV_ERR_NULL;
  if (!aligned16(k_out) || !aligned16(v_out)) return PKV_ERR_UNSUPPORTED;
  if ((int64_t)num_seqs * max_blocks_per_seq > (int64_t)INT_MAX) return PKV_ERR_SHAPE;
  return launch_gather(*cache, block_tables, max_blocks_per_seq, context_lens, cu_seqlens,
                       num_seqs, k_out, v_out, static_cast<hipStream_t>(stream));
}

int pkv_validate_slots_host(const int32_t* slot_mapping, int32_t n, int32_t num_blocks,
                            int32_t one_per_block, int32_t* bad_index) {
  if (bad_index) *bad_index = -1;
  if (n < 0 || num_blocks < 0) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!slot_mapping) return PKV_ERR_NULL;
  const int bad = first_bad_slot(slot_mapping, n, (int64_t)num_blocks * PKV_BLOCK_SIZE,
                                 one_per_block != 0);
  if (bad_index) *bad_index = bad;
  return bad < 0 ? PKV_OK : PKV_ERR_RANGE;
}

int pkv_validate_slots(const int32_t* slot_mapping, int32_t n, int32_t num_blocks,
                       int32_t one_per_block, int32_t* bad_index, void* stream) {
  if (bad_index) *bad_index = -1;
  if (n < 0 || num_blocks < 0) return PKV_ERR_SHAPE;
  if (n == 0) return PKV_OK;
  if (!slot_mapping) return PKV_ERR_NULL;
  int32_t* hs = static_cast<int32_t*>(malloc((size_t)n * sizeof(int32_t)));
  if (!hs) return PKV_ERR_HIP;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int rc;
  if (hipMemcpyAsync(hs, slot_mapping, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    rc = PKV_ERR_HIP;
  else
    rc = pkv_validate_slots_host(hs, n, num_blocks, one_per_block, bad_index);
  free(hs);
  return rc;
}

int pkv_validate_tables(const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* context_lens, int32_t num_seqs, int32_t num_blocks,
                        int32_t* bad_seq, void* stream) {
  if (bad_seq) *bad_seq = -1;
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_blocks < 0 ||
      max_blocks_per_seq > INT_MAX / PKV_BLOCK_SIZE)
    return PKV_ERR_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!block_tables || !context_lens) return PKV_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  size_t nt = (size_t)num_seqs * max_blocks_per_seq;
  int32_t* ht = static_cast<int32_t*>(malloc(nt * sizeof(int32_t)));
  int32_t* hl = static_cast<int32_t*>(malloc((size_t)num_seqs * sizeof(int32_t)));
  int rc = PKV_OK;
  if (!ht || !hl) {
    rc = PKV_ERR_HIP;
  } else if (hipMemcpyAsync(ht, block_tables, nt * sizeof(int32_t), hipMemcpyDeviceToHost, st) !=
                 hipSuccess ||
             hipMemcpyAsync(hl, context_lens, (size_t)num_seqs * sizeof(int32_t),
                            hipMemcpyDeviceToHost, st) != hipSuccess ||
             hipStreamSynchronize(st) != hipSuccess) {
    rc = PKV_ERR_HIP;
  } else {
    for (int s = 0; s < num_seqs && rc == PKV_OK; ++s) {
      int L = hl[s];
      if (L < 0 || L > max_blocks_per_seq * PKV_BLOCK_SIZE) {
        rc = PKV_ERR_RANGE;
      } else {
        int nb = (L + PKV_BLOCK_SIZE - 1) / PKV_BLOCK_SIZE;
        for (int b = 0; b < nb; ++b) {
          int32_t id = ht[(size_t)s * max_blocks_per_seq + b];
          if (id < 0 || id >= num_blocks) {
            rc = PKV_ERR_RANGE;
            break;
          }
        }
      }
      if (rc != PKV_OK && bad_seq) *bad_seq = s;
    }
  }
  free(ht);
  free(hl);
  return rc;
}

}  // extern "C"
