// Byte-moving kernels: slot mapping, cache write (scatter) and gather.
//
// Cache write: each decode step appends the new token's K and V to the cache
// (page "LLM 推理优化深度解析", section "KV Cache 的本质"); the slot of logical
// position t is table[t / 16] * 16 + t % 16 (page "大模型推理的KV Cache管理…",
// section 二, PagedKVCache.append_slot).  All copies move 16-byte chunks with
// consecutive lanes on consecutive addresses.
#include "common.hpp"

namespace pkv {

namespace {

// slots[s][i] for the last ntok positions L - ntok + i of every sequence
// (-1 for a negative position or a length past the table).
__global__ void slot_mapping_kernel(const int32_t* __restrict__ tables, int max_blocks,
                                    const int32_t* __restrict__ lens, int n, int ntok,
                                    int32_t* __restrict__ slots) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)n * ntok) return;
  const int s = (int)(idx / ntok), i = (int)(idx % ntok);
  const int L = lens[s];
  int32_t slot = -1;
  if (L > 0 && L <= max_blocks * kBlock) {
    const int t = L - ntok + i;
    if (t >= 0) slot = tables[(size_t)s * max_blocks + t / kBlock] * kBlock + t % kBlock;
  }
  slots[idx] = slot;
}

// One thread per 16-byte chunk of one (token, KV head) row; rows of K and V
// are copied by the same thread.
__global__ void cache_write_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                   const uint8_t* __restrict__ kn, const uint8_t* __restrict__ vn,
                                   const int32_t* __restrict__ slots, int n, int hkv,
                                   int row_chunks, int64_t num_slots, size_t blk_bytes) {
  int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t per_tok = (int64_t)hkv * row_chunks;
  if (tid >= (int64_t)n * per_tok) return;
  int i = (int)(tid / per_tok);
  int rem = (int)(tid % per_tok);
  int g = rem / row_chunks;
  int c = rem % row_chunks;
  int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;
  int64_t blk = slot / kBlock, off = slot % kBlock;
  size_t row_bytes = (size_t)row_chunks * 16;
  size_t dst = (size_t)blk * blk_bytes + ((size_t)g * kBlock + off) * row_bytes + (size_t)c * 16;
  size_t src = ((size_t)i * hkv + g) * row_bytes + (size_t)c * 16;
  *reinterpret_cast<uint4*>(kc + dst) = *reinterpret_cast<const uint4*>(kn + src);
  *reinterpret_cast<uint4*>(vc + dst) = *reinterpret_cast<const uint4*>(vn + src);
}

// One workgroup per (sequence, logical block): copies up to 16 tokens x all
// KV heads of K and V, 16 bytes per thread per step.
__global__ void gather_kernel(const uint8_t* __restrict__ kc, const uint8_t* __restrict__ vc,
                              const int32_t* __restrict__ tables, int max_blocks,
                              const int32_t* __restrict__ lens, const int32_t* __restrict__ cu,
                              int hkv, int row_chunks, int num_blocks, size_t blk_bytes,
                              uint8_t* __restrict__ ko, uint8_t* __restrict__ vo) {
  const int b = blockIdx.x % max_blocks, s = blockIdx.x / max_blocks;
  int L = lens[s];
  if (L < 0 || L > max_blocks * kBlock) return;
  int t0 = b * kBlock;
  if (t0 >= L) return;
  int ntok = min(kBlock, L - t0);
  int32_t phys = tables[(size_t)s * max_blocks + b];
  if (phys < 0 || phys >= num_blocks) return;
  size_t row_bytes = (size_t)row_chunks * 16;
  int per_tok = hkv * row_chunks;
  int total = ntok * per_tok;
  size_t out0 = (size_t)cu[s] + t0;
  for (int x = threadIdx.x; x < total; x += blockDim.x) {
    int o = x / per_tok;
    int rem = x % per_tok;
    int g = rem / row_chunks, c = rem % row_chunks;
    size_t src = (size_t)phys * blk_bytes + ((size_t)g * kBlock + o) * row_bytes + (size_t)c * 16;
    size_t dst = ((out0 + o) * hkv + g) * row_bytes + (size_t)c * 16;
    *reinterpret_cast<uint4*>(ko + dst) = *reinterpret_cast<const uint4*>(kc + src);
    *reinterpret_cast<uint4*>(vo + dst) = *reinterpret_cast<const uint4*>(vc + src);
  }
}

// Copy-on-write block copy: one workgroup per (pair, K or V); the block's
// every-head region (blk_bytes) is moved in 16-byte pieces, consecutive
// threads on consecutive addresses; the K workgroup also copies the block's
// K parameters and the V workgroup its V parameters: n_par scales (and zero
// points) per block, one per head or one per (head, row).
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    uint8_t* __restrict__ kc, uint8_t* __restrict__ vc, float* __restrict__ ks,
    float* __restrict__ vs, uint8_t* __restrict__ kz, uint8_t* __restrict__ vz,
    const int32_t* __restrict__ pairs, int num_blocks, int n_par, size_t stride_bytes,
    int blk_chunks) {
  const int i = blockIdx.x;
  const bool is_v = blockIdx.y != 0;
  const int src = pairs[2 * i], dst = pairs[2 * i + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint8_t* base = is_v ? vc : kc;
  const uint4* from = reinterpret_cast<const uint4*>(base + (size_t)src * stride_bytes);
  uint4* to = reinterpret_cast<uint4*>(base + (size_t)dst * stride_bytes);
  // non-temporal loads and stores: each byte is moved once (10,000 pairs:
  // 266.4 -> 260.2 us against plain ones)
  for (int c = threadIdx.x; c < blk_chunks; c += blockDim.x) {
    typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
    const u32x4v* f = reinterpret_cast<const u32x4v*>(from + c);
    u32x4v* t = reinterpret_cast<u32x4v*>(to + c);
    __builtin_nontemporal_store(__builtin_nontemporal_load(f), t);
  }
  float* sc = is_v ? vs : ks;
  uint8_t* zp = is_v ? vz : kz;
  for (int j = threadIdx.x; sc != nullptr && j < n_par; j += blockDim.x) {
    sc[(size_t)dst * n_par + j] = sc[(size_t)src * n_par + j];
    if (zp != nullptr) zp[(size_t)dst * n_par + j] = zp[(size_t)src * n_par + j];
  }
}

}  // namespace

int launch_copy_blocks(const pkv_cache_t& c, const int32_t* pairs, int n, hipStream_t st) {
  const bool q8 = is_quantized(c.kv_dtype);
  const bool rows = c.kv_dtype == PKV_U8_ZP;
  const int chunks = (int)(elems_to_bytes(block_elems(c), c.kv_dtype) / 16);
  dim3 grid((unsigned)n, 2), block(256);
  return launch(copy_blocks_kernel, grid, block, st, (uint8_t*)c.k_cache, (uint8_t*)c.v_cache,
                q8 ? c.k_scale : nullptr, q8 ? c.v_scale : nullptr, rows ? c.k_zero : nullptr,
                rows ? c.v_zero : nullptr, pairs, c.num_blocks,
                rows ? c.num_kv_heads * kBlock : c.num_kv_heads, block_stride_bytes(c), chunks);
}

int launch_slot_mapping(const int32_t* tables, int max_blocks, const int32_t* lens, int n,
                        int ntok, int32_t* slots, hipStream_t st) {
  dim3 grid((unsigned)(((int64_t)n * ntok + 255) / 256)), block(256);
  return launch(slot_mapping_kernel, grid, block, st, tables, max_blocks, lens, n, ntok, slots);
}

int launch_cache_write(const pkv_cache_t& c, const void* k, const void* v, const int32_t* slots,
                       int n, hipStream_t st) {
  int row_chunks = (int)(elems_to_bytes(c.head_dim, c.kv_dtype) / 16);
  int64_t threads = (int64_t)n * c.num_kv_heads * row_chunks;
  dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  return launch(cache_write_kernel, grid, block, st, (uint8_t*)c.k_cache, (uint8_t*)c.v_cache,
                (const uint8_t*)k, (const uint8_t*)v, slots, n, c.num_kv_heads, row_chunks,
                (int64_t)c.num_blocks * kBlock, block_stride_bytes(c));
}

int launch_gather(const pkv_cache_t& c, const int32_t* tables, int max_blocks,
                  const int32_t* lens, const int32_t* cu, int num_seqs, void* ko, void* vo,
                  hipStream_t st) {
  int row_chunks = (int)(elems_to_bytes(c.head_dim, c.kv_dtype) / 16);
  dim3 grid((unsigned)((int64_t)max_blocks * num_seqs)), block(256);
  return launch(gather_kernel, grid, block, st, (const uint8_t*)c.k_cache,
                (const uint8_t*)c.v_cache, tables, max_blocks, lens, cu, c.num_kv_heads,
                row_chunks, c.num_blocks, block_stride_bytes(c), (uint8_t*)ko, (uint8_t*)vo);
}

}  // namespace pkv
