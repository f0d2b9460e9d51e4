// Internal helpers shared by the pkv HIP sources (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "pkv.h"

namespace pkv {

constexpr int kBlock = PKV_BLOCK_SIZE;  // tokens per KV block
constexpr int kWave = 64;               // CDNA wavefront width

// Bits of one stored element (FP4 codes are packed two per byte), 0 for an
// unknown type.
inline int elem_bits(int dtype) {
  switch (dtype) {
    case PKV_F32: return 32;
    case PKV_BF16: return 16;
    case PKV_I8: return 8;
    case PKV_FP8_E4M3: return 8;
    case PKV_U8_ZP: return 8;
    case PKV_FP4_E2M1: return 4;
    default: return 0;
  }
}

// Bytes of n stored elements (n even for FP4).
inline int64_t elems_to_bytes(int64_t n, int dtype) { return n * elem_bits(dtype) / 8; }

// Elements of one block of one pool (every KV head's tile).
inline int64_t block_elems(const pkv_cache_t& c) {
  return (int64_t)c.num_kv_heads * c.block_size * c.head_dim;
}

// Pools of codes with binary32 scales (and, for PKV_U8_ZP, zero points).
inline bool is_quantized(int dtype) {
  return dtype == PKV_I8 || dtype == PKV_FP8_E4M3 || dtype == PKV_U8_ZP ||
         dtype == PKV_FP4_E2M1;
}

// Bytes from one block to the next in k_cache / v_cache.
inline size_t block_stride_bytes(const pkv_cache_t& c) {
  const int64_t e = c.block_stride != 0 ? c.block_stride : block_elems(c);
  return (size_t)elems_to_bytes(e, c.kv_dtype);
}

// Launch through hipLaunchKernel so the launch status comes back directly
// instead of through the thread's sticky last-error slot.
template <typename... KArgs, typename... Args>
inline int launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                  Args&&... args) {
  std::tuple<KArgs...> packed(std::forward<Args>(args)...);
  void* ptrs[sizeof...(KArgs)];
  std::apply([&](auto&... a) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&a)), ...);
  }, packed);
  hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0,
                                 stream);
  return e == hipSuccess ? PKV_OK : PKV_ERR_HIP;
}

// ---- device-side helpers ---------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// binary32 -> bfloat16 bits, round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Orders one wavefront's LDS accesses where its lanes exchange data through
// LDS.  The hardware already completes a wave's LDS operations in issue
// order; the fences stop the compiler from treating the other lanes' stores
// as absent, which would let it reuse a value that a lane loaded before them
// or move a load above them.  No instruction is emitted.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Max and sum over lanes l, l^16, l^32 and l^48 (one lane of each 16-lane
// row) with gfx950's row swaps, which stay in the vector unit instead of
// going through LDS like a lane permute.  v_permlane16_swap trades the odd
// rows of its first operand for the even rows of its second, and
// v_permlane32_swap the upper 32 lanes of its first for the lower 32 of its
// second; given a value twice, each lane ends up with its own value in one
// result and its partner's in the other.
// (The max is IEEE maximum, which passes a NaN on; it needs no operand
// quieting, unlike fmaxf.)
__device__ __forceinline__ float rows_max(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float rows_sum(float v) {
  const uint32_t u = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(v);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ---- launchers (defined in the .hip sources) --------------------------------

int launch_slot_mapping(const int32_t* tables, int max_blocks, const int32_t* lens, int n,
                        int ntok, int32_t* slots, hipStream_t st);
int launch_cache_write(const pkv_cache_t& c, const void* k, const void* v, const int32_t* slots,
                       int n, hipStream_t st);
int launch_gather(const pkv_cache_t& c, const int32_t* tables, int max_blocks,
                  const int32_t* lens, const int32_t* cu, int num_seqs, void* ko, void* vo,
                  hipStream_t st);
int launch_copy_blocks(const pkv_cache_t& c, const int32_t* pairs, int n, hipStream_t st);
int launch_quantize(const pkv_cache_t& src, const pkv_cache_t& dst, const int32_t* ids, int n_ids,
                    hipStream_t st);
// Quantized append into a PKV_U8_ZP pool: row i goes to slots[i], or (slots
// null) to position lens[i] - 1 of sequence i through its table.
int launch_cache_write_quant(const pkv_cache_t& c, const void* k, const void* v, int src_dtype,
                             const int32_t* slots, const int32_t* tables, int max_blocks,
                             const int32_t* lens, int n, hipStream_t st);

struct DecodeArgs {
  const pkv_cache_t* cache;
  const void* q;
  int q_dtype;
  const int32_t* tables;
  int max_blocks;
  const int32_t* lens;
  int num_seqs;
  int num_q_heads;
  float scale;
  int partition_tokens;
  void* workspace;
  void* out;
  int out_dtype;
  const void* k_new;   // fused append of position L-1 (decode step), or nullptr
  const void* v_new;
  int ntok;            // query tokens per sequence (1: decode)
  int window;          // sliding window in tokens, 0 for none
  int prefix_blocks;   // >= 0: shared-prefix split over that many common table entries
};
int launch_decode(const DecodeArgs& a, hipStream_t st);

// Balanced split: fewest blocks one wavefront takes.  With 8 a short step
// (a 4096-token window over 8 sequences) made 32 pieces per sequence, and the
// partials' round trip and the combine cost more than the shorter ranges saved:
// 16 took that step from 31.7 to 28.9 us; 24 was slower again.
constexpr int kBalancedMinBlocks = 16;

// Partial slots per (sequence, query head) row for a split setting.  A run of
// n blocks meets at most ceil((n - 1) / 16) + 1 ranges of 16 or more blocks;
// the balanced split cuts a sequence into one run, the shared-prefix split
// into two (its group's P prefix blocks and its own max_blocks - P), so
// ceil((max_blocks - 2) / 16) + 3 <= ceil(max_blocks / 16) + 3 slots cover
// both.
int decode_slots(int max_blocks, int partition_tokens);

// Bytes of the split-context workspace and the offsets of its m, l and count
// parts.
size_t decode_workspace_layout(int64_t rows, int kslots, int D, int64_t num_seqs, size_t* off_m,
                               size_t* off_l, size_t* off_count);

// Compute units of the current device (cached per device), or -1.
int device_cu_count();

}  // namespace pkv
