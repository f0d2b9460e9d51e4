// KV quantization: symmetric 8-bit codes with one binary32 scale per
// (block, KV head) tile (page "大模型推理的KV Cache管理…", section 四: cached
// K/V stored as 8-bit codes and restored as code * scale), and the same
// section's asymmetric scheme (KVQuantizationCache with per-channel
// parameters): uint8 codes with a scale and a zero point per (head, token)
// row of head_dim values, which also makes a one-token append local to its row.
// The per-row codes are those that the page's restore formula (code - zero)
// * scale inverts, over the row's range widened to hold 0 (see AsymRow).
//
// One wavefront per (block, KV head, K-or-V) tile of 16 x head_dim values:
// coalesced 16-byte loads into registers, a wave-wide max of |x|, then
// binary32 division and round-to-nearest-even for every element.  FP8 codes
// follow the OCP E4M3 definition (bias 7, subnormal quantum 2^-9, largest
// finite 448, no infinities); FP4 codes the OCP E2M1 definition (bias 1,
// subnormal quantum 1/2, largest 6), packed two per byte, element 2i in the
// low nibble (the [CSDN] article's section 三 lists FP4 beside INT8 and FP8
// for KV).  Both come from gfx950's conversion instructions, two codes per
// instruction, after a clamp to the largest finite value.  For every finite
// binary32 input they give the nearest code with ties to the even mantissa
// (an exhaustive run against an encoder written from the definitions found
// no difference).
#include "common.hpp"

namespace pkv {

namespace {

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

// Source tiles are read once and codes written once: both carry the
// non-temporal hint (bf16 -> INT8 over 20,000 blocks: 391.6 -> 379.1 us).
__device__ __forceinline__ uint4 load_src16(const void* p) {
  const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(p));
  return uint4{v.x, v.y, v.z, v.w};
}
template <typename T>
__device__ __forceinline__ void store_code(void* p, T v) {
  __builtin_nontemporal_store(v, reinterpret_cast<T*>(p));
}
__device__ __forceinline__ void store_code(void* p, uint2 v) {
  store_code(p, u32x2v{v.x, v.y});
}

// E4M3 codes of four values (element e in byte e): gfx950's OCP conversion
// rounds to nearest, ties to the even mantissa; clamping to +-448 first gives
// the saturation.
__device__ __forceinline__ uint32_t e4m3_word(float y0, float y1, float y2, float y3) {
  auto c = [](float y) { return __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f); };
  s16x2 r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c(y0), c(y1), 1.0f, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, c(y2), c(y3), 1.0f, true);
  return __builtin_bit_cast(uint32_t, r);
}

// E2M1 codes of two values in one byte (the first in the low nibble), put
// into byte `sel` of `w`: the OCP conversion rounds to nearest, ties to the
// even mantissa bit; clamping to +-6 gives the saturation.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t w, float y0, float y1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, __builtin_amdgcn_fmed3f(y0, -6.0f, 6.0f),
                                                 __builtin_amdgcn_fmed3f(y1, -6.0f, 6.0f), 1.0f,
                                                 SEL);
}

enum { Q_I8 = 0, Q_FP8 = 1, Q_FP4 = 2 };

template <typename SrcT, int D, int MODE>
__global__ __launch_bounds__(64) void quantize_kernel(const SrcT* __restrict__ ksrc,
                                                      const SrcT* __restrict__ vsrc,
                                                      uint8_t* __restrict__ kdst,
                                                      uint8_t* __restrict__ vdst,
                                                      float* __restrict__ kscale,
                                                      float* __restrict__ vscale,
                                                      const int32_t* __restrict__ ids,
                                                      int hkv, int num_blocks, int64_t src_stride,
                                                      int64_t dst_stride) {
  constexpr int kElems = kBlock * D;             // values per tile
  constexpr int kPerLane = kElems / kWave;       // 16 (D=64) or 32 (D=128)
  constexpr int kVec = 16 / sizeof(SrcT);        // values per 16-byte load
  constexpr int kLoads = kPerLane / kVec;
  const int lane = threadIdx.x;
  const int g = blockIdx.x % hkv;
  const int idx = blockIdx.x / hkv;
  const int b = ids ? ids[idx] : idx;
  if (b < 0 || b >= num_blocks) return;
  const bool is_v = blockIdx.y != 0;
  const SrcT* src = (is_v ? vsrc : ksrc) + (size_t)b * src_stride + (size_t)g * kElems;
  uint8_t* dst = (is_v ? vdst : kdst) + (size_t)b * dst_stride +
                 (size_t)g * kElems / (MODE == Q_FP4 ? 2 : 1);

  // lane owns values [ld*64*kVec + lane*kVec, +kVec) for each load ld
  float x[kPerLane];
#pragma unroll
  for (int ld = 0; ld < kLoads; ++ld) {
    uint4 raw = load_src16(src + (size_t)ld * kWave * kVec + lane * kVec);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    if constexpr (sizeof(SrcT) == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[ld * kVec + e] = __uint_as_float(w[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[ld * kVec + 2 * e] = bf16_bits_to_f32(w[e] & 0xFFFFu);
        x[ld * kVec + 2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
      }
    }
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) a = fmaxf(a, fabsf(x[i]));
  a = wave_max(a);
  const float sc = MODE == Q_FP8 ? a / 448.0f : MODE == Q_FP4 ? a / 6.0f : a / 127.0f;
  if (lane == 0) (is_v ? vscale : kscale)[(size_t)b * hkv + g] = sc;

  // codes go back in the same element order: kVec bytes per load per lane
  // (kVec / 2 for FP4, two codes per byte); a == 0 gives zero codes
  const bool zero = a == 0.0f;
#pragma unroll
  for (int ld = 0; ld < kLoads; ++ld) {
    const float* y = x + ld * kVec;
    auto q = [&](int e) { return y[e] / sc; };
    if constexpr (MODE == Q_FP4) {
      uint8_t* p = dst + ((size_t)ld * kWave * kVec + lane * kVec) / 2;
      uint32_t w = 0;
      if (!zero) {
        w = e2m1_pair<0>(w, q(0), q(1));
        w = e2m1_pair<1>(w, q(2), q(3));
        if constexpr (kVec == 8) {
          w = e2m1_pair<2>(w, q(4), q(5));
          w = e2m1_pair<3>(w, q(6), q(7));
        }
      }
      if constexpr (kVec == 8)
        store_code(p, w);
      else
        store_code(p, (uint16_t)w);
    } else if constexpr (MODE == Q_FP8) {
      uint8_t* p = dst + (size_t)ld * kWave * kVec + lane * kVec;
      uint32_t w0 = 0, w1 = 0;
      if (!zero) {
        w0 = e4m3_word(q(0), q(1), q(2), q(3));
        if constexpr (kVec == 8) w1 = e4m3_word(q(4), q(5), q(6), q(7));
      }
      if constexpr (kVec == 4)
        store_code(p, w0);
      else
        store_code(p, uint2{w0, w1});
    } else {
      uint8_t c[kVec];
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        float r = rintf(q(e));
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        c[e] = zero ? 0 : (uint8_t)(int8_t)(int)r;
      }
      uint8_t* p = dst + (size_t)ld * kWave * kVec + lane * kVec;
      if constexpr (kVec == 4) {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) w |= (uint32_t)c[e] << (8 * e);
        store_code(p, w);
      } else {
        uint2 w = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          w.x |= (uint32_t)c[e] << (8 * e);
          w.y |= (uint32_t)c[4 + e] << (8 * e);
        }
        store_code(p, w);
      }
    }
  }
}

template <typename SrcT, int D, int MODE>
int launch_q(const pkv_cache_t& src, const pkv_cache_t& dst, const int32_t* ids, int n,
             hipStream_t st) {
  dim3 grid((unsigned)(n * src.num_kv_heads), 2), block(kWave);
  return launch(quantize_kernel<SrcT, D, MODE>, grid, block, st, (const SrcT*)src.k_cache,
                (const SrcT*)src.v_cache, (uint8_t*)dst.k_cache, (uint8_t*)dst.v_cache,
                dst.k_scale, dst.v_scale, ids, src.num_kv_heads, src.num_blocks,
                (int64_t)(block_stride_bytes(src) / sizeof(SrcT)), (int64_t)block_stride_bytes(dst));
}

// Asymmetric row parameters and codes (binary32 steps, ties to even).  The
// row's range is widened to hold 0, so the zero point is the code of 0 and
// never clamps, and each value takes the code whose restored value
// (code - zero) * scale is nearest:
//   lo = min(row min, 0), hi = max(row max, 0), scale = (hi - lo) / 255,
//   zero = clamp(rint(-lo / scale), 0, 255),
//   code = clamp(rint(x / scale) + zero, 0, 255);
// an all-zero row (scale 0) gets zero 0 and codes 0.
struct AsymRow {
  float sc, zf;
  uint8_t zero;
  __device__ __forceinline__ AsymRow(float lo, float hi) {
    lo = fminf(lo, 0.0f);
    hi = fmaxf(hi, 0.0f);
    sc = (hi - lo) / 255.0f;
    zf = 0.0f;
    if (sc != 0.0f) zf = fminf(fmaxf(rintf(-lo / sc), 0.0f), 255.0f);
    zero = (uint8_t)zf;
  }
  __device__ __forceinline__ uint32_t code(float x) const {
    if (sc == 0.0f) return 0u;
    return (uint32_t)fminf(fmaxf(rintf(x / sc) + zf, 0.0f), 255.0f);
  }
};

// Per-row asymmetric quantization of a pool: one wavefront per (block, KV
// head, K-or-V) tile, loaded as in quantize_kernel; the kVec values a lane
// holds per load lie in one row, whose D / kVec lanes are consecutive, so the
// row minimum and maximum are shuffle reductions over that lane group.
template <typename SrcT, int D>
__global__ __launch_bounds__(64) void quantize_rows_kernel(
    const SrcT* __restrict__ ksrc, const SrcT* __restrict__ vsrc, uint8_t* __restrict__ kdst,
    uint8_t* __restrict__ vdst, float* __restrict__ kscale, float* __restrict__ vscale,
    uint8_t* __restrict__ kzero, uint8_t* __restrict__ vzero, const int32_t* __restrict__ ids,
    int hkv, int num_blocks, int64_t src_stride, int64_t dst_stride) {
  constexpr int kElems = kBlock * D;
  constexpr int kVec = 16 / sizeof(SrcT);        // values per 16-byte load
  constexpr int kLoads = kElems / kWave / kVec;
  constexpr int kLpr = D / kVec;                 // lanes per row
  constexpr int kRowsPerLoad = kWave / kLpr;
  const int lane = threadIdx.x;
  const int g = blockIdx.x % hkv;
  const int idx = blockIdx.x / hkv;
  const int b = ids ? ids[idx] : idx;
  if (b < 0 || b >= num_blocks) return;
  const bool is_v = blockIdx.y != 0;
  const SrcT* src = (is_v ? vsrc : ksrc) + (size_t)b * src_stride + (size_t)g * kElems;
  uint8_t* dst = (is_v ? vdst : kdst) + (size_t)b * dst_stride + (size_t)g * kElems;
  float* scale = (is_v ? vscale : kscale) + ((size_t)b * hkv + g) * kBlock;
  uint8_t* zero = (is_v ? vzero : kzero) + ((size_t)b * hkv + g) * kBlock;

#pragma unroll
  for (int ld = 0; ld < kLoads; ++ld) {
    float x[kVec];
    uint4 raw = load_src16(src + (size_t)ld * kWave * kVec + lane * kVec);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    if constexpr (sizeof(SrcT) == 4) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = __uint_as_float(w[e]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[2 * e] = bf16_bits_to_f32(w[e] & 0xFFFFu);
        x[2 * e + 1] = bf16_bits_to_f32(w[e] >> 16);
      }
    }
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int e = 1; e < kVec; ++e) {
      mn = fminf(mn, x[e]);
      mx = fmaxf(mx, x[e]);
    }
#pragma unroll
    for (int o = 1; o < kLpr; o <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, o, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    }
    const AsymRow q(mn, mx);
    const int row = ld * kRowsPerLoad + lane / kLpr;
    if (lane % kLpr == 0) {
      scale[row] = q.sc;
      zero[row] = q.zero;
    }
    uint8_t* p = dst + (size_t)ld * kWave * kVec + lane * kVec;
    if constexpr (kVec == 4) {
      uint32_t c = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) c |= q.code(x[e]) << (8 * e);
      *reinterpret_cast<uint32_t*>(p) = c;
    } else {
      uint2 c = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c.x |= q.code(x[e]) << (8 * e);
        c.y |= q.code(x[4 + e]) << (8 * e);
      }
      *reinterpret_cast<uint2*>(p) = c;
    }
  }
}

// Quantized append: one wavefront per (token, KV head) row pair (K in
// blockIdx.y 0, V in 1); lane l holds values [l * kPer, l * kPer + kPer) of
// the row.  Row i goes to slots[i], or with slots null to position
// lens[i] - 1 of sequence i through its block table.
template <typename SrcT, int D>
__global__ __launch_bounds__(64) void cache_write_quant_kernel(
    const SrcT* __restrict__ kn, const SrcT* __restrict__ vn, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, float* __restrict__ kscale, float* __restrict__ vscale,
    uint8_t* __restrict__ kzero, uint8_t* __restrict__ vzero, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ tables, int max_blocks, const int32_t* __restrict__ lens, int hkv,
    int num_blocks, size_t blk_bytes) {
  constexpr int kPer = D / kWave;   // 1 or 2 values per lane
  const int lane = threadIdx.x;
  const int i = blockIdx.x / hkv, g = blockIdx.x % hkv;
  int64_t slot = -1;
  if (slots != nullptr) {
    slot = slots[i];
  } else {
    const int L = lens[i];
    if (L > 0 && L <= max_blocks * kBlock)
      slot = (int64_t)tables[(size_t)i * max_blocks + (L - 1) / kBlock] * kBlock + (L - 1) % kBlock;
  }
  if (slot < 0 || slot >= (int64_t)num_blocks * kBlock) return;
  const bool is_v = blockIdx.y != 0;
  const SrcT* src = (is_v ? vn : kn) + ((size_t)i * hkv + g) * D + lane * kPer;
  float x[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    if constexpr (sizeof(SrcT) == 4)
      x[e] = src[e];
    else
      x[e] = bf16_bits_to_f32(src[e]);
  }
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int e = 1; e < kPer; ++e) {
    mn = fminf(mn, x[e]);
    mx = fmaxf(mx, x[e]);
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, o, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  }
  const AsymRow q(mn, mx);
  const int64_t blk = slot / kBlock, o = slot % kBlock;
  uint8_t* dst = (is_v ? vc : kc) + (size_t)blk * blk_bytes + ((size_t)g * kBlock + o) * D +
                 lane * kPer;
  if constexpr (kPer == 2)
    *reinterpret_cast<uint16_t*>(dst) = (uint16_t)(q.code(x[0]) | (q.code(x[1]) << 8));
  else
    *dst = (uint8_t)q.code(x[0]);
  if (lane == 0) {
    const size_t r = ((size_t)blk * hkv + g) * kBlock + o;
    (is_v ? vscale : kscale)[r] = q.sc;
    (is_v ? vzero : kzero)[r] = q.zero;
  }
}

template <typename SrcT, int D>
int launch_qrows(const pkv_cache_t& src, const pkv_cache_t& dst, const int32_t* ids, int n,
                 hipStream_t st) {
  dim3 grid((unsigned)(n * src.num_kv_heads), 2), block(kWave);
  return launch(quantize_rows_kernel<SrcT, D>, grid, block, st, (const SrcT*)src.k_cache,
                (const SrcT*)src.v_cache, (uint8_t*)dst.k_cache, (uint8_t*)dst.v_cache,
                dst.k_scale, dst.v_scale, dst.k_zero, dst.v_zero, ids, src.num_kv_heads,
                src.num_blocks, (int64_t)(block_stride_bytes(src) / sizeof(SrcT)),
                (int64_t)block_stride_bytes(dst));
}

template <typename SrcT, int D>
int launch_cwq(const pkv_cache_t& c, const void* k, const void* v, const int32_t* slots,
               const int32_t* tables, int max_blocks, const int32_t* lens, int n,
               hipStream_t st) {
  dim3 grid((unsigned)((int64_t)n * c.num_kv_heads), 2), block(kWave);
  return launch(cache_write_quant_kernel<SrcT, D>, grid, block, st, (const SrcT*)k,
                (const SrcT*)v, (uint8_t*)c.k_cache, (uint8_t*)c.v_cache, c.k_scale, c.v_scale,
                c.k_zero, c.v_zero, slots, tables, max_blocks, lens, c.num_kv_heads,
                c.num_blocks, block_stride_bytes(c));
}

// Quantized append into a pool with one symmetric scale per (block, KV head)
// tile (INT8, E4M3, E2M1).  Each decode step appends one token's K and V
// (page "LLM 推理优化深度解析", section "KV Cache 的本质"); the tile's scale
// covers the rows written so far, so a row whose a / Q exceeds it grows the
// scale and the earlier rows are re-expressed:
//   a = max |x| of the new row, c = a / Q (Q = 127, 448 or 6)
//   row offset r == 0: a fresh tile, s = c (its old contents are ignored)
//   r > 0: s_old = the tile's scale; if c > s_old, s = c and every earlier
//          code becomes encode(decode(code) * s_old / s), else s = s_old
//   new row: code = encode(x / s), zero codes when s == 0
// every step binary32 with ties to even; rows after r are left alone.
// One wavefront per (token, KV head, K-or-V); lane l holds the new row's
// values 2l and 2l + 1 (lanes 32-63 hold none at D = 64), and re-encodes the
// earlier rows 16 code bytes at a time.
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two codes of a 32-bit word to binary32, exact: E4M3 bytes 2K and 2K + 1
// (K = 0, 1), or the two E2M1 codes of byte K (low nibble first).
template <int MODE, int K>
__device__ __forceinline__ f32x2 sym_decode_pair(uint32_t w) {
  if constexpr (MODE == Q_FP8)
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, K == 1);
  else
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, K);
}

template <typename SrcT, int D, int MODE>
__global__ __launch_bounds__(64) void cache_write_sym_kernel(
    const SrcT* __restrict__ kn, const SrcT* __restrict__ vn, uint8_t* __restrict__ kc,
    uint8_t* __restrict__ vc, float* __restrict__ kscale, float* __restrict__ vscale,
    const int32_t* __restrict__ slots, const int32_t* __restrict__ tables, int max_blocks,
    const int32_t* __restrict__ lens, int hkv, int num_blocks, size_t blk_bytes) {
  constexpr float kQ = MODE == Q_I8 ? 127.0f : MODE == Q_FP8 ? 448.0f : 6.0f;
  constexpr int kRowBytes = MODE == Q_FP4 ? D / 2 : D;
  const int lane = threadIdx.x;
  const int i = blockIdx.x / hkv, g = blockIdx.x % hkv;
  int64_t slot = -1;
  if (slots != nullptr) {
    slot = slots[i];
  } else {
    const int L = lens[i];
    if (L > 0 && L <= max_blocks * kBlock)
      slot = (int64_t)tables[(size_t)i * max_blocks + (L - 1) / kBlock] * kBlock + (L - 1) % kBlock;
  }
  if (slot < 0 || slot >= (int64_t)num_blocks * kBlock) return;
  const bool is_v = blockIdx.y != 0;
  const int64_t blk = slot / kBlock;
  const int r = (int)(slot % kBlock);
  uint8_t* tile = (is_v ? vc : kc) + (size_t)blk * blk_bytes + (size_t)g * kBlock * kRowBytes;
  float* scp = (is_v ? vscale : kscale) + (size_t)blk * hkv + g;

  // the new row: values 2 lane and 2 lane + 1
  const bool has = 2 * lane < D;
  float x0 = 0.f, x1 = 0.f;
  if (has) {
    const SrcT* src = (is_v ? vn : kn) + ((size_t)i * hkv + g) * D + 2 * lane;
    if constexpr (sizeof(SrcT) == 4) {
      x0 = src[0];
      x1 = src[1];
    } else {
      x0 = bf16_bits_to_f32(src[0]);
      x1 = bf16_bits_to_f32(src[1]);
    }
  }
  const float a = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
  const float c = a / kQ;
  float s = c;
  if (r > 0) {
    const float s_old = *scp;
    s = s_old;
    if (c > s_old) {
      s = c;
      // re-encode rows 0 .. r-1, 16 code bytes per lane and pass
      const int chunks = r * kRowBytes / 16;
      for (int ch = lane; ch < chunks; ch += kWave) {
        uint4* p = reinterpret_cast<uint4*>(tile + ch * 16);
        const uint4 in = *p;
        const uint32_t w[4] = {in.x, in.y, in.z, in.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if constexpr (MODE == Q_I8) {
            uint32_t acc = 0;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float v = (float)(int8_t)((w[q] >> (8 * e)) & 0xFFu) * s_old;
              const float rr = fminf(fmaxf(rintf(v / s), -127.0f), 127.0f);
              acc |= (uint32_t)(uint8_t)(int8_t)(int)rr << (8 * e);
            }
            o[q] = acc;
          } else if constexpr (MODE == Q_FP8) {
            const f32x2 lo = sym_decode_pair<MODE, 0>(w[q]), hi = sym_decode_pair<MODE, 1>(w[q]);
            const float v0 = lo[0] * s_old, v1 = lo[1] * s_old;
            const float v2 = hi[0] * s_old, v3 = hi[1] * s_old;
            o[q] = e4m3_word(v0 / s, v1 / s, v2 / s, v3 / s);
          } else {
            const f32x2 c0 = sym_decode_pair<MODE, 0>(w[q]), c1 = sym_decode_pair<MODE, 1>(w[q]);
            const f32x2 c2 = sym_decode_pair<MODE, 2>(w[q]), c3 = sym_decode_pair<MODE, 3>(w[q]);
            auto rq = [&](float d) {
              const float v = d * s_old;
              return v / s;
            };
            uint32_t acc = 0;
            acc = e2m1_pair<0>(acc, rq(c0[0]), rq(c0[1]));
            acc = e2m1_pair<1>(acc, rq(c1[0]), rq(c1[1]));
            acc = e2m1_pair<2>(acc, rq(c2[0]), rq(c2[1]));
            acc = e2m1_pair<3>(acc, rq(c3[0]), rq(c3[1]));
            o[q] = acc;
          }
        }
        *p = uint4{o[0], o[1], o[2], o[3]};
      }
    }
  }
  // the new row's codes
  if (has) {
    uint8_t* dst = tile + (size_t)r * kRowBytes;
    const bool zero = s == 0.0f;
    if constexpr (MODE == Q_I8) {
      const float r0 = fminf(fmaxf(rintf(x0 / s), -127.0f), 127.0f);
      const float r1 = fminf(fmaxf(rintf(x1 / s), -127.0f), 127.0f);
      const uint16_t v = zero ? 0 : (uint16_t)((uint8_t)(int8_t)(int)r0 |
                                               ((uint16_t)(uint8_t)(int8_t)(int)r1 << 8));
      *reinterpret_cast<uint16_t*>(dst + 2 * lane) = v;
    } else if constexpr (MODE == Q_FP8) {
      const uint32_t w = zero ? 0u : e4m3_word(x0 / s, x1 / s, 0.f, 0.f);
      *reinterpret_cast<uint16_t*>(dst + 2 * lane) = (uint16_t)(w & 0xFFFFu);
    } else {
      const uint32_t w = zero ? 0u : e2m1_pair<0>(0u, x0 / s, x1 / s);
      dst[lane] = (uint8_t)(w & 0xFFu);
    }
  }
  if (lane == 0) *scp = s;
}

template <typename SrcT, int D, int MODE>
int launch_cws(const pkv_cache_t& c, const void* k, const void* v, const int32_t* slots,
               const int32_t* tables, int max_blocks, const int32_t* lens, int n,
               hipStream_t st) {
  dim3 grid((unsigned)((int64_t)n * c.num_kv_heads), 2), block(kWave);
  return launch(cache_write_sym_kernel<SrcT, D, MODE>, grid, block, st, (const SrcT*)k,
                (const SrcT*)v, (uint8_t*)c.k_cache, (uint8_t*)c.v_cache, c.k_scale, c.v_scale,
                slots, tables, max_blocks, lens, c.num_kv_heads, c.num_blocks,
                block_stride_bytes(c));
}

template <typename SrcT, int D>
int launch_cwq_any(const pkv_cache_t& c, const void* k, const void* v, const int32_t* slots,
                   const int32_t* tables, int max_blocks, const int32_t* lens, int n,
                   hipStream_t st) {
  switch (c.kv_dtype) {
    case PKV_U8_ZP: return launch_cwq<SrcT, D>(c, k, v, slots, tables, max_blocks, lens, n, st);
    case PKV_I8: return launch_cws<SrcT, D, Q_I8>(c, k, v, slots, tables, max_blocks, lens, n, st);
    case PKV_FP8_E4M3:
      return launch_cws<SrcT, D, Q_FP8>(c, k, v, slots, tables, max_blocks, lens, n, st);
    case PKV_FP4_E2M1:
      return launch_cws<SrcT, D, Q_FP4>(c, k, v, slots, tables, max_blocks, lens, n, st);
    default: return PKV_ERR_UNSUPPORTED;
  }
}

template <typename SrcT, int D>
int launch_qd(const pkv_cache_t& src, const pkv_cache_t& dst, const int32_t* ids, int n,
              hipStream_t st) {
  switch (dst.kv_dtype) {
    case PKV_U8_ZP: return launch_qrows<SrcT, D>(src, dst, ids, n, st);
    case PKV_FP8_E4M3: return launch_q<SrcT, D, Q_FP8>(src, dst, ids, n, st);
    case PKV_FP4_E2M1: return launch_q<SrcT, D, Q_FP4>(src, dst, ids, n, st);
    default: return launch_q<SrcT, D, Q_I8>(src, dst, ids, n, st);
  }
}

}  // namespace

int launch_quantize(const pkv_cache_t& src, const pkv_cache_t& dst, const int32_t* ids, int n_ids,
                    hipStream_t st) {
  int n = ids ? n_ids : src.num_blocks;
  if (n == 0) return PKV_OK;
  const bool f32 = src.kv_dtype == PKV_F32;
  if (src.head_dim == 128)
    return f32 ? launch_qd<float, 128>(src, dst, ids, n, st)
               : launch_qd<uint16_t, 128>(src, dst, ids, n, st);
  return f32 ? launch_qd<float, 64>(src, dst, ids, n, st)
             : launch_qd<uint16_t, 64>(src, dst, ids, n, st);
}

int launch_cache_write_quant(const pkv_cache_t& c, const void* k, const void* v, int src_dtype,
                             const int32_t* slots, const int32_t* tables, int max_blocks,
                             const int32_t* lens, int n, hipStream_t st) {
  if (n == 0) return PKV_OK;
  const bool f32 = src_dtype == PKV_F32;
  if (c.head_dim == 128)
    return f32 ? launch_cwq_any<float, 128>(c, k, v, slots, tables, max_blocks, lens, n, st)
               : launch_cwq_any<uint16_t, 128>(c, k, v, slots, tables, max_blocks, lens, n, st);
  return f32 ? launch_cwq_any<float, 64>(c, k, v, slots, tables, max_blocks, lens, n, st)
             : launch_cwq_any<uint16_t, 64>(c, k, v, slots, tables, max_blocks, lens, n, st);
}

}  // namespace pkv
