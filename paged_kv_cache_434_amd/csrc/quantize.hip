// KV quantization: symmetric 8-bit codes with one binary32 scale per
// (block, KV head) tile (page "大模型推理的KV Cache管理…", section 四: cached
// K/V stored as 8-bit codes and restored as code * scale).
//
// One wavefront per (block, KV head, K-or-V) tile of 16 x head_dim values:
// coalesced 16-byte loads into registers, a wave-wide max of |x|, then
// binary32 division and round-to-nearest-even for every element.  FP8 codes
// follow the OCP E4M3 definition (bias 7, subnormal quantum 2^-9, largest
// finite 448, no infinities), computed from the exponent and a rounded
// 3-bit mantissa.
#include "common.hpp"

namespace pkv {

namespace {

// Nearest E4M3 code of y (ties to even mantissa), magnitudes >= 448 clamp to
// 448; the sign bit is the sign of y.  y must not be NaN.
__device__ __forceinline__ uint8_t e4m3_encode(float y) {
  uint32_t sign = __float_as_uint(y) >> 31;
  float ay = fabsf(y);
  uint32_t mag;
  if (ay >= 448.0f) {
    mag = 0x7E;
  } else if (ay < 0.015625f) {                 // below 2^-6: multiples of 2^-9
    mag = (uint32_t)rintf(ay * 512.0f);        // 0..8; 8 is the smallest normal
  } else {
    int e = (int)((__float_as_uint(ay) >> 23) & 0xFF) - 127;  // floor(log2 ay), -6..8
    uint32_t mi = (uint32_t)rintf(ldexpf(ay, 3 - e));         // 8..16
    if (mi == 16) {
      mi = 8;
      e += 1;
    }
    mag = ((uint32_t)(e + 7) << 3) | (mi - 8);
  }
  return (uint8_t)((sign << 7) | mag);
}

template <typename SrcT, int D, bool FP8>
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
  uint8_t* dst = (is_v ? vdst : kdst) + (size_t)b * dst_stride + (size_t)g * kElems;

  // lane owns values [ld*64*kVec + lane*kVec, +kVec) for each load ld
  float x[kPerLane];
#pragma unroll
  for (int ld = 0; ld < kLoads; ++ld) {
    uint4 raw = *reinterpret_cast<const uint4*>(src + (size_t)ld * kWave * kVec + lane * kVec);
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
  const float sc = FP8 ? a / 448.0f : a / 127.0f;
  if (lane == 0) (is_v ? vscale : kscale)[(size_t)b * hkv + g] = sc;

  uint8_t c[kPerLane];
#pragma unroll
  for (int i = 0; i < kPerLane; ++i) {
    if (a == 0.0f) {
      c[i] = 0;
    } else if constexpr (FP8) {
      c[i] = e4m3_encode(x[i] / sc);
    } else {
      float r = rintf(x[i] / sc);
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      c[i] = (uint8_t)(int8_t)(int)r;
    }
  }
  // codes go back in the same element order: kVec bytes per load per lane
#pragma unroll
  for (int ld = 0; ld < kLoads; ++ld) {
    uint8_t* p = dst + (size_t)ld * kWave * kVec + lane * kVec;
    if constexpr (kVec == 4) {
      uint32_t w = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) w |= (uint32_t)c[ld * 4 + e] << (8 * e);
      *reinterpret_cast<uint32_t*>(p) = w;
    } else {
      uint2 w = {0u, 0u};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        w.x |= (uint32_t)c[ld * 8 + e] << (8 * e);
        w.y |= (uint32_t)c[ld * 8 + 4 + e] << (8 * e);
      }
      *reinterpret_cast<uint2*>(p) = w;
    }
  }
}

template <typename SrcT, int D, bool FP8>
int launch_q(const pkv_cache_t& src, const pkv_cache_t& dst, const int32_t* ids, int n,
             hipStream_t st) {
  dim3 grid((unsigned)(n * src.num_kv_heads), 2), block(kWave);
  return launch(quantize_kernel<SrcT, D, FP8>, grid, block, st, (const SrcT*)src.k_cache,
                (const SrcT*)src.v_cache, (uint8_t*)dst.k_cache, (uint8_t*)dst.v_cache,
                dst.k_scale, dst.v_scale, ids, src.num_kv_heads, src.num_blocks,
                (int64_t)(block_stride_bytes(src) / sizeof(SrcT)), (int64_t)block_stride_bytes(dst));
}

template <typename SrcT, int D>
int launch_qd(const pkv_cache_t& src, const pkv_cache_t& dst, const int32_t* ids, int n,
              hipStream_t st) {
  return dst.kv_dtype == PKV_FP8_E4M3 ? launch_q<SrcT, D, true>(src, dst, ids, n, st)
                                      : launch_q<SrcT, D, false>(src, dst, ids, n, st);
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

}  // namespace pkv
