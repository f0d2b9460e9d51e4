// Paged decode attention for gfx950.
//
// out[s][h] = sum_{t < L_s} softmax_t(scale * q[s][h] . k_t) v_t, with k_t and
// v_t found through the block table (16-token blocks, page "LLM 推理优化深度
// 解析", section "PagedAttention：vLLM 的显存碎片治理") and the G = Hq/Hkv query
// heads of a group sharing KV head h / G (same page, section "MQA 与 GQA").
//
// Work split.  A wavefront takes one KV head and all G query heads of its
// group, so every KV byte is read from HBM once.  Fixed split: one wavefront
// per (sequence, KV head, partition of partition_tokens).  Balanced split
// (the default): a persistent grid of as many wavefronts as the GPU holds at
// once cuts each KV head's blocks, all sequences laid end to end, into ranges
// of even work (decode_mfma_balanced_kernel).  Shared prefix: the common blocks run
// once for the queries of 16 / G sequences (decode_mfma_prefix_kernel).
// Several query tokens per sequence take the columns of one or two 16-column
// groups per wavefront, or passes.  The launch index is decoded
// KV-head-fastest: consecutive workgroups go to consecutive XCDs, so with 8
// KV heads every wavefront of one KV head runs on the same XCD and blocks
// shared between sequences (a common prefix) are served by that XCD's L2.
//
// Per 16-token block (bf16 / 8-bit KV, MFMA kernel):
//   1. the K and V tiles ([16][D], contiguous per (block, head)) are read with
//      coalesced 16-byte loads -- lane l takes bytes [16 l, 16 l + 16) of each
//      1 KiB slice -- two blocks ahead of the compute (two register buffers);
//      the partition's block-table entries are loaded once, 64 per vector
//      load, and broadcast from a lane, so no table read sits in front of a
//      tile load;
//   2. V codes are widened to bf16 (exact; INT8 V codes to fp16 1024 + u, also
//      exact), then the tiles are written to LDS with the 16-byte chunks of
//      row t XOR-swizzled by t, so the row-per-lane and column-per-lane reads
//      below are free of bank conflicts; 8- and 4-bit K codes are not widened
//      (step 3);
//   3. S = K q^T on the matrix cores: v_mfma_f32_16x16x32_bf16 with A = K rows
//      (token m = lane % 16) and B = the group's queries (head n = lane % 16,
//      zero for n >= G), D/32 instructions; E4M3 and E2M1 K codes go straight
//      into v_mfma_scale_f32_16x16x128_f8f6f4, INT8 and uint8 K codes into
//      v_mfma_i32_16x16x64_i8, against the query split into a high and a low
//      part in the same format (two or four instructions for D = 128);
//   4. online softmax in base 2: S is scaled by scale*log2(e) (times the
//      block's K scale for 8-bit KV), masked past L by selection, the block
//      maximum per head is shuffled across the four lanes holding that head,
//      and the running maximum only moves (rescaling the accumulator) when the
//      block maximum exceeds it by more than 8, so p <= 2^8;
//   5. O^T += V^T P on the matrix cores: v_mfma_f32_16x16x16_bf16 with A = V^T
//      and B = P, which the QK^T result already holds in the B-operand layout
//      (4 consecutive tokens per lane, head = lane % 16); V^T comes from the
//      row-major LDS tile through gfx950's transposing LDS read (one 8-byte
//      read per instruction instead of four 2-byte ones); for 8-bit KV, P is
//      multiplied by the block's V scale first.  INT8 V codes take an fp16
//      route instead: a byte permute makes two fp16 values 1024 + u at a time,
//      and P V runs on the fp16 MFMA (see widen16_k16).
// Asymmetric per-row pools (value = (code - zero) * scale for each row) run
// the matrix cores on the raw codes: row t's logit is
// scale_t * (q . code_t - zero_t * sum(q)) and the output is
// sum_t p_t scale_t code_t - sum_t p_t scale_t zero_t, so P is multiplied by
// each row's V scale and the second sum is kept beside the accumulator.
// The head index of a lane is lane % 16 in S, P and O alike, so the running
// maximum and sum stay lane-local.
//
// Sliding window: with window W > 0 a query at position p sees only the
// positions p - W < t <= p (page "KV Cache 与 PagedAttention", section
// "三个直接推论": keeping a window of recent tokens saves KV bytes).  The
// blocks before the earliest window of a sequence are left out of its block
// range, so they are never read, and rows outside a column's window are
// masked like rows past the end.
//
// Split context: each piece of a sequence (a fixed partition, or the part of
// a sequence one balanced range covers) writes its (max, sum, normalised
// output) to the workspace and a second kernel (reduce_kernel) combines them
// with the log-sum-exp rule; a sequence in one piece is written directly.
#include <atomic>
#include <type_traits>
#include <mutex>
#include <unordered_map>

#include "common.hpp"

namespace pkv {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __fp16 h16x2 __attribute__((ext_vector_type(2)));   // the packed conversion's type
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
// native clang vector (HIP's u32x4 is a wrapper struct that can keep arrays of
// it out of registers)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxDevices = 64;
// initial running maximum: finite, so exp2(x - m) of a masked logit (-inf)
// is 0 even before the first valid token
constexpr float kNoMax = -3.0e38f;
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag

enum { KV_BF16 = 0, KV_I8 = 1, KV_FP8 = 2, KV_U8Z = 3, KV_FP4 = 4 };
enum { OUT_F32 = 0, OUT_BF16 = 1 };

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer descriptor over [base, base + bytes); loads past `bytes` return
// zero and do not access memory.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// Cache policy bits of a buffer access on gfx950: sc0 = 1, nt = 2, sc1 = 16.
constexpr int kCpolNT = 2;

// K/V tile loads carry the non-temporal hint: a tile is read once per step
// (unless blocks are shared between sequences), and streaming the tiles lets
// the caches keep what every wavefront reads again: block tables, lengths,
// queries.  Measured on the Llama-3-8B-shape step: 117.1 -> 107.2 us.  The
// exception is a launch whose later passes over the query tokens read the
// same tiles again (kMqPasses below): there plain loads keep them in L2.
template <int CPOL>
__device__ __forceinline__ u32x4 buffer_load16_kv(rsrc_t r, int off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL));
}

// Column modes of the MFMA kernels (template parameter MQ): one query token
// per sequence (column n = head n of the group); several tokens that fit one
// pass (k * G <= 16 columns: column n = head n % G of token n / G); several
// passes, whose wavefronts for one (range, KV head) run side by side and share
// the tiles through L2 (balanced split only); several sequences whose
// tables share the range's blocks (a common prefix: column n = head n % G of
// sequence s + n / G), so a shared block is staged once for all of them; and
// two 16-column groups in one wavefront (k * G <= 32, balanced split), whose
// tiles are loaded, staged and read from LDS once for both groups.
enum { kMqOne = 0, kMqPass = 1, kMqPasses = 2, kMqSeqs = 3, kMqPair = 4 };

// Columns of a shared-prefix segment (MQ == kMqSeqs): sequences s .. s +
// nseq - 1 take columns [0, nseq * G); lcol is the context length of this
// lane's column's sequence and lmin the shortest member's.
struct SeqCols {
  int nseq;
  int lcol;
  int lmin;
};

// Byte offset of 16-byte chunk `chunk` of row `row` in an LDS tile of
// 16-bit rows of D elements, chunks XOR-swizzled by the row index, so the
// column-per-lane QK^T reads (16 rows, one chunk) are free of bank conflicts.
// LDS serves 128 bytes, eight 16-byte accesses, per cycle.  A bf16 tile is
// staged by eight lanes writing eight consecutive chunks of a row.  A tile
// widened from 8-bit codes at D = 128 is staged by each lane writing chunks
// 2m and then 2m + 1 of its row (E2M1: 4m + c), so eight lanes would cover 256
// bytes and meet every bank twice.  For those tiles the chunk index is rotated
// first (c -> c / 2 + 8 (c % 2)), which spreads each write over all eight
// bank groups; at D = 64 a row is one 128-byte sweep and the plain swizzle
// already does.
template <int D, int KV>
__device__ __forceinline__ int lds_off(int row, int chunk) {
  constexpr int kChunks = D / 8;
  constexpr bool kRotate = KV != KV_BF16 && D == 128;
  const int c = kRotate ? (chunk >> 1) | ((chunk & 1) * (kChunks / 2)) : chunk;
  return row * (D * 2) + ((c ^ (row & (kChunks - 1))) << 4);
}

// 16 8-bit V codes -> 16 bf16 values (two 16-byte chunks), exact.
// E4M3: the gfx950 conversion instruction, two codes at a time.
// Asymmetric uint8: an unsigned byte converts to binary32 in one instruction,
// and u < 256 has at most 8 significant bits, so its binary32 upper half is u
// in bf16 exactly.  (INT8 V codes take the cheaper fp16 route of widen16_k16;
// K codes are not widened.)
template <int KV>
__device__ __forceinline__ void widen16(u32x4 c, u32x4& lo, u32x4& hi) {
  static_assert(KV == KV_FP8 || KV == KV_U8Z, "E4M3 or uint8 codes");
  const uint32_t w[4] = {c[0], c[1], c[2], c[3]};
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (KV == KV_U8Z) {
      const uint32_t u = w[i];
      const float f0 = (float)(u & 0xFFu);
      const float f1 = (float)((u >> 8) & 0xFFu);
      const float f2 = (float)((u >> 16) & 0xFFu);
      const float f3 = (float)(u >> 24);
      // bytes 2,3 of the low value, then bytes 2,3 of the high value
      o[2 * i] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
      o[2 * i + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    } else {
      bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false);
      bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true);
      o[2 * i] = __builtin_bit_cast(uint32_t, a);
      o[2 * i + 1] = __builtin_bit_cast(uint32_t, b);
    }
  }
  lo = u32x4{o[0], o[1], o[2], o[3]};
  hi = u32x4{o[4], o[5], o[6], o[7]};
}

// 16 INT8 V codes -> 16 fp16 values 1024 + u with u = c + 128, exact: fp16
// 1024 has the bits 0x6400 and a unit in the last place of 1, so a byte
// permute that puts code u under the byte 0x64 makes 1024 + u, two codes per
// permute.  The output takes (1024 + 128) * sum(P) back off.
template <int KV>
__device__ __forceinline__ void widen16_k16(u32x4 c, u32x4& lo, u32x4& hi) {
  constexpr uint32_t kExp = 0x64646464u;
  uint32_t o[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = KV == KV_I8 ? c[i] ^ 0x80808080u : c[i];
    o[2 * i] = __builtin_amdgcn_perm(kExp, u, 0x04010400u);       // u0, u1
    o[2 * i + 1] = __builtin_amdgcn_perm(kExp, u, 0x04030402u);   // u2, u3
  }
  lo = u32x4{o[0], o[1], o[2], o[3]};
  hi = u32x4{o[4], o[5], o[6], o[7]};
}

// 32 E2M1 codes (16 bytes, two per byte, low nibble first) -> 32 bf16
// values (four 16-byte chunks), exact: the gfx950 conversion instruction
// turns the two codes of one byte into two bf16 values.
__device__ __forceinline__ void widen32_fp4(u32x4 c, u32x4 (&o)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t w = c[k];
    o[k] = u32x4{
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2)),
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3))};
  }
}

template <int D, int OUT>
__device__ __forceinline__ void store_out4(void* out, size_t idx, f32x4 v) {
  if constexpr (OUT == OUT_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = v;
  } else {
    uint2 w;
    w.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
    w.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + idx) = w;
  }
}

// ---------------------------------------------------------------------------
// MFMA path: q bf16; KV bf16, int8, E4M3, asymmetric uint8 or E2M1; D = 64 or
// 128; G <= 16.

// Launch-wide arguments of the MFMA kernels.
struct MfmaArgs {
  const uint16_t* q;
  const uint8_t* kc;
  const uint8_t* vc;
  const float* ksc;   // 8-bit pools: scales per (block, head), or per row
  const float* vsc;
  const uint8_t* kz;  // asymmetric per-row pools: zero points per row
  const uint8_t* vz;
  const int32_t* tables;
  const int32_t* lens;
  int max_blocks;
  int num_seqs;
  int hq, hkv, G, num_blocks;
  size_t blk_stride;  // bytes from one block to the next in each pool
  float scale_log2;
  float* ws_m;        // split partials: running maximum (log2 units)
  float* ws_l;        //                 softmax denominator
  float* ws_o;        //                 normalised output row
  int32_t* ws_count;  // balanced split: segments of each sequence
  int kstride;        // partial slots per (sequence, query head)
  int part_blocks;    // fixed split: blocks per partition
  int min_blocks;     // balanced split: fewest blocks one wavefront takes
  int ntok;           // query tokens per sequence (1: decode)
  int tok_per_pass;   // query tokens one wavefront takes (ntok * G columns split in passes)
  int window;         // sliding window in tokens, 0 for none
  int prefix_blocks;  // shared-prefix split: table entries every sequence shares
  int seqs_per_group; //                     sequences whose columns share a wavefront
  void* out;
  const uint8_t* kn;  // fused append (decode step): new K/V rows, or null
  const uint8_t* vn;
  uint8_t* kc_w;
  uint8_t* vc_w;
};

__device__ __forceinline__ int clamp_len(int L, int max_blocks) {
  return (L < 0 || L > max_blocks * kBlock) ? 0 : L;
}

// First logical block any query of a sequence of length L can see: with a
// window W the earliest query (position L - ntok) starts at L - ntok + 1 - W.
__device__ __forceinline__ int first_block(int L, int ntok, int window) {
  if (window <= 0) return 0;
  const int lo = L - ntok + 1 - window;
  return lo > 0 ? lo / kBlock : 0;
}

// Blocks a sequence of length L contributes: [first_block, ceil(L / 16)).
__device__ __forceinline__ int seq_blocks(int L, int ntok, int window) {
  return L > 0 ? (L + kBlock - 1) / kBlock - first_block(L, ntok, window) : 0;
}

// 2^x for the softmax weights: the hardware instruction alone.  A weight
// below 2^-126 of the running maximum comes out as zero rather than as a
// denormal, which no output can tell apart.
__device__ __forceinline__ float exp2_weight(float x) { return __builtin_amdgcn_exp2f(x); }

// Inclusive prefix sum across the wavefront (lane order).
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int readlane_i(int v, int l) { return __builtin_amdgcn_readlane(v, l); }

// Zero output rows of the query heads of KV head g of an empty sequence s
// (every query token of this wavefront's pass).
template <int D, int OUT>
__device__ __forceinline__ void zero_rows(const MfmaArgs& a, int s, int g, int tok0) {
  const int lane = threadIdx.x;
  const int j = lane >> 4, n = lane & 15;
  const int ti = tok0 + n / a.G;
  if (n >= a.G * a.tok_per_pass || ti >= a.ntok) return;
  const size_t row = ((size_t)s * a.ntok + ti) * a.hq + g * a.G + n % a.G;
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    store_out4<D, OUT>(a.out, row * D + 16 * t + 4 * j, f32x4{0.f, 0.f, 0.f, 0.f});
}

// Attention of the G query heads of KV head g of sequence s (length L) over
// its logical blocks [b0, b1).  `whole`: the range is the whole context, so the
// normalised rows go to `out`; otherwise the partial (max, sum, output) goes
// to partial slot `slot` of each row.
template <int D, int KV, int OUT, int NST, int MQ>
__device__ __forceinline__ void mfma_segment(const MfmaArgs& a, int s, int g, int L, int b0,
                                             int b1, int slot, bool whole, int tok0,
                                             uint8_t* lds_k, uint8_t* lds_v, uint8_t* lds_p,
                                             SeqCols sc = SeqCols{1, 0, 0}) {
  constexpr int kBits = KV == KV_BF16 ? 16 : KV == KV_FP4 ? 4 : 8;
  constexpr int kRowBytes = D * kBits / 8;       // bytes of one token's row in HBM
  constexpr int kTile = kBlock * kRowBytes;      // bytes of one (block, head) tile in HBM
  // 16-byte loads per lane per tile (a 512-byte tile leaves lanes 32-63 idle)
  constexpr int kLoads = kTile >= 1024 ? kTile / 1024 : 1;
  // one binary32 scale per (block, head) for K and for V
  constexpr bool kBlockScale = KV == KV_I8 || KV == KV_FP8 || KV == KV_FP4;
  constexpr int kNKK = D / 32;              // QK^T instructions per block
  constexpr int kNT = D / 16;               // PV instructions per block
  // E4M3 and E2M1 K codes enter v_mfma_scale_f32_16x16x128_f8f6f4 as they
  // are stored (A = K rows, 128 codes per row), with the queries as two
  // E4M3 operands (hi + lo): no widening.  Lane (j, n) holds 32 codes of row
  // n; past head_dim they are zero.  E2M1: codes 32 j .. 32 j + 31, one
  // 16-byte load straight into the operand (the four lanes of a row read
  // its 64 bytes, so a load stays contiguous).  E4M3: the tile is loaded
  // linearly and staged in LDS as raw codes (16-byte chunks XOR-swizzled by
  // row), and lane (j, n) reads back chunks 2 j and 2 j + 1 of row n; loading
  // those 32 bytes directly would touch every cache line twice.
  // INT8 K codes take the same raw staging into v_mfma_i32_16x16x64_i8 (two
  // 64-code halves per row), with the queries as two int8 operands (hi, lo):
  // the products are exact integers.  Per-row uint8 codes c are staged as
  // the int8 c - 128 and the row's logit takes (128 - zero) sum(q) back on.
  constexpr bool kIntK = KV == KV_I8 || KV == KV_U8Z;
  constexpr bool kDirectK = KV == KV_FP8 || KV == KV_FP4 || kIntK;
  constexpr int kKLoads = KV == KV_FP4 ? 1 : kLoads;
  const int lane = threadIdx.x;
  const int j = lane >> 4;   // token quad (rows 4j..4j+3 of S) / k-slice
  const int n = lane & 15;   // head column
  const int G = a.G, hq = a.hq, hkv = a.hkv, num_blocks = a.num_blocks;
  // column n of S, P and O: query token ti (several per sequence only in the
  // token modes), sequence s_col (several only for a shared prefix) and head
  // h of the group
  constexpr bool kTok = MQ == kMqPass || MQ == kMqPasses || MQ == kMqPair;
  constexpr bool kSeqs = MQ == kMqSeqs;
  // 16-column groups of this wavefront: group c takes the query tokens
  // tok0 + c * tok_per_pass ..; the tiles are shared by the groups
  constexpr int CG = MQ == kMqPair ? 2 : 1;
  const int s_col = kSeqs ? s + n / G : s;
  const int h = g * G + (MQ != kMqOne ? n % G : n);
  int ti[CG];
  bool has_head[CG];
  size_t out_row[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    ti[c] = kTok ? tok0 + c * a.tok_per_pass + n / G : 0;
    has_head[c] = kTok ? (n < G * a.tok_per_pass && ti[c] < a.ntok)
                       : kSeqs ? n < G * sc.nseq : n < G;
    out_row[c] = kTok ? ((size_t)s * a.ntok + ti[c]) * hq + h : (size_t)s_col * hq + h;
  }
  // last key position + 1 this column may see (causal within the chunk, or
  // its own sequence's length), and with a window the first one (lo_col), and
  // the lowest first position of all columns of this pass (lo_seg): V rows
  // below it are zeroed in LDS
  constexpr int kNoLo = -(1 << 30);
  int lim[CG], lo_col[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    lim[c] = kTok ? L - a.ntok + ti[c] + 1 : kSeqs ? sc.lcol : L;
    lo_col[c] = a.window > 0 ? lim[c] - a.window : kNoLo;
  }
  const int lo_seg = a.window > 0 ? (kTok ? L - a.ntok + tok0 + 1 : L) - a.window : kNoLo;

  f32x4 acc[CG][kNT];
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[c][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // queries of this group as the B operand of S = K q^T: lane (j, n) holds
  // q[h][32 kk + 8 j .. + 8] for each kk
  // queries as the B operand: 8 values per MFMA k-slice, or (direct K) the
  // 32 values that pair with this lane group's K codes in the k order of
  // v_mfma_scale_f32_16x16x128_f8f6f4.  With an E4M3 A operand lane group j
  // holds k = 32 j .. 32 j + 31; with an E2M1 A operand its 32 codes pair
  // with the B bytes of k = 16 j .. 16 j + 15 and 64 + 16 j .. 64 + 16 j + 15
  // (taken from an in-bounds probe of the instruction), so B lane group j
  // holds q[16 j ..] and q[64 + 16 j ..]; past head_dim the values are 0.
  constexpr int kQV = kDirectK ? 4 : kNKK;
  bf16x8 qop[CG][kQV];
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const uint16_t* qrow = a.q + (has_head[c] ? out_row[c] : (size_t)s * a.ntok * hq) * D;
#pragma unroll
    for (int kk = 0; kk < kQV; ++kk) {
      int off = 32 * kk + 8 * j;
      if constexpr (KV == KV_FP8 || kIntK) off = 32 * j + 8 * kk;
      if constexpr (KV == KV_FP4) off = kk < 2 ? 16 * j + 8 * kk : 64 + 16 * j + 8 * (kk - 2);
      bf16x8 v = {};
      if (!kDirectK || off < D) v = *reinterpret_cast<const bf16x8*>(qrow + off);
      qop[c][kk] = has_head[c] ? v : bf16x8{};
    }
  }
  // Direct K: the queries, scaled per head by 2^qe, split into two operands
  // whose sum holds them to a few ulp of bf16 or better.  E4M3: the largest
  // |q| 2^qe lies in [128, 256); hi = nearest E4M3 of q 2^qe and lo = nearest
  // E4M3 of the (exact) remainder, about 8 significant bits together.  INT8:
  // the largest |q| 2^qe lies in [2^12, 2^13); q 2^qe is rounded to an
  // integer u = 128 hi + lo with hi = (u + 64) >> 7 and lo in [-64, 63], both
  // int8, 13 bits in all, and the two integer products are exact.  The logit
  // multiplies by 2^-qe.
  i32x8 qhi8[CG] = {}, qlo8[CG] = {};
  float qinv_d[CG];
  int qsum_i[CG];   // per-row uint8: sum of this lane's integer queries u
#pragma unroll
  for (int c = 0; c < CG; ++c) {
  qinv_d[c] = 1.f;
  qsum_i[c] = 0;
  if constexpr (kDirectK) {
    float mq = 0.f;
#pragma unroll
    for (int kk = 0; kk < kQV; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) mq = fmaxf(mq, fabsf(static_cast<float>(qop[c][kk][e])));
    mq = rows_max(mq);
    constexpr int kTop = kIntK ? 13 : 8;
    const int qe = mq > 0.f ? kTop - __builtin_amdgcn_frexp_expf(mq) : 0;
    qinv_d[c] = __builtin_ldexpf(1.f, -qe);
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = 4 * w + e;   // byte v of the operand
        y[e] = __builtin_ldexpf(static_cast<float>(qop[c][v / 8][v % 8]), qe);
      }
      if constexpr (kIntK) {
        uint32_t hw = 0, lw = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int u = (int)rintf(y[e]);
          qsum_i[c] += u;
          const int hi = (u + 64) >> 7;
          const int lo = u - (hi << 7);
          hw |= (uint32_t)(uint8_t)(int8_t)hi << (8 * e);
          lw |= (uint32_t)(uint8_t)(int8_t)lo << (8 * e);
        }
        qhi8[c][w] = (int)hw;
        qlo8[c][w] = (int)lw;
      } else {
        s16x2 h = {0, 0};
        h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, y[0], y[1], 1.0f, false);
        h = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(h, y[2], y[3], 1.0f, true);
        const uint32_t hw = __builtin_bit_cast(uint32_t, h);
        const f32x2 d01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, 1.0f, false);
        const f32x2 d23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hw, 1.0f, true);
        s16x2 l = {0, 0};
        l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, y[0] - d01[0], y[1] - d01[1], 1.0f,
                                                      false);
        l = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(l, y[2] - d23[0], y[3] - d23[1], 1.0f, true);
        qhi8[c][w] = (int)hw;
        qlo8[c][w] = __builtin_bit_cast(int, l);
      }
    }
  }
  // per-row uint8: the integer queries' sum over the head (exact: at most
  // 128 * 2^13 in magnitude)
  if constexpr (KV == KV_U8Z) qsum_i[c] = (int)rows_sum((float)qsum_i[c]);
  }

  const int32_t* trow = a.tables + (size_t)s * a.max_blocks;
  const size_t blk_stride = a.blk_stride;
  const uint8_t* kbase = a.kc + (size_t)g * kTile;
  const uint8_t* vbase = a.vc + (size_t)g * kTile;

  // Fused append (decode step): the new token is position L-1, row L-1 mod 16
  // of logical block (L-1)/16.  The wavefront whose range holds that block
  // loads the token's K/V row for its KV head now; when it stages that block
  // it puts the row into the LDS tile and stores it into the pool, so it
  // attends over the new token without a separate cache-write launch.  No
  // other wavefront reads that block's tile of this head.
  constexpr int kRowChunks = D * 2 / 16;   // 16-byte chunks of one bf16 row
  int new_b = -1, new_r = 0;
  u32x4 knew = {0u, 0u, 0u, 0u}, vnew = {0u, 0u, 0u, 0u};
  if constexpr (KV == KV_BF16 && !kSeqs) {
    if (a.kn != nullptr && (L - 1) / kBlock >= b0 && (L - 1) / kBlock < b1) {
      new_b = (L - 1) / kBlock;
      new_r = (L - 1) % kBlock;
      if (lane < kRowChunks) {
        const size_t src = ((size_t)s * hkv + g) * (D * 2) + lane * 16;
        knew = *reinterpret_cast<const u32x4*>(a.kn + src);
        vnew = *reinterpret_cast<const u32x4*>(a.vn + src);
      }
    }
  }

  float m[CG], lsum[CG], psum[CG];   // running reference maximum (log2 units); this
                                     // lane's share of the softmax denominator
  // INT8: V codes enter P V as fp16 1024 + u too, and P, which carries the
  // block's V scale, as fp16.  To keep P finite it carries the V scale times
  // vfac = 2^-E, chosen per 64-block chunk so that the chunk's largest V scale
  // times vfac lies in [2^6, 2^7): P <= 2^8 * 2^7 < 65504.  The accumulator is
  // rescaled (exactly, by a power of two) when vfac changes between chunks and
  // divided by vfac at the end.
  constexpr bool kV16 = KV == KV_I8;
  float vfac = 0.f;
  // psum: INT8: this lane's share of sum(P), rescaled like the accumulator;
  // asymmetric rows: of sum_t P_t zero_t, likewise
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    m[c] = kNoMax;
    lsum[c] = 0.f;
    psum[c] = 0.f;
  }

  // The range is walked in chunks of up to 64 blocks.  Per chunk, lane i
  // loads block-table entry i (and, for 8-bit KV, that block's two scales);
  // each block's id is then broadcast from its lane.  Tile loads go through
  // buffer descriptors built per block: a block past the chunk or with an
  // id outside the pool gets a zero-length descriptor, so its loads return
  // zeros without touching memory.  Every iteration therefore issues the
  // same loads and the wait counts stay exact: while block b is computed,
  // the loads of blocks b+1 and b+2 are in flight in two register buffers.
  for (int c0 = b0; c0 < b1; c0 += 64) {
    const int c1 = min(c0 + 64, b1);
    const int tab = (c0 + lane < c1) ? trow[c0 + lane] : -1;
    float ks_l = 1.f, vs_l = 1.f;
    if constexpr (kBlockScale) {
      if (tab >= 0 && tab < num_blocks) {
        ks_l = a.ksc[(size_t)tab * hkv + g];
        vs_l = a.vsc[(size_t)tab * hkv + g];
      }
    }
    if constexpr (kV16) {
      const float vmax = wave_max(tab >= 0 && tab < num_blocks ? fabsf(vs_l) : 0.f);
      const float f = vmax > 0.f ? __builtin_ldexpf(1.f, 7 - __builtin_amdgcn_frexp_expf(vmax))
                                 : 1.f;
      if (f != vfac) {
        if (vfac > 0.f) {
          const float r = f / vfac;
#pragma unroll
          for (int c = 0; c < CG; ++c) {
#pragma unroll
            for (int t = 0; t < kNT; ++t) acc[c][t] *= r;
            psum[c] *= r;
          }
        }
        vfac = f;
      }
    }
    auto phys_of = [&](int b) -> int {
      return b < c1 ? __builtin_amdgcn_readlane(tab, b - c0) : -1;
    };
    // Asymmetric rows: the block's 16 K scales land in lanes 0-15, its 16 V
    // scales in lanes 16-31, its K zero points (4 per dword) in lanes 32-35
    // and its V zero points in lanes 36-39; every other lane's offset lies
    // outside the descriptor's range and reads zero.
    auto load_tile = [&](u32x4 (&kr)[kKLoads], u32x4 (&vr)[kLoads], u32x4& pr, int ph, int bl) {
      const bool in = ph >= 0 && ph < num_blocks;
      const size_t off = in ? (size_t)ph * blk_stride : 0;
      const rsrc_t rk = make_rsrc(kbase + off, in ? kTile : 0);
      // V rows at or past the end are outside the descriptor and load as
      // zeros: bf16 and E4M3 bytes there may encode NaN or infinity, which a
      // zero weight would not cancel
      const int vrows = __builtin_amdgcn_readfirstlane(min(max(L - bl * kBlock, 0), kBlock));
      const rsrc_t rv = make_rsrc(vbase + off, in ? vrows * kRowBytes : 0);
      // tiles other wavefronts read again (later passes, other sequence
      // groups of a shared prefix) stay cached
      constexpr int kCpol = MQ == kMqPasses || MQ == kMqSeqs ? 0 : kCpolNT;
#pragma unroll
      for (int i = 0; i < kKLoads; ++i) {
        if constexpr (KV == KV_FP4) {
          // row n, bytes 16 j .. 16 j + 15 (codes 32 j ..); past head_dim the
          // offset leaves the descriptor and loads zeros
          const int off = 16 * j < kRowBytes ? n * kRowBytes + 16 * j : kTile;
          kr[i] = buffer_load16_kv<kCpol>(rk, off);
        } else {
          kr[i] = buffer_load16_kv<kCpol>(rk, i * 1024 + lane * 16);
        }
      }
#pragma unroll
      for (int i = 0; i < kLoads; ++i) vr[i] = buffer_load16_kv<kCpol>(rv, i * 1024 + lane * 16);
      if constexpr (KV == KV_U8Z) {
        const size_t row0 = in ? ((size_t)ph * hkv + g) * kBlock : 0;
        const rsrc_t rks = make_rsrc(a.ksc + row0, in ? kBlock * 4 : 0);
        const rsrc_t rvs = make_rsrc(a.vsc + row0, in ? kBlock * 4 : 0);
        const rsrc_t rkz = make_rsrc(a.kz + row0, in ? kBlock : 0);
        const rsrc_t rvz = make_rsrc(a.vz + row0, in ? kBlock : 0);
        pr[0] = __builtin_amdgcn_raw_buffer_load_b32(rks, lane * 4, 0, 0);
        pr[1] = __builtin_amdgcn_raw_buffer_load_b32(rvs, (lane - 16) * 4, 0, 0);
        pr[2] = __builtin_amdgcn_raw_buffer_load_b32(rkz, (lane - 32) * 4, 0, 0);
        pr[3] = __builtin_amdgcn_raw_buffer_load_b32(rvz, (lane - 36) * 4, 0, 0);
      }
    };

    // Stage block b from (kr, vr) into LDS, refill the buffer with block
    // b+2, then run QK^T, the softmax update and PV for block b.
    auto process = [&](u32x4 (&kr)[kKLoads], u32x4 (&vr)[kLoads], u32x4& pr, int& ph, int b) {
      const int cur = ph;
      const bool cur_ok = cur >= 0 && cur < num_blocks;
      const int valid = cur_ok ? min(kBlock, L - b * kBlock) : 0;  // valid rows
      const int vlo = lo_seg - b * kBlock;                          // rows below: outside

      // V rows past the end arrive as zeros (see load_tile); rows below a
      // window's first position are zeroed here, for the codes that can
      // encode NaN or infinity (bf16, E4M3).  INT8, uint8 and E2M1 codes are
      // finite, so their rows with zero weight add exactly nothing.
      constexpr bool kZeroLow = KV == KV_BF16 || KV == KV_FP8;
      const bool vlow = kZeroLow && vlo > 0;

      // the previous block's LDS reads come before this block's writes
      wave_sync();
      // ---- stage into LDS as bf16
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        if constexpr (KV == KV_BF16) {
          const int chunk = i * 64 + lane;          // 16-byte chunk of the tile
          const int row = chunk / (D / 8), ch = chunk % (D / 8);
          *reinterpret_cast<u32x4*>(lds_k + lds_off<D, KV>(row, ch)) = kr[i];
          *reinterpret_cast<u32x4*>(lds_v + lds_off<D, KV>(row, ch)) = vr[i];
        } else if constexpr (KV == KV_FP4) {
          const int e0 = (i * 1024 + lane * 16) * 2;   // first of this lane's 32 codes
          const int row = e0 / D, col = e0 % D;
          if (row < kBlock) {
            u32x4 vw[4];
            widen32_fp4(vr[i], vw);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              *reinterpret_cast<u32x4*>(lds_v + lds_off<D, KV>(row, col / 8 + c)) = vw[c];
          }
        } else if constexpr (KV == KV_FP8) {
          const int byte = (i * 64 + lane) * 16;    // first code of this chunk
          const int row = byte / D, col = byte % D; // 16 codes = 2 bf16 chunks
          u32x4 vlo4, vhi;
          widen16<KV>(vr[i], vlo4, vhi);
          *reinterpret_cast<u32x4*>(lds_v + lds_off<D, KV>(row, col / 8)) = vlo4;
          *reinterpret_cast<u32x4*>(lds_v + lds_off<D, KV>(row, col / 8 + 1)) = vhi;
          // raw K codes: chunk c of row r at r * D + 16 (c ^ (r mod D / 16))
          constexpr int kC = D / 16;
          *reinterpret_cast<u32x4*>(lds_k + row * D + 16 * ((col / 16) ^ (row % kC))) = kr[i];
        } else {
          const int byte = (i * 64 + lane) * 16;    // first code of this chunk
          const int row = byte / D, col = byte % D; // 16 codes = 2 bf16 chunks
          u32x4 vlo4, vhi;
          if constexpr (kV16)
            widen16_k16<KV>(vr[i], vlo4, vhi);
          else
            widen16<KV>(vr[i], vlo4, vhi);
          *reinterpret_cast<u32x4*>(lds_v + lds_off<D, KV>(row, col / 8)) = vlo4;
          *reinterpret_cast<u32x4*>(lds_v + lds_off<D, KV>(row, col / 8 + 1)) = vhi;
          // raw K codes, as for E4M3 (uint8: as the int8 c - 128)
          constexpr int kC = D / 16;
          u32x4 kw = kr[i];
          if constexpr (KV == KV_U8Z) kw ^= u32x4{0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
          *reinterpret_cast<u32x4*>(lds_k + row * D + 16 * ((col / 16) ^ (row % kC))) = kw;
        }
      }
      if constexpr (kZeroLow) {
        if (vlow) {   // overwrite the V rows below the window with zeros
#pragma unroll
          for (int i = 0; i < kLoads; ++i) {
            const int chunk = i * 64 + lane;
            const int rb = KV == KV_BF16 ? D * 2 : D;   // tile bytes per row
            const int row = chunk * 16 / rb;
            const int ch = KV == KV_BF16 ? chunk % (D / 8) : (chunk * 16 % D) / 8;
            if (row < vlo) {
              *reinterpret_cast<u32x4*>(lds_v + lds_off<D, KV>(row, ch)) = u32x4{0u, 0u, 0u, 0u};
              if constexpr (KV != KV_BF16)
                *reinterpret_cast<u32x4*>(lds_v + lds_off<D, KV>(row, ch + 1)) = u32x4{0u, 0u, 0u, 0u};
            }
          }
        }
      }
      if constexpr (KV == KV_BF16 && !kSeqs) {
        if (b == new_b && lane < kRowChunks) {   // the appended token's row
          *reinterpret_cast<u32x4*>(lds_k + lds_off<D, KV>(new_r, lane)) = knew;
          *reinterpret_cast<u32x4*>(lds_v + lds_off<D, KV>(new_r, lane)) = vnew;
          if (cur_ok) {
            const size_t dst = (size_t)cur * blk_stride + (size_t)g * kTile + new_r * (D * 2) +
                               lane * 16;
            *reinterpret_cast<u32x4*>(a.kc_w + dst) = knew;
            *reinterpret_cast<u32x4*>(a.vc_w + dst) = vnew;
          }
        }
      }
      float kscale = 1.f, vscale = 1.f;
      if constexpr (kBlockScale) {
        if (b < c1) {
          kscale = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ks_l), b - c0));
          vscale = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(vs_l), b - c0));
        }
      }
      // asymmetric rows: lane (j, n) takes the scales and zero points of its
      // rows 4j..4j+3 through LDS
      f32x4 ks4 = {1.f, 1.f, 1.f, 1.f}, vs4 = {1.f, 1.f, 1.f, 1.f};
      uint32_t kzw = 0u, vzw = 0u;
      if constexpr (KV == KV_U8Z) {
        const uint32_t pw = pr[0] | pr[1] | pr[2] | pr[3];
        if (lane < 40) *reinterpret_cast<uint32_t*>(lds_p + 4 * lane) = pw;
      }
      // every lane's LDS writes come before any lane reads them back
      wave_sync();
      if constexpr (KV == KV_U8Z) {
        ks4 = *reinterpret_cast<const f32x4*>(lds_p + 16 * j);
        vs4 = *reinterpret_cast<const f32x4*>(lds_p + 64 + 16 * j);
        kzw = *reinterpret_cast<const uint32_t*>(lds_p + 128 + 4 * j);
        vzw = *reinterpret_cast<const uint32_t*>(lds_p + 144 + 4 * j);
      }

      // direct K: E2M1 codes leave the buffer before its refill; E4M3 codes
      // come back from LDS (chunks 2 j and 2 j + 1 of row n)
      i32x8 ka = {};
      if constexpr (KV == KV_FP4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) ka[e] = (int)kr[0][e];
      } else if constexpr (KV == KV_FP8 || kIntK) {
        constexpr int kC = D / 16;
        // (always true for D = 128, where the four lane groups cover the row)
        if (kC == 8 || 2 * j < kC) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const u32x4 c = *reinterpret_cast<const u32x4*>(
                lds_k + n * D + 16 * ((2 * j + h) ^ (n % kC)));
#pragma unroll
            for (int e = 0; e < 4; ++e) ka[4 * h + e] = (int)c[e];
          }
        }
      }

      // ---- refill this buffer with block b+NST (zero-length if absent)
      ph = phys_of(b + NST);
      load_tile(kr, vr, pr, ph, b + NST);

      // ---- S = K q^T: lane (j, n) gets S[token 4j + i][head n]
      f32x4 svc[CG];
      int skc[CG][4];   // integer products (INT8, uint8)
#pragma unroll
      for (int c = 0; c < CG; ++c) {
      f32x4 sv = {0.f, 0.f, 0.f, 0.f};
      int sk[4] = {0, 0, 0, 0};
      if constexpr (kIntK) {
        typedef int i32x4 __attribute__((ext_vector_type(4)));
        const i32x4 a0 = {ka[0], ka[1], ka[2], ka[3]}, a1 = {ka[4], ka[5], ka[6], ka[7]};
        const i32x4 h0 = {qhi8[c][0], qhi8[c][1], qhi8[c][2], qhi8[c][3]};
        const i32x4 h1 = {qhi8[c][4], qhi8[c][5], qhi8[c][6], qhi8[c][7]};
        const i32x4 l0 = {qlo8[c][0], qlo8[c][1], qlo8[c][2], qlo8[c][3]};
        const i32x4 l1 = {qlo8[c][4], qlo8[c][5], qlo8[c][6], qlo8[c][7]};
        i32x4 ah = {0, 0, 0, 0}, al = {0, 0, 0, 0};
        ah = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, h0, ah, 0, 0, 0);
        ah = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, h1, ah, 0, 0, 0);
        al = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, l0, al, 0, 0, 0);
        al = __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, l1, al, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) sk[i] = ah[i] * 128 + al[i];
        if constexpr (KV == KV_I8) {
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[i] = (float)sk[i];
        }
      } else if constexpr (kDirectK) {
        constexpr int kFmtA = KV == KV_FP8 ? 0 : 4;   // A operand: E4M3 or E2M1 codes
        sv = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qhi8[c], sv, kFmtA, 0, 0, 127,
                                                              0, 127);
        sv = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qlo8[c], sv, kFmtA, 0, 0, 127,
                                                              0, 127);
      }
#pragma unroll
      for (int kk = 0; kk < (kDirectK ? 0 : kNKK); ++kk) {
        const bf16x8 kop = *reinterpret_cast<const bf16x8*>(lds_k + lds_off<D, KV>(n, 4 * kk + j));
        sv = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qop[c][kk], sv, 0, 0, 0);
      }
      svc[c] = sv;
#pragma unroll
      for (int i = 0; i < 4; ++i) skc[c][i] = sk[i];
      }

      // ---- V^T operands of O^T += V^T P, read now so that their LDS latency
      // passes during the softmax.  Lane (j, n) supplies V[4j + i][16 t + n],
      // i < 4.  ds_read_b64_tr_b16 works on groups of 16 lanes: each lane
      // reads 4 consecutive bf16 and lane 4a + b of the group receives element
      // b of the words read by lanes a, a + 4, a + 8, a + 12.  So lane n of
      // group j reads row 4j + n / 4, columns 16 t + 4 (n % 4) .. + 3 (one
      // 8-byte piece of a 16-byte LDS chunk).
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      s16x4 vt[kNT];
      {
        const int vrow = 4 * j + (n >> 2);
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
          const int col = 16 * t + 4 * (n & 3);
          vt[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4*)(lds_v + lds_off<D, KV>(vrow, col >> 3) +
                                                         (col & 7) * 2));
        }
      }

      // ---- online softmax (base 2), then PV, per column group
#pragma unroll
      for (int c = 0; c < CG; ++c) {
      const f32x4 sv = svc[c];
      const int* sk = skc[c];
      const float cb = a.scale_log2 * kscale * qinv_d[c];
      float x[4];
      float mx = -INFINITY;
      const int vcol = MQ ? (cur_ok ? min(kBlock, lim[c] - b * kBlock) : 0) : valid;
      const int vmin = lo_col[c] - b * kBlock;   // this column's first row in its window
      // one query token per sequence: every row of a block is in range for
      // every column unless the block is the last (or, with a window, the
      // first) of the sequence, so the per-row selects are skipped; a shared
      // prefix block likewise when it ends within the shortest member
      const bool full = kSeqs ? cur_ok && (b + 1) * kBlock <= sc.lmin
                              : !MQ && vcol >= kBlock && vmin <= 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (KV == KV_U8Z)
          // sum u (c - z) = sum u (c - 128) + (128 - z) sum u, all in int32
          x[i] = (float)(sk[i] + (128 - (int)((kzw >> (8 * i)) & 0xFFu)) * qsum_i[c]) *
                 (cb * ks4[i]);
        else
          x[i] = sv[i] * cb;
      }
      if (!full) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!(4 * j + i < vcol && 4 * j + i >= vmin)) x[i] = -INFINITY;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = __builtin_elementwise_maximum(mx, x[i]);
      mx = rows_max(mx);
      const bool bump = mx > m[c] + kRescaleSlack;
      if (__any(bump)) {
        const float mnew = bump ? mx : m[c];
        const float alpha = exp2_weight(m[c] - mnew);
        lsum[c] *= alpha;
        if constexpr (KV == KV_I8 || KV == KV_U8Z) psum[c] *= alpha;
#pragma unroll
        for (int t = 0; t < kNT; ++t) acc[c][t] *= alpha;
        m[c] = mnew;
      }
      f32x4 pw;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float pe = exp2_weight(x[i] - m[c]);
        lsum[c] += pe;
        if constexpr (KV == KV_U8Z)   // rows past the end have p = 0 but may hold any scale
          pw[i] = full || (4 * j + i < vcol && 4 * j + i >= vmin) ? pe * vs4[i] : 0.f;
        else
          pw[i] = pe * (kV16 ? vscale * vfac : vscale);
      }
      if constexpr (kV16) {
        // two paired conversions (toward zero: under 2^-10 relative, finer
        // than bf16 to nearest); sum(P) is taken over the converted values,
        // two at a time by dot products with (1, 1)
        const h16x2 p01 = __builtin_amdgcn_cvt_pkrtz(pw[0], pw[1]);
        const h16x2 p23 = __builtin_amdgcn_cvt_pkrtz(pw[2], pw[3]);
        const f16x4 poh = __builtin_bit_cast(f16x4, __builtin_shufflevector(p01, p23, 0, 1, 2, 3));
        const h16x2 kOnes = {(__fp16)1.0f, (__fp16)1.0f};
        psum[c] = __builtin_amdgcn_fdot2(p01, kOnes, psum[c], false);
        psum[c] = __builtin_amdgcn_fdot2(p23, kOnes, psum[c], false);
        // ---- O^T += V^T P
#pragma unroll
        for (int t = 0; t < kNT; ++t)
          acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, vt[t]), poh,
                                                           acc[c][t], 0, 0, 0);
      } else {
        const bf16x4 pop = __builtin_convertvector(pw, bf16x4);   // two paired conversions
        if constexpr (KV == KV_U8Z) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            psum[c] += static_cast<float>(pop[i]) * (float)((vzw >> (8 * i)) & 0xFFu);
        }
        // ---- O^T += V^T P
#pragma unroll
        for (int t = 0; t < kNT; ++t)
          acc[c][t] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
              __builtin_bit_cast(bf16x4, vt[t]), pop, acc[c][t], 0, 0, 0);
      }
      }
    };

    // NST register buffers in a ring: buffer i holds block b with b % NST == i
    u32x4 kr[NST][kKLoads], vr[NST][kLoads], pr[NST];
    int ph[NST];
#pragma unroll
    for (int i = 0; i < NST; ++i) {
      ph[i] = phys_of(c0 + i);
      load_tile(kr[i], vr[i], pr[i], ph[i], c0 + i);
    }
    for (int b = c0; b < c1; b += NST) {
#pragma unroll
      for (int i = 0; i < NST; ++i)
        process(kr[i], vr[i], pr[i], ph[i], b + i);   // past c1: masked, no memory traffic
    }
  }

  // ---- epilogue: lane (j, n) holds O^T[16 t + 4 j + i][n]
#pragma unroll
  for (int c = 0; c < CG; ++c) {
  const float lt = rows_sum(lsum[c]);
  if constexpr (KV == KV_I8 || KV == KV_U8Z) {
    // INT8 V codes entered as fp16 1024 + (c + 128): take 1152 * sum(P) off
    // every output row; asymmetric rows: take sum_t P_t zero_t off
    const float pt = rows_sum(psum[c]);
    const float voff = KV == KV_I8 ? 1152.f * pt : pt;
#pragma unroll
    for (int t = 0; t < kNT; ++t) acc[c][t] -= voff;
  }
  // a column that saw no key (a query token before the start, or a piece
  // past its causal limit) has lt == 0: zero output, zero weight
  const float inv = lt > 0.f ? (kV16 ? 1.0f / (lt * vfac) : 1.0f / lt) : 0.f;
  if (!has_head[c]) continue;
  if (whole) {
#pragma unroll
    for (int t = 0; t < kNT; ++t)
      store_out4<D, OUT>(a.out, out_row[c] * D + 16 * t + 4 * j, acc[c][t] * inv);
  } else {
    const size_t row = out_row[c] * a.kstride + slot;
#pragma unroll
    for (int t = 0; t < kNT; ++t)
      *reinterpret_cast<f32x4*>(a.ws_o + row * D + 16 * t + 4 * j) = acc[c][t] * inv;
    if (j == 0) {
      a.ws_m[row] = m[c];
      a.ws_l[row] = lt;
    }
  }
  }
}

// Fixed split: one wavefront per (sequence, KV head, partition of
// part_blocks blocks); the launch index is decoded KV-head-fastest.
template <int D, int KV, int OUT, int MQ>
__global__ __launch_bounds__(64) void decode_mfma_kernel(MfmaArgs a, int n_parts) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[kBlock * D * 2];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[kBlock * D * 2];
  __shared__ __attribute__((aligned(16))) uint8_t lds_p[KV == KV_U8Z ? 160 : 16];
  const int g = blockIdx.x % a.hkv;
  const int r = blockIdx.x / a.hkv;
  const int p = r % n_parts;
  const int s = r / n_parts;
  const int L = clamp_len(a.lens[s], a.max_blocks);
  const int nblk = (L + kBlock - 1) / kBlock;
  const int fb = first_block(L, a.ntok, a.window);
  const int parts_s = (nblk - fb + a.part_blocks - 1) / a.part_blocks;
  const int b0 = fb + p * a.part_blocks;
  const int b1 = min(b0 + a.part_blocks, nblk);
  const int tok0 = blockIdx.y * a.tok_per_pass;
  if (b0 >= b1) {
    if (p == 0) zero_rows<D, OUT>(a, s, g, tok0);   // empty sequence
    return;
  }
  mfma_segment<D, KV, OUT, 2, MQ>(a, s, g, L, b0, b1, p, parts_s == 1, tok0, lds_k, lds_v,
                                  lds_p);
}

// Balanced split: a persistent grid of V wavefronts per KV head, one
// generation on the GPU.  For KV head g, the blocks of all sequences are laid
// end to end (sequence 0's blocks, then sequence 1's, ...; T in all, each
// sequence preceded by kSeqStartCost blocks that stand for the cost of
// entering it and are never read, when the ranges stay above min_blocks)
// and wavefront v takes the range
// [v P, v P + P) with P = max(ceil(T / V), min_blocks) (bf16: pairs of ranges
// skewed toward the even XCDs, below), so the wavefronts' work is even and
// they finish together.  A range that covers a sequence's blocks only in part
// yields a partial in slot v - range(R0) of that sequence (R0: the flat
// position of its first real block, range(x) = floor(x / P) for equal
// ranges); the sequence has range(R1 - 1) - range(R0) + 1 pieces, which the
// wavefront holding its first block records for the combine kernel.  The
// wavefronts of one v are consecutive launch indices, so they run side by
// side and read the heads of the same blocks at the same time.
//
// Two blocks in flight per wavefront and two wavefronts per SIMD for every
// format (three or four blocks in flight, and other occupancies, measured
// slower).  INT8 (one query token) asks for three wavefronts per SIMD: with
// its fp16 P V it needs 170 registers and would otherwise drop to two
// (measured on the shared-prefix INT8 workload: 91.8 us at two, 87.4 us at
// three, where two registers are spilled: one 8-byte scratch store and
// reload per two blocks).  Two column groups per wavefront (kMqPair) need
// about 350 registers and run one wavefront per SIMD.
constexpr int kBalStages = 2;
constexpr int kBalWaves = 2;
constexpr int kSeqStartCost = 4;   // blocks charged per sequence start (see the kernel)
template <int D, int KV, int OUT, int MQ>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(
    MQ == kMqPair ? 1 : KV == KV_I8 && !MQ ? 3 : kBalWaves))) void
decode_mfma_balanced_kernel(MfmaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[kBlock * D * 2];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[kBlock * D * 2];
  __shared__ __attribute__((aligned(16))) uint8_t lds_p[KV == KV_U8Z ? 160 : 16];
  const int lane = threadIdx.x;
  // launch index: KV head fastest, then the pass over the query tokens, then
  // the range.  The passes of one (range, KV head) are launched side by side
  // and land on the same XCD, so a later pass finds the tiles the first one
  // fetched in that XCD's L2.
  const int tok_wave = MQ == kMqPair ? 2 * a.tok_per_pass : a.tok_per_pass;
  const int passes = (a.ntok + tok_wave - 1) / tok_wave;
  // bf16 pools (bound by HBM), full generation: consecutive launch indices
  // alternate between even and odd XCDs, and the wavefronts on odd XCDs run
  // 8-11 % slower for the same bytes (on every box and workload measured).
  // So range v takes the parity of its launch index, and even ranges take
  // per + per / 16 blocks, odd ones per - per / 16 (V even; the host rounds
  // it).  Measured on one box against equal ranges, kernel time: 8B step
  // 110.8 -> 109.1 us, 70B 406.4 -> 397.0, long context 174.6 -> 171.0,
  // 8 tokens 129.4 -> 126.3, 70B with 4 tokens 432.0 -> 422.9; with 4 tokens
  // on the 8B shape, a quarter generation, 108.9 -> 111.8, so those keep
  // equal ranges.  Quantized kernels keep equal ranges and one KV head per
  // XCD: over a shared prefix served by the caches, the skew and the split
  // of a head over two XCDs cost 12 % (INT8 81 -> 91 us).
  constexpr bool kSkew = KV == KV_BF16 && (MQ == kMqOne || MQ == kMqPair);
  int g, pass, v;
  if constexpr (kSkew) {
    const unsigned lin = blockIdx.x >> 1;
    g = lin % a.hkv;
    pass = (lin / a.hkv) % passes;
    v = 2 * (int)(lin / (a.hkv * passes)) + (int)(blockIdx.x & 1);
  } else {
    g = blockIdx.x % a.hkv;
    pass = (blockIdx.x / a.hkv) % passes;
    v = blockIdx.x / (a.hkv * passes);
  }
  const int V = gridDim.x / (a.hkv * passes);
  const int B = a.num_seqs;
  const int tok0 = pass * tok_wave;

  // The lengths of the first kLenChunks * 64 sequences are loaded once, all
  // at the same time, and kept in registers for both passes and the walk.
  constexpr int kLenChunks = 4;
  int lc[kLenChunks];
#pragma unroll
  for (int c = 0; c < kLenChunks; ++c) {
    const int si = c * kWave + lane;
    lc[c] = si < B ? clamp_len(a.lens[si], a.max_blocks) : 0;
  }
  // lengths of sequences base .. base+63 in lane order (base a multiple of 64)
  auto len_chunk = [&](int base) -> int {
    const int c = base / kWave;
    int r = 0;
#pragma unroll
    for (int i = 0; i < kLenChunks; ++i)
      if (c == i) r = lc[i];
    if (c >= kLenChunks) {
      const int si = base + lane;
      r = si < B ? clamp_len(a.lens[si], a.max_blocks) : 0;
    }
    return r;
  };

  // pass 1: total (virtual) blocks per KV head, from the inclusive prefix of each
  // 64-sequence chunk (the first chunk's is kept for pass 2, which then needs
  // no second scan when there are at most 64 sequences); zero rows of empty
  // sequences
  //
  // Each sequence counts kSeqStartCost blocks more than it has, placed before
  // its first one and never read: a wavefront that enters a sequence starts
  // its pipeline again (the table entries, then the first tiles, with nothing
  // in flight), which costs it about that much streaming time, so ranges that
  // hold sequence starts take fewer real blocks.  A piece and its slot are
  // counted from the sequence's first real block.  Measured on one box
  // against no start cost (kernel time): 8B 109.0 -> 107.2 us, INT8 8B step
  // 74.8 -> 72.4, E4M3 73.1 -> 71.0, E2M1 49.7 -> 46.5, per-row uint8 78.8 ->
  // 77.5, 1024-token window 54.9 -> 53.0, E4M3 over the shared prefix 77.0 ->
  // 75.3; 2, 3 and 6 blocks gave less overall.
  int total = 0, nseq = 0, incl0 = 0, cnt0 = 0;
  for (int base = 0; base < B; base += kWave) {
    const int si = base + lane;
    const int Ll = len_chunk(base);
    const int nb = seq_blocks(Ll, a.ntok, a.window);
    const int inc = wave_incl_scan(nb);
    const int cnt = wave_incl_scan(nb > 0 ? 1 : 0);
    if (base == 0) {
      incl0 = inc;
      cnt0 = cnt;
    }
    total += readlane_i(inc, kWave - 1);
    nseq += readlane_i(cnt, kWave - 1);
    if (v == 0) {
      uint64_t empty = __ballot(si < B && Ll == 0);
      while (empty) {
        const int e = __ffsll((unsigned long long)empty) - 1;
        empty &= empty - 1;
        zero_rows<D, OUT>(a, base + e, g, tok0);
        if (MQ == kMqPair) zero_rows<D, OUT>(a, base + e, g, tok0 + a.tok_per_pass);
      }
    }
  }
  // the sums above are equal in every lane; say so, so that everything derived
  // from them (ranges, block indices, buffer descriptors) stays in scalar
  // registers instead of being treated as per-lane values
  total = __builtin_amdgcn_readfirstlane(total);
  nseq = __builtin_amdgcn_readfirstlane(nseq);
  // The start cost only where ranges stay above the floor of min_blocks: at
  // the floor the ranges are not balanced in time anyway, and the extra
  // blocks only move range edges off sequence edges (long context with a
  // 4096-token window, 8 sequences: 31.9 -> 34.7 us with the cost).
  const int c = (total + nseq * kSeqStartCost + V - 1) / V > a.min_blocks ? kSeqStartCost : 0;
  auto vblocks = [&](int nb) { return nb > 0 ? nb + c : 0; };
  total += nseq * c;
  incl0 += cnt0 * c;
  const int per = max((total + V - 1) / V, a.min_blocks);
  // skewed pairs of ranges: [2 w per, 2 w per + pe) and [.. + pe, 2 (w + 1) per)
  int x0, x1, pe = per;
  if constexpr (kSkew) {
    const int dsh = per - per / 16 >= a.min_blocks ? per / 16 : 0;
    pe = per + dsh;
    x0 = (v >> 1) * 2 * per + (v & 1) * pe;
    if (x0 >= total) return;
    x1 = min(x0 + ((v & 1) ? per - dsh : pe), total);
  } else {
    x0 = v * per;
    if (x0 >= total) return;
    x1 = min(x0 + per, total);
  }
  auto range_of = [&](int x) {   // the range holding flat position x
    if constexpr (kSkew)
      return 2 * (x / (2 * per)) + ((x % (2 * per)) >= pe ? 1 : 0);
    else
      return x / per;
  };

  // pass 2: the sequence holding flat position x0; the lanes keep the lengths
  // and inclusive prefix of a 64-sequence chunk for the walk below
  int base = 0, carry = 0, s = -1, R0 = 0, Lreg = 0, incl = 0;
  for (; base < B; base += kWave) {
    Lreg = len_chunk(base);
    const int nb = vblocks(seq_blocks(Lreg, a.ntok, a.window));
    incl = (base == 0 ? incl0 : wave_incl_scan(nb)) + carry;
    const uint64_t hit = __ballot(nb > 0 && incl - nb <= x0 && x0 < incl);
    if (hit) {
      const int hl = __ffsll((unsigned long long)hit) - 1;
      s = base + hl;
      R0 = readlane_i(incl - nb, hl);
      break;
    }
    carry = readlane_i(incl, kWave - 1);
  }
  if (s < 0) return;   // unreachable while x0 < total

  int x = x0;
  while (true) {
    const int L = readlane_i(Lreg, s - base);
    const int fb = first_block(L, a.ntok, a.window);
    const int R1 = R0 + vblocks(seq_blocks(L, a.ntok, a.window));
    const int Rr = R0 + c;   // the sequence's first real block
    const int e = min(x1, R1);
    const int xs = max(x, Rr);
    if (xs < e) {
      const int vf = range_of(Rr);
      const int K = range_of(R1 - 1) - vf + 1;
      const int slot = v - vf;
      if (g == 0 && pass == 0 && slot == 0 && lane == 0) a.ws_count[s] = K;
      mfma_segment<D, KV, OUT, kBalStages, MQ>(a, s, g, L, fb + xs - Rr, fb + e - Rr, slot,
                                            K == 1, tok0, lds_k, lds_v, lds_p);
    }
    if (e >= x1) break;
    x = e;
    R0 = R1;
    // next sequence with at least one block (one exists: x < x1 <= total)
    int Lnext = 0;
    while (Lnext == 0 && s + 1 < B) {
      ++s;
      if (s - base >= kWave) {
        carry = readlane_i(incl, kWave - 1);
        base += kWave;
        Lreg = len_chunk(base);
        incl = wave_incl_scan(vblocks(seq_blocks(Lreg, a.ntok, a.window))) + carry;
      }
      Lnext = readlane_i(Lreg, s - base);
    }
    if (Lnext == 0) break;
  }
}

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  return v;
}

// Shared-prefix split.  The first P = prefix_blocks entries of every
// sequence's table are the same physical blocks (a common prompt: page "LLM
// 推理优化深度解析", section "意外的收获：prefix sharing"; page "大模型推理的KV
// Cache管理…", section 二, copy_prefix).  The sequences are taken in groups of
// S = seqs_per_group, whose S * G query heads fill the 16 MFMA columns, and
// for each KV head the work is laid end to end: first every group's P prefix
// blocks (each block staged once for the whole group), then every sequence's
// remaining blocks.  Wavefront v takes the range [v per, v per + per) of that
// order, per = max(ceil(total / V), min_blocks), as the balanced split does.
// A sequence's pieces are the Kp pieces of its group's prefix (slots 0 ..
// Kp - 1) followed by the pieces of its own blocks (slots Kp ...); the
// wavefront holding a sequence's first suffix piece (or, without suffix, the
// first prefix piece of its group) records the piece count for the combine.
// With P = 0 this is the balanced split of one query token per sequence.
// The 8- and 4-bit formats ask for three wavefronts per SIMD (E4M3 would
// otherwise need one register more than three allow).
template <int D, int KV, int OUT>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(
    KV == KV_I8 || KV == KV_FP8 || KV == KV_FP4 ? 3 : kBalWaves))) void
decode_mfma_prefix_kernel(MfmaArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds_k[kBlock * D * 2];
  __shared__ __attribute__((aligned(16))) uint8_t lds_v[kBlock * D * 2];
  __shared__ __attribute__((aligned(16))) uint8_t lds_p[KV == KV_U8Z ? 160 : 16];
  const int lane = threadIdx.x;
  const int g = blockIdx.x % a.hkv;
  const int v = blockIdx.x / a.hkv;
  const int V = gridDim.x / a.hkv;
  const int B = a.num_seqs;
  const int P = a.prefix_blocks;
  const int S = a.seqs_per_group;
  const int G = a.G;
  const int NG = (B + S - 1) / S;

  constexpr int kLenChunks = 4;
  int lc[kLenChunks];
#pragma unroll
  for (int c = 0; c < kLenChunks; ++c) {
    const int si = c * kWave + lane;
    lc[c] = si < B ? clamp_len(a.lens[si], a.max_blocks) : 0;
  }
  auto len_chunk = [&](int base) -> int {
    const int c = base / kWave;
    int r = 0;
#pragma unroll
    for (int i = 0; i < kLenChunks; ++i)
      if (c == i) r = lc[i];
    if (c >= kLenChunks) {
      const int si = base + lane;
      r = si < B ? clamp_len(a.lens[si], a.max_blocks) : 0;
    }
    return r;
  };
  // blocks of a sequence of length L after the shared prefix
  auto suffix_blocks = [&](int L) { return max((L + kBlock - 1) / kBlock - P, 0); };

  // pass 1: suffix blocks in all; zero rows of empty sequences
  int total = 0, incl0 = 0;
  for (int base = 0; base < B; base += kWave) {
    const int si = base + lane;
    const int Ll = len_chunk(base);
    const int inc = wave_incl_scan(suffix_blocks(Ll));
    if (base == 0) incl0 = inc;
    total += readlane_i(inc, kWave - 1);
    if (v == 0) {
      uint64_t empty = __ballot(si < B && Ll == 0);
      while (empty) {
        const int e = __ffsll((unsigned long long)empty) - 1;
        empty &= empty - 1;
        zero_rows<D, OUT>(a, base + e, g, 0);
      }
    }
  }
  const int Tp = NG * P;
  total = __builtin_amdgcn_readfirstlane(total) + Tp;
  const int per = max((total + V - 1) / V, a.min_blocks);
  const int x0 = v * per;
  if (x0 >= total) return;
  const int x1 = min(x0 + per, total);
  // prefix pieces of group q: the wavefronts whose ranges meet [q P, q P + P)
  auto prefix_pieces = [&](int q) { return P > 0 ? ((q + 1) * P - 1) / per - (q * P) / per + 1 : 0; };

  // ---- the shared prefix, one sequence group at a time
  int x = x0;
  while (x < x1 && x < Tp) {
    const int q = x / P;
    const int e = min(x1, (q + 1) * P);
    const int Kp = prefix_pieces(q);
    const int slot = v - (q * P) / per;
    const int s0 = q * S;
    const int nseq = min(S, B - s0);
    const int n = lane & 15;
    const bool col = n < nseq * G;
    const int scol = s0 + (col ? n / G : 0);
    const int lcol = col ? clamp_len(a.lens[scol], a.max_blocks) : 0;
    const int lmax = __builtin_amdgcn_readfirstlane(wave_max_i(lcol));
    const int lmin = __builtin_amdgcn_readfirstlane(wave_min_i(col ? lcol : (1 << 30)));
    const bool has_suffix = suffix_blocks(lcol) > 0;
    if (g == 0 && slot == 0 && lane < 16 && col && n % G == 0 && !has_suffix)
      a.ws_count[scol] = Kp;
    mfma_segment<D, KV, OUT, kBalStages, kMqSeqs>(a, s0, g, lmax, x - q * P, e - q * P, slot,
                                                  Kp == 1 && !has_suffix, 0, lds_k, lds_v,
                                                  lds_p, SeqCols{nseq, lcol, lmin});
    x = e;
  }
  if (x >= x1) return;

  // ---- every sequence's own blocks: positions y = x - Tp of the suffix order
  const int y0 = x - Tp, y1 = x1 - Tp;
  int base = 0, carry = 0, s = -1, R0 = 0, Lreg = 0, incl = 0;
  for (; base < B; base += kWave) {
    Lreg = len_chunk(base);
    const int nb = suffix_blocks(Lreg);
    incl = (base == 0 ? incl0 : wave_incl_scan(nb)) + carry;
    const uint64_t hit = __ballot(nb > 0 && incl - nb <= y0 && y0 < incl);
    if (hit) {
      const int hl = __ffsll((unsigned long long)hit) - 1;
      s = base + hl;
      R0 = readlane_i(incl - nb, hl);
      break;
    }
    carry = readlane_i(incl, kWave - 1);
  }
  if (s < 0) return;   // unreachable while y0 < total suffix blocks

  int y = y0;
  while (true) {
    const int L = readlane_i(Lreg, s - base);
    const int R1 = R0 + suffix_blocks(L);
    const int e = min(y1, R1);
    const int vf = (Tp + R0) / per;
    const int Ks = (Tp + R1 - 1) / per - vf + 1;
    const int Kp = prefix_pieces(s / S);
    const int slot = Kp + v - vf;
    if (g == 0 && slot == Kp && lane == 0) a.ws_count[s] = Kp + Ks;
    mfma_segment<D, KV, OUT, kBalStages, kMqOne>(a, s, g, L, P + y - R0, P + e - R0, slot,
                                                 Kp + Ks == 1, 0, lds_k, lds_v, lds_p);
    if (e >= y1) break;
    y = e;
    R0 = R1;
    int Lnext = 0;
    while (Lnext == 0 && s + 1 < B) {
      ++s;
      if (s - base >= kWave) {
        carry = readlane_i(incl, kWave - 1);
        base += kWave;
        Lreg = len_chunk(base);
        incl = wave_incl_scan(suffix_blocks(Lreg)) + carry;
      }
      Lnext = suffix_blocks(readlane_i(Lreg, s - base)) > 0 ? 1 : 0;
    }
    if (Lnext == 0) break;
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel (q and KV binary32): one wavefront per (sequence, KV head,
// partition); tokens are taken one at a time, each dot product reduced across
// the wavefront, accumulation in binary32.
template <int D, int OUT, int MAXG>
__global__ __launch_bounds__(64) void decode_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ kc, const float* __restrict__ vc,
    const int32_t* __restrict__ tables, int max_blocks, const int32_t* __restrict__ lens, int hq,
    int hkv, int G, int num_blocks, size_t bstride, float scale_log2, int part_blocks, int n_parts,
    int kstride,
    float* __restrict__ ws_m, float* __restrict__ ws_l, float* __restrict__ ws_o,
    void* __restrict__ out, const float* __restrict__ kn, const float* __restrict__ vn,
    float* __restrict__ kc_w, float* __restrict__ vc_w) {
  constexpr int kPer = D / kWave;
  const int lane = threadIdx.x;
  const int g = blockIdx.x % hkv;
  const int r = blockIdx.x / hkv;
  const int p = r % n_parts;
  const int s = r / n_parts;
  int L = lens[s];
  if (L < 0 || L > max_blocks * kBlock) L = 0;
  const int nblk = (L + kBlock - 1) / kBlock;
  const int parts_s = (nblk + part_blocks - 1) / part_blocks;
  const int b0 = p * part_blocks;
  const int b1 = min(b0 + part_blocks, nblk);

  float qv[MAXG][kPer], acc[MAXG][kPer], m[MAXG], l[MAXG];
#pragma unroll
  for (int hh = 0; hh < MAXG; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      acc[hh][e] = 0.f;
      qv[hh][e] = 0.f;
      if (hh < G) qv[hh][e] = q[((size_t)s * hq + g * G + hh) * D + lane * kPer + e];
    }
  }
  if (b0 >= b1) {
    if (p == 0) {
#pragma unroll
      for (int hh = 0; hh < MAXG; ++hh)
        if (hh < G)
#pragma unroll
          for (int e = 0; e < kPer; ++e) {
            const size_t o = ((size_t)s * hq + g * G + hh) * D + lane * kPer + e;
            if constexpr (OUT == OUT_F32) static_cast<float*>(out)[o] = 0.f;
            else static_cast<uint16_t*>(out)[o] = 0;
          }
    }
    return;
  }
  const int32_t* trow = tables + (size_t)s * max_blocks;
  // fused append: the partition holding position L-1 writes the new token
  // into the pool and uses it for that position
  const bool app = kn != nullptr && (L - 1) / kBlock >= b0 && (L - 1) / kBlock < b1;
  float kx[kPer], vx[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) kx[e] = vx[e] = 0.f;
  if (app) {
    const size_t src = ((size_t)s * hkv + g) * D + lane * kPer;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      kx[e] = kn[src + e];
      vx[e] = vn[src + e];
    }
    const int ph = trow[(L - 1) / kBlock];
    if (ph >= 0 && ph < num_blocks) {
      const size_t dst = (size_t)ph * bstride + ((size_t)g * kBlock + (L - 1) % kBlock) * D +
                         lane * kPer;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        kc_w[dst + e] = kx[e];
        vc_w[dst + e] = vx[e];
      }
    }
  }
  for (int b = b0; b < b1; ++b) {
    const int phys = trow[b];
    if (phys < 0 || phys >= num_blocks) continue;
    const int valid = min(kBlock, L - b * kBlock);
    // the block's 16 K and V rows are loaded together (one memory latency per
    // block, not per token); rows past L are loaded but never used
    const size_t base0 = (size_t)phys * bstride + (size_t)g * kBlock * D + lane * kPer;
    float kt[kBlock][kPer], vt[kBlock][kPer];
#pragma unroll
    for (int o = 0; o < kBlock; ++o)
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        kt[o][e] = kc[base0 + (size_t)o * D + e];
        vt[o][e] = vc[base0 + (size_t)o * D + e];
      }
    if (app && (L - 1) / kBlock == b) {   // the appended token's row
      const int o = (L - 1) % kBlock;
#pragma unroll
      for (int oo = 0; oo < kBlock; ++oo)
        if (oo == o)
#pragma unroll
          for (int e = 0; e < kPer; ++e) {
            kt[oo][e] = kx[e];
            vt[oo][e] = vx[e];
          }
    }
    // after the reduce-scatter below lane l holds the dot product of token l / 4
    const int tok = (lane >> 2) & (kBlock - 1);
#pragma unroll
    for (int hh = 0; hh < MAXG; ++hh) {
      if (hh >= G) break;
      // 16 partial dot products per lane, then a butterfly reduce-scatter:
      // after it, every lane holds the full dot product of token lane / 4
      float x[kBlock];
#pragma unroll
      for (int o = 0; o < kBlock; ++o) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < kPer; ++e) d += qv[hh][e] * kt[o][e];
        x[o] = d;
      }
#pragma unroll
      for (int step = 0, half = kBlock / 2; half >= 1; ++step, half >>= 1) {
        const int bit = 32 >> step;                 // lane bits 5, 4, 3, 2
        const bool upper = (lane & bit) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
          const float mine = upper ? x[i + half] : x[i];
          const float other = upper ? x[i] : x[i + half];
          x[i] = mine + __shfl_xor(other, bit, kWave);
        }
      }
      float dot = x[0];
      dot += __shfl_xor(dot, 1, kWave);
      dot += __shfl_xor(dot, 2, kWave);
      const float xl = tok < valid ? dot * scale_log2 : -INFINITY;
      float mx = xl;
#pragma unroll
      for (int o = 4; o < kWave; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
      const float mn = fmaxf(m[hh], mx);
      const float alpha = exp2f(m[hh] - mn);
      const float pe = exp2f(xl - mn);               // 0 for masked tokens
      float ps = pe;
#pragma unroll
      for (int o = 4; o < kWave; o <<= 1) ps += __shfl_xor(ps, o, kWave);
      l[hh] = l[hh] * alpha + ps;
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[hh][e] *= alpha;
#pragma unroll
      for (int o = 0; o < kBlock; ++o) {
        // lanes 4 o .. 4 o + 3 hold token o's weight
        const float po = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pe), 4 * o));
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc[hh][e] += po * vt[o][e];
      }
      m[hh] = mn;
    }
  }
#pragma unroll
  for (int hh = 0; hh < MAXG; ++hh) {
    if (hh >= G) break;
    const size_t row = (size_t)s * hq + g * G + hh;
    const float inv = 1.0f / l[hh];
    if (parts_s == 1) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        const size_t o = row * D + lane * kPer + e;
        if constexpr (OUT == OUT_F32) static_cast<float*>(out)[o] = acc[hh][e] * inv;
        else static_cast<uint16_t*>(out)[o] = f32_to_bf16_bits(acc[hh][e] * inv);
      }
    } else {
      const size_t pr = row * kstride + p;
#pragma unroll
      for (int e = 0; e < kPer; ++e) ws_o[pr * D + lane * kPer + e] = acc[hh][e] * inv;
      if (lane == 0) {
        ws_m[pr] = m[hh];
        ws_l[pr] = l[hh];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Cross-partition combine: one wavefront per (sequence, query head) row with
// more than one partial; M = max_p m_p, w_p = 2^(m_p - M) l_p,
// out = sum_p w_p o_p / sum_p w_p.  Lane p holds partial p's weight (64
// partials at a time); the partial rows are read D/4 lanes per row, several
// rows per load instruction, through a descriptor bounded to this row's
// partials so that every load is issued unconditionally.  The number of
// partials is ceil(blocks / part_blocks) for a fixed split, or the count the
// decode kernel recorded per sequence for a balanced split (`counts`).
// SPEC partial rows are read before the count is known.
template <int D, int OUT, int SPEC>
__global__ __launch_bounds__(64) void reduce_kernel(const float* __restrict__ ws_m,
                                                    const float* __restrict__ ws_l,
                                                    const float* __restrict__ ws_o,
                                                    const int32_t* __restrict__ counts,
                                                    const int32_t* __restrict__ lens,
                                                    int max_blocks, int rows_per_seq,
                                                    int part_blocks, int kstride, int ntok,
                                                    int window, void* __restrict__ out) {
  constexpr int kCols = D / 4;             // lanes per partial row (16-byte pieces)
  constexpr int kRowsPerLoad = kWave / kCols;
  const int row = blockIdx.x;
  const int s = row / rows_per_seq;
  const int lane = threadIdx.x;
  const float* mrow = ws_m + (size_t)row * kstride;
  const float* lrow = ws_l + (size_t)row * kstride;
  // issued together: the length, the piece count and the first 64 partial
  // maxima and sums (slots past the count hold stale values and are masked)
  int L = lens[s];
  const int cnt = counts != nullptr ? counts[s] : 0;
  float m0 = -INFINITY, l0 = 0.f;
  if constexpr (SPEC > 0) {
    m0 = lane < kstride ? mrow[lane] : -INFINITY;
    l0 = lane < kstride ? lrow[lane] : 0.f;
  }
  // the first kSpec partial rows (most sequences have no more pieces), read
  // before the count is known through a descriptor bounded to the row's slots
  // (SPEC = 0: nothing is read ahead; the maxima, sums and rows are read once
  // the count shows more than one piece)
  constexpr int kSpecLoads = SPEC == 0 ? 0 : SPEC > kRowsPerLoad ? SPEC / kRowsPerLoad : 1;
  constexpr int kSpec = kSpecLoads * kRowsPerLoad;
  const int sub0 = lane / kCols, col0 = lane % kCols;
  const rsrc_t rspec = make_rsrc(ws_o + (size_t)row * kstride * D, kstride * D * 4);
  u32x4 spec[kSpecLoads > 0 ? kSpecLoads : 1];
#pragma unroll
  for (int i = 0; i < kSpecLoads; ++i)
    spec[i] = buffer_load16(rspec, ((i * kRowsPerLoad + sub0) * D + col0 * 4) * 4);
  if (L < 0 || L > max_blocks * kBlock) L = 0;
  if (L == 0) return;
  int parts;
  if (counts != nullptr) {
    parts = min(cnt, kstride);
  } else {
    parts = (seq_blocks(L, ntok, window) + part_blocks - 1) / part_blocks;
  }
  if (parts <= 1) return;
  if constexpr (SPEC == 0) {
    m0 = lane < parts ? mrow[lane] : -INFINITY;
    l0 = lane < parts ? lrow[lane] : 0.f;
  }
  float M = lane < parts ? m0 : -INFINITY;
  for (int c = kWave; c < parts; c += kWave)
    if (c + lane < parts) M = fmaxf(M, mrow[c + lane]);
  M = wave_max(M);
  const int sub = lane / kCols, col = lane % kCols;
  const rsrc_t ro = make_rsrc(ws_o + (size_t)row * kstride * D, parts * D * 4);
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int c = 0; c < parts; c += kWave) {
    float wp = 0.f;
    if (c + lane < parts)
      wp = c == 0 ? exp2f(m0 - M) * l0 : exp2f(mrow[c + lane] - M) * lrow[c + lane];
    den += wp;
    const int n64 = min(kWave, parts - c);
    int q0 = 0;
    if (SPEC > 0 && c == 0) {
      // partial rows already loaded; rows past the count are stale memory
      // (possibly NaN bits), so they are left out by selection
#pragma unroll
      for (int i = 0; i < kSpecLoads; ++i) {
        const int pp = i * kRowsPerLoad + sub;
        const float w = __shfl(wp, pp, kWave);
        if (pp < parts) a += w * __builtin_bit_cast(f32x4, spec[i]);
      }
      q0 = kSpec;
    }
#pragma unroll 4
    for (int q = q0; q < n64; q += kRowsPerLoad) {
      const int pp = q + sub;              // partial within this group of 64
      const float w = __shfl(wp, pp & (kWave - 1), kWave);
      const u32x4 v = buffer_load16(ro, ((c + pp) * D + col * 4) * 4);
      a += w * __builtin_bit_cast(f32x4, v);
    }
  }
  den = wave_sum(den);
#pragma unroll
  for (int o = kCols; o < kWave; o <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) a[e] += __shfl_xor(a[e], o, kWave);
  // den == 0: no piece saw a key (query tokens before the start)
  if (sub == 0) store_out4<D, OUT>(out, (size_t)row * D + col * 4, a * (den > 0.f ? 1.0f / den : 0.f));
}

// One-wavefront workgroups of `kernel` that fit on a compute unit at once
// (register and LDS limits); looked up once per kernel.
int resident_waves_per_cu(const void* kernel) {
  static std::mutex mu;
  static std::unordered_map<const void*, int> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(kernel);
  if (it != cache.end()) return it->second;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, kWave, 0) != hipSuccess)
    return -1;
  cache.emplace(kernel, blocks);
  return blocks;
}

// Launch geometry of one decode call.
struct Plan {
  bool balanced;      // balanced split (MFMA path)
  int part_blocks;    // fixed split: blocks per partition
  int n_parts;        // fixed split: partitions per sequence
  int kstride;        // partial slots per row in the workspace
  int cus;            // balanced split: compute units of the device
  int tok_per_pass;   // query tokens per wavefront (tok_per_pass * G <= 16 columns)
  int passes;         // wavefronts per work unit: ceil(ntok / tok_per_pass)
  float *ws_m, *ws_l, *ws_o;
  int32_t* ws_count;
};

template <int D, int OUT>
int run_d_out(const DecodeArgs& a, const Plan& pl, hipStream_t st) {
  const pkv_cache_t& c = *a.cache;
  const int hkv = c.num_kv_heads, hq = a.num_q_heads, G = hq / hkv;
  const float sl2 = a.scale * kLog2e;
  dim3 block(kWave);
  int rc;
  int64_t ranges = 0;   // balanced split: wavefronts per KV head (and pass)
  if (c.kv_dtype == PKV_F32) {
    dim3 grid((unsigned)((int64_t)a.num_seqs * hkv * pl.n_parts));
    rc = launch(decode_f32_kernel<D, OUT, 16>, grid, block, st, (const float*)a.q,
                (const float*)c.k_cache, (const float*)c.v_cache, a.tables, a.max_blocks,
                a.lens, hq, hkv, G, c.num_blocks, block_stride_bytes(c) / sizeof(float), sl2,
                pl.part_blocks, pl.n_parts, pl.kstride,
                pl.ws_m, pl.ws_l, pl.ws_o, a.out, (const float*)a.k_new, (const float*)a.v_new,
                (float*)c.k_cache, (float*)c.v_cache);
  } else {
    MfmaArgs m;
    m.q = (const uint16_t*)a.q;
    m.kc = (const uint8_t*)c.k_cache;
    m.vc = (const uint8_t*)c.v_cache;
    const bool q8 = c.kv_dtype != PKV_BF16;
    m.ksc = q8 ? c.k_scale : nullptr;
    m.vsc = q8 ? c.v_scale : nullptr;
    m.kz = c.kv_dtype == PKV_U8_ZP ? c.k_zero : nullptr;
    m.vz = c.kv_dtype == PKV_U8_ZP ? c.v_zero : nullptr;
    m.tables = a.tables;
    m.lens = a.lens;
    m.max_blocks = a.max_blocks;
    m.num_seqs = a.num_seqs;
    m.hq = hq;
    m.hkv = hkv;
    m.G = G;
    m.num_blocks = c.num_blocks;
    m.blk_stride = block_stride_bytes(c);
    m.scale_log2 = sl2;
    m.ws_m = pl.ws_m;
    m.ws_l = pl.ws_l;
    m.ws_o = pl.ws_o;
    m.ws_count = pl.ws_count;
    m.kstride = pl.kstride;
    m.part_blocks = pl.part_blocks;
    m.min_blocks = kBalancedMinBlocks;
    m.ntok = a.ntok;
    m.tok_per_pass = pl.tok_per_pass;
    m.window = a.window;
    m.prefix_blocks = a.prefix_blocks > 0 ? a.prefix_blocks : 0;
    m.seqs_per_group = G <= 16 ? 16 / G : 1;
    m.out = a.out;
    m.kn = q8 ? nullptr : (const uint8_t*)a.k_new;
    m.vn = q8 ? nullptr : (const uint8_t*)a.v_new;
    m.kc_w = (uint8_t*)c.k_cache;
    m.vc_w = (uint8_t*)c.v_cache;
    // the balanced bf16 kernels of one full generation (one query token, or
    // two column groups) pair their ranges (even, odd): an even count
    auto skew_ranges = [&](int64_t r) {
      return c.kv_dtype == PKV_BF16 ? std::max<int64_t>(2, r & ~(int64_t)1) : r;
    };
    auto go = [&](auto fixed_kernel, auto balanced_kernel) {
      if (pl.balanced) {
        // one generation: as many wavefronts as the GPU holds at once
        const int per_cu = resident_waves_per_cu(reinterpret_cast<const void*>(balanced_kernel));
        if (per_cu <= 0) return (int)PKV_ERR_HIP;
        // several query tokens write k times the partial rows per piece.  bf16
        // steps are bound by HBM with wavefronts to spare, so a quarter of a
        // generation makes a quarter of the pieces (8B shape, 4 tokens: 118.6
        // us at a full generation, 113.8 at half, 109.6 at a quarter; a sixth
        // collapses to 135 us).  The 8- and 4-bit kernels are bound by their
        // arithmetic and need every wavefront (shared prefix, 4 tokens, E4M3:
        // 100.7 us at a full generation, 116.8 at half).
        const int64_t div = a.ntok > 1 && c.kv_dtype == PKV_BF16 ? 4 : 1;
        const int64_t waves = (int64_t)pl.cus * per_cu / div;
        ranges = (waves + hkv - 1) / hkv;
        if (a.ntok <= 1) ranges = skew_ranges(ranges);   // the kMqOne kernel
        dim3 grid((unsigned)(ranges * hkv * pl.passes));
        return launch(balanced_kernel, grid, block, st, m);
      }
      dim3 grid((unsigned)((int64_t)a.num_seqs * hkv * pl.n_parts), (unsigned)pl.passes);
      return launch(fixed_kernel, grid, block, st, m, pl.n_parts);
    };
    // two passes' worth of columns (k * G <= 32) go to one wavefront in the
    // balanced split; more passes get the cached-load kernel, whose passes
    // run side by side; the fixed split launches its passes as separate grid
    // rows, which do not run side by side, so it keeps the streaming one
    const int mq = a.ntok <= 1                       ? kMqOne
                   : pl.balanced && pl.passes == 2 ? kMqPair
                   : pl.balanced && pl.passes > 1  ? kMqPasses
                                                   : kMqPass;
    auto by_kv = [&](auto kv) {
      constexpr int KV = decltype(kv)::value;
      if (a.prefix_blocks >= 0) {
        // shared-prefix split: one generation of wavefronts, as the balanced split
        auto kernel = decode_mfma_prefix_kernel<D, KV, OUT>;
        const int per_cu = resident_waves_per_cu(reinterpret_cast<const void*>(kernel));
        if (per_cu <= 0) return (int)PKV_ERR_HIP;
        const int64_t waves = (int64_t)pl.cus * per_cu;
        ranges = (waves + hkv - 1) / hkv;
        return launch(kernel, dim3((unsigned)(ranges * hkv)), block, st, m);
      }
      if (mq == kMqPair) {
        // two column groups per wavefront: one wavefront per SIMD for D = 128
        // (352 registers for bf16, accumulators in AGPRs), one generation.
        // 8B shape, 8 query tokens: 145.7 us in two passes, 129.1 us; 70B
        // shape, 4 tokens: 468.7 -> 433.4 us.  Half a generation: 141.9 and
        // 482.9 us; three blocks in flight: 131.6 and 439.9 us.
        auto kernel = decode_mfma_balanced_kernel<D, KV, OUT, kMqPair>;
        const int per_cu = resident_waves_per_cu(reinterpret_cast<const void*>(kernel));
        if (per_cu <= 0) return (int)PKV_ERR_HIP;
        const int64_t waves = (int64_t)pl.cus * per_cu;
        ranges = skew_ranges((waves + hkv - 1) / hkv);
        return launch(kernel, dim3((unsigned)(ranges * hkv)), block, st, m);
      }
      if (mq == kMqOne)
        return go(decode_mfma_kernel<D, KV, OUT, kMqOne>,
                  decode_mfma_balanced_kernel<D, KV, OUT, kMqOne>);
      if (mq == kMqPass)
        return go(decode_mfma_kernel<D, KV, OUT, kMqPass>,
                  decode_mfma_balanced_kernel<D, KV, OUT, kMqPass>);
      return go(decode_mfma_kernel<D, KV, OUT, kMqPass>,
                decode_mfma_balanced_kernel<D, KV, OUT, kMqPasses>);
    };
    switch (c.kv_dtype) {
      case PKV_BF16: rc = by_kv(std::integral_constant<int, KV_BF16>{}); break;
      case PKV_I8: rc = by_kv(std::integral_constant<int, KV_I8>{}); break;
      case PKV_FP4_E2M1: rc = by_kv(std::integral_constant<int, KV_FP4>{}); break;
      case PKV_U8_ZP: rc = by_kv(std::integral_constant<int, KV_U8Z>{}); break;
      default: rc = by_kv(std::integral_constant<int, KV_FP8>{}); break;
    }
  }
  // no combine when nothing can be split: a fixed split with one partition
  if (rc != PKV_OK || pl.kstride <= 1 || (!pl.balanced && pl.n_parts <= 1)) return rc;
  dim3 rgrid((unsigned)((int64_t)a.num_seqs * a.ntok * hq));
  // The combine reads the first partial rows of a row before it knows the
  // piece count.  With ranges wavefronts per KV head and B sequences, a
  // sequence has about 1 + ranges / B pieces: read that many rounded up to 2,
  // 4 or 8 (8B shape: 5 pieces, 8 rows; 70B shape: 2 pieces, 2 rows; several
  // query tokens on the 8B shape, half the wavefronts: 3 pieces, 4 rows).
  auto combine = [&](auto kernel) {
    return launch(kernel, rgrid, block, st, (const float*)pl.ws_m, (const float*)pl.ws_l,
                  (const float*)pl.ws_o,
                  (const int32_t*)(pl.balanced ? pl.ws_count : nullptr), a.lens, a.max_blocks,
                  a.ntok * hq, pl.part_blocks, pl.kstride, a.ntok, a.window, a.out);
  };
  // (a shared prefix adds its group's pieces: read 8)
  const int64_t pieces = a.prefix_blocks > 0 ? 8 : pl.balanced ? 1 + ranges / a.num_seqs : 8;
  // Under 1.5 pieces per sequence most rows belong to sequences that one
  // wavefront took whole (their output is already written): read nothing
  // ahead (70B shape, 4 query tokens: 65,536 rows, 102 MB read and 20.5 us
  // with 2 rows ahead; 467.5 against 480.7 us for the step).
  if (a.prefix_blocks <= 0 && pl.balanced && 2 * ranges < a.num_seqs)
    return combine(reduce_kernel<D, OUT, 0>);
  if (pieces <= 2) return combine(reduce_kernel<D, OUT, 2>);
  if (pieces <= 4) return combine(reduce_kernel<D, OUT, 4>);
  return combine(reduce_kernel<D, OUT, 8>);
}

}  // namespace

// Workspace layout for R = B * Hq rows and K partial slots per row:
// o [R][K][D] binary32, then m [R][K], then l [R][K], then (balanced split)
// one int32 count per sequence, each part 256-byte aligned.
size_t decode_workspace_layout(int64_t rows, int kslots, int D, int64_t num_seqs, size_t* off_m,
                               size_t* off_l, size_t* off_count) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  size_t o_bytes = up((size_t)rows * kslots * D * 4);
  size_t m_bytes = up((size_t)rows * kslots * 4);
  size_t c_bytes = up((size_t)num_seqs * 4);
  if (off_m) *off_m = o_bytes;
  if (off_l) *off_l = o_bytes + m_bytes;
  if (off_count) *off_count = o_bytes + 2 * m_bytes;
  return o_bytes + 2 * m_bytes + c_bytes;
}

int device_cu_count() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return -1;
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

int decode_slots(int max_blocks, int partition_tokens) {
  if (partition_tokens == PKV_SPLIT_BALANCED)
    return (max_blocks + kBalancedMinBlocks - 1) / kBalancedMinBlocks + 3;
  const int part_blocks = partition_tokens > 0 ? partition_tokens / kBlock : max_blocks;
  return (max_blocks + part_blocks - 1) / part_blocks;
}

int launch_decode(const DecodeArgs& a, hipStream_t st) {
  const pkv_cache_t& c = *a.cache;
  Plan pl;
  pl.balanced = a.partition_tokens == PKV_SPLIT_BALANCED;
  pl.kstride = decode_slots(a.max_blocks, a.partition_tokens);
  if (pl.balanced) {
    // fp32 pools (a parity path) take the fixed split at the same minimum size
    pl.part_blocks = kBalancedMinBlocks;
    if (c.kv_dtype == PKV_F32) pl.balanced = false;
  } else {
    pl.part_blocks = a.partition_tokens > 0 ? a.partition_tokens / kBlock : a.max_blocks;
  }
  pl.n_parts = (a.max_blocks + pl.part_blocks - 1) / pl.part_blocks;
  pl.cus = 0;
  if (pl.balanced) {
    pl.cus = device_cu_count();
    if (pl.cus <= 0) return PKV_ERR_HIP;
  }
  const int G = a.num_q_heads / c.num_kv_heads;
  pl.tok_per_pass = a.ntok > 1 ? max(1, 16 / G) : 1;
  pl.passes = (a.ntok + pl.tok_per_pass - 1) / pl.tok_per_pass;
  pl.ws_m = pl.ws_l = pl.ws_o = nullptr;
  pl.ws_count = nullptr;
  if (pl.kstride > 1) {
    size_t om, ol, oc;
    decode_workspace_layout((int64_t)a.num_seqs * a.ntok * a.num_q_heads, pl.kstride,
                            c.head_dim, a.num_seqs, &om, &ol, &oc);
    uint8_t* ws = static_cast<uint8_t*>(a.workspace);
    pl.ws_o = reinterpret_cast<float*>(ws);
    pl.ws_m = reinterpret_cast<float*>(ws + om);
    pl.ws_l = reinterpret_cast<float*>(ws + ol);
    pl.ws_count = reinterpret_cast<int32_t*>(ws + oc);
  }
  const bool bf16_out = a.out_dtype == PKV_BF16;
  if (c.head_dim == 128)
    return bf16_out ? run_d_out<128, OUT_BF16>(a, pl, st) : run_d_out<128, OUT_F32>(a, pl, st);
  return bf16_out ? run_d_out<64, OUT_BF16>(a, pl, st) : run_d_out<64, OUT_F32>(a, pl, st);
}

}  // namespace pkv
