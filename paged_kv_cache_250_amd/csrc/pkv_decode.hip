// Paged decode attention for gfx950.
//
// One new query token per sequence attends over the sequence's cached K/V,
// which live in fixed-size blocks scattered through a pool and are found
// through the sequence's block table ("KV Cache Compression & Paged
// Attention Deep Dive", section "Implementation Details: PagedAttention
// Kernel and Page Table": the kernel walks the logical blocks, translates
// each to its physical block and loads K and V from there).  The output of
// query head h is softmax(scale * q_h . K^T) V ("KV Cache Optimization: 3x
// Faster LLM Inference on 24GB VRAM", section "Why Standard Approaches
// Fail"), with query heads h = g*G .. g*G+G-1 sharing KV head g (grouped-
// query attention, same section).
//
// Work decomposition.  One workgroup of NWAVES waves handles one (sequence,
// KV head, partition); partitions are runs of `part` tokens (a multiple of
// the block size).  Each wave streams whole blocks: it loads the block's K
// rows and V channel rows with 64..128-bit loads straight into matrix-core
// operand registers, computes S = K q^T for all G query heads of the group
// on the matrix cores (16x16x32 MFMA, the group padded to 16 heads), runs
// the online softmax in fp32 (running max m and sum l per head), and
// accumulates O^T += V^T P^T on the matrix cores (16x16x16 MFMA).  P is
// split into a high and a low 16-bit part so that the product keeps about
// 16 significant bits of each weight; accumulation is fp32.  The waves of a
// workgroup merge through LDS.  A sequence that fits in one partition is
// written out directly; otherwise each partition leaves (m, l, acc) in the
// workspace and pkv_lse_reduce merges them.
//
// Register layouts (wave64, lane = 16 * g + j, g = lane / 16, j = lane % 16):
//   16x16x32 MFMA  A: row j, k = 8g..8g+7   B: column j, k = 8g..8g+7
//   16x16x16 MFMA  A: row j, k = 4g..4g+3   B: column j, k = 4g..4g+3
//   result         D: rows 4g..4g+3, column j
// Q.K^T: A = K (row j = token j of a 16-token half-block, channels
// 32c+8g..+7 of chunk c), B = Q (column j = query head j of the group, same
// channels) -> lane holds S[token 4g+r][head j].  P.V: A = V^T (row j =
// channel 16t+j, k = tokens 4g..4g+3), B = P^T exactly as S came out ->
// lane holds O^T[channel 16t+4g+r][head j].
#include <cmath>
#include <mutex>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// Build-time tuning knobs (chosen by measurement at the workloads' full
// sizes).  PKV_NWAVES: waves per workgroup.  Units each wave keeps in flight
// ahead of the one it computes, and waves per SIMD, per cache type: 16-bit
// units are 8 KB per wave, so two in flight at one wave per SIMD keep enough
// bytes outstanding (Little's law) with the registers of a whole SIMD; FP8
// units (4 KB) run best with one in flight at two waves per SIMD; INT4 units
// carry 2.5 KB and cheap loads but much arithmetic, so two (unit stream with
// fixed partitions) or three (per-item kernels) in flight at two waves per
// SIMD, and one at three waves per SIMD on the balanced split.
#ifndef PKV_NWAVES
#define PKV_NWAVES 4
#endif
#ifndef PKV_SK_WAVES_PER_EU_16
#define PKV_SK_WAVES_PER_EU_16 1
#endif
#ifndef PKV_SK_DEPTH_16
#define PKV_SK_DEPTH_16 2
#endif
#ifndef PKV_SK_WAVES_PER_EU_Q
#define PKV_SK_WAVES_PER_EU_Q 2
#endif
#ifndef PKV_SK_DEPTH_Q
#define PKV_SK_DEPTH_Q 1
#endif
#ifndef PKV_DEPTH
#define PKV_DEPTH 2
#endif
#ifndef PKV_DEPTH_I4
#define PKV_DEPTH_I4 3
#endif
#ifndef PKV_SK_DEPTH_I4
#define PKV_SK_DEPTH_I4 2
#endif
// INT4 on the balanced split: waves per SIMD and units in flight (INT4
// reads the query at each piece's start, which frees the registers of the
// queries in flight and lets a third wave per SIMD in)
#ifndef PKV_SK_WAVES_PER_EU_I4B
#define PKV_SK_WAVES_PER_EU_I4B 3
#endif
#ifndef PKV_SK_DEPTH_I4B
#define PKV_SK_DEPTH_I4B 1
#endif
#ifndef PKV_SK_WAVES_PER_EU_I4
#define PKV_SK_WAVES_PER_EU_I4 2
#endif
#ifndef PKV_PD_WAVES_PER_EU_I4
#define PKV_PD_WAVES_PER_EU_I4 2
#endif
#ifndef PKV_PD_WAVES_PER_EU
#define PKV_PD_WAVES_PER_EU 2
#endif
// Parts the one-wave merge requests per round (before it knows the part
// count, for the first round): the small batch where runs have few parts
// on average (the stale slots it reads are wasted bytes), the large one
// where they have more (a second round would cost a round trip).
#ifndef PKV_MERGE_BATCH
#define PKV_MERGE_BATCH 8
#endif
#ifndef PKV_MERGE_BATCH_SMALL
#define PKV_MERGE_BATCH_SMALL 4
#endif
constexpr int NWAVES = PKV_NWAVES;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// The two FP8 cache types share layouts, scales and code paths; only the
// code-to-operand conversion differs.
template <int KV>
constexpr bool kFp8 = KV == PKV_FP8_E4M3 || KV == PKV_FP8_E5M2;

// ----------------------------------------------------------- MMA element

template <bool BF>
struct Mma;

template <>
struct Mma<true> {  // bfloat16 operands
  static __device__ __forceinline__ f32x4 k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), c, 0,
                                                   0, 0);
  }
  static __device__ __forceinline__ f32x4 k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bitcast<i16x4>(a), bitcast<i16x4>(b), c, 0,
                                                     0, 0);
  }
  static __device__ __forceinline__ uint32_t enc(float x) {
    return bitcast<uint16_t>((__bf16)x);  // v_cvt_pk_bf16_f32: round to nearest even
  }
  static __device__ __forceinline__ float dec(uint32_t h) { return __uint_as_float(h << 16); }
  // two FP8 codes (bytes 2*HI, 2*HI+1 of w) -> two bf16, exact (E4M3 and
  // E5M2 values have at most 4 significant bits and lie in bf16's range)
  template <int KV, bool HI>
  static __device__ __forceinline__ uint32_t fp8x2(uint32_t w) {
    if constexpr (KV == PKV_FP8_E5M2)
      return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI));
    else
      return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
  }
  static constexpr int P_SHIFT = 0;  // P is scaled by 2^P_SHIFT before the split
};

template <>
struct Mma<false> {  // fp16 operands
  static __device__ __forceinline__ f32x4 k32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(bitcast<f16x8>(a), bitcast<f16x8>(b), c, 0, 0,
                                                  0);
  }
  static __device__ __forceinline__ f32x4 k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(bitcast<f16x4>(a), bitcast<f16x4>(b), c, 0, 0,
                                                 0);
  }
  static __device__ __forceinline__ uint32_t enc(float x) {
    return bitcast<uint16_t>((_Float16)x);
  }
  static __device__ __forceinline__ float dec(uint32_t h) {
    return (float)bitcast<_Float16>((uint16_t)h);
  }
  template <int KV, bool HI>
  static __device__ __forceinline__ uint32_t fp8x2(uint32_t w) {
    if constexpr (KV == PKV_FP8_E5M2)  // an E5M2 code is the top byte of its fp16 value
      return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_bf8(w, 1.0f, HI));
    else
      return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
  // fp16 has a narrow exponent range: weights p in [0, 2^8] (see LAZY) are
  // lifted by 2^6 so that they stay normal numbers down to p = 2^-20 and
  // below 2^14 at the top.
  static constexpr int P_SHIFT = 6;
};

// Two fp32 values -> a 16-bit pair (a in the low half), one packed
// conversion (round to nearest even, as Mma::enc).
template <bool BF>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  if constexpr (BF) return bitcast<uint32_t>(__builtin_convertvector(f32x2{a, b}, bf16x2));
  else return bitcast<uint32_t>(__builtin_convertvector(f32x2{a, b}, f16x2));
}

// INT4 codes as matrix-core operands.  A 4-bit code c placed in the low
// mantissa bits of an fp16 value with a zero exponent field is the subnormal
// c 2^-24 (16 c 2^-24 four bits up), exactly; the matrix cores multiply such
// operands exactly (fp16 subnormals are not flushed).  So a 32-bit word of
// eight codes gives four operand pairs by masking alone: w & 0x000F000F keeps
// the codes at bits 0 and 16, w & 0x00F000F0 those at bits 4 and 20 (times
// 16), and the same masks on w >> 8 the codes at bits 8, 24 and 12, 28.
constexpr uint32_t NIB_LO = 0x000F000Fu, NIB_HI = 0x00F000F0u;

// K: eight codes of one token, channel e at bits 4e ->  operand pairs
// (e0, e4), 16 (e1, e5), (e2, e6), 16 (e3, e7), in units of 2^-24.
__device__ __forceinline__ u32x4 int4_k_operand(uint32_t w) {
  const uint32_t w8 = w >> 8;
  return u32x4{w & NIB_LO, w & NIB_HI, w8 & NIB_LO, w8 & NIB_HI};
}

// V: the word of two 16-channel tiles (a = even, b = odd) for tokens
// 4g + r, token r of parity-t tile at bit 16 (r % 2) + 8 (r / 2) + 4 t ->
// tile a pairs (r0, r1), (r2, r3) and tile b pairs 16 (r0, r1), 16 (r2, r3).
__device__ __forceinline__ void int4_v_operands(uint32_t w, u32x2& ta, u32x2& tb) {
  const uint32_t w8 = w >> 8;
  ta = u32x2{w & NIB_LO, w8 & NIB_LO};
  tb = u32x2{w & NIB_HI, w8 & NIB_HI};
}

// fp16 bits -> fp32 (exact); folded into v_fma_mix operands where it feeds
// a multiply-add.
__device__ __forceinline__ float h_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
__device__ __forceinline__ float h_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// Weight pair times fp16 scales as an fp16 pair and the fp16 rounding of
// the rest: hi = (f16(a0 s0), f16(a1 s1)), lo = (f16(a0 s0 - hi.x),
// f16(a1 s1 - hi.y)), where s0, s1 are the fp16 values in the low halves of
// w0, w1.  The products are mixed-precision FMAs (exact inside, one rounding;
// the +0 addend keeps the multiply an FMA), so the pair costs six VALU
// instructions and no conversions of the scales.
__device__ __forceinline__ void mix_split(float a0, uint32_t w0, float a1, uint32_t w1,
                                          uint32_t& hi, uint32_t& lo) {
  const float x0 = fmaf(a0, h_lo(w0), 0.0f), x1 = fmaf(a1, h_lo(w1), 0.0f);
  const f16x2 h = __builtin_convertvector(f32x2{x0, x1}, f16x2);
  const float r0 = fmaf(a0, h_lo(w0), -(float)h.x), r1 = fmaf(a1, h_lo(w1), -(float)h.y);
  hi = bitcast<uint32_t>(h);
  lo = bitcast<uint32_t>(__builtin_convertvector(f32x2{r0, r1}, f16x2));
}

// --------------------------------------------------------- io load/store

// Eight 16-bit query values as MMA operands: the io type is the operand type
// (INT4 caches convert their queries themselves, see setup_int4).
template <int IO, bool BF>
__device__ __forceinline__ u32x4 q_operand(u32x4 raw) {
  static_assert(IO != PKV_BF16 || BF, "bfloat16 queries feed bfloat16 products");
  return raw;
}

template <int IO, bool BF>
__device__ __forceinline__ u32x4 load_q8(const void* q, int64_t idx) {
  if constexpr (IO == PKV_F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(q) + idx);
    const f32x4 a = p[0], b = p[1];
    u32x4 r;
    r[0] = pack2<BF>(a[0], a[1]);
    r[1] = pack2<BF>(a[2], a[3]);
    r[2] = pack2<BF>(b[0], b[1]);
    r[3] = pack2<BF>(b[2], b[3]);
    return r;
  } else {
    return q_operand<IO, BF>(
        *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(q) + idx));
  }
}

// Stores 4 consecutive fp32 values in the io type.
template <int IO>
__device__ __forceinline__ void store4(void* out, int64_t idx, f32x4 v) {
  if constexpr (IO == PKV_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + idx) = v;
  } else {
    u32x2 w;
    if constexpr (IO == PKV_BF16) {
      w[0] = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
      w[1] = f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16);
    } else {
      w[0] = f32_to_f16_bits(v[0]) | (f32_to_f16_bits(v[1]) << 16);
      w[1] = f32_to_f16_bits(v[2]) | (f32_to_f16_bits(v[3]) << 16);
    }
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + idx) = w;
  }
}

// ------------------------------------------------------ per-block buffers

// A buffer resource over `bytes` bytes at `base`; loads past `bytes` return
// zeros without touching memory, so a zero-sized resource turns every load
// of an absent block into a no-op while keeping the instruction stream (and
// the wait counts) identical for every iteration.
// A wave-uniform pointer moved to scalar registers.  The builtin returns a
// signed int, so each half goes through uint32_t before it is widened: a
// sign-extended low half would corrupt the upper address bits.
__device__ __forceinline__ const char* uniform_ptr(const void* p) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return reinterpret_cast<const char*>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

template <int KV, int D, int P>
struct Geo {
  static constexpr int NC = D / 32;  // Q.K^T chunks of 32 channels
  static constexpr int NT = D / 16;  // P.V tiles of 16 channels
  static constexpr int NH = P / 16;  // 16-token halves
  static constexpr int NG = D / 32;  // INT4 groups per token
  static constexpr bool B16 = (KV == PKV_F16 || KV == PKV_BF16);
  // bytes of one (block, KV head) chunk of a pool and of its metadata
  static constexpr uint32_t KV_CHUNK =
      B16 ? P * D * 2 : (kFp8<KV> ? P * D : P * D / 2);
  static constexpr uint32_t META_CHUNK =
      kFp8<KV> ? P * 4 : (KV == PKV_INT4_ASYM_G32 ? P * NG * 4 : 0);
};

// Every chunk is stored in the order the MFMA operands are consumed, so
// that each lane receives its whole share of a 16-token unit with 16-byte
// loads (8-byte for INT4 at D = 64) and each load instruction of a wave
// covers 1 KB: the vector memory address unit costs about the same per
// instruction whatever its width, and it is the limit when loads are
// narrow.  Lane l = 16 g + j; unit hf holds tokens 16 hf .. 16 hf + 15;
// token 4 g + r of a unit, r < 4.
//
//   K, 16-bit:  [token][D]                       (lane: row j, channels 32c + 8g .. +7)
//   K, FP8:     [token][D/64][g][2][8]           (bytes; channel 32 (2h + s) + 8 g + e)
//   K, INT4:    [token][g][D/32][4 bytes]        (channels 32 c + 8 g + e, e even low nibble)
//   V, 16-bit:  [unit][D/32][j][g][2][4 tokens]  (channel 16 (2s + q) + j)
//   V, FP8:     [unit][D/64][j][g][4][4 tokens]  (bytes; channel 16 (4s + q) + j)
//   V, INT4:    [unit][j][g][D/16][2 bytes]      (tile t, token 4g + r at nibble r)
//   FP8 scales: [token] fp32
//   INT4 meta:  [unit][g][D/32][4 tokens] (s, z) fp16 pairs
template <int KV, int D, int P>
struct BlockBuf {
  using G_ = Geo<KV, D, P>;
  static constexpr int NC = G_::NC, NT = G_::NT, NG = G_::NG;
  static constexpr bool I4 = KV == PKV_INT4_ASYM_G32;
  static constexpr int K_LOADS = G_::B16 ? NC : (kFp8<KV> ? NC / 2 : 1);
  static constexpr int V_LOADS = G_::B16 ? NT / 2 : (kFp8<KV> ? NT / 4 : 1);
  using WT = typename std::conditional<I4 && D == 64, u32x2, u32x4>::type;
  WT k[K_LOADS];
  WT v[V_LOADS];
  f32x4 ks, vs;  // FP8 scales of tokens 4g..4g+3
  u32x4 km, vm;  // INT4 (s, z) of tokens 4g..4g+3, group j % NG
};

// Per-lane byte offsets inside the first unit of a (block, KV head) chunk.
template <int KV, int D, int P>
struct LaneOffsets {
  uint32_t k, v, m;
  __device__ __forceinline__ LaneOffsets(int g, int j) {
    constexpr int NG = Geo<KV, D, P>::NG, NT = Geo<KV, D, P>::NT;
    if constexpr (Geo<KV, D, P>::B16) {
      k = (j * D + 8 * g) * 2;
      v = (j * 4 + g) * 16;
      m = 0;
    } else if constexpr (kFp8<KV>) {
      k = (j * 4 + g) * 16;
      v = (j * 4 + g) * 16;
      m = 16 * g;
    } else {
      k = j * (D / 2) + g * (D / 8);
      v = (j * 4 + g) * (NT * 2);
      m = (g * NG + (j % NG)) * 16;
    }
  }
};

// Cache policy of the pool loads: non-temporal.  Every pool byte is read
// once per call, so the lines are marked to leave the caches first; plain
// loads let the stream push out the lines that are reused (tables, queries,
// partial results) and were measured about 10% slower on the bf16 batch.
constexpr int STREAM = 2;

// Issues the loads of 16-token unit `hf` of a chunk (hf < P / 16).
template <int KV, int D, int P>
__device__ __forceinline__ void load_unit(BlockBuf<KV, D, P>& bb, const LaneOffsets<KV, D, P>& lo,
                                          int hf, __amdgpu_buffer_rsrc_t rk,
                                          __amdgpu_buffer_rsrc_t rv, __amdgpu_buffer_rsrc_t rkm,
                                          __amdgpu_buffer_rsrc_t rvm) {
  using BB = BlockBuf<KV, D, P>;
  constexpr int NG = Geo<KV, D, P>::NG;
  if constexpr (Geo<KV, D, P>::B16) {
#pragma unroll
    for (int c = 0; c < BB::K_LOADS; ++c)
      bb.k[c] = bitcast<u32x4>(
          __builtin_amdgcn_raw_buffer_load_b128(rk, lo.k + c * 64, hf * 32 * D, STREAM));
#pragma unroll
    for (int s = 0; s < BB::V_LOADS; ++s)
      bb.v[s] = bitcast<u32x4>(
          __builtin_amdgcn_raw_buffer_load_b128(rv, lo.v + s * 1024, hf * 32 * D, STREAM));
  } else if constexpr (kFp8<KV>) {
#pragma unroll
    for (int h = 0; h < BB::K_LOADS; ++h)
      bb.k[h] = bitcast<u32x4>(
          __builtin_amdgcn_raw_buffer_load_b128(rk, lo.k + h * 1024, hf * 16 * D, STREAM));
#pragma unroll
    for (int s = 0; s < BB::V_LOADS; ++s)
      bb.v[s] = bitcast<u32x4>(
          __builtin_amdgcn_raw_buffer_load_b128(rv, lo.v + s * 1024, hf * 16 * D, STREAM));
    bb.ks = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(rkm, lo.m, hf * 64, STREAM));
    bb.vs = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(rvm, lo.m, hf * 64, STREAM));
  } else {
    if constexpr (D == 128) {
      bb.k[0] = bitcast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(rk, lo.k, hf * 8 * D, STREAM));
      bb.v[0] = bitcast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(rv, lo.v, hf * 8 * D, STREAM));
    } else {
      bb.k[0] = bitcast<u32x2>(__builtin_amdgcn_raw_buffer_load_b64(rk, lo.k, hf * 8 * D, STREAM));
      bb.v[0] = bitcast<u32x2>(__builtin_amdgcn_raw_buffer_load_b64(rv, lo.v, hf * 8 * D, STREAM));
    }
    bb.km = bitcast<u32x4>(
        __builtin_amdgcn_raw_buffer_load_b128(rkm, lo.m, hf * 16 * NG * 4, STREAM));
    bb.vm = bitcast<u32x4>(
        __builtin_amdgcn_raw_buffer_load_b128(rvm, lo.m, hf * 16 * NG * 4, STREAM));
  }
}

// x from lane (lane & ~3) + C, for every lane.  PKV_QUAD_DPP 0: a
// quad-mode swizzle, which runs in the LDS unit (idle in these kernels) and
// leaves the vector ALU to the arithmetic, at the LDS unit's latency;
// 1: a DPP quad_perm move, one VALU instruction with no round trip.
#ifndef PKV_QUAD_DPP
#define PKV_QUAD_DPP 0
#endif
template <int C>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
  if constexpr (PKV_QUAD_DPP)
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, C * 0x55, 0xF, 0xF, false);
  else
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x8000 | (C * 0x55));
}

// INT4 (s, z) of token 4g + r and group gr, from the lanes that loaded them.
template <int NG>
__device__ __forceinline__ uint32_t int4_meta(const u32x4& m, int r, int gr) {
  const uint32_t x = m[r];
  if constexpr (NG == 4) {
    switch (gr) {
      case 0: return quad_bcast<0>(x);
      case 1: return quad_bcast<1>(x);
      case 2: return quad_bcast<2>(x);
      default: return quad_bcast<3>(x);
    }
  } else {
    return gr == 0 ? quad_bcast<0>(x) : quad_bcast<1>(x);
  }
}

// Units a wave keeps in flight ahead of the one it computes.
template <int KV>
struct Depth {
  static constexpr int value = KV == PKV_INT4_ASYM_G32 ? PKV_DEPTH_I4 : PKV_DEPTH;
};

// ------------------------------------------------------------ the kernels

struct DecodeParams {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const void* k_meta;
  const void* v_meta;
  const int32_t* block_tables;
  const int32_t* ctx_lens;
  float* ws_m;
  float* ws_l;
  float* ws_acc;
  int32_t* ws_np;  // balanced split: parts of each (sequence, KV head)
  int32_t* bad_blocks;  // optional: count of units whose block id is outside the pool
  int32_t Hkv, Hq, G, W, max_ctx;
  int32_t part;     // fixed partitions: tokens per partition
  int32_t P_max;    // partial slots per (sequence, head)
  int32_t num_seqs; // B
  int32_t plan_B;   // > 0: persistent workgroups over plan_B sequences (plan in LDS)
  int32_t workers;  // balanced split: waves in the grid
  int32_t run_cost; // balanced split: cost positions before each run (0: the unit line)
  int64_t num_blocks;
  float scale_log2;  // softmax scale * log2(e)
};

// Scores are kept relative to a reference max per head that moves (and
// rescales the accumulators) only when a score exceeds it by more than LAZY
// (log2 units), so weights stay below 2^LAZY and the common unit needs no
// cross-lane reduction.
constexpr float LAZY = 8.0f;

// State of one wave working on one (sequence, KV head): the query operands
// of the group's heads and the online-softmax accumulators of head j, where
// lane = 16 g + j holds tokens 4g..4g+3 of each 16-token unit.
template <int KV, int IO, int OUT, int D, int P, bool BF>
struct WaveState {
  using BB = BlockBuf<KV, D, P>;
  using G_ = Geo<KV, D, P>;
  using M = Mma<BF>;
  static constexpr int KVT = KV;
  static constexpr int NC = G_::NC, NT = G_::NT, NH = G_::NH, NG = G_::NG;
  // Weights enter the products as p 2^LIFT (times the per-token scale for
  // FP8 V and INT4 V), p <= 2^LAZY.  bfloat16 has the range of fp32; in
  // fp16 the product must stay below 65504: 16-bit caches have no scale
  // (2^(8+6)), E4M3 scales are at most 65504 / 448 < 147 for fp16 inputs
  // (2^8 * 147), E5M2 scales 128 times less (2^(8+7) * 65504 / 57344),
  // INT4 scales at most 2 * 65504 / 15 < 8737 (2^(8-6) * 8737).
  static constexpr int LIFT =
      BF ? 0
         : (KV == PKV_FP8_E4M3 ? 0
                               : (KV == PKV_FP8_E5M2 ? 7
                                                     : (KV == PKV_INT4_ASYM_G32 ? -6 : M::P_SHIFT)));
  static constexpr bool I4 = KV == PKV_INT4_ASYM_G32;
  static_assert(!I4 || !BF, "INT4 caches use fp16 products");
  static __device__ __forceinline__ constexpr float pow2(int e) {
    return e >= 0 ? (float)(1u << e) : 1.0f / (float)(1u << -e);
  }

  int lane, g, j;
  LaneOffsets<KV, D, P> lo;
  u32x4 qop[NC];   // B operand of Q.K^T: head j, channels 32c + 8g .. +7
  float qz[NC];    // INT4: 2^-24 times the sum of the chunk's scaled query channels
  float sl;        // INT4: scale of the raw scores to log2 units (head j)
  f32x4 acc[NT];   // O^T[channel 16t + 4g + r][head j], lifted by 2^LIFT
  float m_run;     // reference max of head j (log2 units), equal in the 4 lane groups
  float l_run;     // sum of weights over this lane's tokens, lifted by 2^LIFT until
                   // finish (then unlifted, and summed over all lanes of head j)
  float zterm[NG];  // INT4: sum of p * z per group over this lane's tokens

  __device__ __forceinline__ WaveState()
      : lane(threadIdx.x & 63), g((threadIdx.x & 63) >> 4), j(threadIdx.x & 15), lo(g, j) {}

  // Loads the query operands of (b, kvh) and clears the accumulators.
  __device__ __forceinline__ void begin(const DecodeParams& prm, int b, int kvh) {
    set_query(prm, b, kvh);
    reset();
  }

  // Takes query values loaded elsewhere in the io type (zeros for heads
  // past the group) and clears the accumulators.
  __device__ __forceinline__ void begin(const u32x4 (&q)[NC], float scale_log2) {
    set_query(q, scale_log2);
    reset();
  }

  // The query operands of (b, kvh), loaded here.
  __device__ __forceinline__ void set_query(const DecodeParams& prm, int b, int kvh) {
    const bool hvalid = j < prm.G;
    const int64_t qbase = ((int64_t)b * prm.Hq + kvh * prm.G + j) * D;
    if constexpr (I4) {
      float qf[NC][8];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int64_t idx = qbase + 32 * c + 8 * g;
        if constexpr (IO == PKV_F32) {
          const f32x4* qp = reinterpret_cast<const f32x4*>(static_cast<const float*>(prm.q) + idx);
          const f32x4 a = hvalid ? qp[0] : f32x4{0, 0, 0, 0}, b2 = hvalid ? qp[1] : f32x4{0, 0, 0, 0};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            qf[c][i] = a[i];
            qf[c][4 + i] = b2[i];
          }
        } else {
          const u32x4 raw = hvalid ? *reinterpret_cast<const u32x4*>(
                                         static_cast<const uint16_t*>(prm.q) + idx)
                                   : u32x4{0, 0, 0, 0};
          decode_q16(raw, qf[c]);
        }
      }
      setup_int4(qf, prm.scale_log2);
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        qop[c] = hvalid ? load_q8<IO, BF>(prm.q, qbase + 32 * c + 8 * g) : u32x4{0, 0, 0, 0};
    }
  }

  // The query operands from values loaded elsewhere in the io type.
  __device__ __forceinline__ void set_query(const u32x4 (&q)[NC], float scale_log2) {
    if constexpr (I4) {
      float qf[NC][8];
#pragma unroll
      for (int c = 0; c < NC; ++c) decode_q16(q[c], qf[c]);
      setup_int4(qf, scale_log2);
    } else {
#pragma unroll
      for (int c = 0; c < NC; ++c) qop[c] = q_operand<IO, BF>(q[c]);
    }
  }

  // Eight 16-bit query values (io type) -> fp32.
  static __device__ __forceinline__ void decode_q16(const u32x4& raw, float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (IO == PKV_BF16) {
        x[2 * i] = __uint_as_float(raw[i] << 16);
        x[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
      } else {
        x[2 * i] = h_lo(raw[i]);
        x[2 * i + 1] = h_hi(raw[i]);
      }
    }
  }

  // INT4 query operands.  Head j's values are scaled by 2^-e so that the
  // largest magnitude of the head lies in [2^14, 2^15) (exact for 16-bit
  // inputs in fp16's normal range), rounded to fp16 and placed in the
  // operand order of int4_k_operand, channels whose codes arrive times 16
  // being divided by 16.  The products then give T = 2^-24 2^-e sum q code,
  // the zero-point term uses qz = 2^-24 times the sum of the same scaled
  // values, and sl = scale * log2(e) * 2^(24 + e) turns a raw score into log2
  // units.
  __device__ __forceinline__ void setup_int4(float (&qf)[NC][8], float scale_log2) {
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(qf[c][i]));
    amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
    int e = 0;
    if (amax > 0.0f) {
      int ex;
      (void)__builtin_frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex)
      e = min(max(ex - 15, -100), 100);
    }
    const float f = __builtin_ldexpf(1.0f, -e), f16th = __builtin_ldexpf(1.0f, -e - 4);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      _Float16 h[8];
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool sixteenth = (i & 1) != 0;  // channels 1, 3, 5, 7: codes times 16
        h[i] = (_Float16)(qf[c][i] * (sixteenth ? f16th : f));
        sum += sixteenth ? 16.0f * (float)h[i] : (float)h[i];
      }
      qop[c] = u32x4{bitcast<uint32_t>(f16x2{h[0], h[4]}), bitcast<uint32_t>(f16x2{h[1], h[5]}),
                     bitcast<uint32_t>(f16x2{h[2], h[6]}), bitcast<uint32_t>(f16x2{h[3], h[7]})};
      sum += __shfl_xor(sum, 16, 64);
      sum += __shfl_xor(sum, 32, 64);
      qz[c] = sum * 5.9604644775390625e-8f;  // 2^-24, exact
    }
    sl = __builtin_ldexpf(scale_log2, 24 + e);
  }

  __device__ __forceinline__ void reset() {
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = f32x4{0, 0, 0, 0};
    m_run = -INFINITY;
    l_run = 0.0f;
#pragma unroll
    for (int gr = 0; gr < NG; ++gr) zterm[gr] = 0.0f;
  }

  // Issues the loads of 16-token unit `hf` of physical block `phys` and
  // returns the number of valid tokens: 0 (and every load empty) when nv is
  // 0 or the block id is outside the pool.
  __device__ __forceinline__ int fetch(BB& bb, const DecodeParams& prm, int kvh, int32_t phys,
                                       int hf, int nv) {
    int64_t chunk = 0;
    if ((uint32_t)phys < (uint32_t)prm.num_blocks && nv > 0) {
      chunk = (int64_t)phys * prm.Hkv + kvh;
    } else {
      // a unit with tokens whose block id is outside the pool is left out
      // of the softmax and counted (phys and nv are wave-uniform)
      if (nv > 0 && prm.bad_blocks && lane == 0) atomicAdd(prm.bad_blocks, 1);
      nv = 0;
    }
    // all of these are wave-uniform; readfirstlane keeps them in scalar
    // registers so that the buffer resources are scalar too
    nv = __builtin_amdgcn_readfirstlane(nv);
    const uint32_t c_lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)chunk);
    const uint32_t c_hi =
        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)chunk >> 32));
    const uint64_t ch = ((uint64_t)c_hi << 32) | c_lo;
    const uint32_t kvb = nv ? G_::KV_CHUNK : 0u;
    const uint32_t mb = nv ? G_::META_CHUNK : 0u;
    const char* kpool = static_cast<const char*>(prm.k_pool);
    const char* vpool = static_cast<const char*>(prm.v_pool);
    const char* kmeta = static_cast<const char*>(prm.k_meta);
    const char* vmeta = static_cast<const char*>(prm.v_meta);
    load_unit<KV, D, P>(bb, lo, hf, make_rsrc(kpool + ch * G_::KV_CHUNK, kvb),
                        make_rsrc(vpool + ch * G_::KV_CHUNK, kvb),
                        make_rsrc(kmeta + ch * G_::META_CHUNK, mb),
                        make_rsrc(vmeta + ch * G_::META_CHUNK, mb));
    return nv;
  }

  // Scores, online softmax and P.V of one loaded unit with nv valid tokens.
  __device__ __forceinline__ void compute(const BB& bb, const int nv, const float scale_log2) {
    accumulate(bb, nv, scores(bb, nv, scale_log2));
  }

  // Scores of the unit's 16 tokens in log2 units (-inf past the end): lane
  // holds tokens 4g..4g+3 of head j.  Depends on the query operands only,
  // not on the softmax state, so a unit's scores can be computed while the
  // previous unit is still being accumulated.
  __device__ __forceinline__ f32x4 scores(const BB& bb, const int nv,
                                          const float scale_log2) const {
    f32x4 s2;
    {
      f32x4 sc = f32x4{0, 0, 0, 0};
      if constexpr (I4) {
        // per group c: T = sum q code on the matrix cores (exact codes), then
        // S T + Z sum q for each token's (S, Z), as mixed-precision FMAs
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const f32x4 t = M::k32(int4_k_operand(bb.k[0][c]), qop[c], f32x4{0, 0, 0, 0});
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t sz = int4_meta<NG>(bb.km, r, c);
            sc[r] = fmaf(h_lo(sz), t[r], fmaf(h_hi(sz), qz[c], sc[r]));
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          u32x4 kop;
          if constexpr (kFp8<KV>) {
            const uint32_t w0 = bb.k[c / 2][2 * (c % 2)], w1 = bb.k[c / 2][2 * (c % 2) + 1];
            kop[0] = M::template fp8x2<KV, false>(w0);
            kop[1] = M::template fp8x2<KV, true>(w0);
            kop[2] = M::template fp8x2<KV, false>(w1);
            kop[3] = M::template fp8x2<KV, true>(w1);
          } else {
            kop = bb.k[c];
          }
          sc = M::k32(kop, qop[c], sc);
        }
        if constexpr (kFp8<KV>) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[r] *= bb.ks[r];
        }
      }
      const float ss = I4 ? sl : scale_log2;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool valid = (4 * g + r) < nv;
        s2[r] = valid ? sc[r] * ss : -INFINITY;
      }
    }
    return s2;
  }

  // Online softmax and P.V of one loaded unit given its scores.
  __device__ __forceinline__ void accumulate(const BB& bb, const int nv, const f32x4 s2) {
    // ---- reference max: moves only when some score passes it by LAZY
    const float lm = fmaxf(fmaxf(s2[0], s2[1]), fmaxf(s2[2], s2[3]));
    if (__any(lm > m_run + LAZY)) {
      float bm = fmaxf(lm, __shfl_xor(lm, 16, 64));
      bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
      const float m_new = fmaxf(m_run, bm);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] *= alpha;
#pragma unroll
      for (int gr = 0; gr < NG; ++gr) zterm[gr] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    // weights come out lifted: p 2^LIFT = exp2(s - (m - LIFT))
    const float m_off = (m_run == -INFINITY ? 0.0f : m_run) - (float)LIFT;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = __builtin_amdgcn_exp2f(s2[r] - m_off);
      l_run += p[r];
    }
    if constexpr (I4) {
      // acc += sum_t (p_t S_t,grp) code_t on the matrix cores; sum_t p_t Z_t,grp
      // is kept per group and added in finish().  p S goes in as an fp16
      // high part and the fp16 rounding of the rest (v_fma_mixlo/hi), which
      // keeps about 22 bits of each weight.  Tokens past the end keep stale
      // metadata (possibly NaN): it is zeroed at its source, once per token,
      // with a select rather than a branch so that the lane broadcasts below
      // stay in uniform control flow
      u32x4 vm;
#pragma unroll
      for (int r = 0; r < 4; ++r) vm[r] = (4 * g + r) < nv ? bb.vm[r] : 0u;
      const float (&pl)[4] = p;
#pragma unroll
      for (int gr = 0; gr < NG; ++gr) {
        uint32_t sz[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sz[r] = int4_meta<NG>(vm, r, gr);
          zterm[gr] = fmaf(pl[r], h_hi(sz[r]), zterm[gr]);
        }
        uint32_t h01, l01, h23, l23;
        mix_split(pl[0], sz[0], pl[1], sz[1], h01, l01);
        mix_split(pl[2], sz[2], pl[3], sz[3], h23, l23);
        const u32x2 phi = {h01, h23}, plo = {l01, l23};
        u32x2 ta, tb;  // tiles 2 gr and 2 gr + 1 (the latter's codes times 16)
        int4_v_operands(bb.v[0][gr], ta, tb);
        acc[2 * gr] = M::k16(ta, phi, acc[2 * gr]);
        acc[2 * gr] = M::k16(ta, plo, acc[2 * gr]);
        acc[2 * gr + 1] = M::k16(tb, phi, acc[2 * gr + 1]);
        acc[2 * gr + 1] = M::k16(tb, plo, acc[2 * gr + 1]);
      }
    } else {
      float pw[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float x = p[r];
        if constexpr (kFp8<KV>) {
          const bool valid = (4 * g + r) < nv;
          x = valid ? x * bb.vs[r] : 0.0f;
        }
        pw[r] = x;
      }
      const u32x2 phi = {pack2<BF>(pw[0], pw[1]), pack2<BF>(pw[2], pw[3])};
      const u32x2 plo = {
          pack2<BF>(pw[0] - M::dec(phi[0] & 0xFFFF), pw[1] - M::dec(phi[0] >> 16)),
          pack2<BF>(pw[2] - M::dec(phi[1] & 0xFFFF), pw[3] - M::dec(phi[1] >> 16))};
      // tokens past the end of the sequence are zeroed in the V operand so
      // that stale pool contents (possibly NaN) cannot reach the accumulator
      uint32_t vmask0 = 0xFFFFFFFFu, vmask1 = 0xFFFFFFFFu;
      if (nv < 16) {  // wave-uniform
        const int t0 = 4 * g;
        vmask0 = (t0 + 0 < nv ? 0x0000FFFFu : 0u) | (t0 + 1 < nv ? 0xFFFF0000u : 0u);
        vmask1 = (t0 + 2 < nv ? 0x0000FFFFu : 0u) | (t0 + 3 < nv ? 0xFFFF0000u : 0u);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        u32x2 vop;
        if constexpr (kFp8<KV>) {
          vop[0] = M::template fp8x2<KV, false>(bb.v[t / 4][t % 4]);
          vop[1] = M::template fp8x2<KV, true>(bb.v[t / 4][t % 4]);
        } else {
          vop = u32x2{bb.v[t / 2][2 * (t % 2)], bb.v[t / 2][2 * (t % 2) + 1]};
        }
        vop[0] &= vmask0;
        vop[1] &= vmask1;
        acc[t] = M::k16(vop, phi, acc[t]);
        acc[t] = M::k16(vop, plo, acc[t]);
      }
    }
  }

  // Totals over the 4 lane groups: afterwards l_run is head j's sum of
  // weights in every lane and acc the unnormalised output (unlifted).
  __device__ __forceinline__ void finish() {
    const float unlift = pow2(-LIFT);
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    l_run *= unlift;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if constexpr (I4) {
        // codes entered as c 2^-24 (odd tiles 16 c 2^-24); zterm of group
        // t/2 (two 16-channel tiles per group of 32)
        float z = zterm[t / 2];
        z += __shfl_xor(z, 16, 64);
        z += __shfl_xor(z, 32, 64);
        acc[t] = acc[t] * ((t & 1) ? 1048576.0f : 16777216.0f) + z;
      }
      acc[t] *= unlift;
    }
  }

  // Normalised output of head j (lanes with j < G).
  __device__ __forceinline__ void store_output(const DecodeParams& prm, int b, int kvh) const {
    if (j >= prm.G) return;
    const float inv = l_run > 0.0f ? 1.0f / l_run : 0.0f;
    const int64_t base = ((int64_t)b * prm.Hq + kvh * prm.G + j) * D;
#pragma unroll
    for (int t = 0; t < NT; ++t) store4<OUT>(prm.out, base + 16 * t + 4 * g, acc[t] * inv);
  }

  // Partial (m, l, acc) of head j into workspace slot k.
  __device__ __forceinline__ void store_partial(const DecodeParams& prm, int b, int kvh,
                                                int k) const {
    if (j >= prm.G) return;
    const int64_t slot = ((int64_t)b * prm.Hq + kvh * prm.G + j) * prm.P_max + k;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      *reinterpret_cast<f32x4*>(prm.ws_acc + slot * D + 16 * t + 4 * g) = acc[t];
    }
    if (g == 0) {
      prm.ws_m[slot] = m_run == -INFINITY ? -INFINITY : m_run * LN2;  // units of the scaled score
      prm.ws_l[slot] = l_run;
    }
  }
};

// Runs `nunits` units through one wave: unit(u, buf) issues the loads of
// unit u (nothing for u >= nunits) and returns its valid tokens.  DEPTH
// units stay in flight ahead of the one being computed; every iteration
// issues the same loads, so the wait before each compute covers exactly the
// oldest unit.  The scheduling barriers keep each unit's loads ahead of the
// previous unit's arithmetic and give the loop head one load order on every
// path.
//
// Pipelined (PKV_PIPELINE, with at least two units in flight): the scores of
// unit L + 1 are computed in the same scheduling region as the softmax and
// P.V of unit L.  The two chains are independent (scores need only the
// query), so while one waits on a matrix-core result, an exponential or a
// lane broadcast, the other has instructions to issue.
#ifndef PKV_PIPELINE
#define PKV_PIPELINE 1
#endif
template <class WS, class UnitFn>
__device__ __forceinline__ void run_units(WS& ws, const float scale_log2, const int nunits,
                                          UnitFn&& unit) {
  constexpr int DEPTH = Depth<WS::KVT>::value;
  constexpr int NB = DEPTH + 1;
  typename WS::BB buf[NB];
  int nv[NB];
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) nv[s] = unit(s, buf[s]);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (PKV_PIPELINE && DEPTH >= 2) {
    f32x4 sc = ws.scores(buf[0], nv[0], scale_log2);
    for (int u0 = 0; u0 < nunits; u0 += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int slot = (k + DEPTH) % NB;
        nv[slot] = unit(u0 + k + DEPTH, buf[slot]);
        __builtin_amdgcn_sched_barrier(0);
        const int nk = (k + 1) % NB;  // unit u0 + k + 1 (its loads were issued earlier)
        const f32x4 sc_next = ws.scores(buf[nk], nv[nk], scale_log2);
        ws.accumulate(buf[k], nv[k], sc);
        sc = sc_next;
        __builtin_amdgcn_sched_barrier(0);
        if (u0 + k + 1 >= nunits) goto done;
      }
    }
  } else {
    for (int u0 = 0; u0 < nunits; u0 += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int slot = (k + DEPTH) % NB;
        nv[slot] = unit(u0 + k + DEPTH, buf[slot]);
        __builtin_amdgcn_sched_barrier(0);
        ws.compute(buf[k], nv[k], scale_log2);
        __builtin_amdgcn_sched_barrier(0);
        if (u0 + k + 1 >= nunits) goto done;
      }
    }
  }
done:;
}

template <int NT>
struct DecodeShared {
  float m[NWAVES][16];
  float l[NWAVES][16];
  f32x4 acc[NWAVES][NT][64];
};

__device__ __forceinline__ int clamp_len(const DecodeParams& prm, int n) {
  return n < 0 ? 0 : (n > prm.max_ctx ? prm.max_ctx : n);
}
__device__ __forceinline__ int clamp_ctx(const DecodeParams& prm, int b) {
  return clamp_len(prm, prm.ctx_lens[b]);
}

// ------------------------------------------------- fixed partitions

// One work item: partition `part` of sequence b for KV head kvh.  The
// NWAVES waves take the partition's blocks in turn (wave w: blocks w,
// w + NWAVES, ...) and merge their results through LDS.
template <int KV, int IO, int OUT, int D, int P, bool BF>
__device__ __forceinline__ void decode_item(const DecodeParams& prm, const int b, const int kvh,
                                            const int part,
                                            DecodeShared<Geo<KV, D, P>::NT>& sh) {
  using WS = WaveState<KV, IO, OUT, D, P, BF>;
  using BB = typename WS::BB;
  constexpr int NT = WS::NT, NH = WS::NH;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Block ids of this wave's next 64 blocks, one per lane, read with a
  // single load issued together with the context length and the query so
  // that the walk over the blocks never waits on the table.  Positions past
  // the table row are clamped into it and never used.
  const int32_t* table = prm.block_tables + (int64_t)b * prm.W;
  const int blk_begin = part * (prm.part / P);
  auto load_ids = [&](int chunk) -> int32_t {
    const int jb = blk_begin + wave + NWAVES * (64 * chunk + lane);
    return table[min(jb, prm.W - 1)];
  };
  int32_t ids = load_ids(0);

  const int n = clamp_ctx(prm, b);
  const int nparts = (n + prm.part - 1) / prm.part;
  WS ws;
  if (n == 0) {
    // empty sequence: zeros, written by the first partition's workgroup
    if (part == 0 && wave == 0) {
      ws.begin(prm, b, kvh);
      ws.store_output(prm, b, kvh);
    }
    return;
  }
  if (part >= nparts) return;
  ws.begin(prm, b, kvh);

  const int tok_end = min(n, (part + 1) * prm.part);
  const int blk_end = (tok_end + P - 1) / P;
  // this wave's blocks: blk_begin + wave + NWAVES * i for i < nbw
  const int nbw = max(0, (blk_end - blk_begin - wave + NWAVES - 1) / NWAVES);
  for (int chunk = 0; 64 * chunk < nbw; ++chunk) {
    if (chunk > 0) ids = load_ids(chunk);
    const int nb = min(64, nbw - 64 * chunk);
    run_units(ws, prm.scale_log2, nb * NH, [&](int u, BB& bb) -> int {
      const int i = u / NH, hf = u % NH;
      int32_t phys = -1;
      int nv = 0;
      if (i < nb) {
        const int jb = blk_begin + wave + NWAVES * (64 * chunk + i);
        phys = __builtin_amdgcn_readlane(ids, i);
        nv = max(0, min(16, tok_end - jb * P - 16 * hf));
      }
      return ws.fetch(bb, prm, kvh, phys, hf, nv);
    });
  }
  ws.finish();

  // ---- merge the waves through LDS; wave w finishes tiles w, w + NWAVES, ...
  const int g = ws.g, j = ws.j;
  if (g == 0) {
    sh.m[wave][j] = ws.m_run;
    sh.l[wave][j] = ws.l_run;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) sh.acc[wave][t][lane] = ws.acc[t];
  __syncthreads();
  float mw[NWAVES];
  float Mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) {
    mw[w] = sh.m[w][j];
    Mx = fmaxf(Mx, mw[w]);
  }
  float fw[NWAVES];
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) {
    fw[w] = mw[w] == -INFINITY ? 0.0f : exp2f(mw[w] - Mx);
    L += fw[w] * sh.l[w][j];
  }
  const bool single = nparts == 1;
  const int h = kvh * prm.G + j;
  for (int t = wave; t < NT; t += NWAVES) {
    f32x4 v = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) v += fw[w] * sh.acc[w][t][lane];
    if (j >= prm.G) continue;
    const int d = 16 * t + 4 * g;
    if (single) {
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      store4<OUT>(prm.out, ((int64_t)b * prm.Hq + h) * D + d, v * inv);
    } else {
      const int64_t slot = ((int64_t)b * prm.Hq + h) * prm.P_max + part;
      *reinterpret_cast<f32x4*>(prm.ws_acc + slot * D + d) = v;
    }
  }
  if (!single && wave == 0 && g == 0 && j < prm.G) {
    const int64_t slot = ((int64_t)b * prm.Hq + h) * prm.P_max + part;
    prm.ws_m[slot] = Mx * LN2;  // back to units of the scaled score
    prm.ws_l[slot] = L;
  }
}

// Exclusive prefix sum over the B sequences of g(clamped context length)
// into S[0..B] (LDS, at least PER_MAX * 64 * NWAVES + 1 entries), by the
// whole workgroup.  The lengths are read with independent, coalesced loads
// (thread t: sequences t, t + 64 NWAVES, ...) and go through LDS, so the
// plan costs one memory round trip; each thread then scans PER_MAX
// consecutive sequences.
template <int PER_MAX, class G>
__device__ __forceinline__ void plan_prefix(int* S, int* wsum, const DecodeParams& prm,
                                            const int B, G&& g) {
  constexpr int NT = 64 * NWAVES;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int n[PER_MAX];
#pragma unroll
  for (int e = 0; e < PER_MAX; ++e) n[e] = prm.ctx_lens[min(e * NT + tid, B - 1)];
#pragma unroll
  for (int e = 0; e < PER_MAX; ++e) {
    const int i = e * NT + tid;
    const int c = n[e] < 0 ? 0 : (n[e] > prm.max_ctx ? prm.max_ctx : n[e]);
    S[i] = i < B ? g(c) : 0;
  }
  __syncthreads();
  int cnt[PER_MAX];
  int run = 0;
#pragma unroll
  for (int e = 0; e < PER_MAX; ++e) {
    run += S[tid * PER_MAX + e];
    cnt[e] = run;  // inclusive prefix within the thread
  }
  int x = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int base = x - run;
  for (int w = 0; w < wave; ++w) base += wsum[w];
#pragma unroll
  for (int e = 0; e < PER_MAX; ++e) {
    const int bb = tid * PER_MAX + e;
    if (bb <= B) S[bb] = base + (e ? cnt[e - 1] : 0);
  }
  if (tid == NT - 1 && B == PER_MAX * NT) S[B] = base + run;
  __syncthreads();
}

// Single pass: one workgroup per (sequence, KV head), its NWAVES waves
// taking alternate blocks and merging through LDS (decode_item with the
// whole context as one partition).
template <int KV, int IO, int OUT, int D, int P, bool BF>
__global__ __launch_bounds__(64 * NWAVES, PKV_PD_WAVES_PER_EU) void paged_decode_kernel(
    const DecodeParams prm) {
  __shared__ DecodeShared<Geo<KV, D, P>::NT> sh;
  const int kvh = blockIdx.x % prm.Hkv;
  const int b = blockIdx.x / prm.Hkv;
  decode_item<KV, IO, OUT, D, P, BF>(prm, b, kvh, 0, sh);
}

// ------------------------------------------------- fixed partitions

// One wave per work item: partition `part` of sequence b for KV head kvh,
// streamed as one run of 16-token units (no merge inside the workgroup).  A
// sequence that fits one partition is written out directly; otherwise the
// partition's (m, l, acc) goes to its workspace slot.
template <int KV, int IO, int OUT, int D, int P, bool BF>
__device__ __forceinline__ void decode_partition(const DecodeParams& prm, const int b,
                                                 const int kvh, const int part) {
  using WS = WaveState<KV, IO, OUT, D, P, BF>;
  using BB = typename WS::BB;
  constexpr int NH = WS::NH;
  const int lane = threadIdx.x & 63;
  // the partition's block ids, one per lane, 64 at a time (positions past
  // the table row are clamped into it and never used)
  const int32_t* table = prm.block_tables + (int64_t)b * prm.W;
  const int blk_begin = part * (prm.part / P);
  auto load_ids = [&](int chunk) -> int32_t {
    return table[min(blk_begin + 64 * chunk + lane, prm.W - 1)];
  };
  int32_t ids = load_ids(0);
  const int n = clamp_ctx(prm, b);
  const int nparts = (n + prm.part - 1) / prm.part;
  WS ws;
  if (n == 0) {  // empty sequence: zeros, written by its first partition's wave
    if (part == 0) {
      ws.begin(prm, b, kvh);
      ws.store_output(prm, b, kvh);
    }
    return;
  }
  if (part >= nparts) return;
  ws.begin(prm, b, kvh);
  const int tok_end = min(n, (part + 1) * prm.part);
  const int nb = (tok_end - part * prm.part + P - 1) / P;  // blocks of the partition
  for (int chunk = 0; 64 * chunk < nb; ++chunk) {
    if (chunk > 0) ids = load_ids(chunk);
    const int nbc = min(64, nb - 64 * chunk);
    run_units(ws, prm.scale_log2, nbc * NH, [&](int u, BB& bb) -> int {
      const int i = u / NH, hf = u % NH;
      int32_t phys = -1;
      int nv = 0;
      if (i < nbc) {
        const int jb = blk_begin + 64 * chunk + i;
        phys = __builtin_amdgcn_readlane(ids, i);
        nv = max(0, min(16, tok_end - jb * P - 16 * hf));
      }
      return ws.fetch(bb, prm, kvh, phys, hf, nv);
    });
  }
  ws.finish();
  if (nparts == 1) ws.store_output(prm, b, kvh);
  else ws.store_partial(prm, b, kvh, part);
}

template <int KV>
struct PdTune {
  static constexpr int WAVES_PER_EU =
      KV == PKV_INT4_ASYM_G32 ? PKV_PD_WAVES_PER_EU_I4 : PKV_PD_WAVES_PER_EU;
};

// Fixed-partition kernel for batches too large for the stream's LDS plan:
// wave t of the grid takes item t = (sequence, partition) * Hkv + KV head,
// so that the waves of a workgroup read the same blocks for neighbouring
// heads.
template <int KV, int IO, int OUT, int D, int P, bool BF>
__global__ __launch_bounds__(64 * NWAVES, PdTune<KV>::WAVES_PER_EU) void partition_decode_kernel(
    const DecodeParams prm) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t w = (int64_t)blockIdx.x * NWAVES + wave;
  const int kvh = (int)(w % prm.Hkv);
  const int64_t r = w / prm.Hkv;
  const int part = (int)(r % prm.P_max);
  const int b = (int)(r / prm.P_max);
  if (b < prm.num_seqs) decode_partition<KV, IO, OUT, D, P, BF>(prm, b, kvh, part);
}

// --------------------------------------------- balanced (stream-K) split

// Each (sequence b, KV head) is a segment of nu_b = ceil(n_b / 16) units of
// 16 tokens; segments are laid end to end (sequence-major, then KV head)
// into U units.  Worker w (a wave) takes the positions [w L / NW,
// (w + 1) L / NW) of a line of length L:
//  - fixed partitions: the unit line itself (L = U);
//  - the balanced split: a cost line on which every segment is preceded by
//    SK_RUN_COST positions for the work a piece costs besides its units (its
//    query, the reset, the closing store: about one unit's time, measured as
//    1.0 us per run in a wave's work on the 70B- and 8B-shaped batches).  A
//    worker's units are those whose positions fall in its range, so a range
//    that ends in the cost before a segment leaves the whole segment to the
//    next worker, and a share crossing many short runs takes fewer units.
// A segment cut by a worker boundary leaves one partial (m, l, acc) per
// worker in the workspace; the merge kernel combines them.  NW never exceeds
// U / SK_MIN_UNITS, so every range covers at least that many positions and
// a segment of nu units has at most nu / SK_MIN_UNITS + 2 parts.
constexpr int SK_MIN_UNITS = 8;
constexpr int SK_PLAN_MAX = 4096;
#ifndef PKV_SK_RUN_COST
#define PKV_SK_RUN_COST 1
#endif

struct SkLine {
  int64_t U;  // length of the line
  int64_t nw;
  __device__ __forceinline__ SkLine(int64_t length, int workers, int64_t units) : U(length) {
    const int64_t cap = units / SK_MIN_UNITS;
    nw = workers < cap ? workers : (cap > 0 ? cap : 1);
  }
  __device__ __forceinline__ int64_t start(int64_t w) const { return w * U / nw; }
  // worker whose range holds position x
  __device__ __forceinline__ int64_t worker_of(int64_t x) const {
    return ((x + 1) * nw - 1) / U;
  }
};

// Position on the cost line of unit u of run (b, kvh): rc positions stand
// before each run, empty sequences' included.
__device__ __forceinline__ int64_t sk_cost(const int* PU, const int Hkv, const int rc,
                                           const int b, const int kvh, const int u) {
  const int pb = PU[b], nu = PU[b + 1] - pb;
  return (int64_t)Hkv * (pb + (int64_t)rc * b) + (int64_t)kvh * (nu + rc) + rc + u;
}

// The first unit (on the unit line) whose cost position is at least y; U
// when there is none.
__device__ __forceinline__ int64_t sk_unit_at(const int* PU, const int B, const int Hkv,
                                              const int rc, const int64_t y, const int64_t U) {
  if (y >= (int64_t)Hkv * (PU[B] + (int64_t)rc * B)) return U;
  int lo = 0, hi = B - 1;  // the largest b with Hkv (PU[b] + rc b) <= y
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)Hkv * (PU[mid] + (int64_t)rc * mid) <= y) lo = mid;
    else hi = mid - 1;
  }
  const int nu = PU[lo + 1] - PU[lo];
  // r < Hkv (nu + rc), which fits 32 bits; nu + rc > 0 (nu > 0 when rc = 0)
  const uint32_t r = (uint32_t)(y - (int64_t)Hkv * (PU[lo] + (int64_t)rc * lo));
  const uint32_t kvh = r / (uint32_t)(nu + rc);
  const int off = (int)(r - kvh * (uint32_t)(nu + rc)) - rc;
  return (int64_t)Hkv * PU[lo] + (int64_t)kvh * nu + (off > 0 ? off : 0);
}

// Per-lane description of unit x0 + lane of a wave's share (one window of
// 64 units): block id, sequence, unit within the sequence's run, context
// length, and kvh | opens-a-piece << 16 | closes-a-piece << 17.  A piece is
// the part of one (sequence, KV head) run inside the share.
struct SkWindow {
  int32_t phys, b, u, n, kf;
};

// Fixed partitions on the same line (pt = units per partition, 0 for the
// balanced split): share boundaries are moved to the nearest partition
// boundary of the run they fall in, so no partition is cut, and a piece
// opens and closes at partition boundaries.
__device__ __forceinline__ int64_t sk_align(const int* PU, const int B, const int Hkv,
                                            const int pt, int64_t x, int64_t U) {
  if (pt == 0 || x >= U) return x;
  int lo = 0, hi = B - 1;  // the sequence whose runs hold unit x
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)Hkv * PU[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  const int nu = PU[lo + 1] - PU[lo];
  const int64_t r = x - (int64_t)Hkv * PU[lo];
  const int64_t kvh = r / nu, u = r - kvh * nu;
  const int64_t ua = min((int64_t)nu, (u + pt / 2) / pt * pt);
  return (int64_t)Hkv * PU[lo] + kvh * nu + ua;
}

template <int NH>
__device__ __forceinline__ SkWindow sk_describe(const DecodeParams& prm, const int* PU,
                                                const int B, const int xs, const int xe,
                                                const int x0, const int pt) {
  const int Hkv = prm.Hkv;
  int x = x0 + (int)(threadIdx.x & 63);
  if (x >= xe) x = xe - 1;  // x0 < xe; lanes past the share repeat its last unit
  int lo = 0, hi = B - 1;   // largest b with Hkv * PU[b] <= x: a sequence with units
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (Hkv * PU[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  const int nu = PU[lo + 1] - PU[lo];
  const int r = x - Hkv * PU[lo];
  const int kvh = r / nu, u = r - kvh * nu;
  SkWindow d;
  d.b = lo;
  d.u = u;
  const bool opens = u == 0 || x == xs || (pt && u % pt == 0);
  const bool closes = u == nu - 1 || x == xe - 1 || (pt && u % pt == pt - 1);
  d.kf = kvh | (opens ? 1 << 16 : 0) | (closes ? 1 << 17 : 0);
  d.n = prm.ctx_lens[lo];
  d.phys = prm.block_tables[(int64_t)lo * prm.W + u / NH];  // u < ceil(n / 16) <= W * NH
  return d;
}

// Scalars that travel with a unit from its loads to its arithmetic.
struct SkInfo {
  int nv, b, kf, u;
};

template <int KV, int D, int P>
struct SkSlot {
  BlockBuf<KV, D, P> bb;
  u32x4 q[D / 32];  // query operands of the piece the unit opens (else zeros)
};

// Log-sum-exp merge of the np parts of run (b, kvh) into the output, by one
// wave: M = max m_k, out = sum e^(m_k - M) acc_k / sum e^(m_k - M) l_k;
// nothing to do when np <= 1 (the decode wrote the output).  `raw` is the
// part count for the balanced split and the context length for fixed
// partitions, as loaded (np follows from it).  Lane tasks are (head,
// 8 channels) pairs of the group; the parts are read BATCH at a time, with
// the maximum kept online.  The first BATCH parts are requested before raw
// is looked at (the reads stay inside the run's G P_max slots), so the read
// of the count and of the parts take one memory round trip together; slots
// at or past np, which may hold another head's parts or stale bytes, are
// left out of every sum.
template <int OUT, int D, int BATCH>
__device__ __forceinline__ void merge_run(const DecodeParams& prm, const int b, const int kvh,
                                          int raw) {
  constexpr int C8 = D / 8;
  const int lane = threadIdx.x & 63;
  // One buffer resource per array over the run's G heads (G P_max slots,
  // the host keeps G P_max D 4 bytes below 2^32), so that it is the same in
  // every lane and the loads need no per-head loop over resources; a lane's
  // head is an offset.
  const int64_t row0 = (int64_t)b * prm.Hq + (int64_t)kvh * prm.G;
  const uint32_t span = (uint32_t)prm.G * (uint32_t)prm.P_max;
  const auto rm = make_rsrc(prm.ws_m + row0 * prm.P_max, span * 4);
  const auto rl = make_rsrc(prm.ws_l + row0 * prm.P_max, span * 4);
  const auto ra = make_rsrc(prm.ws_acc + row0 * prm.P_max * D, span * D * 4);
  for (int t = lane; t < prm.G * C8; t += 64) {
    const int hh = t / C8, c = (t - hh * C8) * 8;
    const int64_t row = row0 + hh;
    const uint32_t s0 = (uint32_t)hh * (uint32_t)prm.P_max;  // the head's first slot
    float M = -INFINITY, L = 0.0f;
    f32x4 a0 = f32x4{0, 0, 0, 0}, a1 = f32x4{0, 0, 0, 0};
    float mk[BATCH], lk[BATCH];
    f32x4 x0[BATCH], x1[BATCH];
    // request parts k0 .. k0 + BATCH - 1
    auto load = [&](const int k0) {
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const uint32_t k = s0 + (uint32_t)(k0 + i);
        mk[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rm, k * 4, 0, 0));
        lk[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, k * 4, 0, 0));
        x0[i] = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(ra, (k * D + c) * 4, 0, 0));
        x1[i] = bitcast<f32x4>(
            __builtin_amdgcn_raw_buffer_load_b128(ra, (k * D + c + 4) * 4, 0, 0));
      }
    };
    // add the requested parts below np, keeping the maximum online
    auto add = [&](const int k0, const int np) {
      float Mb = M;
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        if (k0 + i >= np) mk[i] = -INFINITY;
        Mb = fmaxf(Mb, mk[i]);
      }
      if (Mb > M) {  // the reference moves: rescale what is summed so far
        const float sc = M == -INFINITY ? 0.0f : exp2f((M - Mb) * LOG2E);
        L *= sc;
        a0 *= sc;
        a1 *= sc;
        M = Mb;
      }
      // (stale slots past np may hold anything: selects, not branches, keep
      // them out, so that every requested load is consumed on every path)
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const bool in = k0 + i < np;
        const float wk = mk[i] == -INFINITY ? 0.0f : exp2f((mk[i] - M) * LOG2E);
        const f32x4 z4 = f32x4{0, 0, 0, 0};
        L += in ? wk * lk[i] : 0.0f;
        a0 += in ? wk * x0[i] : z4;
        a1 += in ? wk * x1[i] : z4;
      }
    };
    load(0);
    // the count is first looked at here, after the first parts are requested
    asm volatile("" : "+v"(raw));
    const int np = prm.part == 0 ? raw : (clamp_len(prm, raw) + prm.part - 1) / prm.part;
    add(0, np);
    for (int k0 = BATCH; k0 < np; k0 += BATCH) {
      load(k0);
      add(k0, np);
    }
    if (np <= 1) return;  // (the decode wrote the output)
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    store4<OUT>(prm.out, row * D + c, a0 * inv);
    store4<OUT>(prm.out, row * D + c + 4, a1 * inv);
  }
}

// Tuning per cache type; I4B: the INT4 instantiation for the balanced split
// (fixed partitions keep two waves per SIMD, whose 2,048 waves take the
// 512-token partitions of long contexts evenly).
template <int KV, bool I4B>
struct SkTune {
  static constexpr bool B16 = KV == PKV_F16 || KV == PKV_BF16;
  static constexpr bool I4 = KV == PKV_INT4_ASYM_G32;
  static constexpr int DEPTH =
      B16 ? PKV_SK_DEPTH_16
          : (I4 ? (I4B ? PKV_SK_DEPTH_I4B : PKV_SK_DEPTH_I4) : PKV_SK_DEPTH_Q);
  static constexpr int WAVES_PER_EU =
      B16 ? PKV_SK_WAVES_PER_EU_16
          : (I4 ? (I4B ? PKV_SK_WAVES_PER_EU_I4B : PKV_SK_WAVES_PER_EU_I4)
                : PKV_SK_WAVES_PER_EU_Q);
  // the query operands travel with a piece's first unit, except for INT4,
  // which reads (and converts) them when the piece opens: their registers
  // in flight cost it more than the read (fixed partitions of 512 tokens:
  // 88.9 against 87.6 us), and let a third wave per SIMD in on the
  // balanced split
  static constexpr bool Q_AHEAD = !I4;
};

template <int KV, int IO, int OUT, int D, int P, bool BF, bool I4B = false>
__global__ __launch_bounds__(64 * NWAVES, (SkTune<KV, I4B>::WAVES_PER_EU)) void
streamk_decode_kernel(const DecodeParams prm) {
  static_assert(!I4B || KV == PKV_INT4_ASYM_G32, "the balanced-split tuning is INT4's");
  using WS = WaveState<KV, IO, OUT, D, P, BF>;
  using Slot = SkSlot<KV, D, P>;
  constexpr int NH = WS::NH, NC = WS::NC;
  constexpr int DEPTH = SkTune<KV, I4B>::DEPTH;
  constexpr int NB = DEPTH + 1;
  // fp32 queries are converted at the piece start
  constexpr bool Q_AHEAD = IO != PKV_F32 && SkTune<KV, I4B>::Q_AHEAD;
  constexpr uint32_t QE = IO == PKV_F32 ? 4 : 2;
  __shared__ int PU[SK_PLAN_MAX + 1];  // PU[b] = units of one KV head of sequences before b
  __shared__ int wsum[NWAVES];
  const int B = prm.plan_B;
  plan_prefix<SK_PLAN_MAX / (64 * NWAVES)>(PU, wsum, prm, B, [](int n) { return (n + 15) >> 4; });
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hkv = prm.Hkv;
  const int pt = prm.part / 16;  // fixed partitions: units per partition (0: balanced split)
  const int rc = pt ? 0 : prm.run_cost;  // per-run cost positions (balanced split)
  const int64_t U = (int64_t)Hkv * PU[B];
  const SkLine line(pt ? U : (int64_t)Hkv * (PU[B] + (int64_t)rc * B), prm.workers, U);
  // Empty sequences get their zeros here; for the balanced split's merge,
  // the number of parts of every (sequence, KV head) run (0 when empty).
  for (int e = blockIdx.x * 64 * NWAVES + threadIdx.x; e < B * Hkv; e += gridDim.x * 64 * NWAVES) {
    const int bb = e / Hkv, kv = e - bb * Hkv;
    const int pb = PU[bb], nu = PU[bb + 1] - pb;
    int np = 0;
    if (nu > 0) {
      // the line positions of the run's first and last units
      const int64_t x0 = pt ? (int64_t)Hkv * pb + (int64_t)kv * nu : sk_cost(PU, Hkv, rc, bb, kv, 0);
      np = (int)(line.worker_of(x0 + nu - 1) - line.worker_of(x0) + 1);
    } else {
      const int64_t o = ((int64_t)bb * prm.Hq + (int64_t)kv * prm.G) * D;
      for (int i = 0; i < prm.G * D; i += 4) store4<OUT>(prm.out, o + i, f32x4{0, 0, 0, 0});
    }
    if (pt == 0) prm.ws_np[e] = np;
  }
  const int64_t w = (int64_t)blockIdx.x * NWAVES + wave;
  if (U == 0 || w >= line.nw) return;
  // the worker's units [xs, xe) on the unit line (the balanced split maps
  // both ends at once: lane 0 the start, lane 1 the end)
  int xs, xe;
  if (rc) {
    const int x = (int)sk_unit_at(PU, B, Hkv, rc, line.start(w + (threadIdx.x & 1)), U);
    xs = __builtin_amdgcn_readlane(x, 0);
    xe = __builtin_amdgcn_readlane(x, 1);
  } else {  // the unit line (fixed partitions align the ends to partitions)
    xs = (int)sk_align(PU, B, Hkv, pt, line.start(w), U);
    xe = (int)sk_align(PU, B, Hkv, pt, line.start(w + 1), U);
  }
  const int nun = xe - xs;  // 0 for a range that holds only run costs (or no partition)
  if (nun <= 0) return;

  WS ws;
  const uint32_t qlane = (uint32_t)(ws.j * D + 8 * ws.g) * QE;  // byte offset of head j, chunk 0
  SkWindow cur = sk_describe<NH>(prm, PU, B, xs, xe, xs, pt), nxt = cur;
  if (nun > 64) nxt = sk_describe<NH>(prm, PU, B, xs, xe, xs + 64, pt);
  // on the cost line: the part index of the share's first piece when its
  // run opened in an earlier share (every later piece opens its run here)
  int part0 = 0;
  if (rc && __builtin_amdgcn_readlane(cur.u, 0) > 0)
    part0 = (int)(w - line.worker_of(sk_cost(PU, Hkv, rc, __builtin_amdgcn_readlane(cur.b, 0),
                                             __builtin_amdgcn_readlane(cur.kf, 0) & 0xFFFF, 0)));

  // A piece that opens on the run of the piece before it (fixed partitions:
  // consecutive partitions of one run in one share) keeps that piece's query
  // operands: issue() loads no query for it and its opening sets none.  The
  // two sides see the same sequence of opening pieces, so they agree.
  int iss_run = -1, q_run = -1;

  // Issues the loads of unit L of the share: K/V of its block and, when it
  // opens a piece on a new run, the query operands of that (sequence, KV
  // head).
  auto issue = [&](const int L, Slot& sl) -> SkInfo {
    SkInfo in{0, 0, 0, 0};
    int32_t phys = -1;
    int hf = 0;
    uint32_t qbytes = 0;
    const char* qbase = static_cast<const char*>(prm.q);
    if (L < nun) {
      const int i = L & 63;
      if (i == 0 && L > 0) {
        cur = nxt;
        if (L + 64 < nun) nxt = sk_describe<NH>(prm, PU, B, xs, xe, xs + L + 64, pt);
      }
      phys = __builtin_amdgcn_readlane(cur.phys, i);
      const int u = __builtin_amdgcn_readlane(cur.u, i);
      int n = __builtin_amdgcn_readlane(cur.n, i);
      n = n < 0 ? 0 : (n > prm.max_ctx ? prm.max_ctx : n);
      in.b = __builtin_amdgcn_readlane(cur.b, i);
      in.kf = __builtin_amdgcn_readlane(cur.kf, i);
      in.u = u;
      in.nv = max(0, min(16, n - 16 * u));
      hf = u % NH;
      if (in.kf & (1 << 16)) {
        const int kvh = in.kf & 0xFFFF;
        const int run = in.b * Hkv + kvh;
        if (Q_AHEAD && run != iss_run) {
          qbase += ((int64_t)in.b * prm.Hq + (int64_t)kvh * prm.G) * D * QE;
          qbytes = (uint32_t)prm.G * D * QE;  // heads past the group read as zeros
        }
        iss_run = run;
      }
    }
    const int nv = ws.fetch(sl.bb, prm, in.kf & 0xFFFF, phys, hf, in.nv);
    if constexpr (Q_AHEAD) {
      // only a piece's first unit carries the query: a load instruction
      // costs address-unit time even when it reads nothing
      const uint32_t qb = __builtin_amdgcn_readfirstlane(qbytes);
      if (qb) {
        const auto rq = make_rsrc(uniform_ptr(qbase), qb);
#pragma unroll
        for (int c = 0; c < NC; ++c)
          sl.q[c] =
              bitcast<u32x4>(__builtin_amdgcn_raw_buffer_load_b128(rq, qlane + c * 64, 0, 0));
      }
    }
    in.nv = nv;
    return in;
  };

  // Arithmetic of unit C; closes the piece when the unit is its last.
  // Query operands of the piece unit `in` opens.
  auto set_query = [&](const Slot& sl, const SkInfo& in) {
    const int run = in.b * Hkv + (in.kf & 0xFFFF);
    if (run == q_run) return;  // the previous piece's run: its operands stand
    q_run = run;
    if constexpr (Q_AHEAD) ws.set_query(sl.q, prm.scale_log2);
    else ws.set_query(prm, in.b, in.kf & 0xFFFF);
  };

  // Closes the piece when unit `in` is its last.
  auto close = [&](const SkInfo& in) {
    const int kvh = in.kf & 0xFFFF;
    if (in.kf & (1 << 17)) {
      ws.finish();
      const int pb = PU[in.b], nu = PU[in.b + 1] - pb;
      if (pt) {  // fixed partitions: one piece is one whole partition
        if (nu <= pt) ws.store_output(prm, in.b, kvh);
        else ws.store_partial(prm, in.b, kvh, in.u / pt);
      } else {
        // the balanced split's share is [xs, xe) itself: a run inside it is
        // whole here, and one that opens in it is the run's first part; a
        // run that opened in an earlier share is the share's first piece
        // (on the unit line its index needs a division, done only here)
        const int64_t seg = (int64_t)Hkv * pb + (int64_t)kvh * nu;
        if (seg >= xs && seg + nu <= xe) ws.store_output(prm, in.b, kvh);
        else
          ws.store_partial(prm, in.b, kvh,
                           seg >= xs ? 0 : (rc ? part0 : (int)(w - line.worker_of(seg))));
      }
    }
  };

  // Arithmetic of unit C: opens its piece if it is the first, closes it if
  // it is the last.
  auto process = [&](const Slot& sl, const SkInfo& in) {
    if (in.kf & (1 << 16)) {
      set_query(sl, in);
      ws.reset();
    }
    ws.compute(sl.bb, in.nv, prm.scale_log2);
    close(in);
  };

  Slot ring[NB];
  SkInfo info[NB];
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) info[s] = issue(s, ring[s]);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (PKV_PIPELINE && DEPTH >= 2) {
    // the scores of unit L + 1 are computed alongside the softmax and P.V of
    // unit L (see run_units); a piece's query operands are set up before
    // the scores of its first unit, its accumulators cleared before that
    // unit's accumulation
    set_query(ring[0], info[0]);  // unit 0 opens the share's first piece
    f32x4 sc = ws.scores(ring[0].bb, info[0].nv, prm.scale_log2);
    for (int c0 = 0; c0 < nun; c0 += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int slot = (k + DEPTH) % NB;
        info[slot] = issue(c0 + k + DEPTH, ring[slot]);
        __builtin_amdgcn_sched_barrier(0);
        const int nk = (k + 1) % NB;
        if (info[nk].kf & (1 << 16)) set_query(ring[nk], info[nk]);
        const f32x4 sc_next = ws.scores(ring[nk].bb, info[nk].nv, prm.scale_log2);
        if (info[k].kf & (1 << 16)) ws.reset();
        ws.accumulate(ring[k].bb, info[k].nv, sc);
        close(info[k]);
        sc = sc_next;
        __builtin_amdgcn_sched_barrier(0);
        if (c0 + k + 1 >= nun) goto done;
      }
    }
  } else {
    for (int c0 = 0; c0 < nun; c0 += NB) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int slot = (k + DEPTH) % NB;
        info[slot] = issue(c0 + k + DEPTH, ring[slot]);
        __builtin_amdgcn_sched_barrier(0);
        process(ring[k], info[k]);
        __builtin_amdgcn_sched_barrier(0);
        if (c0 + k + 1 >= nun) goto done;
      }
    }
  }
done:;
}

// ------------------------------------------------------------ merge

// Merge of many parts by NWM waves: wave w takes the batches of eight parts
// starting at 8 w, 8 (w + NWM), ..., keeping (M, L, acc) online, and the
// waves' results are combined through LDS by wave 0.  A long context split
// into 64 partitions is thus read in one round of loads instead of eight
// dependent ones.
template <int NWM>
struct MergeShared {
  float m[NWM][64], l[NWM][64];
  f32x4 a0[NWM][64], a1[NWM][64];
};

template <int OUT, int D, int NWM>
__device__ __forceinline__ void merge_run_waves(const DecodeParams& prm, const int b,
                                                const int h, const int np,
                                                MergeShared<NWM>& sh) {
  constexpr int C8 = D / 8, BATCH = 8;
  static_assert(C8 <= 64, "one task per lane");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  {
    // lane tasks: 8 channels each of query head h
    const bool active = lane < C8;
    const int c = active ? lane * 8 : 0;
    const int64_t row = (int64_t)b * prm.Hq + h;
    const int64_t base = row * prm.P_max;
    const auto rm = make_rsrc(prm.ws_m + base, (uint32_t)np * 4);
    const auto rl = make_rsrc(prm.ws_l + base, (uint32_t)np * 4);
    const auto ra = make_rsrc(prm.ws_acc + base * D, (uint32_t)np * D * 4);
    float M = -INFINITY, L = 0.0f;
    f32x4 a0 = f32x4{0, 0, 0, 0}, a1 = f32x4{0, 0, 0, 0};
    for (int k0 = BATCH * wave; k0 < np; k0 += BATCH * NWM) {
      float mk[BATCH], lk[BATCH];
      f32x4 x0[BATCH], x1[BATCH];
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {  // parts past np read as zeros
        const uint32_t k = (uint32_t)(k0 + i);
        mk[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rm, k * 4, 0, 0));
        lk[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, k * 4, 0, 0));
        x0[i] = bitcast<f32x4>(__builtin_amdgcn_raw_buffer_load_b128(ra, (k * D + c) * 4, 0, 0));
        x1[i] = bitcast<f32x4>(
            __builtin_amdgcn_raw_buffer_load_b128(ra, (k * D + c + 4) * 4, 0, 0));
      }
      float Mb = M;
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        if (k0 + i >= np) mk[i] = -INFINITY;
        Mb = fmaxf(Mb, mk[i]);
      }
      if (Mb > M) {
        const float sc = M == -INFINITY ? 0.0f : exp2f((M - Mb) * LOG2E);
        L *= sc;
        a0 *= sc;
        a1 *= sc;
        M = Mb;
      }
#pragma unroll
      for (int i = 0; i < BATCH; ++i) {
        const float wk = mk[i] == -INFINITY ? 0.0f : exp2f((mk[i] - M) * LOG2E);
        L += wk * lk[i];
        a0 += wk * x0[i];
        a1 += wk * x1[i];
      }
    }
    sh.m[wave][lane] = M;
    sh.l[wave][lane] = L;
    sh.a0[wave][lane] = a0;
    sh.a1[wave][lane] = a1;
    __syncthreads();
    if (wave == 0 && active) {
      float Mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < NWM; ++w) Mx = fmaxf(Mx, sh.m[w][lane]);
      float Lt = 0.0f;
      f32x4 s0 = f32x4{0, 0, 0, 0}, s1 = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < NWM; ++w) {
        const float mw = sh.m[w][lane];
        const float f = mw == -INFINITY ? 0.0f : exp2f((mw - Mx) * LOG2E);
        Lt += f * sh.l[w][lane];
        s0 += f * sh.a0[w][lane];
        s1 += f * sh.a1[w][lane];
      }
      const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
      store4<OUT>(prm.out, row * D + c, s0 * inv);
      store4<OUT>(prm.out, row * D + c + 4, s1 * inv);
    }
    __syncthreads();
  }
}

// The merge step.  The balanced split (a few parts per run): one wave per
// (sequence, KV head).  Fixed partitions of long contexts: one workgroup of
// MERGE_WAVES waves per (sequence, query head), so that the parts, tens of
// KB per head, are read by every CU at once.  With prm.part == 0 the part
// counts are those the balanced split left in the workspace; otherwise they
// follow from the fixed partitions.
constexpr int MERGE_WAVES = 8;

template <int OUT, int D, int NWM, int MB = PKV_MERGE_BATCH>
__global__ __launch_bounds__(64 * NWM) void lse_reduce_kernel(const DecodeParams prm) {
  if constexpr (NWM == 1) {
    const int b = blockIdx.x / prm.Hkv;
    const int kvh = blockIdx.x - b * prm.Hkv;
    // The part count (balanced split) or the context length (fixed
    // partitions) is read by every lane, with a vector load at an offset the
    // compiler takes for a per-lane value (it is zero), so that the value
    // stays in vector registers and merge_run waits for it only after the
    // parts have been requested.  Read as a wave-uniform value it would be
    // waited for before the parts' loads are issued, a memory round trip of
    // its own.
    uint32_t lane0;
    asm volatile("v_mov_b32 %0, 0" : "=v"(lane0));
    const int32_t* src = prm.part == 0 ? prm.ws_np + blockIdx.x : prm.ctx_lens + b;
    const int raw = (int)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(src, 4), lane0, 0, 0);
    merge_run<OUT, D, MB>(prm, b, kvh, raw);  // (writes nothing when there are 0 or 1 parts)
  } else {
    __shared__ MergeShared<NWM> sh;
    const int b = blockIdx.x / prm.Hq;
    const int h = blockIdx.x - b * prm.Hq;
    int np;
    if (prm.part == 0) {  // balanced split: the part count of the head's run
      np = prm.ws_np[b * prm.Hkv + h / prm.G];
    } else {
      const int n = clamp_ctx(prm, b);
      np = (n + prm.part - 1) / prm.part;
    }
    if (np <= 1) return;  // the whole workgroup: written by the decode kernel
    merge_run_waves<OUT, D, NWM>(prm, b, h, np, sh);
  }
}

// ---------------------------------------------------------- host launch

// Workgroups of `kernel` the current GPU holds at once (0 if unknown),
// cached per device.
static int resident_workgroups(const void* kernel, int* cache_dev, int* cache_val) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (*cache_dev == dev) return *cache_val;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * NWAVES, 0) !=
          hipSuccess)
    return 0;
  *cache_val = cus * per_cu;
  *cache_dev = dev;
  return *cache_val;
}

enum class Mode { OnePass, Fixed, Balanced };

// How one call splits the work.
struct Split {
  Mode mode;
  int32_t part;  // Fixed / OnePass: tokens per partition
  int64_t pmax;  // partial slots per (sequence, query head)
};

static Split make_split(const pkv_cache_desc& d, int32_t B, int32_t max_ctx, int32_t partition) {
  const int32_t p = d.block_size;
  const int64_t m = max_ctx < 1 ? 1 : max_ctx;
  if (partition == -1) return {Mode::OnePass, (int32_t)((m + p - 1) / p * p), 1};
  const int64_t nu_max = (m + 15) / 16;
  // the unit offsets are int32 in the kernels
  if (partition == 0 && B <= SK_PLAN_MAX && (int64_t)B * nu_max * d.num_kv_heads <= INT32_MAX)
    return {Mode::Balanced, 0, nu_max / SK_MIN_UNITS + 2};
  const int32_t part = partition > 0 ? partition : 32 * p;  // batches too large for the plan
  return {Mode::Fixed, part, (m + part - 1) / part};
}

// Workspace (4-byte words): for the balanced split first B * Hkv int32 part
// counts (rounded up to 4 words); then m [nm], l [nm], and acc [nm][D] from
// the next 16-byte boundary, with nm = B * Hq * pmax.
static size_t np_words(int64_t B, int64_t Hkv) { return (size_t)((B * Hkv + 3) & ~3); }
static size_t acc_offset_floats(size_t nm) { return (2 * nm + 3) & ~(size_t)3; }
static size_t workspace_floats(const Split& sp, int64_t B, int64_t Hq, int64_t Hkv, int64_t D) {
  if (sp.mode != Mode::Balanced && sp.pmax <= 1) return 0;
  const size_t nm = (size_t)B * Hq * sp.pmax;
  return (sp.mode == Mode::Balanced ? np_words(B, Hkv) : 0) + acc_offset_floats(nm) + nm * D;
}

// phase bit 0: partition kernel, bit 1: merge kernel
template <int KV, int IO, int OUT, int D, int P, bool BF>
static void launch_decode(const DecodeParams& prm, const Split& sp, int B, int phases,
                          hipStream_t s) {
  DecodeParams run = prm;
  if (sp.mode == Mode::Balanced) {
    constexpr bool I4B = KV == PKV_INT4_ASYM_G32;
    static int cache_dev = -1, cache_val = 0;
    int grid = resident_workgroups(
        reinterpret_cast<const void*>(&streamk_decode_kernel<KV, IO, OUT, D, P, BF, I4B>),
        &cache_dev, &cache_val);
    if (grid <= 0) grid = B * prm.Hkv;
    run.plan_B = B;
    run.workers = grid * NWAVES;
    // where runs outnumber the waves, shares cross several runs and each
    // run's piece costs its wave about a unit's time: weigh it on the line
    run.run_cost = (int64_t)B * prm.Hkv > run.workers ? PKV_SK_RUN_COST : 0;
    if (phases & 1)
      hipLaunchKernelGGL((streamk_decode_kernel<KV, IO, OUT, D, P, BF, I4B>), dim3((unsigned)grid),
                         dim3(64 * NWAVES), 0, s, run);
    if (phases & 2) {
      // long contexts over few runs leave many parts per run: merge them with
      // MERGE_WAVES waves per (sequence, query head), as for fixed partitions
      // (and runs whose G P_max parts are too many for the one-wave merge's
      // 32-bit offsets)
      if ((prm.P_max > 8 && (int64_t)run.workers > 8 * (int64_t)B * prm.Hkv) ||
          (int64_t)prm.G * prm.P_max * D * 4 > (int64_t)UINT32_MAX)
        hipLaunchKernelGGL((lse_reduce_kernel<OUT, D, MERGE_WAVES>), dim3((unsigned)(B * prm.Hq)),
                           dim3(64 * MERGE_WAVES), 0, s, run);
      // the average run has about workers / runs + 1 parts
      else if ((int64_t)run.workers <= 2 * (int64_t)B * prm.Hkv)
        hipLaunchKernelGGL((lse_reduce_kernel<OUT, D, 1, PKV_MERGE_BATCH_SMALL>),
                           dim3((unsigned)(B * prm.Hkv)), dim3(64), 0, s, run);
      else
        hipLaunchKernelGGL((lse_reduce_kernel<OUT, D, 1>), dim3((unsigned)(B * prm.Hkv)),
                           dim3(64), 0, s, run);
    }
    return;
  }
  run.workers = 0;
  run.plan_B = 0;
  if ((phases & 1) && sp.mode == Mode::OnePass) {
    hipLaunchKernelGGL((paged_decode_kernel<KV, IO, OUT, D, P, BF>),
                       dim3((unsigned)(B * prm.Hkv)), dim3(64 * NWAVES), 0, s, run);
  } else if ((phases & 1) && B <= SK_PLAN_MAX &&
             (int64_t)B * ((prm.max_ctx + 15) / 16) * prm.Hkv <= INT32_MAX) {
    // fixed partitions on the balanced split's unit stream, with share
    // boundaries at partition boundaries
    static int cache_dev = -1, cache_val = 0;
    int grid = resident_workgroups(
        reinterpret_cast<const void*>(&streamk_decode_kernel<KV, IO, OUT, D, P, BF>), &cache_dev,
        &cache_val);
    if (grid <= 0) grid = B * prm.Hkv;
    run.plan_B = B;
    run.workers = grid * NWAVES;
    hipLaunchKernelGGL((streamk_decode_kernel<KV, IO, OUT, D, P, BF>), dim3((unsigned)grid),
                       dim3(64 * NWAVES), 0, s, run);
    run.workers = 0;
  } else if (phases & 1) {
    // batches too large for the stream's plan: one wave per (sequence,
    // partition, KV head) item
    const int64_t items = (int64_t)B * prm.Hkv * prm.P_max;
    hipLaunchKernelGGL((partition_decode_kernel<KV, IO, OUT, D, P, BF>),
                       dim3((unsigned)((items + NWAVES - 1) / NWAVES)), dim3(64 * NWAVES), 0, s,
                       run);
  }
  run.plan_B = 0;
  if ((phases & 2) && prm.P_max > 1) {
    if (prm.P_max > 8)
      hipLaunchKernelGGL((lse_reduce_kernel<OUT, D, MERGE_WAVES>), dim3((unsigned)(B * prm.Hq)),
                         dim3(64 * MERGE_WAVES), 0, s, run);
    else if (prm.P_max <= PKV_MERGE_BATCH_SMALL)  // every part in the first round
      hipLaunchKernelGGL((lse_reduce_kernel<OUT, D, 1, PKV_MERGE_BATCH_SMALL>),
                         dim3((unsigned)(B * prm.Hkv)), dim3(64), 0, s, run);
    else
      hipLaunchKernelGGL((lse_reduce_kernel<OUT, D, 1>), dim3((unsigned)(B * prm.Hkv)), dim3(64),
                         0, s, run);
  }
}

template <int KV, int IO, int OUT, bool BF>
static void dispatch_dp(const DecodeParams& prm, const Split& sp, int B, int D, int P, int ph,
                        hipStream_t s) {
  if (D == 64) {
    if (P == 16) launch_decode<KV, IO, OUT, 64, 16, BF>(prm, sp, B, ph, s);
    else launch_decode<KV, IO, OUT, 64, 32, BF>(prm, sp, B, ph, s);
  } else {
    if (P == 16) launch_decode<KV, IO, OUT, 128, 16, BF>(prm, sp, B, ph, s);
    else launch_decode<KV, IO, OUT, 128, 32, BF>(prm, sp, B, ph, s);
  }
}

// The output type: the io type, or fp32 from the same arithmetic (the
// PKV_DECODE_OUT_F32 flag).
template <int KV, int IO, bool BF>
static void dispatch_out(const DecodeParams& prm, const Split& sp, bool out32, int B, int D,
                         int P, int ph, hipStream_t s) {
  if constexpr (IO == PKV_F32) {
    dispatch_dp<KV, IO, PKV_F32, BF>(prm, sp, B, D, P, ph, s);
  } else {
    if (out32) dispatch_dp<KV, IO, PKV_F32, BF>(prm, sp, B, D, P, ph, s);
    else dispatch_dp<KV, IO, IO, BF>(prm, sp, B, D, P, ph, s);
  }
}

template <int KV>
static void dispatch_io(const DecodeParams& prm, const Split& sp, int io, bool out32, int B,
                        int D, int P, int ph, hipStream_t s) {
  // MMA operand type: the cache's own type for 16-bit caches, else the io type (bf16 for F32 io)
  if constexpr (KV == PKV_F16) {
    if (io == PKV_F16) dispatch_out<KV, PKV_F16, false>(prm, sp, out32, B, D, P, ph, s);
    else dispatch_out<KV, PKV_F32, false>(prm, sp, out32, B, D, P, ph, s);
  } else if constexpr (KV == PKV_BF16) {
    if (io == PKV_BF16) dispatch_out<KV, PKV_BF16, true>(prm, sp, out32, B, D, P, ph, s);
    else dispatch_out<KV, PKV_F32, true>(prm, sp, out32, B, D, P, ph, s);
  } else if constexpr (KV == PKV_INT4_ASYM_G32) {
    // INT4 codes enter the products as exact fp16 values whatever the io type
    if (io == PKV_F16) dispatch_out<KV, PKV_F16, false>(prm, sp, out32, B, D, P, ph, s);
    else if (io == PKV_BF16) dispatch_out<KV, PKV_BF16, false>(prm, sp, out32, B, D, P, ph, s);
    else dispatch_out<KV, PKV_F32, false>(prm, sp, out32, B, D, P, ph, s);
  } else {
    if (io == PKV_F16) dispatch_out<KV, PKV_F16, false>(prm, sp, out32, B, D, P, ph, s);
    else if (io == PKV_BF16) dispatch_out<KV, PKV_BF16, true>(prm, sp, out32, B, D, P, ph, s);
    else dispatch_out<KV, PKV_F32, true>(prm, sp, out32, B, D, P, ph, s);
  }
}

}  // namespace pkv

using namespace pkv;

extern "C" int32_t pkv_decode_partition(const pkv_cache_desc* desc, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_ctx, int32_t partition) {
  (void)num_q_heads;
  if (validate_desc(desc) != PKV_OK) return -1;
  const Split sp = make_split(*desc, num_seqs, max_ctx, partition);
  if (sp.mode == Mode::Balanced) return 0;
  if (sp.mode == Mode::OnePass) return -1;
  return sp.part;
}

extern "C" size_t pkv_decode_workspace_bytes(const pkv_cache_desc* desc, int32_t num_seqs,
                                             int32_t num_q_heads, int32_t max_ctx,
                                             int32_t partition) {
  if (validate_desc(desc) != PKV_OK || num_seqs < 0 || num_q_heads < 1 || max_ctx < 0) return 0;
  const Split sp = make_split(*desc, num_seqs, max_ctx, partition);
  return workspace_floats(sp, num_seqs, num_q_heads, desc->num_kv_heads, desc->head_dim) *
         sizeof(float);
}

static pkv_status decode_impl(const pkv_cache_desc* desc, const pkv_decode_args* a, int phases,
                              pkv_stream_t stream) {
  if (a && (a->flags & ~(PKV_DECODE_SKIP_MERGE | PKV_DECODE_OUT_F32)))
    return fail(PKV_ERR_INVALID_ARG, "unknown flags 0x%x", a->flags);
  pkv_status st = validate_desc(desc);
  if (st != PKV_OK) return st;
  if (!a) return fail(PKV_ERR_INVALID_ARG, "args is NULL");
  const int32_t B = a->num_seqs, Hq = a->num_q_heads, Hkv = desc->num_kv_heads;
  if (B < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs must be >= 0");
  if (B == 0) return PKV_OK;
  if (Hq < 1 || Hq % Hkv != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", Hq,
                Hkv);
  const int32_t G = Hq / Hkv;
  if (G > 16) return fail(PKV_ERR_UNSUPPORTED, "GQA group of %d heads (at most 16)", G);
  if (a->table_width < 1) return fail(PKV_ERR_INVALID_ARG, "table_width must be >= 1");
  if (a->max_ctx < 0 || (int64_t)a->max_ctx > (int64_t)a->table_width * desc->block_size)
    return fail(PKV_ERR_INVALID_ARG, "max_ctx %d outside [0, table_width * block_size]",
                a->max_ctx);
  if (!a->out || !a->q || !a->k_pool || !a->v_pool || !a->block_tables || !a->ctx_lens)
    return fail(PKV_ERR_INVALID_ARG, "NULL device pointer");
  if (!is_16bit_kv(desc->kv_dtype) && (!a->k_meta || !a->v_meta))
    return fail(PKV_ERR_INVALID_ARG, "quantised caches need k_meta and v_meta");
  if (!(a->scale > 0.0f) || !std::isfinite(a->scale))
    return fail(PKV_ERR_INVALID_ARG, "scale must be positive and finite");
  if (a->partition < -1 || (a->partition > 0 && a->partition % desc->block_size != 0))
    return fail(PKV_ERR_INVALID_ARG,
                "partition must be -1, 0 or a positive multiple of block_size %d",
                desc->block_size);
  const uintptr_t align = reinterpret_cast<uintptr_t>(a->q) | reinterpret_cast<uintptr_t>(a->out) |
                          reinterpret_cast<uintptr_t>(a->k_pool) |
                          reinterpret_cast<uintptr_t>(a->v_pool) |
                          reinterpret_cast<uintptr_t>(a->k_meta) |
                          reinterpret_cast<uintptr_t>(a->v_meta) |
                          reinterpret_cast<uintptr_t>(a->workspace);
  if (align & 15) return fail(PKV_ERR_INVALID_ARG, "device buffers must be 16-byte aligned");

  const Split sp = make_split(*desc, B, a->max_ctx, a->partition);
  if (sp.mode != Mode::Balanced) {
    const int64_t grid = (int64_t)B * Hkv * sp.pmax;
    if (grid > INT32_MAX)
      return fail(PKV_ERR_UNSUPPORTED, "launch grid of %lld workgroups", (long long)grid);
  }
  if ((int64_t)B * Hq > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "too many (sequence, head) pairs");
  DecodeParams prm{};
  prm.out = a->out;
  prm.q = a->q;
  prm.k_pool = a->k_pool;
  prm.v_pool = a->v_pool;
  prm.k_meta = a->k_meta;
  prm.v_meta = a->v_meta;
  prm.block_tables = a->block_tables;
  prm.ctx_lens = a->ctx_lens;
  prm.Hkv = Hkv;
  prm.Hq = Hq;
  prm.G = G;
  prm.W = a->table_width;
  prm.max_ctx = a->max_ctx;
  prm.part = sp.part;
  prm.P_max = (int32_t)sp.pmax;
  prm.num_seqs = B;
  prm.num_blocks = desc->num_blocks;
  prm.scale_log2 = a->scale * LOG2E;
  prm.bad_blocks = a->bad_blocks;
  if (reinterpret_cast<uintptr_t>(a->bad_blocks) & 3)
    return fail(PKV_ERR_INVALID_ARG, "bad_blocks must be 4-byte aligned");
  const size_t need = workspace_floats(sp, B, Hq, Hkv, desc->head_dim) * sizeof(float);
  if (need) {
    if (!a->workspace || a->workspace_bytes < need)
      return fail(PKV_ERR_INVALID_ARG, "workspace of %zu bytes needed, %zu given", need,
                  a->workspace_bytes);
    float* ws = static_cast<float*>(a->workspace);
    if (sp.mode == Mode::Balanced) {
      prm.ws_np = reinterpret_cast<int32_t*>(ws);
      ws += np_words(B, Hkv);
    }
    const size_t nm = (size_t)B * Hq * prm.P_max;
    prm.ws_m = ws;
    prm.ws_l = ws + nm;
    prm.ws_acc = ws + acc_offset_floats(nm);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int D = desc->head_dim, P = desc->block_size, io = desc->io_dtype;
  const bool o32 = (a->flags & PKV_DECODE_OUT_F32) != 0;
  (void)hipGetLastError();  // report only this call's launch errors
  switch (desc->kv_dtype) {
    case PKV_F16: dispatch_io<PKV_F16>(prm, sp, io, o32, B, D, P, phases, s); break;
    case PKV_BF16: dispatch_io<PKV_BF16>(prm, sp, io, o32, B, D, P, phases, s); break;
    case PKV_FP8_E4M3: dispatch_io<PKV_FP8_E4M3>(prm, sp, io, o32, B, D, P, phases, s); break;
    case PKV_FP8_E5M2: dispatch_io<PKV_FP8_E5M2>(prm, sp, io, o32, B, D, P, phases, s); break;
    // a block scale is kept in every per-token entry: read as per-token scales
    case PKV_FP8_E4M3_BLOCK:
      dispatch_io<PKV_FP8_E4M3>(prm, sp, io, o32, B, D, P, phases, s);
      break;
    default: dispatch_io<PKV_INT4_ASYM_G32>(prm, sp, io, o32, B, D, P, phases, s); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "paged decode launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

extern "C" pkv_status pkv_paged_decode(const pkv_cache_desc* desc, const pkv_decode_args* a,
                                       pkv_stream_t stream) {
  const int phases = (a && (a->flags & PKV_DECODE_SKIP_MERGE)) ? 1 : 3;
  return decode_impl(desc, a, phases, stream);
}

extern "C" pkv_status pkv_lse_reduce(const pkv_cache_desc* desc, const pkv_decode_args* a,
                                     pkv_stream_t stream) {
  return decode_impl(desc, a, 2, stream);
}

// ------------------------------------------------ no-allocation entry point

// Split-K partial results of pkv_paged_decode_noalloc live in this
// file-scope device array instead of a caller workspace (each GPU holds its
// own copy from module load until the process ends).  In host code its name
// is only a stand-in: the device address comes from hipGetSymbolAddress,
// taken once per device and kept.
constexpr size_t SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

constexpr int SCRATCH_MAX_DEVICES = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[SCRATCH_MAX_DEVICES];

static pkv_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= SCRATCH_MAX_DEVICES)
    return fail(PKV_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, SCRATCH_MAX_DEVICES);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PKV_ERR_HIP, "hipGetSymbolAddress of the scratch array: %s",
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

extern "C" pkv_status pkv_paged_decode_noalloc(const pkv_cache_desc* desc,
                                               const pkv_decode_args* a, pkv_stream_t stream) {
  pkv_status st = validate_desc(desc);
  if (st != PKV_OK) return st;
  if (!a) return fail(PKV_ERR_INVALID_ARG, "args is NULL");
  if (a->flags & PKV_DECODE_SKIP_MERGE)
    return fail(PKV_ERR_INVALID_ARG, "the merge runs inside pkv_paged_decode_noalloc");
  if (a->workspace || a->workspace_bytes)
    return fail(PKV_ERR_INVALID_ARG, "workspace must be NULL: the library's scratch is used");
  const size_t need = pkv_decode_workspace_bytes(desc, a->num_seqs, a->num_q_heads, a->max_ctx,
                                                 a->partition);
  if (need > SCRATCH_BYTES)
    return fail(PKV_ERR_INVALID_ARG,
                "these sizes need %zu bytes of split-K scratch, at most %zu are available", need,
                SCRATCH_BYTES);
  pkv_decode_args b = *a;
  if (need) {
    st = scratch_address(&b.workspace);
    if (st != PKV_OK) return st;
    b.workspace_bytes = SCRATCH_BYTES;
  }
  return decode_impl(desc, &b, 3, stream);
}
