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
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int NWAVES = 4;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

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
  static __device__ __forceinline__ uint32_t enc(float x) { return f32_to_bf16_bits(x); }
  static __device__ __forceinline__ float dec(uint32_t h) { return __uint_as_float(h << 16); }
  // two fp8 codes (bytes 2*HI, 2*HI+1 of w) -> two bf16, exact
  template <bool HI>
  static __device__ __forceinline__ uint32_t fp8x2(uint32_t w) {
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
  template <bool HI>
  static __device__ __forceinline__ uint32_t fp8x2(uint32_t w) {
    return bitcast<uint32_t>(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
  }
  // fp16 has a narrow exponent range: weights p in [0, 1] are lifted by 2^14
  // so that they stay normal numbers down to p = 2^-28.
  static constexpr int P_SHIFT = 14;
};

template <bool BF>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return Mma<BF>::enc(a) | (Mma<BF>::enc(b) << 16);
}

// Eight 4-bit codes (channel k at bits 4k) -> eight MMA values.
template <bool BF>
__device__ __forceinline__ u32x4 int4x8(uint32_t w) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = pack2<BF>((float)((w >> (8 * i)) & 0xF), (float)((w >> (8 * i + 4)) & 0xF));
  return r;
}

// Four 4-bit codes (token r at bits 4r) -> four MMA values.
template <bool BF>
__device__ __forceinline__ u32x2 int4x4(uint32_t w) {
  u32x2 r;
  r[0] = pack2<BF>((float)(w & 0xF), (float)((w >> 4) & 0xF));
  r[1] = pack2<BF>((float)((w >> 8) & 0xF), (float)((w >> 12) & 0xF));
  return r;
}

// --------------------------------------------------------- io load/store

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
    return *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(q) + idx);
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

template <int KV, int D, int P>
struct BlockBuf {
  static constexpr int NC = D / 32;  // Q.K^T chunks of 32 channels
  static constexpr int NT = D / 16;  // P.V tiles of 16 channels
  static constexpr int NH = P / 16;  // 16-token halves
  static constexpr int NG = D / 32;  // INT4 groups per token
  using KT = typename std::conditional<
      (KV == PKV_F16 || KV == PKV_BF16), u32x4,
      typename std::conditional<KV == PKV_FP8_E4M3, u32x2, uint32_t>::type>::type;
  using VT = typename std::conditional<(KV == PKV_F16 || KV == PKV_BF16), u32x2, uint32_t>::type;
  KT k[NH][NC];
  VT v[NH][NT];
  f32x4 ks[NH], vs[NH];              // FP8 per-token scales of tokens 4g..4g+3
  uint32_t km[NH][4][NG], vm[NH][4][NG];  // INT4 (s, z) pairs of tokens 4g..4g+3
  int nvalid;                        // valid tokens in the block (0 for a bad block id)
};

template <int KV, int D, int P>
__device__ __forceinline__ void load_block(BlockBuf<KV, D, P>& bb, const void* __restrict__ k_pool,
                                           const void* __restrict__ v_pool,
                                           const void* __restrict__ k_meta,
                                           const void* __restrict__ v_meta, int64_t chunk, int g,
                                           int j) {
  using BB = BlockBuf<KV, D, P>;
#pragma unroll
  for (int hf = 0; hf < BB::NH; ++hf) {
    const int ktok = 16 * hf + j;      // K row this lane feeds
    const int vtok = 16 * hf + 4 * g;  // first of the 4 tokens this lane feeds to P.V
#pragma unroll
    for (int c = 0; c < BB::NC; ++c) {
      const int d0 = 32 * c + 8 * g;
      if constexpr (KV == PKV_F16 || KV == PKV_BF16) {
        bb.k[hf][c] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(k_pool) +
                                                       (chunk * P + ktok) * D + d0);
      } else if constexpr (KV == PKV_FP8_E4M3) {
        bb.k[hf][c] = *reinterpret_cast<const u32x2*>(static_cast<const uint8_t*>(k_pool) +
                                                       (chunk * P + ktok) * D + d0);
      } else {
        bb.k[hf][c] = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(k_pool) +
                                                          (chunk * P + ktok) * (D / 2) + d0 / 2);
      }
    }
#pragma unroll
    for (int t = 0; t < BB::NT; ++t) {
      const int ch = 16 * t + j;
      if constexpr (KV == PKV_F16 || KV == PKV_BF16) {
        bb.v[hf][t] = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(v_pool) +
                                                       (chunk * D + ch) * P + vtok);
      } else if constexpr (KV == PKV_FP8_E4M3) {
        bb.v[hf][t] = *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(v_pool) +
                                                          (chunk * D + ch) * P + vtok);
      } else {
        bb.v[hf][t] = *reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(v_pool) +
                                                          (chunk * D + ch) * (P / 2) + vtok / 2);
      }
    }
    if constexpr (KV == PKV_FP8_E4M3) {
      bb.ks[hf] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(k_meta) + chunk * P +
                                                  vtok);
      bb.vs[hf] = *reinterpret_cast<const f32x4*>(static_cast<const float*>(v_meta) + chunk * P +
                                                  vtok);
    }
    if constexpr (KV == PKV_INT4_ASYM_G32) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int gr = 0; gr < BB::NG; ++gr) {
          const int64_t mi = (chunk * P + vtok + r) * BB::NG + gr;
          bb.km[hf][r][gr] = static_cast<const uint32_t*>(k_meta)[mi];
          bb.vm[hf][r][gr] = static_cast<const uint32_t*>(v_meta)[mi];
        }
    }
  }
}

// ------------------------------------------------------------ the kernel

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
  int32_t Hkv, Hq, G, W, max_ctx, part, P_max;
  int64_t num_blocks;
  float scale_log2;  // softmax scale * log2(e)
};

template <int KV, int IO, int D, int P, bool BF>
__global__ __launch_bounds__(64 * NWAVES) void paged_decode_kernel(const DecodeParams prm) {
  using BB = BlockBuf<KV, D, P>;
  using M = Mma<BF>;
  constexpr int NC = BB::NC, NT = BB::NT, NH = BB::NH;

  __shared__ float sm_m[NWAVES][16];
  __shared__ float sm_l[NWAVES][16];
  __shared__ f32x4 sm_acc[NWAVES][NT][64];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4, j = lane & 15;

  const int part = blockIdx.x % prm.P_max;
  const int kvh = (blockIdx.x / prm.P_max) % prm.Hkv;
  const int b = blockIdx.x / (prm.P_max * prm.Hkv);

  int n = prm.ctx_lens[b];
  n = n < 0 ? 0 : (n > prm.max_ctx ? prm.max_ctx : n);
  const int nparts = (n + prm.part - 1) / prm.part;
  const int G = prm.G;
  const int h = kvh * G + j;  // query head of this lane's column
  const bool hvalid = j < G;

  if (n == 0) {
    // empty sequence: zeros, written by the first partition's workgroup
    if (part == 0 && wave == 0 && hvalid) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
        store4<IO>(prm.out, ((int64_t)b * prm.Hq + h) * D + 16 * t + 4 * g, f32x4{0, 0, 0, 0});
    }
    return;
  }
  if (part >= nparts) return;

  const int tok_begin = part * prm.part;
  const int tok_end = min(n, tok_begin + prm.part);
  const int blk_begin = tok_begin / P;
  const int blk_end = (tok_end + P - 1) / P;

  // ---- query operands (B of Q.K^T): head j, channels 32c + 8g .. +7
  u32x4 qop[NC];
  float qsum[NC];  // INT4: sum of the group's query channels
  {
    const int64_t qbase = ((int64_t)b * prm.Hq + h) * D;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qop[c] = hvalid ? load_q8<IO, BF>(prm.q, qbase + 32 * c + 8 * g) : u32x4{0, 0, 0, 0};
      if constexpr (KV == PKV_INT4_ASYM_G32) {
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) s += M::dec(qop[c][i] & 0xFFFF) + M::dec(qop[c][i] >> 16);
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        qsum[c] = s;
      }
    }
  }

  f32x4 acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f32x4{0, 0, 0, 0};
  float m_run = -INFINITY;  // running max of head j (log2 units)
  float l_run = 0.0f;       // partial sum over this lane's tokens
  float zterm[BB::NG];      // INT4: sum of p * z per group (this lane's tokens)
#pragma unroll
  for (int gr = 0; gr < BB::NG; ++gr) zterm[gr] = 0.0f;

  const int64_t chunk_stride = prm.Hkv;
  auto fetch = [&](BB& bb, int jb) {
    int32_t phys = prm.block_tables[(int64_t)b * prm.W + jb];
    int nv = min(P, tok_end - jb * P);
    if ((uint32_t)phys >= (uint32_t)prm.num_blocks) {
      phys = 0;
      nv = 0;
    }
    bb.nvalid = nv;
    load_block<KV, D, P>(bb, prm.k_pool, prm.v_pool, prm.k_meta, prm.v_meta,
                         (int64_t)phys * chunk_stride + kvh, g, j);
  };

  auto compute = [&](BB& bb) {
    const int nv = bb.nvalid;
    float s2[NH][4];
    // ---- scores
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      f32x4 sc;
      if constexpr (KV == PKV_INT4_ASYM_G32) {
        sc = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const f32x4 t = M::k32(int4x8<BF>(bb.k[hf][c]), qop[c], f32x4{0, 0, 0, 0});
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float S = f16_bits_to_f32(bb.km[hf][r][c] & 0xFFFF);
            const float Z = f16_bits_to_f32(bb.km[hf][r][c] >> 16);
            sc[r] += S * t[r] + Z * qsum[c];
          }
        }
      } else {
        sc = f32x4{0, 0, 0, 0};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          u32x4 kop;
          if constexpr (KV == PKV_FP8_E4M3) {
            kop[0] = M::template fp8x2<false>(bb.k[hf][c][0]);
            kop[1] = M::template fp8x2<true>(bb.k[hf][c][0]);
            kop[2] = M::template fp8x2<false>(bb.k[hf][c][1]);
            kop[3] = M::template fp8x2<true>(bb.k[hf][c][1]);
          } else {
            kop = bb.k[hf][c];
          }
          sc = M::k32(kop, qop[c], sc);
        }
        if constexpr (KV == PKV_FP8_E4M3) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sc[r] *= bb.ks[hf][r];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool valid = (16 * hf + 4 * g + r) < nv;
        s2[hf][r] = valid ? sc[r] * prm.scale_log2 : -INFINITY;
      }
    }
    // ---- online softmax (per head j; the 16 tokens of a half sit in lanes j, j+16, j+32, j+48)
    float bm = -INFINITY;
#pragma unroll
    for (int hf = 0; hf < NH; ++hf)
#pragma unroll
      for (int r = 0; r < 4; ++r) bm = fmaxf(bm, s2[hf][r]);
    bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
    bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
    const float m_new = fmaxf(m_run, bm);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    if (__any(alpha != 1.0f)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[t] *= alpha;
#pragma unroll
      for (int gr = 0; gr < BB::NG; ++gr) zterm[gr] *= alpha;
    }
    l_run *= alpha;
    m_run = m_new;
    const float plift = (float)(1 << M::P_SHIFT);
#pragma unroll
    for (int hf = 0; hf < NH; ++hf) {
      float p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = __builtin_amdgcn_exp2f(s2[hf][r] - m_use);
        l_run += p[r];
      }
      // V operands; tokens past the end of the sequence are zeroed so that
      // stale pool contents (possibly NaN) cannot reach the accumulator
      const bool partial = nv < P;
      if constexpr (KV == PKV_INT4_ASYM_G32) {
        // acc += sum_t (p_t s_t,grp) code_t + (sum_t p_t z_t,grp) later
#pragma unroll
        for (int gr = 0; gr < BB::NG; ++gr) {
          float pw[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool valid = (16 * hf + 4 * g + r) < nv;
            const float S = f16_bits_to_f32(bb.vm[hf][r][gr] & 0xFFFF);
            const float Z = f16_bits_to_f32(bb.vm[hf][r][gr] >> 16);
            pw[r] = valid ? p[r] * S * plift : 0.0f;
            zterm[gr] += valid ? p[r] * Z * plift : 0.0f;
          }
          u32x2 phi, plo;
          phi[0] = pack2<BF>(pw[0], pw[1]);
          phi[1] = pack2<BF>(pw[2], pw[3]);
          plo[0] = pack2<BF>(pw[0] - M::dec(phi[0] & 0xFFFF), pw[1] - M::dec(phi[0] >> 16));
          plo[1] = pack2<BF>(pw[2] - M::dec(phi[1] & 0xFFFF), pw[3] - M::dec(phi[1] >> 16));
#pragma unroll
          for (int tt = 0; tt < 2; ++tt) {
            const int t = 2 * gr + tt;
            const u32x2 vop = int4x4<BF>(bb.v[hf][t]);
            acc[t] = M::k16(vop, phi, acc[t]);
            acc[t] = M::k16(vop, plo, acc[t]);
          }
        }
      } else {
        float pw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float x = p[r] * plift;
          if constexpr (KV == PKV_FP8_E4M3) {
            const bool valid = (16 * hf + 4 * g + r) < nv;
            x = valid ? x * bb.vs[hf][r] : 0.0f;
          }
          pw[r] = x;
        }
        u32x2 phi, plo;
        phi[0] = pack2<BF>(pw[0], pw[1]);
        phi[1] = pack2<BF>(pw[2], pw[3]);
        plo[0] = pack2<BF>(pw[0] - M::dec(phi[0] & 0xFFFF), pw[1] - M::dec(phi[0] >> 16));
        plo[1] = pack2<BF>(pw[2] - M::dec(phi[1] & 0xFFFF), pw[3] - M::dec(phi[1] >> 16));
        // mask for the 4 tokens of this lane (16-bit lanes of the V operand)
        uint32_t vmask0 = 0xFFFFFFFFu, vmask1 = 0xFFFFFFFFu;
        if (partial) {
          const int t0 = 16 * hf + 4 * g;
          vmask0 = (t0 + 0 < nv ? 0x0000FFFFu : 0u) | (t0 + 1 < nv ? 0xFFFF0000u : 0u);
          vmask1 = (t0 + 2 < nv ? 0x0000FFFFu : 0u) | (t0 + 3 < nv ? 0xFFFF0000u : 0u);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          u32x2 vop;
          if constexpr (KV == PKV_FP8_E4M3) {
            vop[0] = M::template fp8x2<false>(bb.v[hf][t]);
            vop[1] = M::template fp8x2<true>(bb.v[hf][t]);
          } else {
            vop = bb.v[hf][t];
          }
          vop[0] &= vmask0;
          vop[1] &= vmask1;
          acc[t] = M::k16(vop, phi, acc[t]);
          acc[t] = M::k16(vop, plo, acc[t]);
        }
      }
    }
  };

  // ---- main loop: blocks blk_begin + wave, + NWAVES, ... with one block in flight ahead
  {
    BB buf0, buf1;
    int jb = blk_begin + wave;
    if (jb < blk_end) fetch(buf0, jb);
    while (jb < blk_end) {
      const int jn = jb + NWAVES;
      if (jn < blk_end) fetch(buf1, jn);
      compute(buf0);
      if (jn >= blk_end) break;
      const int jn2 = jn + NWAVES;
      if (jn2 < blk_end) fetch(buf0, jn2);
      compute(buf1);
      jb = jn2;
    }
  }

  // ---- wave epilogue: totals per head over the 4 lane groups
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  const float unlift = 1.0f / (float)(1 << M::P_SHIFT);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if constexpr (KV == PKV_INT4_ASYM_G32) {
      // zterm of group t/2 (D/32 groups of two 16-channel tiles)
      float z = zterm[t / 2];
      z += __shfl_xor(z, 16, 64);
      z += __shfl_xor(z, 32, 64);
      acc[t] += z;
    }
    acc[t] *= unlift;
  }
  if (g == 0) {
    sm_m[wave][j] = m_run;
    sm_l[wave][j] = l_run;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) sm_acc[wave][t][lane] = acc[t];
  __syncthreads();

  // ---- merge the waves; wave w finishes tiles w, w + NWAVES, ...
  float mw[NWAVES];
  float Mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) {
    mw[w] = sm_m[w][j];
    Mx = fmaxf(Mx, mw[w]);
  }
  float fw[NWAVES];
  float L = 0.0f;
#pragma unroll
  for (int w = 0; w < NWAVES; ++w) {
    fw[w] = mw[w] == -INFINITY ? 0.0f : exp2f(mw[w] - Mx);
    L += fw[w] * sm_l[w][j];
  }
  const bool single = nparts == 1;
  for (int t = wave; t < NT; t += NWAVES) {
    f32x4 v = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int w = 0; w < NWAVES; ++w) v += fw[w] * sm_acc[w][t][lane];
    if (!hvalid) continue;
    const int d = 16 * t + 4 * g;
    if (single) {
      const float inv = L > 0.0f ? 1.0f / L : 0.0f;
      store4<IO>(prm.out, ((int64_t)b * prm.Hq + h) * D + d, v * inv);
    } else {
      const int64_t slot = ((int64_t)b * prm.Hq + h) * prm.P_max + part;
      *reinterpret_cast<f32x4*>(prm.ws_acc + slot * D + d) = v;
    }
  }
  if (!single && wave == 0 && g == 0 && hvalid) {
    const int64_t slot = ((int64_t)b * prm.Hq + h) * prm.P_max + part;
    prm.ws_m[slot] = Mx * LN2;  // back to units of the scaled score
    prm.ws_l[slot] = L;
  }
}

// Log-sum-exp merge of the partitions of each (sequence, query head):
// M = max m_k, out = sum e^(m_k - M) acc_k / sum e^(m_k - M) l_k.
template <int IO, int D>
__global__ __launch_bounds__(64) void lse_reduce_kernel(const DecodeParams prm) {
  constexpr int EPL = D / 64;
  const int b = blockIdx.x / prm.Hq;
  const int h = blockIdx.x % prm.Hq;
  const int lane = threadIdx.x;
  int n = prm.ctx_lens[b];
  n = n < 0 ? 0 : (n > prm.max_ctx ? prm.max_ctx : n);
  const int np = (n + prm.part - 1) / prm.part;
  if (np <= 1) return;  // written by the partition kernel
  const int64_t base = ((int64_t)b * prm.Hq + h) * prm.P_max;
  float Mx = -INFINITY;
  for (int k = 0; k < np; ++k) Mx = fmaxf(Mx, prm.ws_m[base + k]);
  float L = 0.0f;
  float a[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) a[e] = 0.0f;
  for (int k = 0; k < np; ++k) {
    const float w = exp2f((prm.ws_m[base + k] - Mx) * LOG2E);
    L += w * prm.ws_l[base + k];
#pragma unroll
    for (int e = 0; e < EPL; ++e) a[e] += w * prm.ws_acc[(base + k) * D + lane * EPL + e];
  }
  const float inv = 1.0f / L;
  const int64_t o = ((int64_t)b * prm.Hq + h) * D + lane * EPL;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    const float x = a[e] * inv;
    if constexpr (IO == PKV_F32)
      static_cast<float*>(prm.out)[o + e] = x;
    else if constexpr (IO == PKV_BF16)
      static_cast<uint16_t*>(prm.out)[o + e] = (uint16_t)f32_to_bf16_bits(x);
    else
      static_cast<uint16_t*>(prm.out)[o + e] = (uint16_t)f32_to_f16_bits(x);
  }
}

// ---------------------------------------------------------- host launch

// phase bit 0: partition kernel, bit 1: merge kernel
template <int KV, int IO, int D, int P, bool BF>
static void launch_decode(const DecodeParams& prm, int B, int phases, hipStream_t s) {
  const int64_t grid = (int64_t)B * prm.Hkv * prm.P_max;
  if (phases & 1)
    hipLaunchKernelGGL((paged_decode_kernel<KV, IO, D, P, BF>), dim3((unsigned)grid),
                       dim3(64 * NWAVES), 0, s, prm);
  if ((phases & 2) && prm.P_max > 1)
    hipLaunchKernelGGL((lse_reduce_kernel<IO, D>), dim3((unsigned)(B * prm.Hq)), dim3(64), 0, s,
                       prm);
}

template <int KV, int IO, bool BF>
static void dispatch_dp(const DecodeParams& prm, int B, int D, int P, int ph, hipStream_t s) {
  if (D == 64) {
    if (P == 16) launch_decode<KV, IO, 64, 16, BF>(prm, B, ph, s);
    else launch_decode<KV, IO, 64, 32, BF>(prm, B, ph, s);
  } else {
    if (P == 16) launch_decode<KV, IO, 128, 16, BF>(prm, B, ph, s);
    else launch_decode<KV, IO, 128, 32, BF>(prm, B, ph, s);
  }
}

template <int KV>
static void dispatch_io(const DecodeParams& prm, int io, int B, int D, int P, int ph,
                        hipStream_t s) {
  // MMA operand type: the cache's own type for 16-bit caches, else the io type (bf16 for F32 io)
  if constexpr (KV == PKV_F16) {
    if (io == PKV_F16) dispatch_dp<KV, PKV_F16, false>(prm, B, D, P, ph, s);
    else dispatch_dp<KV, PKV_F32, false>(prm, B, D, P, ph, s);
  } else if constexpr (KV == PKV_BF16) {
    if (io == PKV_BF16) dispatch_dp<KV, PKV_BF16, true>(prm, B, D, P, ph, s);
    else dispatch_dp<KV, PKV_F32, true>(prm, B, D, P, ph, s);
  } else {
    if (io == PKV_F16) dispatch_dp<KV, PKV_F16, false>(prm, B, D, P, ph, s);
    else if (io == PKV_BF16) dispatch_dp<KV, PKV_BF16, true>(prm, B, D, P, ph, s);
    else dispatch_dp<KV, PKV_F32, true>(prm, B, D, P, ph, s);
  }
}

// Workspace (fp32): m [nm], l [nm], then acc [nm][D] from the first 16-byte
// boundary after l, with nm = B * Hq * P_max.
static size_t acc_offset_floats(size_t nm) { return (2 * nm + 3) & ~(size_t)3; }
static size_t workspace_floats(int64_t B, int64_t Hq, int64_t pmax, int64_t D) {
  const size_t nm = (size_t)B * Hq * pmax;
  return acc_offset_floats(nm) + nm * D;
}

static int32_t resolve_partition(const pkv_cache_desc& d, int32_t B, int32_t max_ctx,
                                 int32_t partition) {
  if (partition == -1) return -1;
  if (partition > 0) return partition;
  // library's choice: one pass when the batch alone fills the GPU or the
  // contexts are short, else 256-token partitions (512 at block size 32)
  const int32_t unit = 16 * d.block_size;
  if (max_ctx <= unit) return -1;
  (void)B;
  return unit;
}

static int32_t part_tokens(const pkv_cache_desc& d, int32_t resolved, int32_t max_ctx) {
  if (resolved > 0) return resolved;
  const int32_t p = d.block_size;
  const int32_t m = max_ctx < 1 ? 1 : max_ctx;
  return (m + p - 1) / p * p;
}

}  // namespace pkv

using namespace pkv;

extern "C" int32_t pkv_decode_partition(const pkv_cache_desc* desc, int32_t num_seqs,
                                        int32_t num_q_heads, int32_t max_ctx, int32_t partition) {
  (void)num_q_heads;
  if (validate_desc(desc) != PKV_OK) return -1;
  return resolve_partition(*desc, num_seqs, max_ctx, partition);
}

extern "C" size_t pkv_decode_workspace_bytes(const pkv_cache_desc* desc, int32_t num_seqs,
                                             int32_t num_q_heads, int32_t max_ctx,
                                             int32_t partition) {
  if (validate_desc(desc) != PKV_OK || num_seqs < 0 || num_q_heads < 1 || max_ctx < 0) return 0;
  const int32_t r = resolve_partition(*desc, num_seqs, max_ctx, partition);
  if (r <= 0) return 0;
  const int64_t pmax = ((int64_t)max_ctx + r - 1) / r;
  if (pmax <= 1) return 0;
  return workspace_floats(num_seqs, num_q_heads, pmax, desc->head_dim) * sizeof(float);
}

static pkv_status decode_impl(const pkv_cache_desc* desc, const pkv_decode_args* a, int phases,
                              pkv_stream_t stream) {
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

  const int32_t resolved = resolve_partition(*desc, B, a->max_ctx, a->partition);
  const int32_t part = part_tokens(*desc, resolved, a->max_ctx);
  const int64_t pmax64 = a->max_ctx > 0 ? ((int64_t)a->max_ctx + part - 1) / part : 1;
  const int64_t grid = (int64_t)B * Hkv * pmax64;
  if (grid > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "launch grid of %lld workgroups", (long long)grid);
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
  prm.part = part;
  prm.P_max = (int32_t)pmax64;
  prm.num_blocks = desc->num_blocks;
  prm.scale_log2 = a->scale * LOG2E;
  if (prm.P_max > 1) {
    const size_t need = workspace_floats(B, Hq, prm.P_max, desc->head_dim) * sizeof(float);
    if (!a->workspace || a->workspace_bytes < need)
      return fail(PKV_ERR_INVALID_ARG, "workspace of %zu bytes needed, %zu given", need,
                  a->workspace_bytes);
    float* ws = static_cast<float*>(a->workspace);
    const size_t nm = (size_t)B * Hq * prm.P_max;
    prm.ws_m = ws;
    prm.ws_l = ws + nm;
    prm.ws_acc = ws + acc_offset_floats(nm);
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int D = desc->head_dim, P = desc->block_size, io = desc->io_dtype;
  switch (desc->kv_dtype) {
    case PKV_F16: dispatch_io<PKV_F16>(prm, io, B, D, P, phases, s); break;
    case PKV_BF16: dispatch_io<PKV_BF16>(prm, io, B, D, P, phases, s); break;
    case PKV_FP8_E4M3: dispatch_io<PKV_FP8_E4M3>(prm, io, B, D, P, phases, s); break;
    default: dispatch_io<PKV_INT4_ASYM_G32>(prm, io, B, D, P, phases, s); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "paged decode launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

extern "C" pkv_status pkv_paged_decode(const pkv_cache_desc* desc, const pkv_decode_args* a,
                                       pkv_stream_t stream) {
  if (a && (a->flags & ~PKV_DECODE_SKIP_MERGE))
    return fail(PKV_ERR_INVALID_ARG, "unknown flags 0x%x", a->flags);
  const int phases = (a && (a->flags & PKV_DECODE_SKIP_MERGE)) ? 1 : 3;
  return decode_impl(desc, a, phases, stream);
}

extern "C" pkv_status pkv_lse_reduce(const pkv_cache_desc* desc, const pkv_decode_args* a,
                                     pkv_stream_t stream) {
  return decode_impl(desc, a, 2, stream);
}
