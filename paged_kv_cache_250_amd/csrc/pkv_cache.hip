// reshape_and_cache: write each new token's K and V into its slot of the
// paged cache, quantising on the way ("Reducing LLM Inference Latency: KV
// Cache Quantization and PagedAttention in vLLM", section "KV Cache
// Quantization: Shrinking the Memory Footprint": K/V are converted to the
// low-precision format before they are stored in the block pool).
//
// One wave per (token, KV head): it reads the token's K and V rows once,
// derives the scales with wave reductions, and scatters the values into the
// chunk layouts the decode kernels read with 16-byte loads (ChunkLayout
// below; the layouts are documented in include/pkv.h).  INT4 V packs two
// tokens per byte, so its nibbles are written with 32-bit atomic and/or;
// every other store owns whole bytes.
#include <algorithm>
#include <vector>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

template <int IO>
__device__ __forceinline__ float load_io(const void* base, int64_t i) {
  if constexpr (IO == PKV_F32) {
    return static_cast<const float*>(base)[i];
  } else if constexpr (IO == PKV_BF16) {
    return __uint_as_float((uint32_t)static_cast<const uint16_t*>(base)[i] << 16);
  } else {
    return f16_bits_to_f32(static_cast<const uint16_t*>(base)[i]);
  }
}

template <int KV>
__device__ __forceinline__ uint16_t to_cache16(float x) {
  return (uint16_t)(KV == PKV_BF16 ? f32_to_bf16_bits(x) : f32_to_f16_bits(x));
}

// FP8: scale = max(max|x| / 448, 1e-12) (one fp32 division), code =
// e4m3(x / scale) ("Reducing LLM Inference Latency...", section "Block-Wise
// Scaling Factors"; here one scale per (token, KV head)).
// E5M2 ("FP8 (Float8) vs INT8 / INT4 Quantization"): the same with its
// largest finite value, 57344, in place of 448.
template <int KV, int EPL>
__device__ __forceinline__ float fp8_scale(const float (&x)[EPL]) {
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) a = fmaxf(a, fabsf(x[e]));
  a = wave_max(a);
  const float s = a / (KV == PKV_FP8_E5M2 ? 57344.0f : 448.0f);
  return fmaxf(s, 1e-12f);
}

// INT4 asymmetric group of 32 channels: s = fp16((max - min) / 15),
// z = fp16(min), code = clamp(rne((x - z) / s), 0, 15), code 0 if s == 0.
template <int EPL>
__device__ __forceinline__ void int4_group(const float (&x)[EPL], uint32_t (&code)[EPL],
                                           uint32_t& sz_bits) {
  constexpr int LANES = 32 / EPL;  // lanes holding one group
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int e = 1; e < EPL; ++e) {
    mn = fminf(mn, x[e]);
    mx = fmaxf(mx, x[e]);
  }
  mn = group_min<LANES>(mn);
  mx = group_max<LANES>(mx);
  const float range = mx - mn;
  const float sf = range / 15.0f;
  const uint32_t sb = f32_to_f16_bits(sf), zb = f32_to_f16_bits(mn);
  const float S = f16_bits_to_f32(sb), Z = f16_bits_to_f32(zb);
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    uint32_t c = 0;
    if (S != 0.0f) {
      const float t = (x[e] - Z) / S;
      const float r = fminf(fmaxf(__builtin_rintf(t), 0.0f), 15.0f);
      c = (uint32_t)r;
    }
    code[e] = c;
  }
  sz_bits = sb | (zb << 16);
}

// Offsets inside one (block, KV head) chunk of the documented layouts
// (include/pkv.h): token t of the block, channel d.  Tokens are grouped in
// units of 16 (hf = t / 16); inside a unit, token 4 g + r.
template <int D>
struct ChunkLayout {
  static constexpr int NT = D / 16, NG = D / 32;
  // 16-bit V, in elements
  static __device__ __forceinline__ int64_t v16(int d, int t) {
    const int T = d / 16, j = d % 16, hf = t / 16, g = (t % 16) / 4, r = t % 4;
    return ((((int64_t)(hf * (NT / 2) + T / 2) * 16 + j) * 4 + g) * 2 + T % 2) * 4 + r;
  }
  // FP8 K, in bytes: per unit [D/64][16 j][4 g][2 (c % 2)][8 e], so that each
  // of the decode's K load instructions reads 1 KB of consecutive bytes
  static __device__ __forceinline__ int64_t k8(int d, int t) {
    const int hf = t / 16, j = t % 16, c = d / 32, g = (d % 32) / 8, e = d % 8;
    return ((((int64_t)hf * (D / 64) + c / 2) * 16 + j) * 4 + g) * 16 + 8 * (c % 2) + e;
  }
  // FP8 V, in bytes
  static __device__ __forceinline__ int64_t v8(int d, int t) {
    const int T = d / 16, j = d % 16, hf = t / 16, g = (t % 16) / 4, r = t % 4;
    return (((int64_t)(hf * (NT / 4) + T / 4) * 16 + j) * 4 + g) * 16 + (T % 4) * 4 + r;
  }
  // INT4 K, byte holding channel d (low nibble for even d % 8)
  static __device__ __forceinline__ int64_t k4(int d, int t) {
    const int c = d / 32, g = (d % 32) / 8, e = d % 8;
    return (int64_t)t * (D / 2) + g * (D / 8) + 4 * c + e / 2;
  }
  // INT4 V, 32-bit word holding token t of channel d, and the nibble's bit
  // offset in it: one word per (unit, j, g, pair of 16-channel tiles), token
  // 4 g + r of tile parity T % 2 at bit 16 (r % 2) + 8 (r / 2) + 4 (T % 2),
  // so that masking the word with 0x000F000F (and its 8-bit shift) yields the
  // token pairs of the even tile, and with 0x00F000F0 those of the odd one
  static __device__ __forceinline__ int64_t v4_word(int d, int t) {
    const int T = d / 16, j = d % 16, hf = t / 16, g = (t % 16) / 4;
    return ((int64_t)(hf * 16 + j) * 4 + g) * NG + T / 2;
  }
  static __device__ __forceinline__ uint32_t v4_shift(int d, int t) {
    const int r = t % 4;
    return 16u * (uint32_t)(r & 1) + 8u * (uint32_t)(r >> 1) + 4u * (uint32_t)((d / 16) & 1);
  }
  // INT4 (s, z) word of group gr
  static __device__ __forceinline__ int64_t m4(int gr, int t) {
    const int hf = t / 16, g = (t % 16) / 4, r = t % 4;
    return ((int64_t)(hf * 4 + g) * NG + gr) * 4 + r;
  }
};

// Requantises the FP8 codes of tokens 0 .. off-1 of one (block, KV head)
// chunk from scale s_old to s_new: code' = e4m3(fp32(fp32(code * s_old) /
// s_new)), NaN codes kept.  Both layouts interleave tokens inside a unit of
// 16 (a unit is D 16-byte vectors): in K the vector v holds token
// 16 (v / D) + (v % D) / 4 % 16 in all its bytes; in V byte b of vector v
// holds token 16 (v / D) + 4 (v % 4) + b % 4.  The wave loads every vector
// it needs before it changes any, so one call costs one round trip to
// memory.
template <int D, int P>
__device__ __forceinline__ void requant_block(uint8_t* chunk, int which, int off, float s_old,
                                              float s_new) {
  constexpr int NV = P * D / 16 / 64;  // 16-byte vectors per lane covering a chunk
  const int lane = threadIdx.x;
  uint4* vec = reinterpret_cast<uint4*>(chunk);
  const int nvec = (off + 15) / 16 * D;  // the units holding tokens below off
  uint4 w[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = lane + 64 * i;
    if (v < nvec) w[i] = vec[v];
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = lane + 64 * i;
    if (v >= nvec) continue;
    uint32_t word[4] = {w[i].x, w[i].y, w[i].z, w[i].w};
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const int tok = which ? 16 * (v / D) + 4 * (v % 4) + (b & 3) : 16 * (v / D) + (v % D) / 4 % 16;
      if (tok >= off) continue;
      const uint32_t sh = 8u * (uint32_t)(b & 3);
      const float c = e4m3_to_f32((word[b >> 2] >> sh) & 0xFFu);
      if (c != c) continue;  // NaN codes are kept
      const uint32_t code = f32_to_e4m3((c * s_old) / s_new);
      word[b >> 2] = (word[b >> 2] & ~(0xFFu << sh)) | (code << sh);
    }
    vec[v] = make_uint4(word[0], word[1], word[2], word[3]);
  }
  // the whole-vector stores cover the new token's V bytes too: they must land
  // before the new token's own byte stores
  __threadfence_block();
}

template <int KV, int IO, int D, int P>
__global__ __launch_bounds__(64) void reshape_and_cache_kernel(
    const void* __restrict__ k, const void* __restrict__ v, const int64_t* __restrict__ slots,
    int32_t Hkv, int64_t num_slots, void* __restrict__ k_pool, void* __restrict__ v_pool,
    void* __restrict__ k_meta, void* __restrict__ v_meta) {
  constexpr int EPL = D / 64;  // channels per lane
  const int64_t i = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int64_t slot = slots[i];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot / P;
  const int off = (int)(slot % P);
  const int64_t chunk = blk * Hkv + h;
  const int64_t in_base = (i * Hkv + h) * D;
  using L = ChunkLayout<D>;
  // block-scaled FP8: both old block scales are requested before anything
  // is stored, so the two reads cost one round trip
  float s_old_kv[2] = {0.0f, 0.0f};
  if constexpr (KV == PKV_FP8_E4M3_BLOCK) {
    if (off > 0) {
      s_old_kv[0] = static_cast<const float*>(k_meta)[chunk * P];
      s_old_kv[1] = static_cast<const float*>(v_meta)[chunk * P];
    }
  }

#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const void* src = which ? v : k;
    float x[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) x[e] = load_io<IO>(src, in_base + lane * EPL + e);

    if constexpr (KV == PKV_F16 || KV == PKV_BF16) {
      uint16_t* pool = static_cast<uint16_t*>(which ? v_pool : k_pool);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int d = lane * EPL + e;
        const int64_t idx = chunk * P * D + (which ? L::v16(d, off) : (int64_t)off * D + d);
        pool[idx] = to_cache16<KV>(x[e]);
      }
    } else if constexpr (KV == PKV_FP8_E4M3_BLOCK) {
      // one scale per (block, KV head): raise it to this token's and, if it
      // grows, requantise the block's earlier tokens from their codes
      uint8_t* pool = static_cast<uint8_t*>(which ? v_pool : k_pool);
      float* sc = static_cast<float*>(which ? v_meta : k_meta) + chunk * P;
      float s_new = fp8_scale<PKV_FP8_E4M3, EPL>(x);
      if (off > 0) {
        const float s_old = s_old_kv[which];  // the block's scale, kept in every entry
        s_new = fmaxf(s_old, s_new);
        if (s_new > s_old) requant_block<D, P>(pool + chunk * P * D, which, off, s_old, s_new);
      }
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int d = lane * EPL + e;
        const int64_t idx = chunk * P * D + (which ? L::v8(d, off) : L::k8(d, off));
        pool[idx] = (uint8_t)f32_to_e4m3(x[e] / s_new);
      }
      if (lane < P) sc[lane] = s_new;
    } else if constexpr (KV == PKV_FP8_E4M3 || KV == PKV_FP8_E5M2) {
      uint8_t* pool = static_cast<uint8_t*>(which ? v_pool : k_pool);
      const float scale = fp8_scale<KV, EPL>(x);
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int d = lane * EPL + e;
        const int64_t idx = chunk * P * D + (which ? L::v8(d, off) : L::k8(d, off));
        const float y = x[e] / scale;
        pool[idx] = (uint8_t)(KV == PKV_FP8_E5M2 ? f32_to_e5m2(y) : f32_to_e4m3(y));
      }
      if (lane == 0) static_cast<float*>(which ? v_meta : k_meta)[chunk * P + off] = scale;
    } else {  // INT4
      uint32_t code[EPL];
      uint32_t sz;
      int4_group<EPL>(x, code, sz);
      constexpr int LANES = 32 / EPL;
      if ((lane % LANES) == 0) {
        const int gr = lane / LANES;
        static_cast<uint32_t*>(which ? v_meta : k_meta)[chunk * P * (D / 32) + L::m4(gr, off)] =
            sz;
      }
      uint8_t* pool = static_cast<uint8_t*>(which ? v_pool : k_pool);
      const int64_t cbase = chunk * P * (D / 2);
      if (which == 0) {
        // channel pairs (even, odd) share a byte of the token's row
        if constexpr (EPL == 2) {
          pool[cbase + L::k4(lane * 2, off)] = (uint8_t)(code[0] | (code[1] << 4));
        } else {
          const uint32_t hi = __shfl_down(code[0], 1, 64);
          if ((lane & 1) == 0) pool[cbase + L::k4(lane, off)] = (uint8_t)(code[0] | (hi << 4));
        }
      } else {
        // the tokens of a word belong to different calls or waves, hence
        // the atomics
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const int d = lane * EPL + e;
          uint32_t* word = reinterpret_cast<uint32_t*>(pool + cbase) + L::v4_word(d, off);
          const uint32_t shift = L::v4_shift(d, off);
          atomicAnd(word, ~(0xFu << shift));
          atomicOr(word, code[e] << shift);
        }
      }
    }
  }
}

template <int KV, int IO, int D, int P>
static void launch_rc(const pkv_cache_desc& d, const void* k, const void* v, int32_t N,
                      const int64_t* slots, void* kp, void* vp, void* km, void* vm,
                      hipStream_t s) {
  dim3 grid((unsigned)N, (unsigned)d.num_kv_heads);
  hipLaunchKernelGGL((reshape_and_cache_kernel<KV, IO, D, P>), grid, dim3(64), 0, s, k, v, slots,
                     d.num_kv_heads, d.num_blocks * d.block_size, kp, vp, km, vm);
}

template <int KV, int IO>
static void dispatch_rc_dp(const pkv_cache_desc& d, const void* k, const void* v, int32_t N,
                           const int64_t* slots, void* kp, void* vp, void* km, void* vm,
                           hipStream_t s) {
  if (d.head_dim == 64) {
    if (d.block_size == 16) launch_rc<KV, IO, 64, 16>(d, k, v, N, slots, kp, vp, km, vm, s);
    else launch_rc<KV, IO, 64, 32>(d, k, v, N, slots, kp, vp, km, vm, s);
  } else {
    if (d.block_size == 16) launch_rc<KV, IO, 128, 16>(d, k, v, N, slots, kp, vp, km, vm, s);
    else launch_rc<KV, IO, 128, 32>(d, k, v, N, slots, kp, vp, km, vm, s);
  }
}

template <int KV>
static void dispatch_rc_io(const pkv_cache_desc& d, const void* k, const void* v, int32_t N,
                           const int64_t* slots, void* kp, void* vp, void* km, void* vm,
                           hipStream_t s) {
  switch (d.io_dtype) {
    case PKV_F16: dispatch_rc_dp<KV, PKV_F16>(d, k, v, N, slots, kp, vp, km, vm, s); break;
    case PKV_BF16: dispatch_rc_dp<KV, PKV_BF16>(d, k, v, N, slots, kp, vp, km, vm, s); break;
    default: dispatch_rc_dp<KV, PKV_F32>(d, k, v, N, slots, kp, vp, km, vm, s); break;
  }
}

pkv_status launch_reshape_and_cache(const pkv_cache_desc& d, const void* k, const void* v,
                                    int32_t N, const int64_t* slots, void* k_pool, void* v_pool,
                                    void* k_meta, void* v_meta, pkv_stream_t stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();  // report only this call's launch errors
  switch (d.kv_dtype) {
    case PKV_F16: dispatch_rc_io<PKV_F16>(d, k, v, N, slots, k_pool, v_pool, k_meta, v_meta, s); break;
    case PKV_BF16: dispatch_rc_io<PKV_BF16>(d, k, v, N, slots, k_pool, v_pool, k_meta, v_meta, s); break;
    case PKV_FP8_E4M3:
      dispatch_rc_io<PKV_FP8_E4M3>(d, k, v, N, slots, k_pool, v_pool, k_meta, v_meta, s);
      break;
    case PKV_FP8_E5M2:
      dispatch_rc_io<PKV_FP8_E5M2>(d, k, v, N, slots, k_pool, v_pool, k_meta, v_meta, s);
      break;
    case PKV_FP8_E4M3_BLOCK:
      dispatch_rc_io<PKV_FP8_E4M3_BLOCK>(d, k, v, N, slots, k_pool, v_pool, k_meta, v_meta, s);
      break;
    default:
      dispatch_rc_io<PKV_INT4_ASYM_G32>(d, k, v, N, slots, k_pool, v_pool, k_meta, v_meta, s);
      break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "reshape_and_cache launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

// copy_blocks: copy-on-write of shared, partly filled blocks ("KV Cache
// Compression & Paged Attention Deep Dive": forked sequences share blocks
// and copy on write).  All KV heads of a block are adjacent in every array
// (chunk = block * Hkv + head), so one block is one contiguous span per
// array.  Workgroup (x, y) copies a 16 KB tile of array y (K pool, V pool,
// K meta, V meta) of one pair: 256 threads, four 16-byte vectors each, all
// four loads issued before the first store.  The work is a plain HBM copy,
// so nothing here is a contraction.
struct CopySpans {
  uint4* base[4];
  int64_t vecs[4];  // 16-byte vectors of one block in each array (0: absent)
};

constexpr int kCopyThreads = 256;
constexpr int kCopyVecs = 4;
constexpr int kCopyTile = kCopyThreads * kCopyVecs;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(
    const int32_t* __restrict__ pairs, int32_t num_blocks, int32_t tiles_per_pair,
    CopySpans sp) {
  const int a = blockIdx.y;
  const int64_t nv = sp.vecs[a];
  const int32_t pair = (int32_t)(blockIdx.x / (uint32_t)tiles_per_pair);
  const int32_t tile = (int32_t)(blockIdx.x - (uint32_t)pair * (uint32_t)tiles_per_pair);
  const int64_t first = (int64_t)tile * kCopyTile;
  if (first >= nv) return;
  const int32_t src = pairs[2 * (int64_t)pair], dst = pairs[2 * (int64_t)pair + 1];
  if (src == dst || (uint32_t)src >= (uint32_t)num_blocks || (uint32_t)dst >= (uint32_t)num_blocks)
    return;
  const uint4* from = sp.base[a] + (int64_t)src * nv;
  uint4* to = sp.base[a] + (int64_t)dst * nv;
  uint4 v[kCopyVecs];
#pragma unroll
  for (int i = 0; i < kCopyVecs; ++i) {
    const int64_t x = first + i * kCopyThreads + threadIdx.x;
    if (x < nv) v[i] = from[x];
  }
#pragma unroll
  for (int i = 0; i < kCopyVecs; ++i) {
    const int64_t x = first + i * kCopyThreads + threadIdx.x;
    if (x < nv) to[x] = v[i];
  }
}

static pkv_status launch_copy_blocks(const pkv_cache_desc& d, const int32_t* pairs, int32_t n,
                              void* k_pool, void* v_pool, void* k_meta, void* v_meta,
                              pkv_stream_t stream) {
  size_t pool_bytes = 0, meta_bytes = 0;
  pkv_cache_bytes(&d, &pool_bytes, &meta_bytes);
  const int64_t pool_vecs = (int64_t)(pool_bytes / (size_t)d.num_blocks / 16);
  const int64_t meta_vecs = (int64_t)(meta_bytes / (size_t)d.num_blocks / 16);
  CopySpans sp{};
  sp.base[0] = static_cast<uint4*>(k_pool);
  sp.base[1] = static_cast<uint4*>(v_pool);
  sp.base[2] = static_cast<uint4*>(k_meta);
  sp.base[3] = static_cast<uint4*>(v_meta);
  sp.vecs[0] = sp.vecs[1] = pool_vecs;
  sp.vecs[2] = sp.vecs[3] = meta_vecs;
  const int arrays = meta_vecs ? 4 : 2;
  const int64_t tiles = (pool_vecs + kCopyTile - 1) / kCopyTile;
  if ((int64_t)n * tiles > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "%d pairs of %lld tiles exceed one launch", n,
                (long long)tiles);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)(n * tiles), (unsigned)arrays),
                     dim3(kCopyThreads), 0, s, pairs, (int32_t)d.num_blocks, (int32_t)tiles, sp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PKV_ERR_HIP, "copy_blocks launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}

// Swap moves: gather device blocks into consecutive staging slots (to the
// host) or scatter staging slots into device blocks (from the host).  A
// staging slot holds one block of every array back to back (K, V, K meta,
// V meta), the host pool's block format.  The block ids of one launch ride
// in the kernel arguments; workgroup (x, y) moves a 16 KB tile of array y
// of one block, as copy_blocks_kernel does.
constexpr int kMoveIds = 128;

struct MoveIds {
  int32_t id[kMoveIds];  // device block of slot first_slot + i
  int32_t count;
  int32_t first_slot;
};

__global__ __launch_bounds__(kCopyThreads) void move_blocks_kernel(MoveIds ids, int32_t tiles,
                                                                   CopySpans sp,
                                                                   uint4* __restrict__ staging,
                                                                   int64_t slot_vecs,
                                                                   int32_t to_staging) {
  const int a = blockIdx.y;
  const int64_t nv = sp.vecs[a];
  const int32_t k = (int32_t)(blockIdx.x / (uint32_t)tiles);
  const int32_t tile = (int32_t)(blockIdx.x - (uint32_t)k * (uint32_t)tiles);
  const int64_t first = (int64_t)tile * kCopyTile;
  if (first >= nv || k >= ids.count) return;
  int64_t off = 0;  // offset of array a inside a staging slot
  for (int i = 0; i < a; ++i) off += sp.vecs[i];
  uint4* blk = sp.base[a] + (int64_t)ids.id[k] * nv;
  uint4* slot = staging + (int64_t)(ids.first_slot + k) * slot_vecs + off;
  const uint4* from = to_staging ? blk : slot;
  uint4* to = to_staging ? slot : blk;
  uint4 v[kCopyVecs];
#pragma unroll
  for (int i = 0; i < kCopyVecs; ++i) {
    const int64_t x = first + i * kCopyThreads + threadIdx.x;
    if (x < nv) v[i] = from[x];
  }
#pragma unroll
  for (int i = 0; i < kCopyVecs; ++i) {
    const int64_t x = first + i * kCopyThreads + threadIdx.x;
    if (x < nv) to[x] = v[i];
  }
}

static CopySpans spans_of(const pkv_cache_desc& d, void* k_pool, void* v_pool, void* k_meta,
                          void* v_meta) {
  size_t pool_bytes = 0, meta_bytes = 0;
  pkv_cache_bytes(&d, &pool_bytes, &meta_bytes);
  CopySpans sp{};
  sp.base[0] = static_cast<uint4*>(k_pool);
  sp.base[1] = static_cast<uint4*>(v_pool);
  sp.base[2] = static_cast<uint4*>(k_meta);
  sp.base[3] = static_cast<uint4*>(v_meta);
  sp.vecs[0] = sp.vecs[1] = (int64_t)(pool_bytes / (size_t)d.num_blocks / 16);
  sp.vecs[2] = sp.vecs[3] = (int64_t)(meta_bytes / (size_t)d.num_blocks / 16);
  return sp;
}

// Launches the gather (to_staging) or scatter of pairs [i0, i1) through
// slots 0 .. i1 - i0 - 1.
static void launch_moves(const CopySpans& sp, const int32_t* pairs, int32_t i0, int32_t i1,
                         uint4* staging, int64_t slot_vecs, int32_t to_staging, hipStream_t s) {
  const int arrays = sp.vecs[2] ? 4 : 2;
  const int32_t tiles = (int32_t)((sp.vecs[0] + kCopyTile - 1) / kCopyTile);
  for (int32_t c = i0; c < i1; c += kMoveIds) {
    MoveIds ids{};
    ids.count = std::min(kMoveIds, i1 - c);
    ids.first_slot = c - i0;
    for (int32_t k = 0; k < ids.count; ++k) ids.id[k] = pairs[2 * (c + k)];
    hipLaunchKernelGGL(move_blocks_kernel, dim3((unsigned)(ids.count * tiles), (unsigned)arrays),
                       dim3(kCopyThreads), 0, s, ids, tiles, sp, staging, slot_vecs, to_staging);
  }
}

}  // namespace pkv

using namespace pkv;

extern "C" pkv_status pkv_reshape_and_cache(const pkv_cache_desc* desc, const void* k,
                                            const void* v, int32_t N,
                                            const int64_t* slot_mapping, void* k_pool,
                                            void* v_pool, void* k_meta, void* v_meta,
                                            pkv_stream_t stream) {
  pkv_status st = validate_desc(desc);
  if (st != PKV_OK) return st;
  if (N < 0) return fail(PKV_ERR_INVALID_ARG, "N must be >= 0");
  if (N == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool)
    return fail(PKV_ERR_INVALID_ARG, "NULL device pointer");
  if (!is_16bit_kv(desc->kv_dtype) && (!k_meta || !v_meta))
    return fail(PKV_ERR_INVALID_ARG, "quantised caches need k_meta and v_meta");
  if (desc->kv_dtype == PKV_INT4_ASYM_G32 && (reinterpret_cast<uintptr_t>(v_pool) & 3))
    return fail(PKV_ERR_INVALID_ARG, "INT4 v_pool must be 4-byte aligned");
  if (desc->kv_dtype == PKV_FP8_E4M3_BLOCK &&
      ((reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & 15))
    return fail(PKV_ERR_INVALID_ARG, "block-scaled FP8 pools must be 16-byte aligned");
  if (desc->num_kv_heads > 65535) return fail(PKV_ERR_UNSUPPORTED, "too many KV heads");
  return launch_reshape_and_cache(*desc, k, v, N, slot_mapping, k_pool, v_pool, k_meta, v_meta,
                                  stream);
}

extern "C" pkv_status pkv_copy_blocks(const pkv_cache_desc* desc, const int32_t* pairs, int32_t n,
                                      void* k_pool, void* v_pool, void* k_meta, void* v_meta,
                                      pkv_stream_t stream) {
  pkv_status st = validate_desc(desc);
  if (st != PKV_OK) return st;
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return PKV_OK;
  if (!pairs || !k_pool || !v_pool) return fail(PKV_ERR_INVALID_ARG, "NULL device pointer");
  const bool quant = !is_16bit_kv(desc->kv_dtype);
  if (quant && (!k_meta || !v_meta))
    return fail(PKV_ERR_INVALID_ARG, "quantised caches need k_meta and v_meta");
  for (const void* ptr : {(const void*)k_pool, (const void*)v_pool,
                          quant ? (const void*)k_meta : nullptr,
                          quant ? (const void*)v_meta : nullptr})
    if (reinterpret_cast<uintptr_t>(ptr) & 15)
      return fail(PKV_ERR_INVALID_ARG, "pools and metadata must be 16-byte aligned");
  return launch_copy_blocks(*desc, pairs, n, k_pool, v_pool, quant ? k_meta : nullptr,
                            quant ? v_meta : nullptr, stream);
}

extern "C" size_t pkv_swap_block_bytes(const pkv_cache_desc* desc) {
  if (validate_desc(desc) != PKV_OK) return 0;
  size_t pool_bytes = 0, meta_bytes = 0;
  pkv_cache_bytes(desc, &pool_bytes, &meta_bytes);
  return 2 * (pool_bytes + meta_bytes) / (size_t)desc->num_blocks;
}

extern "C" pkv_status pkv_swap_blocks(const pkv_cache_desc* desc, const int32_t* pairs, int32_t n,
                                      int32_t to_host, void* k_pool, void* v_pool, void* k_meta,
                                      void* v_meta, void* host_pool, int64_t num_host_blocks,
                                      void* staging, size_t staging_bytes, pkv_stream_t stream) {
  pkv_status st = validate_desc(desc);
  if (st != PKV_OK) return st;
  if (n < 0) return fail(PKV_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return PKV_OK;
  const bool quant = !is_16bit_kv(desc->kv_dtype);
  if (!pairs || !k_pool || !v_pool || !host_pool || !staging || (quant && (!k_meta || !v_meta)))
    return fail(PKV_ERR_INVALID_ARG, "NULL pointer");
  for (const void* ptr : {(const void*)k_pool, (const void*)v_pool, (const void*)staging,
                          quant ? (const void*)k_meta : nullptr,
                          quant ? (const void*)v_meta : nullptr})
    if (reinterpret_cast<uintptr_t>(ptr) & 15)
      return fail(PKV_ERR_INVALID_ARG, "pools, metadata and staging must be 16-byte aligned");
  const size_t bb = pkv_swap_block_bytes(desc);
  if (staging_bytes < bb)
    return fail(PKV_ERR_INVALID_ARG, "staging holds %zu bytes, one block is %zu", staging_bytes,
                bb);
  if (num_host_blocks < 0) return fail(PKV_ERR_INVALID_ARG, "num_host_blocks must be >= 0");
  std::vector<char> seen_d((size_t)desc->num_blocks, 0), seen_h((size_t)num_host_blocks, 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = pairs[2 * i], h = pairs[2 * i + 1];
    if (b < 0 || b >= desc->num_blocks || h < 0 || h >= num_host_blocks)
      return fail(PKV_ERR_INVALID_ARG, "pair %d (%d, %d) outside the pools", i, b, h);
    if (seen_d[b]++ || seen_h[h]++)
      return fail(PKV_ERR_INVALID_ARG, "pair %d repeats a block", i);
  }
  const CopySpans sp = spans_of(*desc, k_pool, v_pool, quant ? k_meta : nullptr,
                                quant ? v_meta : nullptr);
  const int64_t slot_vecs = (int64_t)(bb / 16);
  const int32_t cap = (int32_t)std::min<size_t>(staging_bytes / bb, (size_t)n);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  uint4* stg = static_cast<uint4*>(staging);
  char* host = static_cast<char*>(host_pool);
  (void)hipGetLastError();
  for (int32_t i0 = 0; i0 < n; i0 += cap) {
    const int32_t i1 = std::min(n, i0 + cap);
    if (to_host) launch_moves(sp, pairs, i0, i1, stg, slot_vecs, 1, s);
    // one copy per run of consecutive host blocks
    for (int32_t r0 = i0; r0 < i1;) {
      int32_t r1 = r0 + 1;
      while (r1 < i1 && pairs[2 * r1 + 1] == pairs[2 * (r1 - 1) + 1] + 1) ++r1;
      char* hp = host + (size_t)pairs[2 * r0 + 1] * bb;
      char* dp = reinterpret_cast<char*>(stg) + (size_t)(r0 - i0) * bb;
      const size_t bytes = (size_t)(r1 - r0) * bb;
      hipError_t e = to_host ? hipMemcpyAsync(hp, dp, bytes, hipMemcpyDeviceToHost, s)
                             : hipMemcpyAsync(dp, hp, bytes, hipMemcpyHostToDevice, s);
      if (e != hipSuccess)
        return fail(PKV_ERR_HIP, "swap copy failed: %s", hipGetErrorString(e));
      r0 = r1;
    }
    if (!to_host) launch_moves(sp, pairs, i0, i1, stg, slot_vecs, 0, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "swap launch failed: %s", hipGetErrorString(e));
  return PKV_OK;
}
