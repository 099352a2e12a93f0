/*
 * Paged decode attention -- CPU oracle (test infrastructure only).
 *
 * This file is the plain, slow reference that the HIP path is checked
 * against.  It shares no code, header or table with the HIP library.  Only
 * tests, the smoke check and the bench's CPU baseline load it.
 *
 * Everything here is written from the definitions on the pages:
 *
 *  - The KV cache of a sequence lives in fixed-size blocks of p tokens taken
 *    from one shared pool; a per-sequence block table maps logical block
 *    t / p to a physical block, and token t sits at offset t % p
 *    ("Reducing LLM Inference Latency: KV Cache Quantization and
 *    PagedAttention in vLLM", section "PagedAttention: Solving VRAM
 *    Fragmentation", block-manager emulation).
 *  - Attention of one query head is softmax(q K^T / sqrt(d)) V over the
 *    cached tokens ("KV Cache Optimization: 3x Faster LLM Inference on 24GB
 *    VRAM", section "Why Standard Approaches Fail"); under grouped-query
 *    attention G query heads share one KV head (same section).  Query head
 *    h reads KV head h / G (reading: contiguous groups).
 *  - Decode: only the new token's query is computed; the context length n
 *    counts the new token, whose K/V were written to the cache first
 *    ("Optimizing LLM Inference: KV Cache and PagedAttention Explained",
 *    section "The Inference Bottleneck").
 *  - FP8 E4M3 storage with an absmax scale: scale = max|x| / 448 clamped
 *    below by 1e-12, code = e4m3(x / scale), x^ = code * scale
 *    ("Reducing LLM Inference Latency...", section "Block-Wise Scaling
 *    Factors").  Reading: one scale per (token, KV head), fp32 arithmetic
 *    with one rounding per operation, round-to-nearest-even into e4m3,
 *    saturating at +-448.
 *  - FP8 E4M3 with one scale per (block, KV head), as the page's snippet
 *    computes it ("Block-Wise Scaling Factors": one absmax scale for the
 *    tokens of a block).  Reading: tokens arrive one at a time in offset
 *    order; a token at offset 0 opens the block with its own scale; a later
 *    token raises the block scale to max(block scale, its own scale) and,
 *    when it grows, the block's earlier tokens are requantised from their
 *    codes: code' = e4m3(fp32(fp32(code * s_old) / s_new)) (NaN codes are
 *    kept).  The scale is stored in each of the block's p scale entries, so
 *    reading is the same as for per-token scales.
 *  - FP8 E5M2 (same page, section "FP8 (Float8) vs INT8 / INT4
 *    Quantization": 1 sign, 5 exponent, 2 mantissa bits, the range of
 *    fp16).  Reading: the same absmax scale with E5M2's largest finite
 *    value, 57344, in place of 448, and the same layouts and metadata.
 *  - INT4 group-wise storage ("Optimizing KV-Cache Memory Footprint in
 *    High-Throughput LLM Serving", section 4; KIVI's asymmetric groups of
 *    32 in "KV Cache Compression & Paged Attention Deep Dive", section "KV
 *    Cache Quantization").  Reading: per (token, KV head, 32 channels):
 *    s = fp16((max - min) / 15), z = fp16(min), code = clamp(rne((x - z) /
 *    s), 0, 15) (code 0 when s == 0), x^ = fma(code, s, z) in fp32.
 *
 * Pool layouts (the byte format the library also uses; per layer):
 *   f16/bf16 : K [N_blk][Hkv][p][D] 16-bit, V [N_blk][Hkv][D][p] 16-bit
 *   fp8_e4m3 : K [N_blk][Hkv][p][D] u8,     V [N_blk][Hkv][D][p] u8,
 *              k_scale, v_scale [N_blk][Hkv][p] fp32
 *   int4     : K [N_blk][Hkv][p][D/2] u8 (channel 2j in the low nibble of byte
 *              j, 2j+1 in the high nibble), V [N_blk][Hkv][D][p/2] u8 (token 2i
 *              in the low nibble of byte i, 2i+1 in the high nibble),
 *              k_meta, v_meta [N_blk][Hkv][p][D/32][2] fp16 bits (s, z)
 *
 * Attention is computed in fp64 on the dequantised cache values (the
 * exact value of each stored element).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum {
  ORC_F16 = 0,
  ORC_BF16 = 1,
  ORC_FP8_E4M3 = 2,
  ORC_INT4 = 3,
  ORC_F32 = 4,
  ORC_FP8_E5M2 = 5,
  ORC_FP8_E4M3_BLOCK = 6
};

static int is_fp8(int kv) {
  return kv == ORC_FP8_E4M3 || kv == ORC_FP8_E5M2 || kv == ORC_FP8_E4M3_BLOCK;
}
/* code format of an FP8 cache type */
static int fp8_format(int kv) { return kv == ORC_FP8_E5M2 ? ORC_FP8_E5M2 : ORC_FP8_E4M3; }

/* ---------------------------------------------------------------- formats */

/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h) {
  int sign = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24);
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(1.0 + f / 1024.0, e - 15);
  return sign ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double orc_bf16_to_f64(uint16_t h) {
  int sign = h >> 15, e = (h >> 7) & 0xFF, f = h & 0x7F;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133);
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(1.0 + f / 128.0, e - 127);
  return sign ? -v : v;
}

/* Round an fp64 value to a binary format with `mbits` fraction bits and
 * minimum normal exponent `emin` (below it the quantum stays 2^(emin-mbits):
 * subnormals); returns the rounded value (round half to even).  A rounded
 * magnitude above `maxfin`, the largest finite value, becomes +-inf, or
 * +-maxfin when `sat` is set. */
static double round_binary(double x, int mbits, int emin, double maxfin, int sat) {
  if (x != x) return x;
  double a = fabs(x);
  if (a == 0.0) return x;
  int e;
  frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) -> a in [2^(e-1), 2^e) */
  int exp_unbiased = e - 1;
  if (exp_unbiased < emin) exp_unbiased = emin; /* subnormal range: fixed quantum */
  double quantum = ldexp(1.0, exp_unbiased - mbits);
  double q = nearbyint(a / quantum) * quantum; /* exact scaling; nearbyint is RNE */
  if (q > maxfin) {
    /* the rounded value leaves the finite range */
    q = sat ? maxfin : INFINITY;
  }
  return x < 0 ? -q : q;
}

uint16_t orc_f64_to_f16_bits(double x) {
  if (x != x) return 0x7E00;
  double r = round_binary(x, 10, -14, 65504.0, 0);
  uint16_t sign = signbit(r) ? 0x8000 : 0;
  double a = fabs(r);
  if (isinf(a)) return sign | 0x7C00;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int ue = e - 1;
  if (ue < -14) /* subnormal: a = f * 2^-24 */
    return sign | (uint16_t)(a * 16777216.0);
  uint16_t frac = (uint16_t)((ldexp(a, -ue) - 1.0) * 1024.0);
  return sign | (uint16_t)((ue + 15) << 10) | frac;
}

uint16_t orc_f64_to_bf16_bits(double x) {
  if (x != x) return 0x7FC0;
  double r = round_binary(x, 7, -126, 3.3895313892515355e38, 0);
  uint16_t sign = signbit(r) ? 0x8000 : 0;
  double a = fabs(r);
  if (isinf(a)) return sign | 0x7F80;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int ue = e - 1;
  if (ue < -126) return sign | (uint16_t)ldexp(a, 133);
  uint16_t frac = (uint16_t)((ldexp(a, -ue) - 1.0) * 128.0);
  return sign | (uint16_t)((ue + 127) << 7) | frac;
}

/* OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 fraction bits; no
 * infinities; S.1111.111 is NaN, so the largest finite magnitude is
 * 1.75 * 2^8 = 448. */
double orc_e4m3_to_f64(uint8_t c) {
  int sign = c >> 7, e = (c >> 3) & 0xF, f = c & 0x7;
  double v;
  if (e == 15 && f == 7)
    return NAN;
  if (e == 0)
    v = ldexp((double)f, -9);
  else
    v = ldexp(1.0 + f / 8.0, e - 7);
  return sign ? -v : v;
}

/* Round to nearest even into E4M3, saturating at +-448. */
uint8_t orc_f64_to_e4m3(double x) {
  if (x != x) return 0x7F;
  double r = round_binary(x, 3, -6, 448.0, 1);
  uint8_t sign = signbit(r) ? 0x80 : 0;
  double a = fabs(r);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int ue = e - 1;
  if (ue < -6) return sign | (uint8_t)ldexp(a, 9); /* subnormal: a = f * 2^-9 */
  uint8_t frac = (uint8_t)((ldexp(a, -ue) - 1.0) * 8.0);
  return sign | (uint8_t)((ue + 7) << 3) | frac;
}

/* OCP FP8 E5M2: 1 sign, 5 exponent (bias 15), 2 fraction bits; exponent
 * field 31 holds the infinities (fraction 0) and NaNs; largest finite
 * 1.75 * 2^15 = 57344; subnormals f * 2^-16. */
double orc_e5m2_to_f64(uint8_t c) {
  int sign = c >> 7, e = (c >> 2) & 0x1F, f = c & 0x3;
  double v;
  if (e == 31)
    v = f ? NAN : INFINITY;
  else if (e == 0)
    v = ldexp((double)f, -16);
  else
    v = ldexp(1.0 + f / 4.0, e - 15);
  return sign ? -v : v;
}

/* Round to nearest even into E5M2, saturating at +-57344. */
uint8_t orc_f64_to_e5m2(double x) {
  if (x != x) return 0x7F;
  double r = round_binary(x, 2, -14, 57344.0, 1);
  uint8_t sign = signbit(r) ? 0x80 : 0;
  double a = fabs(r);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);
  int ue = e - 1;
  if (ue < -14) return sign | (uint8_t)ldexp(a, 16); /* subnormal: a = f * 2^-16 */
  uint8_t frac = (uint8_t)((ldexp(a, -ue) - 1.0) * 4.0);
  return sign | (uint8_t)((ue + 15) << 2) | frac;
}

/* ------------------------------------------------------- quantisation */

/* FP8 with one absmax scale for a row of D values (fp32 inputs); fmt is
 * ORC_FP8_E4M3 (largest finite 448) or ORC_FP8_E5M2 (57344). */
void orc_fp8_quantize_row_fmt(const float* x, int D, int fmt, uint8_t* codes, float* scale_out) {
  const float fmax = fmt == ORC_FP8_E5M2 ? 57344.0f : 448.0f;
  float a = 0.0f;
  for (int d = 0; d < D; ++d) {
    float ax = fabsf(x[d]);
    if (ax > a) a = ax;
  }
  volatile float s = a / fmax; /* one fp32 division */
  float scale = s < 1e-12f ? 1e-12f : s;
  for (int d = 0; d < D; ++d) {
    volatile float y = x[d] / scale; /* one fp32 division */
    codes[d] = fmt == ORC_FP8_E5M2 ? orc_f64_to_e5m2((double)y) : orc_f64_to_e4m3((double)y);
  }
  *scale_out = scale;
}

void orc_fp8_quantize_row(const float* x, int D, uint8_t* codes, float* scale_out) {
  orc_fp8_quantize_row_fmt(x, D, ORC_FP8_E4M3, codes, scale_out);
}

float orc_fp8_dequant_fmt(uint8_t code, float scale, int fmt) {
  double c = fmt == ORC_FP8_E5M2 ? orc_e5m2_to_f64(code) : orc_e4m3_to_f64(code);
  volatile float v = (float)c * scale; /* one fp32 rounding */
  return v;
}

float orc_fp8_dequant(uint8_t code, float scale) {
  return orc_fp8_dequant_fmt(code, scale, ORC_FP8_E4M3);
}

/* INT4 asymmetric min/max quantisation of one group of `n` values. */
void orc_int4_quantize_group(const float* x, int n, uint8_t* codes, uint16_t* s_bits,
                             uint16_t* z_bits) {
  float mn = x[0], mx = x[0];
  for (int i = 1; i < n; ++i) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  volatile float range = mx - mn;
  volatile float sf = range / 15.0f;
  uint16_t sb = orc_f64_to_f16_bits((double)sf);
  uint16_t zb = orc_f64_to_f16_bits((double)mn);
  float S = (float)orc_f16_to_f64(sb), Z = (float)orc_f16_to_f64(zb);
  for (int i = 0; i < n; ++i) {
    int c = 0;
    if (S != 0.0f) {
      volatile float diff = x[i] - Z;
      volatile float t = diff / S;
      double r = nearbyint((double)t); /* exact fp32 value, rounded half to even */
      if (r < 0.0) r = 0.0;
      if (r > 15.0) r = 15.0;
      c = (int)r;
    }
    codes[i] = (uint8_t)c;
  }
  *s_bits = sb;
  *z_bits = zb;
}

float orc_int4_dequant(int code, uint16_t s_bits, uint16_t z_bits) {
  float S = (float)orc_f16_to_f64(s_bits), Z = (float)orc_f16_to_f64(z_bits);
  return fmaf((float)code, S, Z);
}

/* ------------------------------------------------------------ descriptor */

typedef struct {
  int kv_dtype;  /* ORC_F16 / ORC_BF16 / ORC_FP8_E4M3 / ORC_INT4 */
  int in_dtype;  /* dtype of new K/V and of Q: ORC_F16 / ORC_BF16 / ORC_F32 */
  int Hkv, D, p;
  int64_t num_blocks;
} orc_desc;

static double load_in(const void* base, int dtype, int64_t i) {
  if (dtype == ORC_F16) return orc_f16_to_f64(((const uint16_t*)base)[i]);
  if (dtype == ORC_BF16) return orc_bf16_to_f64(((const uint16_t*)base)[i]);
  return (double)((const float*)base)[i];
}

/* Write N new tokens' K and V ([N][Hkv][D] in in_dtype) to their slots.
 * slot < 0 skips the token.  Returns 0, or -1 on a slot outside the pool. */
int orc_reshape_and_cache(const orc_desc* ds, const void* k, const void* v, int N,
                          const int64_t* slots, void* k_pool, void* v_pool, void* k_meta,
                          void* v_meta) {
  const int H = ds->Hkv, D = ds->D, p = ds->p;
  float* row = (float*)malloc(sizeof(float) * (size_t)D);
  uint8_t* codes = (uint8_t*)malloc((size_t)D);
  for (int i = 0; i < N; ++i) {
    int64_t slot = slots[i];
    if (slot < 0) continue;
    if (slot >= ds->num_blocks * p) {
      free(row);
      free(codes);
      return -1;
    }
    int64_t blk = slot / p;
    int off = (int)(slot % p);
    for (int h = 0; h < H; ++h) {
      for (int which = 0; which < 2; ++which) {
        const void* src = which ? v : k;
        void* pool = which ? v_pool : k_pool;
        void* meta = which ? v_meta : k_meta;
        int64_t in_base = ((int64_t)i * H + h) * D;
        int64_t chunk = (blk * H + h); /* (block, head) chunk index */
        for (int d = 0; d < D; ++d) row[d] = (float)load_in(src, ds->in_dtype, in_base + d);
        if (ds->kv_dtype == ORC_F16 || ds->kv_dtype == ORC_BF16) {
          uint16_t* P = (uint16_t*)pool;
          for (int d = 0; d < D; ++d) {
            uint16_t b = ds->kv_dtype == ORC_F16 ? orc_f64_to_f16_bits(row[d])
                                                 : orc_f64_to_bf16_bits(row[d]);
            int64_t idx = which ? (chunk * D + d) * p + off     /* V: [D][p] */
                                : (chunk * p + off) * D + d;    /* K: [p][D] */
            P[idx] = b;
          }
        } else if (ds->kv_dtype == ORC_FP8_E4M3_BLOCK) {
          uint8_t* P = (uint8_t*)pool;
          float* S = (float*)meta + chunk * p;
          float tok;
          orc_fp8_quantize_row_fmt(row, D, ORC_FP8_E4M3, codes, &tok); /* its own scale */
          float s_new = tok;
          if (off > 0) {
            const float s_old = S[0];
            if (s_old > s_new) s_new = s_old;
            if (s_new > s_old) /* requantise the block's earlier tokens */
              for (int t = 0; t < off; ++t)
                for (int d = 0; d < D; ++d) {
                  int64_t idx = which ? (chunk * D + d) * p + t : (chunk * p + t) * D + d;
                  double c = orc_e4m3_to_f64(P[idx]);
                  if (c != c) continue; /* NaN codes are kept */
                  volatile float v = (float)c * s_old;
                  volatile float y = v / s_new;
                  P[idx] = orc_f64_to_e4m3((double)y);
                }
          }
          for (int d = 0; d < D; ++d) {
            volatile float y = row[d] / s_new;
            int64_t idx = which ? (chunk * D + d) * p + off : (chunk * p + off) * D + d;
            P[idx] = orc_f64_to_e4m3((double)y);
          }
          for (int t = 0; t < p; ++t) S[t] = s_new;
        } else if (is_fp8(ds->kv_dtype)) {
          uint8_t* P = (uint8_t*)pool;
          float scale;
          orc_fp8_quantize_row_fmt(row, D, ds->kv_dtype, codes, &scale);
          for (int d = 0; d < D; ++d) {
            int64_t idx = which ? (chunk * D + d) * p + off : (chunk * p + off) * D + d;
            P[idx] = codes[d];
          }
          ((float*)meta)[chunk * p + off] = scale;
        } else {
          uint8_t* P = (uint8_t*)pool;
          uint16_t* M = (uint16_t*)meta;
          int ng = D / 32;
          for (int g = 0; g < ng; ++g) {
            uint16_t sb, zb;
            orc_int4_quantize_group(row + 32 * g, 32, codes + 32 * g, &sb, &zb);
            int64_t mi = ((chunk * p + off) * ng + g) * 2;
            M[mi] = sb;
            M[mi + 1] = zb;
          }
          if (which == 0) {
            for (int j = 0; j < D / 2; ++j)
              P[(chunk * p + off) * (D / 2) + j] = (uint8_t)(codes[2 * j] | (codes[2 * j + 1] << 4));
          } else {
            for (int d = 0; d < D; ++d) {
              uint8_t* byte = &P[(chunk * D + d) * (p / 2) + off / 2];
              int sh = (off & 1) ? 4 : 0;
              *byte = (uint8_t)((*byte & ~(0xF << sh)) | (codes[d] << sh));
            }
          }
        }
      }
    }
  }
  free(row);
  free(codes);
  return 0;
}

/* Exact value of cached element (block, head, token offset, channel). */
static double cached_value(const orc_desc* ds, int which, const void* pool, const void* meta,
                           int64_t blk, int h, int off, int d) {
  const int H = ds->Hkv, D = ds->D, p = ds->p;
  int64_t chunk = blk * H + h;
  if (ds->kv_dtype == ORC_F16 || ds->kv_dtype == ORC_BF16) {
    int64_t idx = which ? (chunk * D + d) * p + off : (chunk * p + off) * D + d;
    uint16_t b = ((const uint16_t*)pool)[idx];
    return ds->kv_dtype == ORC_F16 ? orc_f16_to_f64(b) : orc_bf16_to_f64(b);
  }
  if (is_fp8(ds->kv_dtype)) {
    int64_t idx = which ? (chunk * D + d) * p + off : (chunk * p + off) * D + d;
    uint8_t c = ((const uint8_t*)pool)[idx];
    float scale = ((const float*)meta)[chunk * p + off];
    return (double)orc_fp8_dequant_fmt(c, scale, fp8_format(ds->kv_dtype));
  }
  int code;
  if (which == 0) {
    uint8_t byte = ((const uint8_t*)pool)[(chunk * p + off) * (D / 2) + d / 2];
    code = (d & 1) ? (byte >> 4) : (byte & 0xF);
  } else {
    uint8_t byte = ((const uint8_t*)pool)[(chunk * D + d) * (p / 2) + off / 2];
    code = (off & 1) ? (byte >> 4) : (byte & 0xF);
  }
  int64_t mi = ((chunk * p + off) * (D / 32) + d / 32) * 2;
  const uint16_t* M = (const uint16_t*)meta;
  return (double)orc_int4_dequant(code, M[mi], M[mi + 1]);
}

/* Dequantised K and V of positions 0..n-1 of one sequence and KV head,
 * gathered through the block table into contiguous [n][D] fp64 arrays. */
int orc_gather(const orc_desc* ds, const void* k_pool, const void* v_pool, const void* k_meta,
               const void* v_meta, const int32_t* table_row, int n, int h, double* K,
               double* V) {
  const int D = ds->D, p = ds->p;
  for (int t = 0; t < n; ++t) {
    int32_t blk = table_row[t / p];
    if (blk < 0 || blk >= ds->num_blocks) return -1;
    int off = t % p;
    for (int d = 0; d < D; ++d) {
      K[(int64_t)t * D + d] = cached_value(ds, 0, k_pool, k_meta, blk, h, off, d);
      V[(int64_t)t * D + d] = cached_value(ds, 1, v_pool, v_meta, blk, h, off, d);
    }
  }
  return 0;
}

/* Paged decode attention over the whole context of every selected
 * sequence.  q: [B][Hq][D] in in_dtype; block_tables [B][W]; ctx_lens [B].
 * seq_mask (may be NULL) selects the sequences to compute; others are left
 * untouched.  out: [B][Hq][D] fp64.  scale is the fp32 softmax scale.
 * If partition > 0, also writes each partition's running max m, sum l and
 * unnormalised accumulator: part_m, part_l [B][Hq][P_max],
 * part_acc [B][Hq][P_max][D] (entries past a sequence's last partition are
 * left untouched).  Partitions are ranges [partition*k, partition*(k+1)) of
 * logical token positions.  Returns 0, or -1 on an invalid table entry. */
int orc_paged_attention(const orc_desc* ds, const void* q, const void* k_pool,
                        const void* v_pool, const void* k_meta, const void* v_meta,
                        const int32_t* block_tables, const int32_t* ctx_lens, int B, int Hq,
                        int W, float scale, const uint8_t* seq_mask, double* out,
                        int partition, int P_max, double* part_m, double* part_l,
                        double* part_acc) {
  const int H = ds->Hkv, D = ds->D, G = Hq / H;
  const double sigma = (double)scale;
  int err = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : err)
  for (int64_t bg = 0; bg < (int64_t)B * H; ++bg) {
    int b = (int)(bg / H), g = (int)(bg % H);
    if (seq_mask && !seq_mask[b]) continue;
    int n = ctx_lens[b];
    if (n < 0 || n > W * ds->p) {
      err |= 1;
      continue;
    }
    double* K = (double*)malloc(sizeof(double) * ((size_t)n * D + 1));
    double* V = (double*)malloc(sizeof(double) * ((size_t)n * D + 1));
    double* s = (double*)malloc(sizeof(double) * ((size_t)n + 1));
    if (orc_gather(ds, k_pool, v_pool, k_meta, v_meta, block_tables + (int64_t)b * W, n, g, K,
                   V) != 0) {
      err |= 1;
      free(K);
      free(V);
      free(s);
      continue;
    }
    for (int hh = 0; hh < G; ++hh) {
      int h = g * G + hh;
      double qv[256];
      for (int d = 0; d < D; ++d) qv[d] = load_in(q, ds->in_dtype, ((int64_t)b * Hq + h) * D + d);
      double* o = out + ((int64_t)b * Hq + h) * D;
      for (int t = 0; t < n; ++t) {
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qv[d] * K[(int64_t)t * D + d];
        s[t] = sigma * acc;
      }
      /* whole-context softmax */
      double m = -INFINITY;
      for (int t = 0; t < n; ++t)
        if (s[t] > m) m = s[t];
      double l = 0.0;
      for (int d = 0; d < D; ++d) o[d] = 0.0;
      for (int t = 0; t < n; ++t) {
        double e = exp(s[t] - m);
        l += e;
        for (int d = 0; d < D; ++d) o[d] += e * V[(int64_t)t * D + d];
      }
      for (int d = 0; d < D; ++d) o[d] = n > 0 ? o[d] / l : 0.0;
      /* per-partition statistics */
      if (partition > 0 && part_m) {
        int np = (n + partition - 1) / partition;
        for (int k = 0; k < np && k < P_max; ++k) {
          int t0 = k * partition, t1 = t0 + partition < n ? t0 + partition : n;
          double mk = -INFINITY;
          for (int t = t0; t < t1; ++t)
            if (s[t] > mk) mk = s[t];
          double lk = 0.0;
          double* ak = part_acc + (((int64_t)b * Hq + h) * P_max + k) * D;
          for (int d = 0; d < D; ++d) ak[d] = 0.0;
          for (int t = t0; t < t1; ++t) {
            double e = exp(s[t] - mk);
            lk += e;
            for (int d = 0; d < D; ++d) ak[d] += e * V[(int64_t)t * D + d];
          }
          part_m[((int64_t)b * Hq + h) * P_max + k] = mk;
          part_l[((int64_t)b * Hq + h) * P_max + k] = lk;
        }
      }
    }
    free(K);
    free(V);
    free(s);
  }
  return err ? -1 : 0;
}

/* Log-sum-exp merge of per-partition (m_k, l_k, acc_k) into the normalised
 * output: M = max m_k, o = sum e^(m_k - M) acc_k / sum e^(m_k - M) l_k. */
void orc_lse_merge(int np, const double* m, const double* l, const double* acc, int D,
                   double* out) {
  double M = -INFINITY;
  for (int k = 0; k < np; ++k)
    if (m[k] > M) M = m[k];
  double L = 0.0;
  for (int d = 0; d < D; ++d) out[d] = 0.0;
  for (int k = 0; k < np; ++k) {
    double w = exp(m[k] - M);
    L += w * l[k];
    for (int d = 0; d < D; ++d) out[d] += w * acc[(int64_t)k * D + d];
  }
  for (int d = 0; d < D; ++d) out[d] = np > 0 ? out[d] / L : 0.0;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* ------------------------------------------------ array helpers (tests) */

void orc_e4m3_encode_array(const double* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_e4m3(x[i]);
}
void orc_e4m3_decode_array(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_to_f64(c[i]);
}
void orc_f16_encode_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_f16_bits(x[i]);
}
void orc_bf16_encode_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_bf16_bits(x[i]);
}
void orc_f16_decode_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f16_to_f64(h[i]);
}
void orc_bf16_decode_array(const uint16_t* h, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f64(h[i]);
}
void orc_fp8_quantize_rows(const float* x, int64_t rows, int D, uint8_t* codes, float* scales) {
  for (int64_t r = 0; r < rows; ++r) orc_fp8_quantize_row(x + r * D, D, codes + r * D, scales + r);
}
void orc_fp8_quantize_rows_fmt(const float* x, int64_t rows, int D, int fmt, uint8_t* codes,
                               float* scales) {
  for (int64_t r = 0; r < rows; ++r)
    orc_fp8_quantize_row_fmt(x + r * D, D, fmt, codes + r * D, scales + r);
}
void orc_fp8_dequant_array_fmt(const uint8_t* c, const float* scale_per_row, int64_t rows, int D,
                               int fmt, float* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int d = 0; d < D; ++d)
      out[r * D + d] = orc_fp8_dequant_fmt(c[r * D + d], scale_per_row[r], fmt);
}
void orc_e5m2_encode_array(const double* x, int64_t n, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f64_to_e5m2(x[i]);
}
void orc_e5m2_decode_array(const uint8_t* c, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e5m2_to_f64(c[i]);
}
void orc_fp8_dequant_array(const uint8_t* c, const float* scale_per_row, int64_t rows, int D,
                           float* out) {
  for (int64_t r = 0; r < rows; ++r)
    for (int d = 0; d < D; ++d) out[r * D + d] = orc_fp8_dequant(c[r * D + d], scale_per_row[r]);
}
void orc_int4_quantize_rows(const float* x, int64_t rows, int D, uint8_t* codes, uint16_t* s,
                            uint16_t* z) {
  int ng = D / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int g = 0; g < ng; ++g)
      orc_int4_quantize_group(x + r * D + 32 * g, 32, codes + r * D + 32 * g, s + r * ng + g,
                              z + r * ng + g);
}
void orc_int4_dequant_array(const uint8_t* codes, const uint16_t* s, const uint16_t* z,
                            int64_t rows, int D, float* out) {
  int ng = D / 32;
  for (int64_t r = 0; r < rows; ++r)
    for (int d = 0; d < D; ++d)
      out[r * D + d] = orc_int4_dequant(codes[r * D + d], s[r * ng + d / 32], z[r * ng + d / 32]);
}
