/*
 * kivi_oracle.c -- plain, slow CPU oracle for KIVI packed-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY (see kivi_oracle.h).  Built with gcc, -O2,
 * -ffp-contract=off and no fast-math, so every float operation below is one
 * IEEE-754 binary32 (or binary64) operation in the order written.
 *
 * Method source: web page "Literature audit -- Group 2 (KV-cache compression
 * primary sources)", section "1. KIVI -- kivi2024", list "Core algorithm
 * (implementation-grade)"; "KIVI item N" below means item N of that list.
 *
 * Points the page leaves open, and the reading taken here:
 *   - round(): round half to even (rintf in the default rounding mode).
 *   - (X - z)/s: true IEEE fp32 division.
 *   - max == min gives s = 0: all codes 0, zero = min, no division.
 *   - codes are clamped to [0, 2^B - 1] (provably a no-op for finite input).
 *   - a scale is stored as fp32; a zero point (the group minimum, which is
 *     an fp16 input value) is stored as that fp16 value, exactly.
 *   - fp16-scale layout (a cache with scale_fp16 set; the pages fix no
 *     storage precision for s): s is computed in fp32 as above, rounded to
 *     the nearest binary16 value (ties to even), and the codes are chosen
 *     for that stored scale -- Q = round((X - z) / s16), clamped -- so that
 *     dequantization reads exactly what quantization used.  A scale that
 *     rounds to zero is stored as zero and gives all codes 0, as max == min
 *     does.  s16 is finite for every fp16 input (max - min <= 131008, so s
 *     <= 43670 for B >= 2).
 *   - prefill with t % R == 0 quantizes every key (the prose rule "keep the
 *     last t mod R keys"), leaving the key window empty.
 *   - the cache is updated before attention runs, so attention sees all t
 *     tokens, the newest included.
 *   - the mask is additive, one fp32 per (batch row, token); a row whose
 *     every score is -inf yields a zero output.
 *   - GQA: query head hq reads KV head hq / (Hq / H).
 *   - scores are divided by sqrt(head_dim).
 */
#include "kivi_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ fp16 */

float kivi_oracle_half_to_float(uint16_t h) {
  /* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
  int sign = (h >> 15) & 1;
  int expo = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double v;
  if (expo == 0) {
    v = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
  } else if (expo == 31) {
    v = frac ? NAN : INFINITY;
  } else {
    v = ldexp((double)(1024 + frac), expo - 25);  /* (1 + frac/1024) 2^(e-15) */
  }
  return (float)(sign ? -v : v);                  /* exact: 11 bits fit */
}

/* An fp32 value that is exactly a binary16 value -> its bit pattern.  The
 * zero points stored in the cache are such values (minima of fp16 inputs).
 * Returns 0 and the pattern, or -1 when the value has no exact fp16 form. */
int kivi_oracle_float_to_half(float f, uint16_t *out) {
  const uint16_t sign = signbit(f) ? 0x8000u : 0u;
  const double a = fabs((double)f);
  if (a == 0.0) { *out = sign; return 0; }
  if (!(a <= 65504.0)) return -1;                       /* inf, nan, too large */
  if (a < ldexp(1.0, -14)) {                            /* subnormal: frac 2^-24 */
    const double frac = ldexp(a, 24);
    if (frac != floor(frac)) return -1;
    *out = (uint16_t)(sign | (uint16_t)frac);
    return 0;
  }
  int ex;
  (void)frexp(a, &ex);                                  /* a = m 2^ex, m in [0.5, 1) */
  const double frac = (ldexp(a, 1 - ex) - 1.0) * 1024.0; /* a = (1 + frac/1024) 2^(ex-1) */
  if (frac != floor(frac)) return -1;
  *out = (uint16_t)(sign | (uint16_t)((ex - 1 + 15) << 10) | (uint16_t)frac);
  return 0;
}

/* fp32 -> binary16, rounded to nearest, ties to even (IEEE 754
 * roundTiesToEven), written from the format's definition: magnitudes below
 * 2^-14 are multiples of 2^-24 (subnormals), those in [2^e, 2^(e+1)) for
 * e >= -14 multiples of 2^(e-10); a magnitude that rounds to 2^16 or more
 * (65520 and up) becomes infinity.  NaN -> the quiet NaN 0x7e00. */
uint16_t kivi_oracle_half_rne(float f) {
  const uint16_t sign = signbit(f) ? 0x8000u : 0u;
  if (isnan(f)) return 0x7e00u;
  const double a = fabs((double)f);
  if (isinf(a)) return (uint16_t)(sign | 0x7c00u);
  int ex = -14;                                   /* exponent of the quantum's binade */
  if (a >= ldexp(1.0, -14)) {
    (void)frexp(a, &ex);                          /* a in [2^(ex-1), 2^ex) */
    ex -= 1;
  }
  const double quantum = ldexp(1.0, ex - 10);
  const double n = a / quantum;                   /* exact: a power-of-two scaling */
  double r = floor(n);
  const double frac = n - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  /* subnormal: the pattern is r itself.  Normal: exponent field ex + 15
   * and fraction r - 1024, i.e. (ex + 14) * 1024 + r; a round up to r = 2048
   * gives the next binade's first pattern, and r = 1024 from the subnormal
   * range the smallest normal one. */
  long bits;
  if (ex == -14 && r < 1024.0)
    bits = (long)r;
  else
    bits = (long)(ex + 14) * 1024 + (long)r;
  if (bits >= 0x7c00) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (uint16_t)bits);
}

/* -------------------------------------------------------------- quantizer */

/* KIVI item 1: z = min(X), s = (max(X) - min(X)) / (2^B - 1),
 * Q = round((X - z) / s).  All arithmetic in fp32. */
void kivi_oracle_quantize_group(const float *x, int n, int bits, uint8_t *codes,
                                float *scale, float *zero) {
  float mn = x[0], mx = x[0];
  for (int i = 1; i < n; ++i) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  const int qmax = (1 << bits) - 1;
  const float s = (mx - mn) / (float)qmax;
  const float z = mn;
  for (int i = 0; i < n; ++i) {
    int q = 0;
    if (s != 0.0f) {
      float r = rintf((x[i] - z) / s);
      q = (int)r;
      if (q < 0) q = 0;
      if (q > qmax) q = qmax;
    }
    codes[i] = (uint8_t)q;
  }
  *scale = s;
  *zero = z;
}

/* KIVI item 1 for the fp16-scale layout: the same s and z as above, s then
 * rounded to binary16 (s16), and the codes chosen for s16. */
void kivi_oracle_quantize_group_s16(const float *x, int n, int bits, uint8_t *codes,
                                    uint16_t *scale_bits, float *zero) {
  float mn = x[0], mx = x[0];
  for (int i = 1; i < n; ++i) {
    if (x[i] < mn) mn = x[i];
    if (x[i] > mx) mx = x[i];
  }
  const int qmax = (1 << bits) - 1;
  const float s = (mx - mn) / (float)qmax;
  const uint16_t sb = kivi_oracle_half_rne(s);
  const float s16 = kivi_oracle_half_to_float(sb);
  const float z = mn;
  for (int i = 0; i < n; ++i) {
    int q = 0;
    if (s16 != 0.0f) {
      float r = rintf((x[i] - z) / s16);
      q = (int)r;
      if (q < 0) q = 0;
      if (q > qmax) q = qmax;
    }
    codes[i] = (uint8_t)q;
  }
  *scale_bits = sb;
  *zero = z;
}

/* KIVI item 1: dequantization Q*s + z, as an fp32 product then an fp32 sum. */
float kivi_oracle_dequant(uint32_t code, float scale, float zero) {
  float p = (float)code * scale;
  return p + zero;
}

/* ---------------------------------------------------------------- packing */

void kivi_oracle_pack_codes(const uint8_t *codes, int n, int bits, uint32_t *words) {
  const int per_word = 32 / bits;
  const int n_words = (n + per_word - 1) / per_word;
  for (int w = 0; w < n_words; ++w) words[w] = 0;
  for (int e = 0; e < n; ++e)
    words[e / per_word] |= (uint32_t)codes[e] << (bits * (e % per_word));
}

void kivi_oracle_unpack_codes(const uint32_t *words, int n, int bits, uint8_t *codes) {
  const int per_word = 32 / bits;
  const uint32_t mask = (1u << bits) - 1u;
  for (int e = 0; e < n; ++e)
    codes[e] = (uint8_t)((words[e / per_word] >> (bits * (e % per_word))) & mask);
}

/* Code of element e in a packed run (same bit order as the packer above). */
static uint32_t code_at(const uint32_t *words, int e, int bits) {
  const int per_word = 32 / bits;
  return (words[e / per_word] >> (bits * (e % per_word))) & ((1u << bits) - 1u);
}

/* ---------------------------------------------------------------- layout */

static int bits_ok(int bits) { return bits == 2 || bits == 4; }

static int shape_ok(int D, int bits, int G) {
  return bits_ok(bits) && G > 0 && D > 0 && (G % (32 / bits)) == 0 &&
         (D % G) == 0 && (128 % G) == 0 && D <= 1024;
}

#define TOKENS_PER_RECORD 128

/* Byte offsets of the sections of a record (kivi_oracle.h). */
typedef struct {
  int64_t kc, ks, kz, vc, vs, vz, size;
} record_t;

/* sb: bytes per stored scale, 4 (fp32) or 2 (fp16-scale layout) */
static int record_of(int D, int kb, int vb, int G, int sb, record_t *r) {
  if (!shape_ok(D, kb, G) || !shape_ok(D, vb, G) || (sb != 4 && sb != 2)) return -1;
  const int64_t groups = TOKENS_PER_RECORD / G;
  r->kc = 0;
  r->ks = r->kc + (int64_t)TOKENS_PER_RECORD * D * kb / 8;
  r->kz = r->ks + groups * D * sb;
  r->vc = r->kz + groups * D * 2;
  r->vs = r->vc + (int64_t)TOKENS_PER_RECORD * D * vb / 8;
  r->vz = r->vs + (int64_t)(D / G) * TOKENS_PER_RECORD * sb;
  r->size = r->vz + (int64_t)(D / G) * TOKENS_PER_RECORD * 2;
  return 0;
}

static int scale_bytes(const kivi_oracle_cache *c) { return c->scale_fp16 ? 2 : 4; }

int64_t kivi_oracle_record_bytes(int D, int k_bits, int v_bits, int G) {
  record_t r;
  return record_of(D, k_bits, v_bits, G, 4, &r) ? 0 : r.size;
}

int64_t kivi_oracle_record_bytes_s(int D, int k_bits, int v_bits, int G, int scale_fp16) {
  record_t r;
  return record_of(D, k_bits, v_bits, G, scale_fp16 ? 2 : 4, &r) ? 0 : r.size;
}

/* A stored scale as a float: an fp32 word, or an fp16 one (exact). */
static float scale_load(const kivi_oracle_cache *c, const uint8_t *p) {
  if (c->scale_fp16) return kivi_oracle_half_to_float(*(const uint16_t *)p);
  return *(const float *)p;
}

/* Start of the record holding token tau of slab bh. */
static uint8_t *record_at(const kivi_oracle_cache *c, const record_t *r, int64_t bh,
                          int64_t tau) {
  return c->blocks + (bh * (c->capacity / TOKENS_PER_RECORD) + tau / TOKENS_PER_RECORD) * r->size;
}

/* Where key group g (tokens g G .. g G + G - 1) of channel ch of slab bh is
 * stored: its code words, scale and zero. */
typedef struct {
  uint32_t *codes;
  uint8_t *scale;     /* fp32 or fp16 (scale_bytes) */
  uint16_t *zero;
} key_slot_t;

static key_slot_t key_slot(const kivi_oracle_cache *c, const record_t *r, int64_t bh,
                           int64_t g, int ch) {
  const int G = c->group, D = c->head_dim;
  uint8_t *rec = record_at(c, r, bh, g * G);
  const int64_t local = ((g * G) % TOKENS_PER_RECORD) / G;   /* group within the record */
  const int64_t i = local * D + ch;
  key_slot_t k;
  k.codes = (uint32_t *)(rec + r->kc) + i * (G * c->k_bits / 32);
  k.scale = rec + r->ks + i * scale_bytes(c);
  k.zero = (uint16_t *)(rec + r->kz) + i;
  return k;
}

/* Where token tau of slab bh keeps its value codes, and the scale / zero of
 * its channel group gc. */
static uint32_t *value_codes(const kivi_oracle_cache *c, const record_t *r, int64_t bh,
                             int64_t tau) {
  uint8_t *rec = record_at(c, r, bh, tau);
  return (uint32_t *)(rec + r->vc) + (tau % TOKENS_PER_RECORD) * (c->head_dim * c->v_bits / 32);
}
static uint8_t *value_scale(const kivi_oracle_cache *c, const record_t *r, int64_t bh,
                            int64_t tau, int gc) {
  uint8_t *rec = record_at(c, r, bh, tau);
  return rec + r->vs + (gc * TOKENS_PER_RECORD + tau % TOKENS_PER_RECORD) * scale_bytes(c);
}

/* KIVI item 1 on one group of the cache's layout: codes, the stored scale
 * (written at `scale`) and the zero point. */
static void quantize_into(const kivi_oracle_cache *c, const float *x, int n, int bits,
                          uint8_t *codes, uint8_t *scale, float *zero) {
  if (c->scale_fp16) {
    kivi_oracle_quantize_group_s16(x, n, bits, codes, (uint16_t *)scale, zero);
  } else {
    kivi_oracle_quantize_group(x, n, bits, codes, (float *)scale, zero);
  }
}
static uint16_t *value_zero(const kivi_oracle_cache *c, const record_t *r, int64_t bh,
                            int64_t tau, int gc) {
  uint8_t *rec = record_at(c, r, bh, tau);
  return (uint16_t *)(rec + r->vz) + gc * TOKENS_PER_RECORD + tau % TOKENS_PER_RECORD;
}

/* Quantize one key group -- G consecutive tokens of channel ch -- and store it
 * at group index g of slab bh.  KIVI item 2. */
static int put_key_group(const kivi_oracle_cache *c, const record_t *r, const float *x,
                         int64_t bh, int64_t g, int ch) {
  uint8_t q[TOKENS_PER_RECORD];
  float z;
  key_slot_t k = key_slot(c, r, bh, g, ch);
  quantize_into(c, x, c->group, c->k_bits, q, k.scale, &z);
  kivi_oracle_pack_codes(q, c->group, c->k_bits, k.codes);
  return kivi_oracle_float_to_half(z, k.zero);
}

/* Quantize one value row -- all D channels of token tau, in groups of G
 * consecutive channels -- and store it.  KIVI item 3. */
static int put_value_row(const kivi_oracle_cache *c, const record_t *r, const float *x,
                         int64_t bh, int64_t tau) {
  uint8_t q[1024];
  const int D = c->head_dim, G = c->group;
  for (int g = 0; g < D / G; ++g) {
    float z;
    quantize_into(c, x + g * G, G, c->v_bits, q + g * G, value_scale(c, r, bh, tau, g), &z);
    if (kivi_oracle_float_to_half(z, value_zero(c, r, bh, tau, g))) return -1;
  }
  kivi_oracle_pack_codes(q, D, c->v_bits, value_codes(c, r, bh, tau));
  return 0;
}

/* ------------------------------------------------------------- the cache */

static int cache_ok(const kivi_oracle_cache *c) {
  record_t r;
  return c && c->blocks && c->k_res && c->v_res &&
         record_of(c->head_dim, c->k_bits, c->v_bits, c->group, scale_bytes(c), &r) == 0 &&
         c->residual > 0 && c->residual % c->group == 0 && c->capacity > 0 &&
         c->capacity % TOKENS_PER_RECORD == 0 && c->capacity % c->residual == 0 &&
         c->n_tokens >= 0 && c->n_tokens <= c->capacity;
}

int kivi_oracle_pack_keys(const kivi_oracle_cache *dst, const uint16_t *k, int64_t T,
                          int64_t off) {
  record_t r;
  if (!cache_ok(dst) || T < 0 || off < 0 || T % dst->group || off % dst->group ||
      off + T > dst->capacity)
    return -1;
  record_of(dst->head_dim, dst->k_bits, dst->v_bits, dst->group, scale_bytes(dst), &r);
  const int D = dst->head_dim, G = dst->group;
  float x[TOKENS_PER_RECORD];
  for (int64_t bh = 0; bh < (int64_t)dst->batch * dst->n_kv_heads; ++bh)
    for (int64_t g = 0; g < T / G; ++g)
      for (int ch = 0; ch < D; ++ch) {
        for (int i = 0; i < G; ++i)
          x[i] = kivi_oracle_half_to_float(k[(bh * T + g * G + i) * D + ch]);
        if (put_key_group(dst, &r, x, bh, off / G + g, ch)) return -1;
      }
  return 0;
}

int kivi_oracle_pack_values(const kivi_oracle_cache *dst, const uint16_t *v, int64_t T,
                            int64_t off) {
  record_t r;
  if (!cache_ok(dst) || T < 0 || off < 0 || off + T > dst->capacity) return -1;
  record_of(dst->head_dim, dst->k_bits, dst->v_bits, dst->group, scale_bytes(dst), &r);
  const int D = dst->head_dim;
  float x[1024];
  for (int64_t bh = 0; bh < (int64_t)dst->batch * dst->n_kv_heads; ++bh)
    for (int64_t tau = 0; tau < T; ++tau) {
      for (int ch = 0; ch < D; ++ch)
        x[ch] = kivi_oracle_half_to_float(v[(bh * T + tau) * D + ch]);
      if (put_value_row(dst, &r, x, bh, off + tau)) return -1;
    }
  return 0;
}

/* KIVI item 4, one token at a time.  For each arriving token tau:
 *   values: the fp16 queue holds the last min(tau, R) values; adding tau
 *           would make R+1, so when tau >= R the oldest (token tau-R, in slot
 *           tau % R) is popped and quantized first;
 *   both:   the new key and value go into slot tau % R;
 *   keys:   the fp16 key buffer holds tokens [tau - tau%R, tau]; when it holds
 *           R tokens the whole block is quantized and the buffer empties. */
int kivi_oracle_append(kivi_oracle_cache *c, const uint16_t *k_new,
                       const uint16_t *v_new, int64_t n_new) {
  record_t r;
  if (!cache_ok(c) || n_new < 0 || c->n_tokens + n_new > c->capacity) return -1;
  record_of(c->head_dim, c->k_bits, c->v_bits, c->group, scale_bytes(c), &r);
  const int D = c->head_dim, G = c->group, R = c->residual;
  const int64_t BH = (int64_t)c->batch * c->n_kv_heads;
  float *x = (float *)malloc(sizeof(float) * (size_t)(R > D ? R : D));
  if (!x) return -1;
  int rc = 0;
  for (int64_t i = 0; i < n_new && rc == 0; ++i) {
    const int64_t tau = c->n_tokens;
    const int64_t slot = tau % R;
    for (int64_t bh = 0; bh < BH && rc == 0; ++bh) {
      uint16_t *kres = c->k_res + bh * R * D;
      uint16_t *vres = c->v_res + bh * R * D;
      if (tau >= R) {  /* value queue would reach R+1: pop token tau-R */
        for (int ch = 0; ch < D; ++ch) x[ch] = kivi_oracle_half_to_float(vres[slot * D + ch]);
        rc |= put_value_row(c, &r, x, bh, tau - R);
      }
      memcpy(kres + slot * D, k_new + (bh * n_new + i) * D, sizeof(uint16_t) * D);
      memcpy(vres + slot * D, v_new + (bh * n_new + i) * D, sizeof(uint16_t) * D);
      if ((tau + 1) % R == 0) {  /* key buffer holds R tokens: quantize all */
        const int64_t first = tau + 1 - R;
        for (int ch = 0; ch < D; ++ch)
          for (int g = 0; g < R / G; ++g) {
            for (int j = 0; j < G; ++j)
              x[j] = kivi_oracle_half_to_float(kres[(int64_t)(g * G + j) * D + ch]);
            rc |= put_key_group(c, &r, x, bh, first / G + g, ch);
          }
      }
    }
    c->n_tokens = tau + 1;
  }
  free(x);
  return rc ? -1 : 0;
}

/* Key tau of (bh) as the attention sees it: dequantized if its R-block has
 * been quantized, else the fp16 value from the window. */
static float key_at(const kivi_oracle_cache *c, const record_t *r, int64_t bh, int64_t tau,
                    int ch) {
  const int64_t t = c->n_tokens, R = c->residual, G = c->group, D = c->head_dim;
  const int64_t n_kq = t - t % R;
  if (tau < n_kq) {
    key_slot_t k = key_slot(c, r, bh, tau / G, ch);
    const uint32_t q = code_at(k.codes, (int)(tau % G), c->k_bits);
    return kivi_oracle_dequant(q, scale_load(c, k.scale), kivi_oracle_half_to_float(*k.zero));
  }
  return kivi_oracle_half_to_float(c->k_res[(bh * R + tau % R) * D + ch]);
}

static float value_at(const kivi_oracle_cache *c, const record_t *r, int64_t bh, int64_t tau,
                      int ch) {
  const int64_t t = c->n_tokens, R = c->residual, G = c->group, D = c->head_dim;
  const int64_t n_vq = t > R ? t - R : 0;
  if (tau < n_vq) {
    const uint32_t q = code_at(value_codes(c, r, bh, tau), ch, c->v_bits);
    const int gc = (int)(ch / G);
    return kivi_oracle_dequant(q, scale_load(c, value_scale(c, r, bh, tau, gc)),
                               kivi_oracle_half_to_float(*value_zero(c, r, bh, tau, gc)));
  }
  return kivi_oracle_half_to_float(c->v_res[(bh * R + tau % R) * D + ch]);
}

int kivi_oracle_materialize(const kivi_oracle_cache *c, float *k_hat, float *v_hat) {
  record_t r;
  if (!cache_ok(c)) return -1;
  record_of(c->head_dim, c->k_bits, c->v_bits, c->group, scale_bytes(c), &r);
  const int64_t BH = (int64_t)c->batch * c->n_kv_heads, t = c->n_tokens;
  const int D = c->head_dim;
  for (int64_t bh = 0; bh < BH; ++bh)
    for (int64_t tau = 0; tau < t; ++tau)
      for (int ch = 0; ch < D; ++ch) {
        if (k_hat) k_hat[(bh * t + tau) * D + ch] = key_at(c, &r, bh, tau, ch);
        if (v_hat) v_hat[(bh * t + tau) * D + ch] = value_at(c, &r, bh, tau, ch);
      }
  return 0;
}

/* KIVI item 5 for one (batch row, query head): scores q.K^T / sqrt(d) over
 * every cached key (quantized ones dequantized, window ones in fp16), plus the
 * mask, softmax, then the probability-weighted sum of the values.  The page's
 * concat / split into quantized and full-precision parts is a partition of
 * the same sums.  Element values are fp32; sums are fp64. */
static int attend_one(const kivi_oracle_cache *c, const uint16_t *q, int n_q_heads,
                      const float *mask, int b, int hq, double *score, float *out) {
  const int D = c->head_dim;
  const int64_t t = c->n_tokens;
  const int n_rep = n_q_heads / c->n_kv_heads;
  const int64_t bh = (int64_t)b * c->n_kv_heads + hq / n_rep;
  record_t r;
  record_of(D, c->k_bits, c->v_bits, c->group, scale_bytes(c), &r);
  float qv[1024];
  for (int ch = 0; ch < D; ++ch)
    qv[ch] = kivi_oracle_half_to_float(q[((int64_t)b * n_q_heads + hq) * D + ch]);
  double m = -INFINITY;
  for (int64_t tau = 0; tau < t; ++tau) {
    double acc = 0.0;
    for (int ch = 0; ch < D; ++ch) acc += (double)qv[ch] * (double)key_at(c, &r, bh, tau, ch);
    acc = acc / sqrt((double)D);
    if (mask) acc += (double)mask[(int64_t)b * t + tau];
    score[tau] = acc;
    if (acc > m) m = acc;
  }
  for (int ch = 0; ch < D; ++ch) out[ch] = 0.0f;
  if (t == 0 || m == -INFINITY) return 0;  /* empty or fully masked row */
  double l = 0.0;
  for (int64_t tau = 0; tau < t; ++tau) {
    score[tau] = exp(score[tau] - m);
    l += score[tau];
  }
  double o[1024];
  for (int ch = 0; ch < D; ++ch) o[ch] = 0.0;
  for (int64_t tau = 0; tau < t; ++tau) {
    const double p = score[tau] / l;
    for (int ch = 0; ch < D; ++ch) o[ch] += p * (double)value_at(c, &r, bh, tau, ch);
  }
  for (int ch = 0; ch < D; ++ch) out[ch] = (float)o[ch];
  return 0;
}

int kivi_oracle_decode_attn_heads(const kivi_oracle_cache *c, const uint16_t *q,
                                  int n_q_heads, const float *mask, int b,
                                  int h0, int h1, float *out) {
  if (!cache_ok(c) || n_q_heads <= 0 || n_q_heads % c->n_kv_heads || b < 0 ||
      b >= c->batch || h0 < 0 || h1 > n_q_heads || h0 > h1)
    return -1;
  double *score = (double *)malloc(sizeof(double) * (size_t)(c->n_tokens + 1));
  if (!score) return -1;
  for (int hq = h0; hq < h1; ++hq)
    attend_one(c, q, n_q_heads, mask, b, hq, score, out + (int64_t)(hq - h0) * c->head_dim);
  free(score);
  return 0;
}

int kivi_oracle_decode_attn(const kivi_oracle_cache *c, const uint16_t *q,
                            int n_q_heads, const float *mask, float *out) {
  if (!cache_ok(c) || n_q_heads <= 0 || n_q_heads % c->n_kv_heads) return -1;
  for (int b = 0; b < c->batch; ++b) {
    int rc = kivi_oracle_decode_attn_heads(
        c, q, n_q_heads, mask, b, 0, n_q_heads,
        out + (int64_t)b * n_q_heads * c->head_dim);
    if (rc) return rc;
  }
  return 0;
}
