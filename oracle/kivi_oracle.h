/*
 * kivi_oracle.h -- plain, slow CPU oracle for KIVI packed-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file or the library built from it: only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg use it.  It shares no source with
 * the HIP library.
 *
 * Source of the method: the web page "Literature audit -- Group 2 (KV-cache
 * compression primary sources)", section "1. KIVI -- kivi2024", list "Core
 * algorithm (implementation-grade)", items 1-6 (cited below as "KIVI item N").
 *
 * Every pointer is a host pointer.  fp16 data is passed as raw IEEE binary16
 * bit patterns (uint16_t).  All arrays are owned by the caller.
 *
 * Storage layout (the same contract the GPU library follows).  The quantized
 * part of each (batch row b, KV head h) slab is a run of records, one per 128
 * consecutive tokens: record j of slab bh holds tokens [128 j, 128 j + 128)
 * and sits at byte ((bh * (cap/128)) + j) * RB of the `blocks` array, where
 * RB = kivi_oracle_record_bytes(D, kb, vb, G).  A record holds, in order:
 *   key codes   u32 [128/G][D][G*kb/32]  key group g (tokens 128 j + G g ..)
 *                                        of channel c: its token e at word
 *                                        e/(32/kb), bits kb*(e%(32/kb))
 *                                        (KIVI item 2: per-channel groups of G
 *                                        tokens, packed along tokens)
 *   key scales  f32 [128/G][D]
 *   key zeros   f16 [128/G][D]           the group minimum, an fp16 input
 *                                        value, stored exactly
 *   value codes u32 [128][D*vb/32]       token tau: channel e at word
 *                                        e/(32/vb), bits vb*(e%(32/vb))
 *                                        (KIVI item 3: per-token groups of G
 *                                        channels, packed along channels)
 *   value scales f32 [D/G][128]
 *   value zeros  f16 [D/G][128]
 * G divides 128; cap is a multiple of 128.  With scale_fp16 set, both scale
 * sections hold binary16 values instead ([128/G][D] and [D/G][128] of 2
 * bytes), the sections after them moving up accordingly.
 *   key/value residual fp16 [B][H][R][D]  token tau in slot tau % R
 */
#ifndef KIVI_ORACLE_H
#define KIVI_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kivi_oracle_cache {
  int32_t batch, n_kv_heads, head_dim;
  int32_t k_bits, v_bits, group, residual;
  int64_t capacity;
  int64_t n_tokens;
  uint8_t *blocks;             /* [B][H][cap/128] records */
  uint16_t *k_res, *v_res;
  int32_t scale_fp16;          /* 0: fp32 scales; 1: fp16 scales */
} kivi_oracle_cache;

/* Bytes of one 128-token record; 0 for shapes the layout does not take.
 * _s: the same for fp32 (scale_fp16 0) or fp16 (1) scales. */
int64_t kivi_oracle_record_bytes(int D, int k_bits, int v_bits, int G);
int64_t kivi_oracle_record_bytes_s(int D, int k_bits, int v_bits, int G, int scale_fp16);

/* binary16 bit pattern -> float (exact). */
float kivi_oracle_half_to_float(uint16_t h);
/* float holding a binary16 value -> its bit pattern; 0, or -1 if inexact. */
int kivi_oracle_float_to_half(float f, uint16_t *out);

/* KIVI item 1: asymmetric round-to-nearest group quantizer. */
void kivi_oracle_quantize_group(const float *x, int n, int bits, uint8_t *codes,
                                float *scale, float *zero);
/* float -> binary16 bit pattern, round to nearest, ties to even. */
uint16_t kivi_oracle_half_rne(float f);
/* KIVI item 1 with the scale stored as binary16: s rounded to fp16 (its bit
 * pattern in *scale_bits), codes chosen for the rounded scale. */
void kivi_oracle_quantize_group_s16(const float *x, int n, int bits, uint8_t *codes,
                                    uint16_t *scale_bits, float *zero);
/* KIVI item 1: dequantization code*scale + zero (fp32 multiply, then add). */
float kivi_oracle_dequant(uint32_t code, float scale, float zero);

/* Bit packing of n codes of `bits` bits into u32 words (lowest bits first). */
void kivi_oracle_pack_codes(const uint8_t *codes, int n, int bits, uint32_t *words);
void kivi_oracle_unpack_codes(const uint32_t *words, int n, int bits, uint8_t *codes);

/* KIVI item 2: per-channel key quantization, G consecutive tokens per group.
 * k: fp16 [B][H][T][D] (B, H, D from dst); T % G == 0; off % G == 0.  Writes
 * the key sections for tokens [off, off + T) of dst's records; nothing else
 * of dst changes.  Returns 0 or -1. */
int kivi_oracle_pack_keys(const kivi_oracle_cache *dst, const uint16_t *k, int64_t T,
                          int64_t off);

/* KIVI item 3: per-token value quantization, G consecutive channels per group.
 * v: fp16 [B][H][T][D].  Writes the value sections for tokens [off, off + T).
 * Returns 0 or -1. */
int kivi_oracle_pack_values(const kivi_oracle_cache *dst, const uint16_t *v, int64_t T,
                            int64_t off);

/* KIVI item 4: append n_new tokens (k_new, v_new: fp16 [B][H][n_new][D]) one
 * at a time through the fp16 residual window.  Returns 0 or -1. */
int kivi_oracle_append(kivi_oracle_cache *c, const uint16_t *k_new,
                       const uint16_t *v_new, int64_t n_new);

/* Dequantized view of the cache: k_hat, v_hat f32 [B][H][n_tokens][D]. */
int kivi_oracle_materialize(const kivi_oracle_cache *c, float *k_hat, float *v_hat);

/* KIVI item 5: decode-step attention over the mixed packed/fp16 cache.
 * q: fp16 [B][Hq][D]; mask: additive f32 [B][n_tokens] or NULL;
 * out: f32 [B][Hq][D].  Query head hq reads KV head hq / (Hq/H).
 * Returns 0 or -1. */
int kivi_oracle_decode_attn(const kivi_oracle_cache *c, const uint16_t *q,
                            int n_q_heads, const float *mask, float *out);

/* Same computation restricted to batch row b and query heads [h0, h1); out is
 * f32 [h1-h0][D].  Used to sample large workloads one head at a time. */
int kivi_oracle_decode_attn_heads(const kivi_oracle_cache *c, const uint16_t *q,
                                  int n_q_heads, const float *mask, int b,
                                  int h0, int h1, float *out);

#ifdef __cplusplus
}
#endif
#endif /* KIVI_ORACLE_H */
