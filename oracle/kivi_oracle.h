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
 * Storage layout (the same contract the GPU library follows; the packing
 * direction is the page's: keys packed along tokens, values along channels):
 *   key codes   u32 [B][H][cap/G][D][G*kb/32]   token e of a group at word
 *                                               e/(32/kb), bits kb*(e%(32/kb))
 *   key scale   f32 [B][H][cap/G][D]            (and key zero, same shape)
 *   value codes u32 [B][H][cap][D*vb/32]        channel e at word e/(32/vb),
 *                                               bits vb*(e%(32/vb))
 *   value scale f32 [B][H][D/G][cap]            (and value zero, same shape)
 *   key/value residual fp16 [B][H][R][D]        token tau in slot tau % R
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
  uint32_t *k_codes; float *k_scale, *k_zero;
  uint32_t *v_codes; float *v_scale, *v_zero;
  uint16_t *k_res, *v_res;
} kivi_oracle_cache;

/* binary16 bit pattern -> float (exact). */
float kivi_oracle_half_to_float(uint16_t h);

/* KIVI item 1: asymmetric round-to-nearest group quantizer. */
void kivi_oracle_quantize_group(const float *x, int n, int bits, uint8_t *codes,
                                float *scale, float *zero);
/* KIVI item 1: dequantization code*scale + zero (fp32 multiply, then add). */
float kivi_oracle_dequant(uint32_t code, float scale, float zero);

/* Bit packing of n codes of `bits` bits into u32 words (lowest bits first). */
void kivi_oracle_pack_codes(const uint8_t *codes, int n, int bits, uint32_t *words);
void kivi_oracle_unpack_codes(const uint32_t *words, int n, int bits, uint8_t *codes);

/* KIVI item 2: per-channel key quantization, G consecutive tokens per group.
 * k: fp16 [B][H][T][D]; T % G == 0; dst_token_offset % G == 0.  Writes groups
 * [off/G, (off+T)/G) of a destination with capacity `cap`.  Returns 0 or -1. */
int kivi_oracle_pack_keys(const uint16_t *k, int B, int H, int64_t T, int D,
                          int bits, int G, uint32_t *codes, float *scale,
                          float *zero, int64_t cap, int64_t dst_token_offset);

/* KIVI item 3: per-token value quantization, G consecutive channels per group.
 * v: fp16 [B][H][T][D].  Writes rows [off, off+T).  Returns 0 or -1. */
int kivi_oracle_pack_values(const uint16_t *v, int B, int H, int64_t T, int D,
                            int bits, int G, uint32_t *codes, float *scale,
                            float *zero, int64_t cap, int64_t dst_token_offset);

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
