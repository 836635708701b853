/*
 * kivi.h -- C ABI of libkivi.so: KIVI 2/4-bit packed KV cache and decode
 * attention read straight from it, for AMD Instinct MI355X (gfx950).
 *
 * Method source: web page "Literature audit -- Group 2 (KV-cache compression
 * primary sources)", section "1. KIVI -- kivi2024", list "Core algorithm
 * (implementation-grade)", items 1-6 ("KIVI item N" below), and the same
 * section's note that the released code supports grouped-query attention.
 *
 * Conventions for every call
 *   - Pointers marked (device) are HIP device pointers; everything else is
 *     host memory.  The caller owns every buffer; the library allocates and
 *     frees nothing.
 *   - fp16 tensors are IEEE binary16, passed as untyped pointers.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default
 *     stream.  Calls enqueue kernels and return without synchronizing.
 *   - Arguments are validated on the host before any HIP call.  A rejected
 *     call returns a negative status, enqueues nothing and changes nothing;
 *     kivi_last_error() then describes the failure (per thread).
 *   - Results are deterministic: no floating-point atomics, and the split of
 *     the token range is a fixed function of the shape.
 *
 * Storage layout of a cache (b < batch, h < n_kv_heads, G = group,
 * D = head_dim, R = residual, cap = capacity, kb/vb = key/value bits).  The
 * quantized part of each (b, h) slab is a run of cap/128 records, one per
 * 128 consecutive tokens; record j of slab (b, h) holds tokens [128 j,
 * 128 j + 128) and starts at byte ((b * n_kv_heads + h) * (cap/128) + j) *
 * RB of `blocks`, RB = kivi_record_bytes(D, kb, vb, G).  A record holds, in
 * this order (each section a multiple of 16 bytes):
 *   key codes    u32 [128/G][D][G*kb/32]  key group g of the record (tokens
 *                                         128 j + G g ..) and channel c:
 *                                         token e of the group in word
 *                                         e/(32/kb), bits kb*(e % (32/kb))
 *                                         (KIVI item 2: per-channel groups
 *                                         of G tokens, packed along tokens)
 *   key scales   f32 [128/G][D]
 *   key zeros    f16 [128/G][D]           the group minimum, an fp16 input
 *                                         value, stored exactly
 *   value codes  u32 [128][D*vb/32]       token tau of the record: channel e
 *                                         in word e/(32/vb), bits vb*(e %
 *                                         (32/vb)) (KIVI item 3: per-token
 *                                         groups of G channels, packed along
 *                                         channels)
 *   value scales f32 [D/G][128]           channel group, token of the record
 *   value zeros  f16 [D/G][128]
 * With scale_fp16 = 1 both scale sections hold binary16 values ([128/G][D]
 * and [D/G][128] of 2 bytes; RB = kivi_record_bytes_ex(D, kb, vb, G, 1)),
 * the sections after them moving up accordingly.
 *   k_res    fp16 [B][H][R][D]              the fp16 residual window (KIVI
 *   v_res    fp16 [B][H][R][D]              item 4); token tau lives in slot
 *                                           tau % R
 * Every byte a 128-token block of one slab needs is one contiguous record,
 * so attention streams the store in long sequential runs.
 * With t = n_tokens: keys [0, t - t%R) are in the records and keys
 * [t - t%R, t) in k_res; values [0, max(0, t-R)) are in the records and the
 * last min(t, R) values in v_res.
 *
 * Quantizer (KIVI item 1), bit-exact with an fp32 CPU reference: per group,
 * z = min x, s = (max x - min x) / (2^B - 1) (IEEE fp32 division), code =
 * clamp(round_half_even((x - z) / s), 0, 2^B - 1); a group with max == min
 * stores s = 0 and all-zero codes.  fp16-scale layout (scale_fp16 = 1; the
 * page fixes no storage precision for s, and its item 6 puts storage on the
 * hyperparameter axis): s is rounded to the nearest binary16 value (ties to
 * even) and the codes are chosen for that stored scale, code =
 * clamp(round_half_even((x - z) / s16), 0, 2^B - 1); a scale that rounds to
 * 0 gives all-zero codes.  At 2 bits, G 32, D 128 a record is 12,288 bytes
 * instead of 14,336.
 */
#ifndef KIVI_H
#define KIVI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  KIVI_OK = 0,
  KIVI_ERR_INVALID_ARG = -1, /* a shape, bit width, pointer or option is invalid */
  KIVI_ERR_CAPACITY = -2,    /* the write would pass the cache capacity          */
  KIVI_ERR_WORKSPACE = -3,   /* the workspace is smaller than required            */
  KIVI_ERR_HIP = -4          /* a HIP launch failed (detail in kivi_last_error)   */
};

/* A KV cache for one attention layer.  Host struct; the array pointers are
 * (device) memory owned by the caller, laid out as described above.  A new
 * cache has n_tokens = 0 and needs no initialisation of its arrays.
 * Constraints: k_bits, v_bits in {2, 4}; group divides 128 and head_dim and
 * is a multiple of 32/bits for both; head_dim <= 256; residual % group == 0;
 * capacity a positive multiple of 128 and of residual; 0 <= n_tokens <=
 * capacity; batch * n_kv_heads <= 65535; blocks, k_res and v_res 16-byte
 * aligned.
 *
 * Ragged batch (row_tokens != NULL): the rows are independent sequences of
 * different lengths, as in serving, where the batch holds requests of
 * different context lengths (the setting of the throughput measurement on
 * the "Literature audit" page, section "1. KIVI -- kivi2024", "Original
 * evaluation setting").  row_tokens is a host array of `batch` counts; row
 * b holds row_tokens[b] tokens (0 <= row_tokens[b] <= capacity), stored by
 * the rules above with t = row_tokens[b], and batch <= 256.  n_tokens is
 * then not read: every call that changes the counts writes the longest one
 * into it.  The records and windows of row b, taken alone, form a cache of
 * batch 1 (blocks + b * n_kv_heads * (capacity/128) * RB unless paged, k_res
 * and v_res + b * n_kv_heads * R * D elements), so a row's storage is
 * independent of the others'.  A row is emptied by setting its count to 0 (nothing on the
 * device changes; later appends overwrite what it held).  A mask for a
 * ragged batch is f32 [B][max_b row_tokens[b]] (plus one for
 * kivi_decode_step); entries past a row's length are not read.
 *
 * Paged cache (page_table != NULL): `blocks` is a pool of n_pages pages, a
 * page being n_kv_heads consecutive records (one per KV head) of one
 * 128-token block of one row; record j of slab (b, h) is record h of page
 * page_table[b * (capacity/128) + j], i.e. at byte (page * n_kv_heads + h) *
 * RB of `blocks`.  Rows then hold only the pages their tokens use, in any
 * order, so that short rows of a ragged batch do not hold a long row's
 * memory (the same serving setting).  The caller keeps, for every row, the
 * entries of the blocks its tokens use -- and of the block an append writes
 * into -- pointing at pages no other (row, block) uses.  The table lives in device memory and is not
 * checked on the host: an entry outside [0, n_pages) is clamped into the
 * pool (a caller error whose results are unspecified; no access leaves the
 * pool).  page_table 4-byte aligned; n_pages * n_kv_heads * RB < 2^62. */
typedef struct kivi_cache {
  int32_t batch;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t k_bits;
  int32_t v_bits;
  int32_t group;     /* G: tokens per key group and channels per value group */
  int32_t residual;  /* R: fp16 window length                              */
  int64_t capacity;  /* maximum number of tokens                           */
  int64_t n_tokens;  /* t: changed only by kivi_append, kivi_decode_step */
  uint8_t *blocks;   /* [B][H][capacity/128] records                       */
  uint16_t *k_res;
  uint16_t *v_res;
  int64_t *row_tokens; /* NULL, or host [batch]: per-row token counts      */
  const int32_t *page_table; /* NULL, or (device) int32 [batch][capacity/128] */
  int64_t n_pages;     /* pages in `blocks` when page_table is set         */
  int32_t scale_fp16;  /* 0: fp32 scales; 1: fp16 scales (see above)       */
} kivi_cache;

/* Bytes of one 128-token record for a shape (0 if the shape is invalid);
 * a cache's `blocks` array holds batch * n_kv_heads * capacity/128 of them. */
size_t kivi_record_bytes(int32_t head_dim, int32_t k_bits, int32_t v_bits, int32_t group);
/* The same for either scale precision: scale_fp16 0 (fp32 scales, as
 * kivi_record_bytes) or 1 (fp16 scales); 0 for an invalid shape or flag. */
size_t kivi_record_bytes_ex(int32_t head_dim, int32_t k_bits, int32_t v_bits, int32_t group,
                            int32_t scale_fp16);

/* KIVI item 2: quantize keys per channel in groups of `group` consecutive
 * tokens and store them in the records of `dst` (packed along tokens).
 *   dst      a cache descriptor: its shape and `blocks` say where the codes,
 *            scales and zeros go; n_tokens and the windows are neither read
 *            nor changed.
 *   k_fp16   (device) fp16 [batch][n_kv_heads][T][head_dim], token-major.
 *   The T tokens become tokens [dst_token_offset, dst_token_offset + T).
 *   Requires T % group == 0, dst_token_offset % group == 0 and the range
 *   inside the capacity.  T == 0 is a no-op. */
int kivi_pack_keys(const kivi_cache *dst, const void *k_fp16, int64_t T,
                   int64_t dst_token_offset, void *stream);

/* KIVI item 3: quantize values per token in groups of `group` consecutive
 * channels and store them in the records of `dst` (packed along channels).
 *   v_fp16   (device) fp16 [batch][n_kv_heads][T][head_dim].
 *   Tokens go to [dst_token_offset, dst_token_offset + T) (any offset); the
 *   rest as for kivi_pack_keys. */
int kivi_pack_values(const kivi_cache *dst, const void *v_fp16, int64_t T,
                     int64_t dst_token_offset, void *stream);

/* KIVI item 4: append n_new tokens to the cache through the fp16 window.
 * The result is bit-identical to appending them one at a time: for each
 * token tau, if tau >= R the value in slot tau % R (token tau - R) is
 * quantized into its record first; the new key and value then take slot
 * tau % R; when tau + 1 is a multiple of R the R keys of the window are
 * quantized into their records.  Appending T tokens to an empty cache is
 * the prefill rule: keys [0, T - T%R) and values [0, T - R) quantized, the
 * rest kept in fp16.
 *   k_new_fp16, v_new_fp16  (device) fp16 [B][H][n_new][D].
 *   n_new >= 0; KIVI_ERR_CAPACITY if n_tokens + n_new > capacity.
 * On success c->n_tokens grows by n_new (on the host, at once; the kernels
 * run in stream order). */
int kivi_append(kivi_cache *c, const void *k_new_fp16, const void *v_new_fp16,
                int64_t n_new, void *stream);

/* KIVI item 4 for one row of a ragged batch (row_tokens != NULL): append
 * n_new tokens to row b alone, by the rule of kivi_append, e.g. the prefill
 * of a new request into an emptied row.
 *   k_new_fp16, v_new_fp16  (device) fp16 [H][n_new][D].
 * KIVI_ERR_CAPACITY if row_tokens[b] + n_new > capacity; KIVI_ERR_INVALID_ARG
 * for a cache without row_tokens.  On success row_tokens[b] grows by n_new
 * and n_tokens becomes the longest row. */
int kivi_append_row(kivi_cache *c, int32_t b, const void *k_new_fp16, const void *v_new_fp16,
                    int64_t n_new, void *stream);

/* Bytes of workspace kivi_decode_attn needs for this cache shape and query
 * head count at any n_tokens up to the capacity. 0 on invalid arguments. */
size_t kivi_decode_attn_workspace_bytes(const kivi_cache *c, int32_t n_q_heads);

/* KIVI item 5: one decode step of attention over the cache.  For query head
 * hq of batch row b (KV head hq / (n_q_heads / n_kv_heads)):
 *   s_tau = q . K_tau / sqrt(D) + mask[b][tau]   for tau < t,
 *   out   = sum_tau softmax(s)_tau V_tau,
 * where K_tau, V_tau are the dequantized codes (code * scale + zero) where
 * quantized and the fp16 window values otherwise.  A row whose scores are
 * all -inf gives zeros; t == 0 gives zeros.
 *   q_fp16    (device) fp16 [B][n_q_heads][D]; n_q_heads % n_kv_heads == 0.
 *   mask      (device) f32 [B][n_tokens] additive, indexed by token, or NULL.
 *   out       (device) f32 [B][n_q_heads][D].
 *   workspace (device) at least kivi_decode_attn_workspace_bytes() bytes.
 * Append first, then attend: the cache must already hold the current token. */
int kivi_decode_attn(const kivi_cache *c, const void *q_fp16, int32_t n_q_heads,
                     const float *mask, float *out, void *workspace,
                     size_t workspace_bytes, void *stream);

/* kivi_decode_attn without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The partial results go to a scratch
 * array of 16 MiB that the library holds on each GPU it runs on until the
 * process ends; the call allocates nothing.  Arguments as for
 * kivi_decode_attn (automatic plan).  KIVI_ERR_WORKSPACE, before anything
 * runs, when this call's partials pass 16 MiB: (D + 4) x 4 bytes for each
 * of batch x n_q_heads x S partial slots, where the matrix kernel plans S =
 * its workgroups per slab (about one workgroup per CU, shared out among the
 * batch x n_kv_heads slabs) plus one per 32 tokens of the window (at most 10
 * for R = 128).  Every call on a
 * GPU shares its array: calls that overlap on one GPU (several streams or
 * threads) race and must be serialized by the caller.  Each call writes
 * every slot it reads, so no state carries over between calls. */
int kivi_decode_attn_noalloc(const kivi_cache *c, const void *q_fp16, int32_t n_q_heads,
                             const float *mask, float *out, void *stream);


/* Same as kivi_decode_attn with explicit tuning, for tests and sweeps:
 *   tokens_per_split  0 = automatic, else a positive multiple of 64.
 *   path              KIVI_PATH_AUTO (the matrix-core kernel where the shape
 *                     allows -- with 4-bit codes and one query head per KV
 *                     head only from 18 blocks of 128 tokens per row on --
 *                     else the vector kernel where it allows, else the
 *                     scalar kernel), KIVI_PATH_GENERIC (scalar kernel for
 *                     every token), KIVI_PATH_MATRIX (matrix-core kernel:
 *                     head_dim 128, G 32, 1, 2 or 4 query heads per KV
 *                     head, 16-byte aligned q, record array and windows;
 *                     2-bit keys and values in any cache, or 4-bit keys,
 *                     values or both in a contiguous cache of a uniform
 *                     batch) or
 *                     KIVI_PATH_VECTOR (vector kernel: 2- or 4-bit codes,
 *                     head_dim 128, G 32, R a multiple of 32, 1 or an even
 *                     number (at most 64) of query heads per KV head,
 *                     capacity below 2^26 tokens and a slab's records below
 *                     4 GB).  A
 *                     forced path the shape does not allow is rejected.
 * The workspace must hold kivi_decode_attn_workspace_bytes_ex() bytes. */
enum { KIVI_PATH_AUTO = 0, KIVI_PATH_GENERIC = 1, KIVI_PATH_MATRIX = 2, KIVI_PATH_VECTOR = 3 };
int kivi_decode_attn_ex(const kivi_cache *c, const void *q_fp16, int32_t n_q_heads,
                        const float *mask, float *out, void *workspace,
                        size_t workspace_bytes, int32_t tokens_per_split,
                        int32_t path, void *stream);
size_t kivi_decode_attn_workspace_bytes_ex(const kivi_cache *c, int32_t n_q_heads,
                                           int32_t tokens_per_split, int32_t path);

/* KIVI items 4 and 5 in one call: one decode step that appends one token
 * and attends over the cache that results, i.e. the same cache state and
 * (within the attention tolerance) the same output as
 *   kivi_append(c, k_new, v_new, 1); kivi_decode_attn(c, q, ...).
 * Where the default path takes the matrix-core kernel (KIVI_PATH_AUTO of
 * kivi_decode_attn_ex, for the cache after the append) and q, k_new and
 * v_new are 16-byte aligned, the append runs inside the attention launch: the new
 * key and value are read from k_new / v_new, the value that leaves the
 * window and a key block the token completes are quantized by the
 * workgroups that attend over them, and the cache writes happen where no
 * other workgroup reads.  Otherwise the two calls above run in turn.
 *   k_new_fp16, v_new_fp16  (device) fp16 [B][H][D], the new token.
 *   q_fp16, out             as for kivi_decode_attn.
 *   mask                    (device) f32 [B][n_tokens + 1] or NULL.
 *   workspace               at least kivi_decode_attn_workspace_bytes().
 * KIVI_ERR_CAPACITY if the cache is full; the workspace is checked before
 * anything runs.  On success c->n_tokens grows by one. */
int kivi_decode_step(kivi_cache *c, const void *k_new_fp16, const void *v_new_fp16,
                     const void *q_fp16, int32_t n_q_heads, const float *mask,
                     float *out, void *workspace, size_t workspace_bytes, void *stream);

/* A second workload on the packed cache: token selection by attention mass
 * and attention over the selected tokens, after the web page "HCAttention:
 * Extreme KV Cache Compression via Heterogeneous Attention Computing for
 * LLMs" (a review), section "What carries the argument": approximate scores
 * from quantized keys (Eq. 3), here the KIVI scores over the packed cache,
 * and the smallest prefix of the tokens sorted by score whose mass reaches
 * tau (Eq. 4); the output over the selected set (Eq. 5) renormalized, as the
 * review's major comment 2 asks to state.  For every (b, hq), with s_j = q .
 * K_j / sqrt(D) + mask[b][j] as in kivi_decode_attn and a = softmax(s):
 *   S   = the smallest set of tokens, taken in decreasing order of s (equal
 *         scores by increasing token index), whose mass sum_S a reaches
 *         tau; tokens of mass zero (-inf scores) are never selected, and when
 *         the others do not reach tau they are all selected;
 *   out = sum_{j in S} a_j V_j / sum_{j in S} a_j.
 * The selection is per call (per query); nothing leaves the cache.  Masses
 * are summed in fixed point (units of 2^-36 of the largest e^(s - max)), so
 * the selection is deterministic; a token whose mass is below 2^-37 of the
 * largest counts as mass zero.  Uniform caches (row_tokens NULL) with fewer
 * than 2^27 tokens.
 *   tau         in (0, 1].
 *   q_fp16, mask, out as for kivi_decode_attn.
 *   n_selected  (device) int32 [B][n_q_heads] or NULL: |S| of each row.
 *   sel_mask    (device) uint32 [B][n_q_heads][ceil(t / 32)] or NULL: bit
 *               j % 32 of word j / 32 set when token j is in S.
 *   workspace   (device, 256-byte aligned) at least
 *               kivi_select_attn_workspace_bytes() bytes. */
int kivi_select_attn(const kivi_cache *c, const void *q_fp16, int32_t n_q_heads,
                     const float *mask, float tau, float *out, int32_t *n_selected,
                     uint32_t *sel_mask, void *workspace, size_t workspace_bytes, void *stream);
/* Bytes of workspace kivi_select_attn needs for this cache shape at any
 * n_tokens up to the capacity (0 on invalid arguments). */
size_t kivi_select_attn_workspace_bytes(const kivi_cache *c, int32_t n_q_heads);

/* Static description of a status code. */
const char *kivi_status_string(int status);
/* Detail of the last failing call on this thread ("" if none). */
const char *kivi_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* KIVI_H */
