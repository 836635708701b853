// kivi_internal.hpp -- launchers behind the C ABI (host side declarations).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kivi_device.hpp"

namespace kivi {

// Quantize key groups [g_first, g_first + n_groups) of every (batch, head)
// slab (BH slabs) from `src` into the packed store (KIVI item 2).
hipError_t launch_key_groups(const TokenSource &src, int64_t g_first, int64_t n_groups,
                             int64_t BH, const Layout &L, hipStream_t s);

// Quantize value rows [tau_first, tau_first + n_rows) of every slab from `src`
// into the packed store (KIVI item 3).
hipError_t launch_value_rows(const TokenSource &src, int64_t tau_first, int64_t n_rows,
                             int64_t BH, const Layout &L, hipStream_t s);

// Copy new tokens into window slots: keys for tokens [k_from, t0 + n_new),
// values for [v_from, t0 + n_new); token tau goes to slot tau % R.
hipError_t launch_write_window(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_res,
                               uint16_t *v_res, int64_t t0, int64_t n_new, int64_t k_from,
                               int64_t v_from, int64_t BH, int R, int D, hipStream_t s);

// Pack fast paths for a contiguous fp16 input [BH][T_in][D] (the pack entry
// points and the prefill): key tiles (whole groups from destination group
// g_first on) and value tokens (destination tokens from tau_first on, a
// multiple of 64).  Shapes: D in {64, 128, 256}, G a power of two in [16, 64]
// with G * D * 2 <= 16 KB.
bool pack_tiles_supported(int D, int G, int bits);
// x holds T_in rows per slab; the first n_rows are packed.
hipError_t launch_key_tiles(const uint16_t *x, int64_t T_in, int64_t n_rows, int64_t g_first,
                            int64_t BH, const Layout &L, hipStream_t s);
hipError_t launch_value_tokens(const uint16_t *x, int64_t T_in, int64_t n_rows, int64_t tau_first,
                               int64_t BH, const Layout &L, hipStream_t s);

// Single-token append (the decode step), fused into one kernel: pops the
// value leaving the window into the packed store and writes the new key and
// value into their window slot (the key only if `key_to_window`).  Shapes:
// G and 32 / bits powers of two of at most 64, D <= 256.
__host__ __device__ inline bool append_one_supported(int D, int G, int bits) {
  const int per = 32 / bits;
  return D <= 256 && G <= 64 && (G & (G - 1)) == 0 && per <= G && D % G == 0;
}
hipError_t launch_append_one(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_res,
                             uint16_t *v_res, int64_t t0, int64_t BH, int R, bool key_to_window,
                             const Layout &L, hipStream_t s);
// The same for a ragged batch (row b = slab / H appends token rows.n[b]),
// including the key block a row's token completes.
hipError_t launch_append_one_rows(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_res,
                                  uint16_t *v_res, int64_t BH, int H, int R,
                                  const RowCounts &rows, const Layout &L, hipStream_t s);

// The selection rule of one (b, hq) row: a token is selected when its score
// key (an order-preserving map of the float, select_key) is above `key`, or
// equal to it with index <= `cut`.
struct SelectRow {
  uint32_t key;
  int32_t cut;
  float m;          // the row's largest score (-inf: nothing selected)
  int32_t count;    // tokens selected
};
__device__ __forceinline__ uint32_t select_key(float s) {
  const uint32_t u = __float_as_uint(s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ bool select_takes(const SelectRow &r, float s, int64_t tau) {
  const uint32_t k = select_key(s);
  return s > -INFINITY && (k > r.key || (k == r.key && tau <= r.cut));
}

// Everything the decode kernels read.
struct DecodeArgs {
  Layout L;              // the packed store
  const uint16_t *k_res;
  const uint16_t *v_res;
  const uint16_t *q;     // [B][Hq][D]
  const float *mask;     // [B][t] or nullptr
  float *part;           // partials [B][Hq][S_total][D + 4]: acc[D], m, l, (pad)
  float *out;            // [B][Hq][D]
  int32_t B, H, D, kb, vb, G, R, Hq, n_rep;
  int64_t cap, t, n_kq, n_vq;
  float sm_scale;        // 1 / sqrt(D)
  int32_t S_total;       // partial slots per (b, hq)
  // Fused decode step (matrix kernel only): t_new >= 0 is the token this
  // launch appends (t_new = t - 1).  Its key and value come from k_new /
  // v_new ([B][H][D] fp16) instead of the window slots; the value it pushes
  // out of the window (token t_new - R, when t_new >= R) is quantized by the
  // window-role workgroup that attends over it, which stores it in the cache
  // and then puts the new value into its slot; when t is a multiple of R,
  // the window-role workgroups of keys [t - R, t) quantize their key groups
  // and store them.  t_new = -1: a plain attention call that writes nothing
  // to the cache.
  const uint16_t *k_new;
  const uint16_t *v_new;
  int64_t t_new;
  // Scores-only launches: s = q . K / sqrt(D) + mask of token tau of
  // (b, hq) at scores[(b Hq + hq) cap + tau].  Selected-attention launches
  // read them there, and the selection rule of row (b, hq) at sel[b Hq + hq].
  float *scores;
  const SelectRow *sel;
  // Scores-only matrix launches, when rmax is set: the largest score each
  // wave stored of row (b, hq) at rmax[(b Hq + hq) rmax_n + k] (k: the
  // wave's item share, or a window chunk), -inf for a wave with none; the
  // selection then takes the row's largest score from these rmax_n values.
  float *rmax;
  int32_t rmax_n;
};

// Scalar kernel over tokens [tok_begin, t): `n_splits` splits of
// `tokens_per_split`, writing partial slots [slot_base, slot_base + n_splits).
// With `rows` (a ragged batch), row b attends over rows->n[b] tokens; splits
// past a row's end write empty partials.
hipError_t launch_decode_generic(const DecodeArgs &a, int64_t tok_begin, int tokens_per_split,
                                 int n_splits, int slot_base, hipStream_t s,
                                 const RowCounts *rows = nullptr);

// Vector kernel for 2/4-bit caches with G = 32 and D = 128 (shapes in
// decode_vector_supported).  `rows` as for the scalar kernel.
bool decode_vector_supported(const DecodeArgs &a);
hipError_t launch_decode_vector(const DecodeArgs &a, int tokens_per_split, int n_splits,
                                hipStream_t s, const RowCounts *rows = nullptr);

bool decode_matrix_supported(const DecodeArgs &a);
// Tokens [0, n_main) of a row go to the matrix kernel's block role: whole
// 128-token blocks of quantized keys and values.  In a fused step the value
// leaving the window (token t_new - R) is quantized by the window role, so
// the blocks stop before it.
__host__ __device__ inline int64_t matrix_main(const RowSpan &r, int R) {
  const int64_t lim = r.t_new >= R ? r.t_new - R : r.n_vq;
  return lim / kRecTokens * kRecTokens;
}
// Window chunks (32 tokens each) that cover tokens [n_main, t).
__host__ __device__ inline int matrix_window_chunks(int64_t t, int64_t n_main) {
  return (int)((t - n_main + 31) / 32);
}
int decode_matrix_window_chunks(const DecodeArgs &a, int64_t n_main);
// One launch of n_groups workgroups per slab (n_groups * B * H in all); the
// waves of a workgroup take window chunks of [n_main, t) and blocks of its
// share of [0, n_main) from a counter in LDS.  Partial slots: one per
// workgroup (its waves' blocks), then one per window chunk.
int decode_matrix_waves(const DecodeArgs &a);
hipError_t launch_decode_matrix(const DecodeArgs &a, int64_t n_main, int n_groups,
                                hipStream_t s);
// launch_decode_matrix and launch_decode_matrix_rows also take 4-bit codes
// (G = 32, D = 128, 1, 2 or 4 query heads per KV head), attention and the
// fused step: 4-bit keys and values in any cache, 4-bit keys or values alone
// in a contiguous cache of a uniform batch (decode_matrix4_supported).
bool decode_matrix4_supported(const DecodeArgs &a, bool ragged);
// Ragged batch: row b attends over t[b] tokens (after the append of a
// fused step); per KV head, share u of n_shares is workgroup
// share[u] >> 8 & 4095 of the share[u] >> 20 workgroups of row share[u] &
// 255.  a.t is the longest row (the mask's row stride); a.S_total must hold
// every row's slots.
struct MatrixRows {
  int32_t t[kMaxRows];
  uint32_t share[kMaxRows];
};
template <bool RAGGED>
using MatrixRowArg = typename std::conditional<RAGGED, MatrixRows, NoRows>::type;
hipError_t launch_decode_matrix_rows(const DecodeArgs &a, const MatrixRows &rows, int n_shares,
                                     hipStream_t s);
// The selection workload on the matrix kernel's shapes, with the plan of
// launch_decode_matrix (no fused step): the scores of every token into
// DecodeArgs::scores, and the attention over the tokens DecodeArgs::sel
// selects (partials as launch_decode_matrix, merged by launch_combine when
// n_groups > 1).
hipError_t launch_scores_matrix(const DecodeArgs &a, int64_t n_main, int n_groups, hipStream_t s);
hipError_t launch_selected_matrix(const DecodeArgs &a, int64_t n_main, int n_groups,
                                  hipStream_t s);

// The scores of every token (DecodeArgs::scores), in splits of
// tokens_per_split tokens: the vector kernel's shapes, and any shape.
hipError_t launch_scores_vector(const DecodeArgs &a, int tokens_per_split, int n_splits,
                                hipStream_t s);
hipError_t launch_scores_generic(const DecodeArgs &a, int tokens_per_split, int n_splits,
                                 hipStream_t s);

// Token selection by attention mass on the scores (select.hip): per (b, hq)
// row, the smallest set of tokens in decreasing score order (equal scores by
// increasing index) whose softmax mass reaches tau.
// sel_mask (optional) gets bit tau % 32 of word tau / 32 of its row's
// ceil(t / 32) words for the selected tokens.
hipError_t launch_select_rows(const DecodeArgs &a, float tau, SelectRow *rows,
                              int32_t *n_selected, uint32_t *sel_mask, hipStream_t s);
// Attention over the selected tokens of every row (a.scores, a.sel): the
// scores are read instead of computed, and a token the row's rule does not
// select scores -inf; otherwise as launch_decode_vector /
// launch_decode_generic.
hipError_t launch_selected_vector(const DecodeArgs &a, int tokens_per_split, int n_splits,
                                  hipStream_t s);
hipError_t launch_selected_generic(const DecodeArgs &a, int tokens_per_split, int n_splits,
                                   hipStream_t s);

// Log-sum-exp merge of the S_total partial slots into `out`.  With
// `slots`, the rows of batch row b merge their first slots->n[b] slots, and
// rows with none are left as they are (their output is already written).
hipError_t launch_combine(const DecodeArgs &a, hipStream_t s, const RowCounts *slots = nullptr);

}  // namespace kivi
