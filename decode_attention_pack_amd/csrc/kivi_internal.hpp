// kivi_internal.hpp -- launchers behind the C ABI (host side declarations).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kivi_device.hpp"

namespace kivi {

// Quantize key groups [g_first, g_first + n_groups) of every (batch, head)
// slab (BH slabs) from `src` into the key layout (KIVI item 2).
hipError_t launch_key_groups(const TokenSource &src, int64_t g_first, int64_t n_groups,
                             int64_t BH, int bits, int G, int D, int64_t cap,
                             uint32_t *codes, float *scale, float *zero, hipStream_t s);

// Quantize value rows [tau_first, tau_first + n_rows) of every slab from `src`
// into the value layout (KIVI item 3).
hipError_t launch_value_rows(const TokenSource &src, int64_t tau_first, int64_t n_rows,
                             int64_t BH, int bits, int G, int D, int64_t cap,
                             uint32_t *codes, float *scale, float *zero, hipStream_t s);

// Copy new tokens into window slots: keys for tokens [k_from, t0 + n_new),
// values for [v_from, t0 + n_new); token tau goes to slot tau % R.
hipError_t launch_write_window(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_res,
                               uint16_t *v_res, int64_t t0, int64_t n_new, int64_t k_from,
                               int64_t v_from, int64_t BH, int R, int D, hipStream_t s);

// Pack fast paths for a contiguous fp16 input [BH][T][D] (the pack entry
// points): key tiles (T % G == 0; groups g_first.. of the destination) and
// value tokens (destination tokens tau_first..).  Shapes: D in {64, 128, 256},
// G a power of two with G * D * 2 <= 16 KB and G <= 64.
bool pack_tiles_supported(int D, int G, int bits);
// x holds T_in rows per slab; the first n_rows are packed.
hipError_t launch_key_tiles(const uint16_t *x, int64_t T_in, int64_t n_rows, int64_t g_first,
                            int64_t BH, int bits, int G, int D, int64_t cap, uint32_t *codes,
                            float *scale, float *zero, hipStream_t s);
hipError_t launch_value_tokens(const uint16_t *x, int64_t T_in, int64_t n_rows, int64_t tau_first,
                               int64_t BH, int bits, int G, int D, int64_t cap, uint32_t *codes,
                               float *scale, float *zero, hipStream_t s);

// Single-token append (the decode step), fused into one kernel: pops the
// value leaving the window into the value layout and writes the new key and
// value into their window slot (the key only if `key_to_window`).  Shapes:
// G and 32 / bits powers of two of at most 64, D <= 256.
__host__ __device__ inline bool append_one_supported(int D, int G, int bits) {
  const int per = 32 / bits;
  return D <= 256 && G <= 64 && (G & (G - 1)) == 0 && per <= G && D % G == 0;
}
hipError_t launch_append_one(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_res,
                             uint16_t *v_res, int64_t t0, int64_t BH, int R, int D, int G,
                             int bits, int64_t cap, bool key_to_window, uint32_t *codes,
                             float *scale, float *zero, hipStream_t s);

// Everything the decode kernels read.
struct DecodeArgs {
  const uint32_t *k_codes;
  const float *k_scale;
  const float *k_zero;
  const uint32_t *v_codes;
  const float *v_scale;
  const float *v_zero;
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
};

// Scalar kernel over tokens [tok_begin, t): `n_splits` splits of
// `tokens_per_split`, writing partial slots [slot_base, slot_base + n_splits).
hipError_t launch_decode_generic(const DecodeArgs &a, int64_t tok_begin, int tokens_per_split,
                                 int n_splits, int slot_base, hipStream_t s);

// Matrix-core kernel for 2-bit caches with G = 32, D = 128 and 1, 2 or 4
// query heads per KV head.  Returns hipErrorInvalidValue for other shapes.
bool decode_vector_supported(const DecodeArgs &a);
hipError_t launch_decode_vector(const DecodeArgs &a, int tokens_per_split, int n_splits,
                                hipStream_t s);

bool decode_matrix_supported(const DecodeArgs &a);
// Window chunks (32 tokens each) that cover tokens [n_main, t).
int decode_matrix_window_chunks(const DecodeArgs &a, int64_t n_main);
// One launch: block role over [0, n_main) in n_splits splits (partial slots
// [0, n_splits)), window role over [n_main, t) (slots after those).
hipError_t launch_decode_matrix(const DecodeArgs &a, int64_t n_main, int tokens_per_split,
                                int n_splits, hipStream_t s);

// Log-sum-exp merge of the S_total partial slots into `out`.
hipError_t launch_combine(const DecodeArgs &a, hipStream_t s);

}  // namespace kivi
