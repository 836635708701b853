// decode_generic.hip -- scalar (VALU) decode attention over the KIVI cache,
// and the split-K log-sum-exp combine.
//
// Method source: web page "Literature audit -- Group 2 (KV-cache compression
// primary sources)", section "1. KIVI -- kivi2024", list "Core algorithm
// (implementation-grade)", item 5 (attention over quantized keys/values plus
// the fp16 window) and item 4 (which tokens are quantized).
//
// This kernel handles any shape the ABI accepts.  It dequantizes one element
// at a time and is meant for the fp16 window, ragged tails and shapes the
// matrix-core kernel does not cover.  One workgroup owns a token range of one
// (batch row, KV head) and up to 8 of that head's query heads, keeps an
// online softmax (running max m, running sum l) and writes (acc[D], m, l) as
// a partial; the combine kernel merges the partials of all splits.
#include <math.h>

#include "kivi_internal.hpp"

namespace kivi {

namespace {

constexpr int kThreads = 256;
constexpr int kHeads = 8;     // most query heads per workgroup
constexpr int kChunk = 256;   // tokens per inner step (one per thread)

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace

// grid: (n_splits, H * head_chunks, B); block: 256.  NH (1, 2, 4 or 8) query
// heads per workgroup: the smallest power of two covering the heads per KV
// head, up to 8, so that MHA shapes do not carry 8 heads' worth of products.
// A ragged batch (RAGGED): row b holds rows.n[b] tokens; a.t is the mask's
// row stride.  MODE 1 (scores): only the scores s = q . K / sqrt(D) + mask of
// every token, into a.scores[(b Hq + hq) cap + tau] (no softmax, no values).
// MODE 2 (selected): attention whose scores are read from a.scores, with
// -inf for a token that the row's selection rule (a.sel) does not take.
template <int NH, bool RAGGED, int MODE>
__global__ void __launch_bounds__(kThreads)
decode_generic_kernel(DecodeArgs a, int64_t tok_begin, int tokens_per_split, int slot_base,
                      int head_chunks, RowArg<RAGGED> rows) {
  constexpr bool SCORES = MODE == 1, SELECTED = MODE == 2;
  __shared__ float q_s[NH][256];
  __shared__ float p_s[NH][kChunk];
  __shared__ float stat_s[NH][2];   // new m, alpha
  __shared__ float red_s[kThreads];

  const int tid = threadIdx.x;
  const int split = blockIdx.x;
  const int h = blockIdx.y / head_chunks;
  const int hc = blockIdx.y % head_chunks;
  const int b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.H + h;
  const int hq0 = h * a.n_rep + hc * NH;
  const int nh = min(NH, a.n_rep - hc * NH);
  const int D = a.D;

  RowSpan rs;
  if constexpr (RAGGED)
    rs = row_span(rows.n[b], a.R, false);
  else
    rs = RowSpan{a.t, a.n_kq, a.n_vq, -1};
  int64_t s0 = tok_begin + (int64_t)split * tokens_per_split;
  int64_t s1 = s0 + tokens_per_split;
  if (s1 > rs.t) s1 = rs.t;

  for (int i = tid; i < NH * D; i += kThreads) {
    const int j = i / D, c = i % D;
    q_s[j][c] = j < nh ? h2f(a.q[((int64_t)b * a.Hq + hq0 + j) * D + c]) : 0.0f;
  }

  float m[NH], l[NH], acc[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.0f;
    acc[j] = 0.0f;
  }
  const int c_own = tid % D;           // value channel owned in the V phase
  const int n_par = kThreads / D;      // token parities sharing a channel
  const int par = tid / D;
  // value code word, bit offset and channel group of channel c_own
  const int vper = 32 / a.vb;
  const int vword = c_own / vper;
  const int vsh = a.vb * (c_own % vper);
  const uint32_t vmsk = (1u << a.vb) - 1u;
  const int vgrp = c_own / a.G;
  const Layout &L = a.L;
  __syncthreads();

  for (int64_t c0 = s0; c0 < s1; c0 += kChunk) {
    // scores: one token per thread, all heads of the chunk at once
    const int64_t tau = c0 + tid;
    float sc[NH];
#pragma unroll
    for (int j = 0; j < NH; ++j) sc[j] = 0.0f;
    if (SELECTED && tau < s1) {
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const int64_t r = (int64_t)b * a.Hq + hq0 + (j < nh ? j : 0);
        const float sv = a.scores[r * a.cap + tau];
        sc[j] = j < nh && select_takes(a.sel[r], sv, tau) ? sv : -INFINITY;
      }
    } else if (tau < s1) {
      // key channel c of token tau as attention sees it: code * scale + zero
      // (fp32 multiply, then add) below n_kq, else the fp16 window row; the
      // per-token index arithmetic (group, word, bit offset) is done once
      if (tau < rs.n_kq) {
        const int per = 32 / a.kb;
        const int words = a.G / per;
        const int64_t g = tau / a.G;
        const int e = (int)(tau - g * a.G);
        // the group's channels are consecutive in its record
        const uint32_t *cw = L.key_codes(bh, g, 0) + e / per;
        const uint8_t *ks = L.key_scales(bh, g);
        const uint16_t *kz = L.key_zero(bh, g, 0);
        const int sh = a.kb * (e % per);
        const uint32_t msk = (1u << a.kb) - 1u;
        for (int c = 0; c < D; ++c) {
          const uint32_t code = (cw[c * words] >> sh) & msk;
          const float k = __fadd_rn(__fmul_rn((float)code, L.scale_at(ks, c)), h2f(kz[c]));
#pragma unroll
          for (int j = 0; j < NH; ++j) sc[j] = fmaf(q_s[j][c], k, sc[j]);
        }
      } else {
        const uint16_t *row = a.k_res + (bh * a.R + tau % a.R) * D;
        for (int c = 0; c < D; ++c) {
          const float k = h2f(row[c]);
#pragma unroll
          for (int j = 0; j < NH; ++j) sc[j] = fmaf(q_s[j][c], k, sc[j]);
        }
      }
      const float mk = a.mask ? a.mask[(int64_t)b * a.t + tau] : 0.0f;
#pragma unroll
      for (int j = 0; j < NH; ++j) sc[j] = sc[j] * a.sm_scale + mk;
    } else {
#pragma unroll
      for (int j = 0; j < NH; ++j) sc[j] = -INFINITY;
    }
    if constexpr (SCORES) {
      if (tau < s1)
        for (int j = 0; j < nh; ++j)
          a.scores[((int64_t)b * a.Hq + hq0 + j) * a.cap + tau] = sc[j];
      continue;
    }
#pragma unroll
    for (int j = 0; j < NH; ++j) p_s[j][tid] = sc[j];
    __syncthreads();

    // online softmax statistics, one wave per head
    const int wave = tid >> 6, lane = tid & 63;
    for (int j = wave; j < nh; j += kThreads / 64) {
      float cm = -INFINITY;
      for (int i = lane; i < kChunk; i += 64) cm = fmaxf(cm, p_s[j][i]);
      cm = wave_max(cm);
      const float mn = fmaxf(m[j], cm);
      float sum = 0.0f;
      for (int i = lane; i < kChunk; i += 64) {
        const float p = mn == -INFINITY ? 0.0f : expf(p_s[j][i] - mn);
        p_s[j][i] = p;
        sum += p;
      }
      sum = wave_sum(sum);
      if (lane == 0) {
        stat_s[j][0] = mn;
        stat_s[j][1] = mn == -INFINITY ? 1.0f : expf(m[j] - mn);
        red_s[j] = sum;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      if (j < nh) {
        const float alpha = stat_s[j][1];
        m[j] = stat_s[j][0];
        l[j] = l[j] * alpha + red_s[j];
        acc[j] *= alpha;
      }
    }

    // values: thread owns channel c_own and every n_par-th token; value
    // channel c_own of token tv is code * scale + zero below n_vq, else the
    // fp16 window row
    const int64_t cend = (c0 + kChunk < s1) ? c0 + kChunk : s1;
    for (int64_t tv = c0 + par; tv < cend; tv += n_par) {
      float v;
      if (tv < rs.n_vq) {
        const uint32_t code = (L.value_codes(bh, tv)[vword] >> vsh) & vmsk;
        v = __fadd_rn(__fmul_rn((float)code, L.value_scale(bh, tv, vgrp)),
                      h2f(*L.value_zero(bh, tv, vgrp)));
      } else {
        v = h2f(a.v_res[(bh * a.R + tv % a.R) * D + c_own]);
      }
      const int i = (int)(tv - c0);
#pragma unroll
      for (int j = 0; j < NH; ++j) acc[j] = fmaf(p_s[j][i], v, acc[j]);
    }
    __syncthreads();
  }

  if constexpr (SCORES) return;
  // merge the n_par token parities of each channel, then write the partial
  for (int j = 0; j < nh; ++j) {
    red_s[tid] = acc[j];
    __syncthreads();
    if (tid < D) {
      float s = 0.0f;
      for (int p = 0; p < n_par; ++p) s += red_s[p * D + tid];
      float *dst = a.part + (((int64_t)b * a.Hq + hq0 + j) * a.S_total + slot_base + split) *
                                (int64_t)(D + 4);
      dst[tid] = s;
      if (tid == 0) {
        dst[D] = m[j];
        dst[D + 1] = l[j];
      }
    }
    __syncthreads();
  }
}

// Merge of two log-sum-exp partials (m, l, acc): the result has m = max of
// the two and both sums rescaled to it; an empty partial has m = -inf.
__device__ __forceinline__ void lse_merge(float &m, float &l, float4 &o, float m2, float l2,
                                          float4 o2) {
  const float mn = fmaxf(m, m2);
  const float f1 = m == -INFINITY ? 0.0f : __expf(m - mn);
  const float f2 = m2 == -INFINITY ? 0.0f : __expf(m2 - mn);
  l = l * f1 + l2 * f2;
  o.x = o.x * f1 + o2.x * f2;
  o.y = o.y * f1 + o2.y * f2;
  o.z = o.z * f1 + o2.z * f2;
  o.w = o.w * f1 + o2.w * f2;
  m = mn;
}

// grid: (B * Hq, ceil(D / 32)); block: 256.
// out = sum_s acc_s e^(m_s - M) / sum_s l_s e^(m_s - M), M = max_s m_s, over
// the S_total partial slots of one (batch row, query head).  Thread
// (slot group sg = 8 wave + lane / 8, channel quad cq = lane % 8) merges
// slots s = sg (mod 32) for 4 channels with a running maximum, loading up to
// 8 of its slots at once; the 8 slot groups of a wave merge through lane
// shuffles and the 4 waves through LDS.  A workgroup covers 32 channels, so
// most rows need one round trip to memory.
// With RAGGED, row b merges its first slots.n[b] slots (the partial stride
// stays S_total) and a row with none is skipped.
template <bool RAGGED>
__global__ void __launch_bounds__(256) combine_kernel(DecodeArgs a, RowArg<RAGGED> slots) {
  __shared__ float red_m[4][8];
  __shared__ float red_l[4][8];
  __shared__ float4 red_o[4][8];
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sg = wave * 8 + (lane >> 3), cq = lane & 7;
  int S = a.S_total;
  if constexpr (RAGGED) {
    S = slots.n[row / a.Hq];
    if (S == 0) return;   // the whole workgroup: S is uniform
  }
  const int D = a.D, stride = D + 4;
  const int c = blockIdx.y * 32 + cq * 4;
  const bool c_ok = c < D;               // D is a multiple of 8
  const float *p = a.part + row * a.S_total * (int64_t)stride;

  float M = -INFINITY, L = 0.0f;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = sg; s0 < S; s0 += 32 * 8) {
    float2 ml[8];
    float4 acc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + 32 * u;
      ml[u] = make_float2(-INFINITY, 0.0f);
      acc[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (s < S) {
        const float *ps = p + (int64_t)s * stride;
        ml[u] = *(const float2 *)(ps + D);
        if (c_ok) acc[u] = *(const float4 *)(ps + c);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (ml[u].x == -INFINITY) continue;
      lse_merge(M, L, o, ml[u].x, ml[u].y, acc[u]);
    }
  }
  // the 8 slot groups of this wave: lanes with the same channel quad
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(M, off), l2 = __shfl_xor(L, off);
    const float4 o2 = make_float4(__shfl_xor(o.x, off), __shfl_xor(o.y, off),
                                  __shfl_xor(o.z, off), __shfl_xor(o.w, off));
    lse_merge(M, L, o, m2, l2, o2);
  }
  if (lane < 8) {
    red_m[wave][lane] = M;
    red_l[wave][lane] = L;
    red_o[wave][lane] = o;
  }
  __syncthreads();
  if (threadIdx.x < 8 && c_ok) {
    M = red_m[0][cq];
    L = red_l[0][cq];
    o = red_o[0][cq];
#pragma unroll
    for (int w = 1; w < 4; ++w) lse_merge(M, L, o, red_m[w][cq], red_l[w][cq], red_o[w][cq]);
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    *(float4 *)(a.out + row * D + c) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  }
}

template <bool RAGGED, int MODE>
static void launch_generic(const DecodeArgs &a, dim3 grid, hipStream_t s, int64_t tok_begin,
                           int tps, int slot_base, int head_chunks, const RowArg<RAGGED> &rows) {
  if (a.n_rep == 1)
    hipLaunchKernelGGL((decode_generic_kernel<1, RAGGED, MODE>), grid, dim3(kThreads), 0, s, a,
                       tok_begin, tps, slot_base, head_chunks, rows);
  else if (a.n_rep == 2)
    hipLaunchKernelGGL((decode_generic_kernel<2, RAGGED, MODE>), grid, dim3(kThreads), 0, s, a,
                       tok_begin, tps, slot_base, head_chunks, rows);
  else if (a.n_rep <= 4)
    hipLaunchKernelGGL((decode_generic_kernel<4, RAGGED, MODE>), grid, dim3(kThreads), 0, s, a,
                       tok_begin, tps, slot_base, head_chunks, rows);
  else
    hipLaunchKernelGGL((decode_generic_kernel<kHeads, RAGGED, MODE>), grid, dim3(kThreads), 0,
                       s, a, tok_begin, tps, slot_base, head_chunks, rows);
}

hipError_t launch_decode_generic(const DecodeArgs &a, int64_t tok_begin, int tokens_per_split,
                                 int n_splits, int slot_base, hipStream_t s,
                                 const RowCounts *rows) {
  if (n_splits <= 0) return hipSuccess;
  if (rows && a.B > kMaxRows) return hipErrorInvalidValue;
  const int head_chunks = (a.n_rep + kHeads - 1) / kHeads;
  dim3 grid((unsigned)n_splits, (unsigned)(a.H * head_chunks), (unsigned)a.B);
  if (rows)
    launch_generic<true, 0>(a, grid, s, tok_begin, tokens_per_split, slot_base, head_chunks,
                                *rows);
  else
    launch_generic<false, 0>(a, grid, s, tok_begin, tokens_per_split, slot_base, head_chunks,
                                 NoRows{});
  return hipGetLastError();
}

hipError_t launch_selected_generic(const DecodeArgs &a, int tokens_per_split, int n_splits,
                                   hipStream_t s) {
  if (n_splits <= 0) return hipSuccess;
  if (!a.scores || !a.sel) return hipErrorInvalidValue;
  const int head_chunks = (a.n_rep + kHeads - 1) / kHeads;
  dim3 grid((unsigned)n_splits, (unsigned)(a.H * head_chunks), (unsigned)a.B);
  launch_generic<false, 2>(a, grid, s, 0, tokens_per_split, 0, head_chunks, NoRows{});
  return hipGetLastError();
}

hipError_t launch_scores_generic(const DecodeArgs &a, int tokens_per_split, int n_splits,
                                 hipStream_t s) {
  if (n_splits <= 0) return hipSuccess;
  if (!a.scores) return hipErrorInvalidValue;
  const int head_chunks = (a.n_rep + kHeads - 1) / kHeads;
  dim3 grid((unsigned)n_splits, (unsigned)(a.H * head_chunks), (unsigned)a.B);
  launch_generic<false, 1>(a, grid, s, 0, tokens_per_split, 0, head_chunks, NoRows{});
  return hipGetLastError();
}

hipError_t launch_combine(const DecodeArgs &a, hipStream_t s, const RowCounts *slots) {
  if (a.D % 8 != 0 || a.S_total <= 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(a.B * a.Hq), (unsigned)((a.D + 31) / 32));
  if (slots) {
    if (a.B > kMaxRows) return hipErrorInvalidValue;
    for (int b = 0; b < a.B; ++b)
      if (slots->n[b] < 0 || slots->n[b] > a.S_total) return hipErrorInvalidValue;
    hipLaunchKernelGGL((combine_kernel<true>), grid, dim3(256), 0, s, a, *slots);
  } else {
    hipLaunchKernelGGL((combine_kernel<false>), grid, dim3(256), 0, s, a, NoRows{});
  }
  return hipGetLastError();
}

}  // namespace kivi
