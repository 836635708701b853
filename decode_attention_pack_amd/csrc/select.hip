// select.hip -- token selection by attention mass on the packed cache, and
// attention over the selected tokens.
//
// Method source: web page "HCAttention: Extreme KV Cache Compression via
// Heterogeneous Attention Computing for LLMs" (a review of that paper),
// section "What carries the argument": Eq. (3) (approximate attention scores
// from quantized keys; here the KIVI scores q . K / sqrt(D) over the packed
// cache, KIVI item 5 of the page "Literature audit -- Group 2", section 1)
// and Eq. (4) (keep the smallest prefix of the tokens sorted by score whose
// mass reaches tau); the same review's major comment 2 on Eq. (5) (the
// output over the selected set, here renormalized).
//
// The selection of one (batch row, query head) row: the row's largest score,
// a histogram of token counts and probability masses over buckets of the
// distance to it, the bucket where the mass counted from the top reaches tau,
// then that bucket's tokens sorted by (score, index) in LDS.  A bucket too
// crowded to sort falls back to a radix select over the scores'
// order-preserving 32-bit keys in three passes (11, 11 and 10 bits).  Masses
// are e^(s - max) in fixed point (units of 2^-36, 64-bit integer sums), so
// the histograms, and with them the selection, do not depend on the order of
// the additions.  Equal scores are taken by increasing token index.  The
// scores come from the matrix, vector or scalar kernel's scores mode, and the
// attention over the selected tokens is the same kernel's selected-attention
// mode reading them back.
#include <math.h>

#include "kivi_internal.hpp"

namespace kivi {

namespace {

// 16 waves per row: each pass over a row's scores keeps up to eight 16-byte
// loads in flight per thread, so a 32k-token row is one round of loads.
constexpr int kSThreads = 1024;

// The score a key stands for (select_key's inverse).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// e^(s - m) in units of 2^-36: at most 2^36, so a row of up to 2^27 tokens
// sums in 64 bits.  A -inf score has mass 0.
__device__ __forceinline__ uint64_t fixed_mass(float s, float m) {
  return (uint64_t)rintf(expf(s - m) * 68719476736.0f);
}

// Inclusive scans over the threads of a workgroup (counts and masses).
__device__ __forceinline__ void block_scan(uint32_t &c, uint64_t &w, uint32_t *sc, uint64_t *sw) {
  const int tid = threadIdx.x;
  sc[tid] = c;
  sw[tid] = w;
  __syncthreads();
  for (int off = 1; off < kSThreads; off <<= 1) {
    const uint32_t c2 = tid >= off ? sc[tid - off] : 0u;
    const uint64_t w2 = tid >= off ? sw[tid - off] : 0u;
    __syncthreads();
    sc[tid] += c2;
    sw[tid] += w2;
    __syncthreads();
  }
  c = sc[tid];
  w = sw[tid];
  __syncthreads();
}

}  // namespace

// Rows whose crossing bucket holds more tokens than the sort list: the
// selection by radix passes over the score keys (select_rows_radix).
constexpr int kSortCap = 2048;
// Buckets of the score distance below the row's largest score, and the span
// they cover: a token more than kSpan below it has mass below e^-25.6
// (about 2^-37) of the largest and counts as mass zero.
constexpr int kNB = 4096;
constexpr float kSpan = 25.6f;

// Mass of a token scoring s in a row whose largest score is m.
__device__ __forceinline__ uint64_t token_mass(float s, float m) {
  return s - m >= -kSpan ? fixed_mass(s, m) : 0u;
}

// f(i, s) for every score s = sr[i], i < t, of a row (16-byte aligned):
// thread k takes the float4s k, k + kSThreads, ..., eight of them loaded
// before any is used, so that each thread keeps several loads in flight.
template <typename F>
__device__ __forceinline__ void for_scores(const float *sr, int t, F f) {
  const int tid = threadIdx.x;
  const int n4 = t / 4;
  const float4 *s4 = (const float4 *)sr;
  int v = tid;
  for (; v + 7 * kSThreads < n4; v += 8 * kSThreads) {
    float4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = s4[v + u * kSThreads];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = 4 * (v + u * kSThreads);
      f(i, x[u].x);
      f(i + 1, x[u].y);
      f(i + 2, x[u].z);
      f(i + 3, x[u].w);
    }
  }
  for (; v < n4; v += kSThreads) {
    const float4 x = s4[v];
    f(4 * v, x.x);
    f(4 * v + 1, x.y);
    f(4 * v + 2, x.z);
    f(4 * v + 3, x.w);
  }
  for (int i = 4 * n4 + tid; i < t; i += kSThreads) f(i, sr[i]);
}

// The radix selection of one row (kSThreads threads), given the row's largest
// score m and the mass to reach: three passes over the keys (11, 11, 10
// bits), each a histogram of counts and masses under the prefix fixed so
// far, then the ties at the threshold key by index.
__device__ SelectRow select_rows_radix(const float *sr, int t, float m, float tau,
                                       uint32_t *h_cnt, uint64_t *h_mass, uint32_t *s_c,
                                       uint64_t *s_w, uint32_t *s_u, uint64_t *s_u64) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0u, pmask = 0u;
  uint64_t need = 0u;
  uint32_t c_above = 0u, n_at = 0u;
  uint64_t w_at = 0u;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nb = pass == 2 ? 1024 : 2048;
    for (int i = tid; i < nb; i += kSThreads) {
      h_cnt[i] = 0u;
      h_mass[i] = 0u;
    }
    __syncthreads();
    for_scores(sr, t, [&](int, float s) {
      const uint64_t w = token_mass(s, m);
      const uint32_t k = select_key(s);
      if (w > 0u && (k & pmask) == prefix) {
        const uint32_t bkt = (k >> shift) & (uint32_t)(nb - 1);
        atomicAdd(&h_cnt[bkt], 1u);
        atomicAdd((unsigned long long *)&h_mass[bkt], (unsigned long long)w);
      }
    });
    __syncthreads();
    const int per = nb / kSThreads;   // thread k: buckets nb - per k - 1 down
    uint32_t c = 0u;
    uint64_t w = 0u;
    for (int i = 0; i < per; ++i) {
      c += h_cnt[nb - 1 - per * tid - i];
      w += h_mass[nb - 1 - per * tid - i];
    }
    const uint32_t c_own = c;
    const uint64_t w_own = w;
    block_scan(c, w, s_c, s_w);
    if (pass == 0) {
      const uint64_t total = s_w[kSThreads - 1];
      __syncthreads();
      need = tau >= 1.0f ? total : (uint64_t)ceil((double)tau * (double)total);
      need = need < 1u ? 1u : (need > total ? total : need);
    }
    const uint64_t w_before = w - w_own;
    if (w_before < need && need <= w) {
      uint32_t cb = c - c_own;
      uint64_t wb = w_before;
      for (int i = 0; i < per; ++i) {
        const int bkt = nb - 1 - per * tid - i;
        if (wb + h_mass[bkt] >= need) {
          s_u[0] = (uint32_t)bkt;
          s_u[1] = cb;
          s_u64[0] = wb;
          break;
        }
        cb += h_cnt[bkt];
        wb += h_mass[bkt];
      }
    }
    __syncthreads();
    const uint32_t bkt = s_u[0];
    need -= s_u64[0];
    c_above += s_u[1];
    prefix |= bkt << shift;
    pmask |= (uint32_t)(nb - 1) << shift;
    n_at = h_cnt[bkt];
    w_at = h_mass[bkt];
    __syncthreads();
  }
  // every token at the threshold key has the same mass; the first n_tie of
  // them in index order are selected
  const uint64_t w_one = w_at / n_at;
  const uint32_t n_tie = (uint32_t)((need + w_one - 1u) / w_one);
  int cut = 0x7FFFFFFF;
  if (n_tie < n_at) {
    const int per = (t + kSThreads - 1) / kSThreads;   // thread k: tokens [k per, (k + 1) per)
    const int i0 = tid * per, i1 = min(t, i0 + per);
    uint32_t c = 0u;
    for (int i = i0; i < i1; ++i) c += (select_key(sr[i]) == prefix) ? 1u : 0u;
    const uint32_t c_own = c;
    uint64_t unused = 0u;
    block_scan(c, unused, s_c, s_w);
    const uint32_t before = c - c_own;
    if (before < n_tie && n_tie <= c) {
      uint32_t k = before;
      for (int i = i0; i < i1; ++i) {
        if (select_key(sr[i]) == prefix && ++k == n_tie) {
          s_u[0] = (uint32_t)i;
          break;
        }
      }
    }
    __syncthreads();
    cut = (int)s_u[0];
    __syncthreads();
  }
  return SelectRow{prefix, cut, m, (int32_t)(c_above + n_tie)};
}

// grid: B * Hq rows; block: kSThreads.  Row r = b Hq + hq over a.t scores.
// 1. the row's largest score m; 2. a histogram of token counts and masses
// over kNB buckets of the distance m - s (bucket 0 the closest), and the
// bucket where the mass counted from the top reaches tau; 3. that bucket's
// tokens, sorted by score (then index) in LDS, and the prefix of them that
// completes the mass.  A score lower than another never lands in a lower
// bucket, so the tokens of the buckets above all precede the bucket's in
// the selection order.
// 4. (sel_mask) the row's selection bits, 32 tokens per word.
__global__ void __launch_bounds__(kSThreads)
select_rows_kernel(DecodeArgs a, float tau, SelectRow *rows, int32_t *n_selected,
                   uint32_t *sel_mask) {
  // the histograms (counts, masses) and, after them, the sort list share LDS
  __shared__ uint64_t h_mass[kNB];
  __shared__ uint32_t h_cnt[kNB];
  __shared__ uint32_t s_c[kSThreads];
  __shared__ uint64_t s_w[kSThreads];
  __shared__ float s_max[kSThreads / 64];
  __shared__ uint32_t s_u[4];
  __shared__ uint64_t s_u64[2];
  uint64_t *list = h_mass;   // (score key << 32 | ~index), after the histogram is read
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int t = (int)a.t;
  const float *sr = a.scores + row * a.cap;

  // the row's largest score: from the scores launch's per-wave maxima where
  // it recorded them, else from the row itself
  float m = -INFINITY;
  if (a.rmax) {
    for (int k = tid; k < a.rmax_n; k += kSThreads) m = fmaxf(m, a.rmax[row * a.rmax_n + k]);
  } else {
    for_scores(sr, t, [&](int, float s) { m = fmaxf(m, s); });
  }
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((tid & 63) == 0) s_max[tid >> 6] = m;
  __syncthreads();
  m = s_max[0];
#pragma unroll
  for (int w8 = 1; w8 < kSThreads / 64; ++w8) m = fmaxf(m, s_max[w8]);
  const int words = (t + 31) / 32;
  if (m == -INFINITY) {   // no token (t == 0) or every score -inf: nothing selected
    if (tid == 0) {
      rows[row] = SelectRow{0xFFFFFFFFu, -1, -INFINITY, 0};
      if (n_selected) n_selected[row] = 0;
    }
    if (sel_mask)
      for (int wd = tid; wd < words; wd += kSThreads) sel_mask[row * words + wd] = 0u;
    return;
  }
  const float inv_w = (float)kNB / kSpan;
  auto bucket_of = [&](float s) { return min(kNB - 1, (int)((m - s) * inv_w)); };

  for (int i = tid; i < kNB; i += kSThreads) {
    h_cnt[i] = 0u;
    h_mass[i] = 0u;
  }
  __syncthreads();
  for_scores(sr, t, [&](int, float s) {
    const uint64_t w = token_mass(s, m);
    if (w > 0u) {
      const int bkt = bucket_of(s);
      atomicAdd(&h_cnt[bkt], 1u);
      atomicAdd((unsigned long long *)&h_mass[bkt], (unsigned long long)w);
    }
  });
  __syncthreads();
  // thread k: buckets per k .. per k + per - 1 (closest first)
  constexpr int per = kNB / kSThreads;
  uint32_t c = 0u;
  uint64_t w = 0u;
  for (int i = 0; i < per; ++i) {
    c += h_cnt[per * tid + i];
    w += h_mass[per * tid + i];
  }
  const uint32_t c_own = c;
  const uint64_t w_own = w;
  block_scan(c, w, s_c, s_w);
  const uint64_t total = s_w[kSThreads - 1];
  __syncthreads();
  uint64_t need = tau >= 1.0f ? total : (uint64_t)ceil((double)tau * (double)total);
  need = need < 1u ? 1u : (need > total ? total : need);
  const uint64_t w_before = w - w_own;
  if (w_before < need && need <= w) {
    uint32_t cb = c - c_own;
    uint64_t wb = w_before;
    for (int i = 0; i < per; ++i) {
      const int bkt = per * tid + i;
      if (wb + h_mass[bkt] >= need) {
        s_u[0] = (uint32_t)bkt;
        s_u[1] = cb;
        s_u[2] = h_cnt[bkt];
        s_u64[0] = wb;
        break;
      }
      cb += h_cnt[bkt];
      wb += h_mass[bkt];
    }
  }
  __syncthreads();
  const int beta = (int)s_u[0];
  const uint32_t c_above = s_u[1], n_at = s_u[2];
  need -= s_u64[0];
  SelectRow res;
  if (n_at > (uint32_t)kSortCap) {
    // a crowded bucket (many near-equal scores): the radix passes
    __syncthreads();
    res = select_rows_radix(sr, t, m, tau, h_cnt, h_mass, s_c, s_w, s_u, s_u64);
  } else {
    // 3. the bucket's tokens into the list, padded to a power of two with
    // entries that sort last
    int n_pad = 1;
    while (n_pad < (int)n_at) n_pad <<= 1;
    if (tid == 0) s_u[3] = 0u;
    __syncthreads();
    for (int i = tid; i < n_pad; i += kSThreads) list[i] = 0u;
    __syncthreads();
    // (the bucket test first: the mass, an exponential, only for the few
    // tokens in the bucket -- it is zero only in the last, clamped bucket)
    for_scores(sr, t, [&](int i, float s) {
      if (bucket_of(s) == beta) {
        if (token_mass(s, m) > 0u) {
          const uint32_t slot = atomicAdd(&s_u[3], 1u);
          list[slot] = ((uint64_t)select_key(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
        }
      }
    });
    __syncthreads();
    // bitonic sort, descending: larger key first, then smaller index
    for (int k = 2; k <= n_pad; k <<= 1) {
      for (int j = k >> 1; j > 0; j >>= 1) {
        for (int i = tid; i < n_pad; i += kSThreads) {
          const int p = i ^ j;
          if (p > i) {
            const uint64_t x = list[i], y = list[p];
            const bool desc = (i & k) == 0;
            if (desc ? x < y : x > y) {
              list[i] = y;
              list[p] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    // the first entries whose masses reach `need`: a scan of the masses in
    // sorted order, per2 consecutive entries per thread
    const int per2 = (n_pad + kSThreads - 1) / kSThreads;
    uint32_t cnt = 0u;
    uint64_t acc = 0u;
    for (int i = tid * per2; i < min(n_pad, (tid + 1) * per2); ++i) {
      const uint64_t e = list[i];
      if (e != 0u) {
        ++cnt;
        acc += fixed_mass(key_score((uint32_t)(e >> 32)), m);
      }
    }
    const uint32_t cnt_own = cnt;
    const uint64_t acc_own = acc;
    block_scan(cnt, acc, s_c, s_w);
    const uint64_t before = acc - acc_own;
    if (before < need && need <= acc) {
      uint64_t run = before;
      uint32_t k = cnt - cnt_own;
      for (int i = tid * per2; i < min(n_pad, (tid + 1) * per2); ++i) {
        const uint64_t e = list[i];
        run += fixed_mass(key_score((uint32_t)(e >> 32)), m);
        ++k;
        if (run >= need) {
          s_u[0] = (uint32_t)(e >> 32);
          s_u[1] = 0xFFFFFFFFu - (uint32_t)e;
          s_u[2] = k;
          break;
        }
      }
    }
    __syncthreads();
    res = SelectRow{s_u[0], (int32_t)s_u[1], m, (int32_t)(c_above + s_u[2])};
  }
  if (tid == 0) {
    rows[row] = res;
    if (n_selected) n_selected[row] = res.count;
  }
  if (sel_mask) {
    for (int wd = tid; wd < words; wd += kSThreads) {
      uint32_t bits = 0u;
      for (int e = 0; e < 32 && 32 * wd + e < t; ++e)
        bits |= select_takes(res, sr[32 * wd + e], 32 * wd + e) ? 1u << e : 0u;
      sel_mask[row * words + wd] = bits;
    }
  }
}

hipError_t launch_select_rows(const DecodeArgs &a, float tau, SelectRow *rows,
                              int32_t *n_selected, uint32_t *sel_mask, hipStream_t s) {
  // rows of scores are read as float4s: 16-byte aligned rows
  if (!a.scores || !rows || a.t < 0 || a.t > a.cap || a.t >= ((int64_t)1 << 27) ||
      a.cap % 4 != 0 || ((uintptr_t)a.scores & 15) != 0 || !(tau > 0.0f && tau <= 1.0f))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(select_rows_kernel, dim3((unsigned)(a.B * a.Hq)), dim3(kSThreads), 0, s, a,
                     tau, rows, n_selected, sel_mask);
  return hipGetLastError();
}

}  // namespace kivi
