// kivi_device.hpp -- device-side helpers shared by the KIVI HIP kernels.
//
// Method source: web page "Literature audit -- Group 2 (KV-cache compression
// primary sources)", section "1. KIVI -- kivi2024", list "Core algorithm
// (implementation-grade)" ("KIVI item N").
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace kivi {

__device__ __forceinline__ float h2f(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

// fp32 -> binary16 bit pattern, round to nearest even: exact for a value
// that is an fp16 value (a zero point, the minimum of fp16 inputs).
__device__ __forceinline__ uint16_t f2h_bits(float f) {
  return __half_as_ushort(__float2half_rn(f));
}

// Tokens per record of the packed store.
constexpr int kRecTokens = 128;

// The packed store of a cache (include/kivi.h): each (batch row, KV head)
// slab is a run of records, one per 128 tokens, each holding the key codes,
// key scales, key zeros (fp16), value codes, value scales and value zeros
// (fp16) of its tokens, in that order.  Section offsets are multiples of 16
// bytes.  Key groups (KIVI item 2, G tokens of one channel) and value groups
// (KIVI item 3, G channels of one token) both lie inside one record, since G
// divides 128.
// Paged cache (pt set): `blocks` is a pool of n_pages pages of H records (one
// per KV head), and record j of slab (b, h) is record h of page
// pt[b nrec + j].  A page index outside [0, n_pages) is clamped into the
// pool: a caller error, whose results are unspecified, never makes an access
// leave it.
// Scales are fp32, or binary16 in the fp16-scale layout (sb == 2), where the
// stored scale is s rounded to the nearest binary16 value and the codes are
// chosen for it (stored_scale).
struct Layout {
  uint8_t *blocks;
  int64_t rec;        // bytes per record
  int64_t nrec;       // records per slab (capacity / 128)
  int32_t kc, ks, kz, vc, vs, vz;   // section offsets in bytes
  int32_t D, G, kb, vb;
  int32_t sb;         // bytes per stored scale: 4, or 2 (fp16 scales)
  const int32_t *pt;  // page table [B][nrec] (device) or nullptr
  int64_t n_pages;
  int32_t H;          // KV heads: records per page

  // record of 128-token block j of slab bh
  __host__ __device__ __forceinline__ uint8_t *record_at(int64_t bh, int64_t j) const {
    if (pt == nullptr) return blocks + (bh * nrec + j) * rec;
    // batch x heads fits 16 bits (the ABI's limit): 32-bit division
    const uint32_t b = (uint32_t)bh / (uint32_t)H, h = (uint32_t)bh - b * (uint32_t)H;
    int64_t p = pt[(int64_t)b * nrec + j];
    p = p < 0 ? 0 : (p >= n_pages ? n_pages - 1 : p);
    return blocks + (p * H + (int64_t)h) * rec;
  }
  __host__ __device__ __forceinline__ uint8_t *record(int64_t bh, int64_t tau) const {
    return record_at(bh, tau / kRecTokens);
  }
  // key group g (tokens g G .. g G + G - 1) of channel c
  __host__ __device__ __forceinline__ int64_t key_index(int64_t g, int c) const {
    return ((g * G) % kRecTokens / G) * D + c;
  }
  __device__ __forceinline__ uint32_t *key_codes(int64_t bh, int64_t g, int c) const {
    return (uint32_t *)(record(bh, g * G) + kc) + key_index(g, c) * (G * kb / 32);
  }
  __device__ __forceinline__ float key_scale(int64_t bh, int64_t g, int c) const {
    const uint8_t *p = record(bh, g * G) + ks + key_index(g, c) * sb;
    return sb == 2 ? h2f(*(const uint16_t *)p) : *(const float *)p;
  }
  // element i of a run of stored scales starting at p
  __device__ __forceinline__ float scale_at(const uint8_t *p, int64_t i) const {
    return sb == 2 ? h2f(((const uint16_t *)p)[i]) : ((const float *)p)[i];
  }
  // the scales of key group g, channels 0 .. D-1 (a run for scale_at)
  __device__ __forceinline__ const uint8_t *key_scales(int64_t bh, int64_t g) const {
    return record(bh, g * G) + ks + key_index(g, 0) * sb;
  }
  // s: a stored_scale value (exact in the layout's precision)
  __device__ __forceinline__ void put_key_scale(int64_t bh, int64_t g, int c, float s) const {
    uint8_t *p = record(bh, g * G) + ks + key_index(g, c) * sb;
    if (sb == 2)
      *(uint16_t *)p = f2h_bits(s);
    else
      *(float *)p = s;
  }
  __device__ __forceinline__ uint16_t *key_zero(int64_t bh, int64_t g, int c) const {
    return (uint16_t *)(record(bh, g * G) + kz) + key_index(g, c);
  }
  // token tau: its code row, and the scale / zero of its channel group gc
  __device__ __forceinline__ uint32_t *value_codes(int64_t bh, int64_t tau) const {
    return (uint32_t *)(record(bh, tau) + vc) + (tau % kRecTokens) * (D * vb / 32);
  }
  __device__ __forceinline__ float value_scale(int64_t bh, int64_t tau, int gc) const {
    const uint8_t *p = record(bh, tau) + vs + (gc * kRecTokens + tau % kRecTokens) * sb;
    return sb == 2 ? h2f(*(const uint16_t *)p) : *(const float *)p;
  }
  __device__ __forceinline__ void put_value_scale(int64_t bh, int64_t tau, int gc,
                                                  float s) const {
    uint8_t *p = record(bh, tau) + vs + (gc * kRecTokens + tau % kRecTokens) * sb;
    if (sb == 2)
      *(uint16_t *)p = f2h_bits(s);
    else
      *(float *)p = s;
  }
  __device__ __forceinline__ uint16_t *value_zero(int64_t bh, int64_t tau, int gc) const {
    return (uint16_t *)(record(bh, tau) + vz) + gc * kRecTokens + tau % kRecTokens;
  }
};

// Section offsets and record size for a shape; rec = 0 if the layout does
// not take it (bits other than 2 and 4, G not dividing 128 or D).
inline Layout make_layout(uint8_t *blocks, int D, int kb, int vb, int G, int64_t cap,
                          bool scale_fp16 = false) {
  Layout L{};
  L.blocks = blocks;
  L.D = D;
  L.G = G;
  L.kb = kb;
  L.vb = vb;
  L.sb = scale_fp16 ? 2 : 4;
  const bool ok = (kb == 2 || kb == 4) && (vb == 2 || vb == 4) && G > 0 && D > 0 &&
                  kRecTokens % G == 0 && D % G == 0 && G % (32 / kb) == 0 &&
                  G % (32 / vb) == 0;
  if (!ok) return L;
  const int groups = kRecTokens / G;
  L.kc = 0;
  L.ks = L.kc + kRecTokens * D * kb / 8;
  L.kz = L.ks + groups * D * L.sb;
  L.vc = L.kz + groups * D * 2;
  L.vs = L.vc + kRecTokens * D * vb / 8;
  L.vz = L.vs + (D / G) * kRecTokens * L.sb;
  L.rec = L.vz + (D / G) * kRecTokens * 2;
  L.nrec = cap / kRecTokens;
  return L;
}

// Token accounting of a sequence holding t tokens (KIVI item 4): keys [0,
// n_kq) and values [0, n_vq) are in the records, the rest in the fp16
// window.  t_new >= 0 marks a launch that appends token t_new = t - 1 itself
// (the fused decode step); -1 a plain attention call.
struct RowSpan {
  int64_t t, n_kq, n_vq, t_new;
};
__host__ __device__ __forceinline__ RowSpan row_span(int64_t t, int R, bool appends) {
  RowSpan r;
  r.t = t;
  r.n_kq = t - t % R;
  r.n_vq = t > R ? t - R : 0;
  r.t_new = appends ? t - 1 : -1;
  return r;
}

// A ragged batch: batch row b holds its own token count.  Per-row tables
// travel in the kernel arguments of a launch (nothing is copied to the
// device), which bounds a ragged batch at kMaxRows rows.
constexpr int kMaxRows = 256;
struct RowCounts {
  int32_t n[kMaxRows];
};
struct NoRows {};
template <bool RAGGED>
using RowArg = typename std::conditional<RAGGED, RowCounts, NoRows>::type;

// Where token tau of one (batch, head) slab comes from when it is quantized:
// tokens below `t0` are read from the fp16 window `res` (slot tau % R); tokens
// from `t0` on are read from the caller's input `inp`, whose row 0 is token
// `t0`.  The pack entry points use only `inp`; append uses both.
struct TokenSource {
  const uint16_t *res;   // [BH][R][D] or nullptr
  const uint16_t *inp;   // [BH][n_inp][D]
  int64_t t0;            // first token held by `inp`
  int64_t n_inp;         // rows of `inp` per slab
  int32_t R;
  int32_t D;
  __device__ __forceinline__ const uint16_t *row(int64_t bh, int64_t tau) const {
    if (tau < t0) return res + (bh * R + tau % R) * (int64_t)D;
    return inp + (bh * n_inp + (tau - t0)) * (int64_t)D;
  }
};

// Group minimum and maximum with the rule of a sequential scan in element
// order: on ties the earlier element wins.  Values only tie with a
// different bit pattern for +0.0 / -0.0, where the stored zero point (and a
// constant group's scale) keeps the sign of the first zero, as in the fp32
// CPU reference.
__device__ __forceinline__ float first_min(float mn, float x) { return x < mn ? x : mn; }
__device__ __forceinline__ float first_max(float mx, float x) { return x > mx ? x : mx; }

// Group minimum and maximum of v[0..N) with the sequential rule, using the
// hardware min/max: they can differ from the sequential scan only when the
// result is a zero (+0.0 / -0.0 ties), and then the scan's answer is the
// first zero in element order, found by a second pass that rarely runs.
template <int N>
__device__ __forceinline__ void group_first_min_max(const float (&v)[N], float &mn, float &mx) {
  mn = v[0];
  mx = v[0];
#pragma unroll
  for (int i = 1; i < N; ++i) {
    mn = fminf(mn, v[i]);
    mx = fmaxf(mx, v[i]);
  }
  if (mn == 0.0f || mx == 0.0f) {
    float z = 0.0f;
    for (int i = N - 1; i >= 0; --i)
      if (v[i] == 0.0f) z = v[i];        // ends at the first zero
    if (mn == 0.0f) mn = z;
    if (mx == 0.0f) mx = z;
  }
}

// The same over aligned groups of `width` lanes (a power of two, at most 64)
// holding consecutive elements in lane order: a butterfly in which the lane
// block with the lower indices wins ties, so every lane ends with the result
// of the sequential scan.
__device__ __forceinline__ void lanes_first_min_max(float &mn, float &mx, int lane, int width) {
  for (int o = 1; o < width; o <<= 1) {
    const float pmn = __shfl_xor(mn, o), pmx = __shfl_xor(mx, o);
    if ((lane & o) == 0) {   // this lane's block comes first
      mn = pmn < mn ? pmn : mn;
      mx = pmx > mx ? pmx : mx;
    } else {
      mn = mn < pmn ? mn : pmn;
      mx = mx > pmx ? mx : pmx;
    }
  }
}

// KIVI item 1: the asymmetric round-to-nearest quantizer, bit-exact with an
// fp32 CPU reference.  s = (max - min) / (2^B - 1) uses IEEE fp32 division
// (the HIP default: correctly rounded), the code is round-half-to-even of
// (x - min) / s, clamped to [0, 2^B - 1]; s == 0 gives code 0.
__device__ __forceinline__ float group_scale(float mn, float mx, int bits) {
  return (mx - mn) / (float)((1 << bits) - 1);
}

// The scale a group stores and quantizes with: s, or in the fp16-scale
// layout s rounded to the nearest binary16 value (v_cvt_f16_f32: round to
// nearest even, subnormals kept); a scale that rounds to 0 gives all codes 0.
__device__ __forceinline__ float stored_scale(float s, const Layout &L) {
  return L.sb == 2 ? h2f(f2h_bits(s)) : s;
}

__device__ __forceinline__ uint32_t quant_code(float x, float z, float s, int bits) {
  if (s == 0.0f) return 0u;
  float r = rintf((x - z) / s);
  const float qmax = (float)((1 << bits) - 1);
  r = fminf(fmaxf(r, 0.0f), qmax);
  return (uint32_t)r;
}

// The same code as quant_code, with the division done once per group: r is
// v_rcp_f32(s) (relative error <= 2^-23).  q = (x - z) * r then lies within
// |(x - z) / s| * 2^-21.5 < 1e-5 of the correctly rounded quotient (the
// quotient is at most 15, or 22.5 with an fp16 scale rounded down from a
// subnormal value: 1.5 x 15), so both round to the same integer unless q is
// within 1e-5 of a half-integer; those rare elements take the exact IEEE
// division.
__device__ __forceinline__ uint32_t quant_code_r(float x, float z, float s, float r, int bits) {
  if (s == 0.0f) return 0u;
  const float u = x - z;
  float q = rintf(u * r);
  if (fabsf(u * r - q) > 0.49999f) q = rintf(u / s);
  const float qmax = (float)((1 << bits) - 1);
  q = fminf(fmaxf(q, 0.0f), qmax);
  return (uint32_t)q;
}

// quant_code_r over the n values of one group, with the same arithmetic: the
// near-tie test of every value comes first, and the division runs only in a
// lane that has a value near a tie, so the common path has no branch per
// value.
template <int N>
__device__ __forceinline__ void quant_codes_r(const float (&x)[N], float z, float s, float r,
                                              int bits, uint32_t (&c)[N]) {
  if (s == 0.0f) {
#pragma unroll
    for (int i = 0; i < N; ++i) c[i] = 0u;
    return;
  }
  float q[N];
  bool near = false;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float u = x[i] - z;
    q[i] = rintf(u * r);
    near = near || fabsf(u * r - q[i]) > 0.49999f;
  }
  if (near) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const float u = x[i] - z;
      if (fabsf(u * r - q[i]) > 0.49999f) q[i] = rintf(u / s);
    }
  }
  const float qmax = (float)((1 << bits) - 1);
#pragma unroll
  for (int i = 0; i < N; ++i) c[i] = (uint32_t)fminf(fmaxf(q[i], 0.0f), qmax);
}

}  // namespace kivi
