// decode_vector.hip -- vector-unit decode attention over the KIVI cache for
// head_dim 128, group size 32, 2- or 4-bit key and value codes and one or an
// even number of query heads per KV head (the MHA and 2-way GQA shapes, which
// give the matrix cores too little to do, and the 4-bit GQA shapes the matrix
// kernel does not take).
//
// Method source: web page "Literature audit -- Group 2 (KV-cache compression
// primary sources)", section "1. KIVI -- kivi2024", list "Core algorithm
// (implementation-grade)", item 5 (attention over quantized keys/values plus
// the fp16 window), item 4 (which tokens are quantized) and items 2-3
// (per-channel key groups, per-token value groups).
//
// Work split.  A workgroup (4 waves) owns a token range of one (batch row,
// KV head) slab and its NH query heads.  Wave w takes the 32-token groups
// w, w + 4, ... of the range and keeps its own online softmax (m, l, acc),
// so the token loop has no workgroup barrier; the four waves merge once at
// the end and write one (acc[128], m, l) partial for the split combine.
//
// Keys, per 32-token group: lane i owns channels 2i and 2i+1 and reads
// their codes for all 32 tokens with one or two 16-byte loads (the group's
// codes are one contiguous block of 128 channel rows).  For each 16-token
// half it forms 16 partial dot products (q_c s_c) code + q_c z_c over its
// two channels; a reduce-scatter across the 64 lanes (lane swaps for lane
// bits 5 and 4, DPP mirrors for bits 3 and 2, quad swaps for bits 1 and 0)
// leaves the score of token i >> 2 of the half in lane i.
//
// Values: lane i takes token i >> 2 of each half and channel quarter i & 3
// (32 channels, which are one value group: one scale and zero per token),
// reads the quarter's codes with one 8- or 16-byte load and accumulates
// p s code into 32 registers; the zero-point term p z is kept per lane and
// added once at the end.  The fp16 windows are read in the same lane
// layouts.
#include <math.h>

#include "kivi_internal.hpp"
#include "lane_ops.hpp"

namespace kivi {

namespace {

constexpr int kVD = 128;       // head_dim
constexpr int kVG = 32;        // group size (tokens of a key group, channels of a value group)
constexpr int kVWaves = 4;
constexpr int kVThreads = 64 * kVWaves;

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Bytes 0, 1 (HI false) or 2, 3 (HI true) of x, each holding a code 0..15,
// as floats.  Read as an fp8 E4M3 number, a byte c < 16 is c * 2^-9 (the
// subnormals and the first binade are evenly spaced), so the scaled
// conversion by 2^9 returns c exactly, two codes per instruction.
template <bool HI>
__device__ __forceinline__ f32x2 code_pair(uint32_t x) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8((int)x, 512.0f, HI);
}

// Codes of one 32-bit word as floats, code k (bits [BITS k, BITS k + BITS))
// in f[k].
template <int BITS>
__device__ __forceinline__ void unpack_word(uint32_t w, float (&f)[32 / BITS]) {
  if constexpr (BITS == 4) {
    // byte i of lo holds code 2i, byte i of hi code 2i + 1
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    const f32x2 a = code_pair<false>(lo), b = code_pair<true>(lo);
    const f32x2 c = code_pair<false>(hi), d = code_pair<true>(hi);
    f[0] = a.x; f[2] = a.y; f[4] = b.x; f[6] = b.y;
    f[1] = c.x; f[3] = c.y; f[5] = d.x; f[7] = d.y;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // byte i of m holds code 4i + r
      const uint32_t m = (w >> (2 * r)) & 0x03030303u;
      const f32x2 a = code_pair<false>(m), b = code_pair<true>(m);
      f[r] = a.x; f[4 + r] = a.y; f[8 + r] = b.x; f[12 + r] = b.y;
    }
  }
}

template <int N4>
__device__ __forceinline__ void load_words(const uint32_t *p, uint32_t *w) {
#pragma unroll
  for (int i = 0; i < N4; ++i) {
    const uint4 v = *(const uint4 *)(p + 4 * i);
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
}

// Reduce-scatter of the 16 per-lane partial sums v[e] (e = token of a
// 16-token half) over all 64 lanes: returns, in lane i, the sum over every
// lane of v[i >> 2].  Lane bit 5 picks token bit 3, lane bit 4 token bit 2
// (lane swaps), lane bits 3 and 2 token bits 1 and 0 (a row mirror and a
// half-row mirror pair each lane with one whose bit differs); the four lanes
// of a quad then hold partial sums of the same token and add up.
__device__ __forceinline__ float reduce_tokens(float (&v)[16], int lane) {
  lane_swap32x4(v[0], v[8], v[1], v[9], v[2], v[10], v[3], v[11]);
  lane_swap32x4(v[4], v[12], v[5], v[13], v[6], v[14], v[7], v[15]);
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] += v[i + 8];
  lane_swap16x4(v[0], v[4], v[1], v[5], v[2], v[6], v[3], v[7]);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] += v[i + 4];
  const bool b3 = lane & 8, b2 = lane & 4;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float x = b3 ? v[i + 2] : v[i], y = b3 ? v[i] : v[i + 2];
    v[i] = x + dpp_mov<0x140>(y);   // row mirror
  }
  {
    const float x = b2 ? v[1] : v[0], y = b2 ? v[0] : v[1];
    v[0] = x + dpp_mov<0x141>(y);   // half-row mirror
  }
  float r = v[0] + dpp_mov<0xB1>(v[0]);   // quad_perm [1, 0, 3, 2]
  return r + dpp_mov<0x4E>(r);            // quad_perm [2, 3, 0, 1]
}

__device__ __forceinline__ float wave_max_all(float v) { return group_max(row_max(v)); }
__device__ __forceinline__ float wave_sum_all(float v) { return group_sum(row_sum(v)); }

__device__ __forceinline__ float uniform(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

}  // namespace

// grid: (n_splits, H * head_chunks, B); block: 256 (4 waves).  A ragged
// batch (RAGGED): row b holds rows.n[b] tokens; a.t is the mask's row
// stride.
// MODE 1 (scores): only the scores s = q . K / sqrt(D) + mask of every
// token, into a.scores[(b Hq + hq) cap + tau] (no softmax, no values).
// MODE 2 (selected): attention whose scores are read from a.scores, with -inf
// for a token that the row's selection rule (a.sel) does not take; no keys
// are read.
template <int KB, int VB, int NH, bool RAGGED, int MODE, bool PAGED, bool S16>
__global__ void __launch_bounds__(kVThreads)
    __attribute__((amdgpu_waves_per_eu(2)))   // two waves per SIMD: the compiler may use 256 VGPRs
decode_vector_kernel(DecodeArgs a, int tokens_per_split, int head_chunks, int direct,
                     RowArg<RAGGED> rows) {
  constexpr bool SCORES = MODE == 1, SELECTED = MODE == 2;
  __shared__ float red_s[kVWaves][NH][kVD];
  __shared__ float stat_s[kVWaves][NH][2];

  constexpr int KPW = 32 / KB;   // key tokens per code word
  constexpr int KWH = KB / 2;    // key code words per channel and 16-token half
  constexpr int VPW = 32 / VB;   // value channels per code word
  constexpr int VWQ = VB;        // value code words per token and 32-channel quarter

  const int lane = threadIdx.x & 63;
  // wave-uniform, so that group indices and their branches stay scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int split = blockIdx.x;
  const int h = blockIdx.y / head_chunks;
  const int hc = blockIdx.y % head_chunks;
  const int b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.H + h;
  const int hq0 = h * a.n_rep + hc * NH;
  const int qd = lane & 3;    // value channels 32 qd .. 32 qd + 31 (one value group)
  const int tq = lane >> 2;   // token of each 16-token half this lane scores and accumulates

  // token and group indices within a slab fit 32 bits (cap < 2^26)
  RowSpan rs;
  if constexpr (RAGGED)
    rs = row_span(rows.n[b], a.R, false);
  else
    rs = RowSpan{a.t, a.n_kq, a.n_vq, -1};
  const int s0 = split * tokens_per_split;
  const int s1 = (int)min((int64_t)s0 + tokens_per_split, rs.t);
  const int g_end = (s1 + kVG - 1) / kVG;
  const int t_all = (int)rs.t, n_kq = (int)rs.n_kq, n_vq = (int)rs.n_vq, R = a.R;

  // q of channels 2 lane, 2 lane + 1, times 1/sqrt(D)
  float q0[NH], q1[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    const uint32_t qq = *(const uint32_t *)(a.q + ((int64_t)b * a.Hq + hq0 + j) * kVD + 2 * lane);
    q0[j] = h2f((uint16_t)(qq & 0xFFFFu)) * a.sm_scale;
    q1[j] = h2f((uint16_t)(qq >> 16)) * a.sm_scale;
  }

  float m[NH], lsum[NH], acc[NH][32], az[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    m[j] = -INFINITY;
    lsum[j] = 0.0f;
    az[j] = 0.0f;
#pragma unroll
    for (int c = 0; c < 32; ++c) acc[j][c] = 0.0f;
  }

  // Slab base pointer (wave-uniform, so it stays in scalar registers) and
  // 32-bit byte offsets: each load is a scalar base plus one 32-bit vector
  // offset, with no 64-bit address arithmetic per lane.  A 32-token group g
  // lies in record g / 4 of the slab, as its group g % 4; a slab's records
  // span less than 4 GB (decode_vector_supported).
  const Layout &L = a.L;
  const char *slab = (const char *)L.blocks + bh * L.nrec * L.rec;
  const uint32_t rec = (uint32_t)L.rec;
  const char *kres = (const char *)(a.k_res + bh * a.R * kVD);
  const char *vres = (const char *)(a.v_res + bh * a.R * kVD);
  // (selected attention: the mask is part of the stored scores)
  const char *mrow = a.mask && !SELECTED ? (const char *)(a.mask + (int64_t)b * a.t) : nullptr;
  SelectRow selr[NH];
  if constexpr (SELECTED) {
#pragma unroll
    for (int j = 0; j < NH; ++j) selr[j] = a.sel[(int64_t)b * a.Hq + hq0 + j];
  }
  const uint32_t kc_lane = (uint32_t)L.kc + (uint32_t)lane * (2 * KB) * 4u;
  // fp16-scale layout (S16): scales of 2 bytes, the sections after them
  // moved up
  const uint32_t ks_lane = (uint32_t)L.ks + (uint32_t)lane * (S16 ? 4u : 8u);
  const uint32_t kz_lane = (uint32_t)L.kz + (uint32_t)lane * 4u;
  const uint32_t kr_lane = (uint32_t)lane * 4u;
  const uint32_t vc_lane = (uint32_t)L.vc + (uint32_t)qd * VWQ * 4u;
  const uint32_t vs_lane = (uint32_t)L.vs + (uint32_t)qd * (kRecTokens * (S16 ? 2u : 4u));
  const uint32_t vz_lane = (uint32_t)L.vz + (uint32_t)qd * (kRecTokens * 2u);
  const uint32_t vr_lane = (uint32_t)qd * 64u;

  // The code, scale and zero words of a group (and the mask entries of the
  // lane's tokens) are loaded one group ahead, so their latency overlaps the
  // arithmetic of the group before.  The loads are unconditional: every
  // group below g_end lies inside the capacity (the words of a window group
  // are loaded and not used) and the mask index is clamped to the last token.
  // fp16 scales stay raw words until they are used, so that no fetch waits
  // for its own loads to widen them
  struct Raw {
    uint32_t kw[2 * KB];
    std::conditional_t<S16, uint32_t, float2> ks;
    float2 kz;
    uint32_t vw[2][VWQ];
    std::conditional_t<S16, uint32_t, float> vs[2];
    float vz[2], mk[2];
    float ss[SELECTED ? NH : 1][2];   // stored scores (selected attention)
  };
  // paged cache: the row's line of the page table and the head's record in
  // a page, set once.  The entries of 64 records from pg_first on sit one per
  // lane in pg_v (one vector load per 64 records); a record's entry is read
  // from its lane, so no fetch waits on a scalar load of the table.
  const int32_t *pg_row = PAGED ? L.pt + (int64_t)b * L.nrec : nullptr;
  const char *pg_base = PAGED ? (const char *)L.blocks + (int64_t)h * L.rec : nullptr;
  const int64_t pg_stride = (int64_t)a.H * L.rec;
  int pg_first = 0;
  int32_t pg_v = 0;
  auto pg_load = [&](int first) {
    pg_first = first;
    pg_v = pg_row[min(first + lane, (int)L.nrec - 1)];
  };
  if constexpr (PAGED) pg_load((s0 / kVG) >> 2);
  auto fetch = [&](int g, Raw &r) {
    // the group's record: an offset into the slab, or a page of a paged cache
    const char *recp = slab;
    uint32_t r0 = (uint32_t)(g >> 2) * rec;
    if constexpr (PAGED) {
      const int ri = g >> 2;
      if (ri - pg_first >= 64) pg_load(ri);
      int64_t p = __builtin_amdgcn_readlane(pg_v, ri - pg_first);
      p = p < 0 ? 0 : (p >= L.n_pages ? L.n_pages - 1 : p);
      recp = pg_base + p * pg_stride;
      r0 = 0u;
    }
    const uint32_t lg = (uint32_t)(g & 3);               // group within the record
    if constexpr (!SELECTED) {
      load_words<KB / 2>((const uint32_t *)(recp + (r0 + lg * (kVD * KB * 4u) + kc_lane)), r.kw);
      if constexpr (S16)
        r.ks = *(const uint32_t *)(recp + (r0 + lg * (kVD * 2u) + ks_lane));
      else
        r.ks = *(const float2 *)(recp + (r0 + lg * (kVD * 4u) + ks_lane));
      const uint32_t zz = *(const uint32_t *)(recp + (r0 + lg * (kVD * 2u) + kz_lane));
      r.kz = make_float2(h2f((uint16_t)(zz & 0xFFFFu)), h2f((uint16_t)(zz >> 16)));
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const uint32_t tl = lg * kVG + 16 * hh + tq;       // token within the record
      const uint32_t tau = (uint32_t)(g * kVG + 16 * hh + tq);
      if constexpr (SELECTED) {
        // groups below g_end lie inside the capacity, and so inside the row
#pragma unroll
        for (int j = 0; j < NH; ++j)
          r.ss[j][hh] = a.scores[((int64_t)b * a.Hq + hq0 + j) * a.cap + tau];
      } else {
        r.mk[hh] = mrow ? *(const float *)(mrow + (uint32_t)min((int)tau, t_all - 1) * 4u) : 0.0f;
      }
      if constexpr (SCORES) continue;
      const uint32_t *src = (const uint32_t *)(recp + (r0 + tl * (kVD * VB / 8u) + vc_lane));
      if constexpr (VWQ == 4) {
        const uint4 v = *(const uint4 *)src;
        r.vw[hh][0] = v.x;
        r.vw[hh][1] = v.y;
        r.vw[hh][2] = v.z;
        r.vw[hh][3] = v.w;
      } else {
        const uint2 v = *(const uint2 *)src;
        r.vw[hh][0] = v.x;
        r.vw[hh][1] = v.y;
      }
      if constexpr (S16)
        r.vs[hh] = *(const uint16_t *)(recp + (r0 + vs_lane + tl * 2u));
      else
        r.vs[hh] = *(const float *)(recp + (r0 + vs_lane + tl * 4u));
      r.vz[hh] = h2f(*(const uint16_t *)(recp + (r0 + vz_lane + tl * 2u)));
    }
  };

  // one 32-token group: scores, online softmax update, value accumulation
  auto process = [&](int gi, const Raw &cur) __attribute__((always_inline)) {
    const int t0 = gi * kVG;
    float sc[NH][2];
    if constexpr (SELECTED) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int tau = t0 + 16 * hh + tq;
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          const float sv = cur.ss[j][hh];
          sc[j][hh] = tau < s1 && select_takes(selr[j], sv, tau) ? sv : -INFINITY;
        }
      }
    } else {
      const bool quantized = t0 < n_kq;     // n_kq is a multiple of the group size
      float ksx, ksy;
      if constexpr (S16) {
        ksx = h2f((uint16_t)(cur.ks & 0xFFFFu));
        ksy = h2f((uint16_t)(cur.ks >> 16));
      } else {
        ksx = cur.ks.x;
        ksy = cur.ks.y;
      }
      float qs0[NH], qs1[NH], qz[NH];
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        qs0[j] = q0[j] * ksx;
        qs1[j] = q1[j] * ksy;
        qz[j] = fmaf(q1[j], cur.kz.y, q0[j] * cur.kz.x);
      }
      // fp16 key window: token tau sits in row tau mod R; R is a multiple of
      // the group size, so the group's tokens sit in consecutive rows
      const int row0 = quantized ? 0 : (int)((uint32_t)t0 % (uint32_t)R);

#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        float part[NH][16];
        if (quantized) {
#pragma unroll
          for (int j = 0; j < NH; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) part[j][e] = qz[j];
#pragma unroll
          for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
            for (int wi = 0; wi < KWH; ++wi) {
              float f[KPW];
              unpack_word<KB>(cur.kw[ch * KB + hh * KWH + wi], f);
#pragma unroll
              for (int k = 0; k < KPW; ++k)
#pragma unroll
                for (int j = 0; j < NH; ++j)
                  part[j][wi * KPW + k] =
                      fmaf(ch ? qs1[j] : qs0[j], f[k], part[j][wi * KPW + k]);
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int tau = t0 + 16 * hh + e;
            // rows past the split end are inside the window array; their
            // products are dropped
            const uint32_t kk =
                *(const uint32_t *)(kres + ((uint32_t)(row0 + 16 * hh + e) * (kVD * 2u) + kr_lane));
            const float k0 = tau < s1 ? h2f((uint16_t)(kk & 0xFFFFu)) : 0.0f;
            const float k1 = tau < s1 ? h2f((uint16_t)(kk >> 16)) : 0.0f;
#pragma unroll
            for (int j = 0; j < NH; ++j) part[j][e] = fmaf(q1[j], k1, q0[j] * k0);
          }
        }
        const bool valid = t0 + 16 * hh + tq < s1;
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          const float v = reduce_tokens(part[j], lane) + cur.mk[hh];
          sc[j][hh] = valid ? v : -INFINITY;
        }
      }
    }
    if constexpr (SCORES) {
      // every token's score sits in the four lanes of its tq; one writes it
      if ((lane & 3) == 0) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int tau = t0 + 16 * hh + tq;
          if (tau < s1) {
#pragma unroll
            for (int j = 0; j < NH; ++j)
              a.scores[((int64_t)b * a.Hq + hq0 + j) * a.cap + tau] = sc[j][hh];
          }
        }
      }
      return;
    }

    // online softmax of this wave over the group's 32 tokens
    float p[NH][2];
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      const float gmax = uniform(wave_max_all(fmaxf(sc[j][0], sc[j][1])));
      if (gmax > m[j]) {
        const float alpha = m[j] == -INFINITY ? 0.0f : __expf(m[j] - gmax);
        lsum[j] *= alpha;
        az[j] *= alpha;
#pragma unroll
        for (int c = 0; c < 32; ++c) acc[j][c] *= alpha;
        m[j] = gmax;
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) p[j][hh] = m[j] == -INFINITY ? 0.0f : __expf(sc[j][hh] - m[j]);
      lsum[j] += p[j][0] + p[j][1];
    }

    // values of token tq of each half, channels 32 qd .. 32 qd + 31
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int tau = t0 + 16 * hh + tq;
      if (tau < s1) {
        if (tau < n_vq) {
          float ps[NH];
          float vsc;
          if constexpr (S16)
            vsc = h2f((uint16_t)cur.vs[hh]);
          else
            vsc = cur.vs[hh];
#pragma unroll
          for (int j = 0; j < NH; ++j) {
            ps[j] = p[j][hh] * vsc;
            az[j] = fmaf(p[j][hh], cur.vz[hh], az[j]);
          }
#pragma unroll
          for (int wi = 0; wi < VWQ; ++wi) {
            float f[VPW];
            unpack_word<VB>(cur.vw[hh][wi], f);
#pragma unroll
            for (int k = 0; k < VPW; ++k)
#pragma unroll
              for (int j = 0; j < NH; ++j)
                acc[j][wi * VPW + k] = fmaf(ps[j], f[k], acc[j][wi * VPW + k]);
          }
        } else {
          const uint16_t *row =
              (const uint16_t *)(vres + (((uint32_t)tau % (uint32_t)R) * (kVD * 2u) + vr_lane));
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint4 v = *(const uint4 *)(row + 8 * i);
            const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float x0 = h2f((uint16_t)(vv[k] & 0xFFFFu));
              const float x1 = h2f((uint16_t)(vv[k] >> 16));
#pragma unroll
              for (int j = 0; j < NH; ++j) {
                acc[j][8 * i + 2 * k] = fmaf(p[j][hh], x0, acc[j][8 * i + 2 * k]);
                acc[j][8 * i + 2 * k + 1] = fmaf(p[j][hh], x1, acc[j][8 * i + 2 * k + 1]);
              }
            }
          }
        }
      }
    }
  };

  // two register sets alternate as the current group and the one ahead
  const int g_first = s0 / kVG + wave;
  Raw ra, rb;
  if (g_first < g_end) fetch(g_first, ra);
  for (int gi = g_first; gi < g_end;) {
    fetch(min(gi + kVWaves, g_end - 1), rb);
    process(gi, ra);
    gi += kVWaves;
    if (gi >= g_end) break;
    fetch(min(gi + kVWaves, g_end - 1), ra);
    process(gi, rb);
    gi += kVWaves;
  }
  if constexpr (SCORES) return;

  // Per wave: fold in the zero-point sum, then sum acc over the 16 token
  // lanes of each channel quarter (lane bits 5..2).  Bits 5 and 4 scatter
  // the 32 channels (lane swaps); bits 3 and 2 are summed whole (rotations
  // by 4 and 8 within a row), leaving channels 32 qd + 16 b5 + 8 b4 + i
  // (i < 8) in the four lanes of that (b5, b4, qd).
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    float *v = acc[j];
#pragma unroll
    for (int c = 0; c < 32; ++c) v[c] += az[j];
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      lane_swap32x4(v[i], v[i + 16], v[i + 1], v[i + 17], v[i + 2], v[i + 18], v[i + 3], v[i + 19]);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] += v[i + 16];
    lane_swap16x4(v[0], v[8], v[1], v[9], v[2], v[10], v[3], v[11]);
    lane_swap16x4(v[4], v[12], v[5], v[13], v[6], v[14], v[7], v[15]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float x = v[i] + v[i + 8];
      x += dpp_mov<0x124>(x);
      x += dpp_mov<0x128>(x);
      v[i] = x;
    }
    // lane bits 3..2 pick which two of the eight sums this lane stores
    const int base = 32 * qd + 16 * ((lane >> 5) & 1) + 8 * ((lane >> 4) & 1);
    const int k = (lane >> 2) & 3;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if ((i >> 1) == k) red_s[wave][j][base + i] = v[i];
    const float l_w = wave_sum_all(lsum[j]) * 0.25f;   // every token sits in four lanes
    if (lane == 0) {
      stat_s[wave][j][0] = m[j];
      stat_s[wave][j][1] = l_w;
    }
  }
  __syncthreads();

  // merge the four waves and write the partial (acc, m, l) of this split
  for (int i = threadIdx.x; i < NH * kVD; i += kVThreads) {
    const int j = i / kVD, c = i % kVD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kVWaves; ++w) M = fmaxf(M, stat_s[w][j][0]);
    float o = 0.0f, L = 0.0f;
#pragma unroll
    for (int w = 0; w < kVWaves; ++w) {
      const float mw = stat_s[w][j][0];
      const float f = mw == -INFINITY ? 0.0f : __expf(mw - M);
      o = fmaf(red_s[w][j][c], f, o);
      L = fmaf(stat_s[w][j][1], f, L);
    }
    if (direct) {
      // a single split: this is the whole softmax, normalized here
      a.out[((int64_t)b * a.Hq + hq0 + j) * kVD + c] = o * (L > 0.0f ? 1.0f / L : 0.0f);
    } else {
      float *dst =
          a.part + (((int64_t)b * a.Hq + hq0 + j) * a.S_total + split) * (int64_t)(kVD + 4);
      dst[c] = o;
      if (c == 0) {
        dst[kVD] = M;
        dst[kVD + 1] = L;
      }
    }
  }
}

bool decode_vector_supported(const DecodeArgs &a) {
  // 16-byte code loads (records and their sections are multiples of 16
  // bytes); q is read 4 bytes at a time; 32-bit offsets within a slab's
  // records and 32-bit token indices
  const bool aligned = ((uintptr_t)a.L.blocks & 15) == 0 && ((uintptr_t)a.v_res & 15) == 0 &&
                       ((uintptr_t)a.k_res & 3) == 0 && ((uintptr_t)a.q & 3) == 0;
  return a.D == kVD && a.G == kVG && (a.kb == 2 || a.kb == 4) && (a.vb == 2 || a.vb == 4) &&
         (a.n_rep == 1 || (a.n_rep % 2 == 0 && a.n_rep <= 64)) && a.R % kVG == 0 &&
         a.cap % kVG == 0 &&
         a.cap < ((int64_t)1 << 26) && a.L.nrec * a.L.rec < ((int64_t)1 << 32) && aligned;
}

// One query head per KV head: NH = 1.  An even number: NH = 2, and n_rep / 2
// workgroups per (split, slab), each for two of the heads (four heads in one
// workgroup would not fit two waves per SIMD).
template <int KB, int VB, bool RAGGED, int MODE, bool PAGED, bool S16>
static void launch_bits(const DecodeArgs &a, dim3 grid, int tps, int direct, hipStream_t s,
                        const RowArg<RAGGED> &rows) {
  if (a.n_rep == 1) {
    hipLaunchKernelGGL((decode_vector_kernel<KB, VB, 1, RAGGED, MODE, PAGED, S16>), grid, dim3(kVThreads),
                       0, s, a, tps, 1, direct, rows);
  } else {
    if constexpr (MODE == 1) {
      // scores only: no value accumulators, so one workgroup takes every
      // head of the KV head and reads its keys once
      if (a.n_rep == 4) {
        hipLaunchKernelGGL((decode_vector_kernel<KB, VB, 4, RAGGED, MODE, PAGED, S16>), grid,
                           dim3(kVThreads), 0, s, a, tps, 1, direct, rows);
        return;
      }
      if (a.n_rep == 8) {
        hipLaunchKernelGGL((decode_vector_kernel<KB, VB, 8, RAGGED, MODE, PAGED, S16>), grid,
                           dim3(kVThreads), 0, s, a, tps, 1, direct, rows);
        return;
      }
    }
    const int chunks = a.n_rep / 2;
    grid.y *= chunks;
    hipLaunchKernelGGL((decode_vector_kernel<KB, VB, 2, RAGGED, MODE, PAGED, S16>), grid, dim3(kVThreads),
                       0, s, a, tps, chunks, direct, rows);
  }
}

template <bool RAGGED, int MODE, bool PAGED, bool S16>
static void launch_bits_layout(const DecodeArgs &a, dim3 grid, int tps, int direct, hipStream_t s,
                               const RowArg<RAGGED> &rows) {
  if (a.kb == 2 && a.vb == 2)
    launch_bits<2, 2, RAGGED, MODE, PAGED, S16>(a, grid, tps, direct, s, rows);
  else if (a.kb == 2)
    launch_bits<2, 4, RAGGED, MODE, PAGED, S16>(a, grid, tps, direct, s, rows);
  else if (a.vb == 2)
    launch_bits<4, 2, RAGGED, MODE, PAGED, S16>(a, grid, tps, direct, s, rows);
  else
    launch_bits<4, 4, RAGGED, MODE, PAGED, S16>(a, grid, tps, direct, s, rows);
}

// A paged cache (PAGED) and the fp16-scale layout (S16) take their own
// instantiations, so that the contiguous fp32-scale ones keep their
// registers and schedule.
template <bool RAGGED, int MODE>
static void launch_all_bits(const DecodeArgs &a, dim3 grid, int tps, int direct, hipStream_t s,
                            const RowArg<RAGGED> &rows) {
  const bool s16 = a.L.sb == 2;
  if (a.L.pt) {
    if (s16)
      launch_bits_layout<RAGGED, MODE, true, true>(a, grid, tps, direct, s, rows);
    else
      launch_bits_layout<RAGGED, MODE, true, false>(a, grid, tps, direct, s, rows);
  } else {
    if (s16)
      launch_bits_layout<RAGGED, MODE, false, true>(a, grid, tps, direct, s, rows);
    else
      launch_bits_layout<RAGGED, MODE, false, false>(a, grid, tps, direct, s, rows);
  }
}

// With a single split (n_splits == 1) the kernel writes the normalized
// output itself and no combine pass is needed; otherwise it writes one
// partial per split.
hipError_t launch_decode_vector(const DecodeArgs &a, int tokens_per_split, int n_splits,
                                hipStream_t s, const RowCounts *rows) {
  if (n_splits <= 0) return hipSuccess;
  if (!decode_vector_supported(a) || tokens_per_split % kVG != 0) return hipErrorInvalidValue;
  if (rows && a.B > kMaxRows) return hipErrorInvalidValue;
  dim3 grid((unsigned)n_splits, (unsigned)a.H, (unsigned)a.B);
  const int direct = n_splits == 1;
  if (rows)
    launch_all_bits<true, 0>(a, grid, tokens_per_split, direct, s, *rows);
  else
    launch_all_bits<false, 0>(a, grid, tokens_per_split, direct, s, NoRows{});
  return hipGetLastError();
}

hipError_t launch_selected_vector(const DecodeArgs &a, int tokens_per_split, int n_splits,
                                  hipStream_t s) {
  if (n_splits <= 0) return hipSuccess;
  if (!decode_vector_supported(a) || tokens_per_split % kVG != 0 || !a.scores || !a.sel)
    return hipErrorInvalidValue;
  dim3 grid((unsigned)n_splits, (unsigned)a.H, (unsigned)a.B);
  launch_all_bits<false, 2>(a, grid, tokens_per_split, n_splits == 1, s, NoRows{});
  return hipGetLastError();
}

hipError_t launch_scores_vector(const DecodeArgs &a, int tokens_per_split, int n_splits,
                                hipStream_t s) {
  if (n_splits <= 0) return hipSuccess;
  if (!decode_vector_supported(a) || tokens_per_split % kVG != 0 || !a.scores)
    return hipErrorInvalidValue;
  dim3 grid((unsigned)n_splits, (unsigned)a.H, (unsigned)a.B);
  launch_all_bits<false, 1>(a, grid, tokens_per_split, 0, s, NoRows{});
  return hipGetLastError();
}

}  // namespace kivi
