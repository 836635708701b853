// decode_matrix.hip -- matrix-core (MFMA) decode attention over the packed
// KIVI cache, for 2-bit keys and values, group 32, head_dim 128 and 1, 2 or 4
// query heads per KV head.
//
// Method source: web page "Literature audit -- Group 2 (KV-cache compression
// primary sources)", section "1. KIVI -- kivi2024", list "Core algorithm
// (implementation-grade)", item 5: scores q.deq(K)^T over the quantized keys,
// softmax, then P.deq(V) over the quantized values.  This kernel covers the
// tokens whose key AND value are both quantized, in blocks of 128 tokens; the
// fp16 window and the ragged tail go to the scalar kernel, and the combine
// kernel merges both.
//
// Algebra.  With a key group's scale s and zero z (per channel c, 32 tokens),
//   q . K_tau = sum_c (q_c s_c) code_{c,tau} + sum_c q_c z_c,
// and for values (scale/zero per token tau and 32-channel group),
//   sum_tau p_tau V_{tau,c} = sum_tau (p_tau s_tau) code_{tau,c} + sum_tau p_tau z_tau.
// The first sums are dense contractions with small-integer codes, done on the
// matrix cores as fp16 x fp16 -> fp32 products.  Codes 0..3 are exact as fp16
// values; the fp32 factors (q s) and (p s) are split into an fp16 high part
// and an fp16 low part (the rounding residual), each multiplied in its own
// MFMA, which keeps about 22 significant bits.  The zero-point sums are plain
// fp32 dot products.
//
// Operand delivery.  The 2-bit codes are packed along tokens for keys and
// along channels for values, i.e. along the axis that is NOT contracted.  The
// gfx950 LDS transpose read (ds_read_b64_tr_b4) turns 16 rows of 64 bits into
// 16 columns of 4-bit nibbles across a 16-lane group, which puts a pair of
// codes per nibble exactly where the MFMA B operand wants it: a lane then
// holds, for one token (keys) or one channel (values), the codes of 16
// consecutive contraction indices.  Masking a dword with 0x00030003-style
// masks places two codes in the low mantissa bits of two fp16 halves, i.e. as
// the subnormal value code * 2^(pos - 24); the position factor 2^pos is taken
// out of the matching A element, and 2^-24 out of the result.
#include <math.h>

#include "kivi_internal.hpp"

namespace kivi {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef int i2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i2 lds_i2;
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = 128;
constexpr int kG = 32;
constexpr int kBT = 128;   // tokens per block
#ifndef KIVI_MATRIX_KEY_LO
#define KIVI_MATRIX_KEY_LO 1
#endif
#ifndef KIVI_MATRIX_VALUE_LO
#define KIVI_MATRIX_VALUE_LO 1
#endif

// One block of the packed cache, staged in LDS exactly as it sits in HBM
// (except the value scale/zero, gathered per channel group).
struct alignas(16) Stage {
  uint32_t kc[1024];   // 4 key groups x 128 channels x 2 words
  float ks[512];       // [4 groups][128 channels]
  float kz[512];
  uint32_t vc[1024];   // 128 tokens x 8 words
  float vs[512];       // [4 channel groups][128 tokens]
  float vz[512];
};


__device__ __forceinline__ void load_lds(const void *g, lds_void *l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
}

// Stage block `blk` (tokens [128 blk, 128 blk + 128)) of slab bh.
__device__ __forceinline__ void stage_block(const DecodeArgs &a, int64_t bh, int64_t blk,
                                           Stage *s, int lane) {
  const int64_t tau0 = blk * kBT;
  const int64_t g0 = tau0 / kG;
  const uint32_t *kc = a.k_codes + (bh * (a.cap / kG) + g0) * (kD * 2);
  const float *ks = a.k_scale + (bh * (a.cap / kG) + g0) * kD;
  const float *kz = a.k_zero + (bh * (a.cap / kG) + g0) * kD;
  const uint32_t *vc = a.v_codes + (bh * a.cap + tau0) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    load_lds(kc + i * 256 + lane * 4, (lds_void *)(s->kc + i * 256));
    load_lds(vc + i * 256 + lane * 4, (lds_void *)(s->vc + i * 256));
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    load_lds(ks + i * 256 + lane * 4, (lds_void *)(s->ks + i * 256));
    load_lds(kz + i * 256 + lane * 4, (lds_void *)(s->kz + i * 256));
    const int gch = 2 * i + (lane >> 5);
    const int64_t off = (bh * 4 + gch) * a.cap + tau0 + (lane & 31) * 4;
    load_lds(a.v_scale + off, (lds_void *)(s->vs + i * 256));
    load_lds(a.v_zero + off, (lds_void *)(s->vz + i * 256));
  }
}

__device__ __forceinline__ i2 tr4(const uint32_t *p) {
  return __builtin_amdgcn_ds_read_tr4_b64_v2i32((lds_i2 *)p);
}

// B operand from one transposed dword: even (low 2 bits of each nibble) and
// odd (high 2 bits, which come out 4x larger) halves.  Element 2r+e of the
// result holds nibble r+4e.
__device__ __forceinline__ void split_codes(uint32_t x, h8 &be, h8 &bo) {
  const uint32_t x8 = x >> 8;
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  u4 e = {x & 0x00030003u, x & 0x00300030u, x8 & 0x00030003u, x8 & 0x00300030u};
  u4 o = {x & 0x000C000Cu, x & 0x00C000C0u, x8 & 0x000C000Cu, x8 & 0x00C000C0u};
  be = __builtin_bit_cast(h8, e);
  bo = __builtin_bit_cast(h8, o);
}

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false)));
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false)));
  return v;
}

__device__ __forceinline__ float row_sum(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
  return v;
}

// The workgroup is a single wave, whose LDS accesses complete in order, so
// sharing data through LDS between its lanes needs only the wave's own LDS
// operations to finish -- not the memory fence of a workgroup barrier, which
// would also wait for the prefetch DMA in flight.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Wait for this wave's outstanding global->LDS copies.
__device__ __forceinline__ void wait_staged() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Sum over the 4 lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// hi/lo fp16 split of x*y: hi = rn16(x*y), lo = rn16(x*y - hi).
__device__ __forceinline__ void split_mul(float x, float y, _Float16 &hi, _Float16 &lo) {
  hi = (_Float16)(x * y);
  lo = (_Float16)__builtin_fmaf(x, y, -(float)hi);
}

}  // namespace

// grid: (n_split, H, B); block: one wave.  Split `split` covers tokens
// [split * tps, min(n_main, (split + 1) * tps)).
template <int NREP>
__global__ void __launch_bounds__(64)
decode_matrix_kernel(DecodeArgs a, int64_t n_main, int tps) {
  static_assert(NREP == 1 || NREP == 2 || NREP == 4, "query heads per KV head");
  constexpr int GA = 16 / NREP;       // key groups per A operand
  // Separate objects, so the compiler can tell that writes to the small
  // arrays never touch the stage buffer being filled by DMA.
  __shared__ Stage sm_st[2];
  __shared__ __attribute__((aligned(16))) float sm_p[4][kBT];   // probabilities, per head
  __shared__ __attribute__((aligned(16))) float sm_bias[16];
  __shared__ __attribute__((aligned(16))) float sm_zt[16];
  __shared__ __attribute__((aligned(16))) float sm_alpha[4];

  const int lane = threadIdx.x;
  const int i = lane & 15;
  const int kg = lane >> 4;
  const int split = blockIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.H + hk;
  const int64_t blk_begin = (int64_t)split * tps / kBT;
  int64_t blk_end = ((int64_t)split + 1) * tps / kBT;
  if (blk_end * kBT > n_main) blk_end = n_main / kBT;

  // --- roles of this lane
  // A operand of the key contraction: row m = i is (head h_a, group slot g_a)
  const int h_a = min(i / GA, NREP - 1);
  const int g_a = (i % GA) & 3;
  // A operand of the value contraction: row m = i is (head h_v, channel group c_v)
  const int h_v = min(i / 4, NREP - 1);
  const int c_v = i & 3;
  // score / output lanes: rows 4 kg .. 4 kg + 3 of the MFMA result
  const bool k_valid = (NREP == 4) || (NREP == 2 && (kg & 1) == 0) || (NREP == 1 && kg == 0);
  const int h_s = (kg * NREP) / 4;               // head of the scores this lane holds
  const bool v_valid = kg < NREP;                // head of the outputs this lane holds = kg

  // q of head h_a at this lane's 32 key channels, odd channels scaled by 1/16
  float qa[4][8];
  {
    const uint16_t *q = a.q + ((int64_t)b * a.Hq + hk * NREP + h_a) * kD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c0 = 64 * (ks >> 1) + 16 * kg + 8 * (ks & 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) qa[ks][j] = h2f(q[c0 + j]) * ((j & 1) ? 0.0625f : 1.0f);
    }
  }

  // The key-side A operand is q * s_k * 2^ek, with ek kept so that the
  // largest |q| times the block's largest key scale stays below 2^14 (no fp16
  // overflow for any fp16 input range).  qa carries the current 2^ek.
  float qmax = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) qmax = fmaxf(qmax, fabsf(qa[ks][j]) * ((j & 1) ? 16.0f : 1.0f));
  qmax = row_max(qmax);
  qmax = fmaxf(qmax, __shfl_xor(qmax, 16));
  qmax = fmaxf(qmax, __shfl_xor(qmax, 32));
  int ek_run = 0;

  const float LOG2E = 1.4426950408889634f;
  const float c_even = 16777216.0f * a.sm_scale * LOG2E;   // 2^24 / sqrt(D) * log2(e)
  const float c_odd = 0.25f * c_even;
  const float c_bias = a.sm_scale * LOG2E;

  // The value-side A operand is p * s_v * 2^ev, with the power of two ev set
  // per block from the block's largest value scale so that the fp16 split
  // stays in the normal range (p can be as small as 2^-20 and still matter).
  int ev_run = 0;
  float m_run = -INFINITY;     // running max (log2 units), head h_s
  float l_run = 0.0f;          // this lane's share of the running sum
  float zt_e = 0.0f, zt_o = 0.0f;   // value zero-point sums, row (h_v, c_v)
  f4 dv[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g) dv[g][0] = dv[g][1] = (f4){0, 0, 0, 0};

  if (blk_begin < blk_end) stage_block(a, bh, blk_begin, &sm_st[0], lane);

  for (int64_t blk = blk_begin; blk < blk_end; ++blk) {
    const int cur = (int)((blk - blk_begin) & 1);
    wait_staged();
    const Stage &st = sm_st[cur];
    // Transposed code reads first: the LDS transpose read carries no alias
    // information, so the compiler orders it behind every outstanding LDS
    // DMA; issuing the next block's DMA after these reads keeps it in flight
    // during the arithmetic below.
    i2 xk[4][2], xv[2][4];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int rho = 0; rho < 2; ++rho)
        xk[g][rho] = tr4(st.kc + g * 256 + (64 * rho + 16 * kg + i) * 2);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        xv[u][g] = tr4(st.vc + (32 * kg + 16 * u + i) * 8 + g * 2);
    // mask values of this lane's tokens, read before the DMA is issued (a
    // plain load would otherwise wait for the whole DMA to land)
    float mk[4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) mk[g][0] = mk[g][1] = 0.0f;
    if (a.mask) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float2 m2 = *(const float2 *)(a.mask + (int64_t)b * a.t + blk * kBT + 32 * g + 2 * i);
        mk[g][0] = m2.x * LOG2E;
        mk[g][1] = m2.y * LOG2E;
      }
    }
    // largest value scale of the block -> exponent ev for this block
    int ev;
    {
      const f4 v0 = *(const f4 *)(st.vs + lane * 8);
      const f4 v1 = *(const f4 *)(st.vs + lane * 8 + 4);
      float mx = fmaxf(fmaxf(fmaxf(v0[0], v0[1]), fmaxf(v0[2], v0[3])),
                       fmaxf(fmaxf(v1[0], v1[1]), fmaxf(v1[2], v1[3])));
      mx = row_max(mx);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // mx < 2^e with e = frexp exponent; p <= 1, so p * s * 2^(14 - e) < 2^14
      ev = mx > 0.0f ? 14 - __builtin_amdgcn_frexp_expf(mx) : 0;
      ev = __builtin_amdgcn_readfirstlane(ev);
    }
    {
      const f4 k0 = *(const f4 *)(st.ks + lane * 8);
      const f4 k1 = *(const f4 *)(st.ks + lane * 8 + 4);
      float mx = fmaxf(fmaxf(fmaxf(k0[0], k0[1]), fmaxf(k0[2], k0[3])),
                       fmaxf(fmaxf(k1[0], k1[1]), fmaxf(k1[2], k1[3])));
      mx = row_max(mx);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float prod = mx * qmax;
      int ek = prod > 0.0f ? 14 - __builtin_amdgcn_frexp_expf(prod) : ek_run;
      ek = __builtin_amdgcn_readfirstlane(ek);
      if (ek != ek_run) {
        const float f = __builtin_amdgcn_ldexpf(1.0f, ek - ek_run);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
          for (int j = 0; j < 8; ++j) qa[ks][j] *= f;
        ek_run = ek;
      }
    }
    if (blk + 1 < blk_end) stage_block(a, bh, blk + 1, &sm_st[cur ^ 1], lane);

    // ---- key side: A = hi/lo(q s), bias = q . z
    h8 ah[4], al[4];
    float be_e = 0.0f, be_o = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c0 = 64 * (ks >> 1) + 16 * kg + 8 * (ks & 1);
      const float *sp = st.ks + g_a * kD + c0;
      const float *zp = st.kz + g_a * kD + c0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int j = r + 4 * e;
          _Float16 hi, lo;
          split_mul(qa[ks][j], sp[j], hi, lo);
          ah[ks][2 * r + e] = hi;
          al[ks][2 * r + e] = lo;
          if (j & 1) be_o = fmaf(qa[ks][j], zp[j], be_o);
          else be_e = fmaf(qa[ks][j], zp[j], be_e);
        }
      }
    }
    float bias = group_sum(fmaf(16.0f, be_o, be_e));
    if (kg == 0) sm_bias[i] = bias;

    f4 dk[4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      dk[g][0] = dk[g][1] = (f4){0, 0, 0, 0};
#pragma unroll
      for (int rho = 0; rho < 2; ++rho) {
        const i2 x = xk[g][rho];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          h8 be, bo;
          split_codes((uint32_t)x[d], be, bo);
          const int ks = 2 * rho + d;
          dk[g][0] = mfma(ah[ks], be, dk[g][0]);
          if (KIVI_MATRIX_KEY_LO) dk[g][0] = mfma(al[ks], be, dk[g][0]);
          dk[g][1] = mfma(ah[ks], bo, dk[g][1]);
          if (KIVI_MATRIX_KEY_LO) dk[g][1] = mfma(al[ks], bo, dk[g][1]);
        }
      }
    }
    wave_lds_sync();

    // ---- scores and online softmax (lanes holding head h_s)
    if (k_valid) {
      const f4 bias4 = *(const f4 *)(sm_bias + 4 * kg);
      const float un = __builtin_amdgcn_ldexpf(1.0f, -ek_run);    // undo 2^ek
      float s2[4][2];
      float bmax = -INFINITY;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float bb = bias4[g] * (c_bias * un);
        s2[g][0] = fmaf(dk[g][0][g], c_even * un, bb);
        s2[g][1] = fmaf(dk[g][1][g], c_odd * un, bb);
        s2[g][0] += mk[g][0];
        s2[g][1] += mk[g][1];
        bmax = fmaxf(bmax, fmaxf(s2[g][0], s2[g][1]));
      }
      bmax = row_max(bmax);
      const float m_new = fmaxf(m_run, bmax);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      float lsum = 0.0f;
      const float sc_e = __builtin_amdgcn_ldexpf(1.0f, ev);        // 2^ev
      const float sc_o = __builtin_amdgcn_ldexpf(1.0f, ev - 4);    // odd tokens: / 16
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float p0 = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s2[g][0] - m_new);
        const float p1 = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s2[g][1] - m_new);
        lsum += p0 + p1;
        float2 pp = make_float2(p0 * sc_e, p1 * sc_o);
        *(float2 *)(&sm_p[h_s][32 * g + 2 * i]) = pp;
      }
      l_run = fmaf(l_run, alpha, lsum);
      m_run = m_new;
      if (i == 0) sm_alpha[h_s] = alpha;
    }
    wave_lds_sync();

    // ---- value side: A = hi/lo(p s), zero-point sums p . z
    {
      // accumulators are in units of 2^ev_run; move them to 2^ev
      const float rescale = __builtin_amdgcn_ldexpf(1.0f, ev - ev_run);
      ev_run = ev;
      const float av = (v_valid ? sm_alpha[kg] : 1.0f) * rescale;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        dv[g][0][g] *= av;
        dv[g][1][g] *= av;
      }
      const float ar = sm_alpha[h_v] * rescale;
      zt_e *= ar;
      zt_o *= ar;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      h8 vh[2], vl[2];
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int t0 = 32 * kg + 16 * u + 8 * d;
        const float *pp = &sm_p[h_v][t0];
        const float *sp = st.vs + c_v * kBT + t0;
        const float *zp = st.vz + c_v * kBT + t0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int j = r + 4 * e;
            _Float16 hi, lo;
            split_mul(pp[j], sp[j], hi, lo);
            vh[d][2 * r + e] = hi;
            vl[d][2 * r + e] = lo;
            if (j & 1) zt_o = fmaf(pp[j], zp[j], zt_o);
            else zt_e = fmaf(pp[j], zp[j], zt_e);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const i2 x = xv[u][g];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          h8 be, bo;
          split_codes((uint32_t)x[d], be, bo);
          dv[g][0] = mfma(vh[d], be, dv[g][0]);
          if (KIVI_MATRIX_VALUE_LO) dv[g][0] = mfma(vl[d], be, dv[g][0]);
          dv[g][1] = mfma(vh[d], bo, dv[g][1]);
          if (KIVI_MATRIX_VALUE_LO) dv[g][1] = mfma(vl[d], bo, dv[g][1]);
        }
      }
    }
  }

  // ---- write the partial (acc[128], m, l) of each query head
  const float zt = group_sum(fmaf(16.0f, zt_o, zt_e));
  if (kg == 0) sm_zt[i] = zt;
  const float l_head = row_sum(l_run);
  wave_lds_sync();
  const int slot_stride = kD + 2;
  if (v_valid) {
    const f4 z4 = *(const f4 *)(sm_zt + 4 * kg);
    float *dst = a.part + (((int64_t)b * a.Hq + hk * NREP + kg) * a.S_total + split) * slot_stride;
    const float unit = __builtin_amdgcn_ldexpf(1.0f, -ev_run);      // undo 2^ev
    const float ce = __builtin_amdgcn_ldexpf(1.0f, 24 - ev_run);    // and the code's 2^-24
    const float co = __builtin_amdgcn_ldexpf(1.0f, 22 - ev_run);    // odd channels came out 4x
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float2 o = make_float2(fmaf(dv[g][0][g], ce, z4[g] * unit),
                             fmaf(dv[g][1][g], co, z4[g] * unit));
      *(float2 *)(dst + 32 * g + 2 * i) = o;
    }
  }
  if (k_valid && i == 0) {
    float *dst = a.part + (((int64_t)b * a.Hq + hk * NREP + h_s) * a.S_total + split) * slot_stride;
    dst[kD] = m_run == -INFINITY ? -INFINITY : m_run * 0.6931471805599453f;
    dst[kD + 1] = l_head;
  }
}

bool decode_matrix_supported(const DecodeArgs &a) {
  return a.kb == 2 && a.vb == 2 && a.G == kG && a.D == kD &&
         (a.n_rep == 1 || a.n_rep == 2 || a.n_rep == 4);
}

hipError_t launch_decode_matrix(const DecodeArgs &a, int64_t n_main, int tokens_per_split,
                                int n_splits, hipStream_t s) {
  if (!decode_matrix_supported(a) || n_main % kBT != 0 || tokens_per_split % kBT != 0)
    return hipErrorInvalidValue;
  if (n_splits <= 0) return hipSuccess;
  dim3 grid((unsigned)n_splits, (unsigned)a.H, (unsigned)a.B);
  switch (a.n_rep) {
    case 1:
      hipLaunchKernelGGL(decode_matrix_kernel<1>, grid, dim3(64), 0, s, a, n_main, tokens_per_split);
      break;
    case 2:
      hipLaunchKernelGGL(decode_matrix_kernel<2>, grid, dim3(64), 0, s, a, n_main, tokens_per_split);
      break;
    default:
      hipLaunchKernelGGL(decode_matrix_kernel<4>, grid, dim3(64), 0, s, a, n_main, tokens_per_split);
      break;
  }
  return hipGetLastError();
}

}  // namespace kivi
