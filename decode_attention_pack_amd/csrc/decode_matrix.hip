// decode_matrix.hip -- matrix-core (MFMA) decode attention over the packed
// KIVI cache, for 2-bit keys and values, group 32, head_dim 128 and 1, 2 or 4
// query heads per KV head.
//
// Method source: web page "Literature audit -- Group 2 (KV-cache compression
// primary sources)", section "1. KIVI -- kivi2024", list "Core algorithm
// (implementation-grade)", item 5: scores q.deq(K)^T over the quantized keys,
// softmax, then P.deq(V) over the quantized values.  The matrix-core role of
// this kernel covers the tokens whose key AND value are both quantized, in
// whole blocks of 128 tokens; a second role, in the same launch, covers the
// rest (the fp16 window and the quantized tokens past the last whole block)
// with scalar arithmetic.  Each workgroup writes a partial (acc, m, l) and
// the combine kernel merges them.
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
// consecutive contraction indices.  A shift and an and-or place a code c in
// the top mantissa bits of an fp16 1.0, giving the exact normal value 1 + c/4
// (low code of a nibble) or 1 + c/16 (high code); a packed fp16 subtraction
// of 1 leaves c/4 or c/16, exact and normal (or zero).  Two encodings that
// skip the subtraction lose accuracy on the matrix core: codes as fp16
// subnormals (it keeps only ~14 bits when it adds the two products of one
// register whose B halves are subnormal), and 1 + c/4 with the sum of A
// removed afterwards (the large constant part cancels, and the rounding of
// the fp32 accumulation is magnified 4x and 16x).
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

// B operand from one transposed dword holding nibbles 0..7.  Element 2r+e of
// `be` is c/4 for the low code c of nibble r+4e, element 2r+e of `bo` is c/16
// for its high code (exact fp16 values).
__device__ __forceinline__ void split_codes(uint32_t x, h8 &be, h8 &bo) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  const uint32_t l8 = x << 8, l4 = x << 4, r4 = x >> 4, r8 = x >> 8;
  const uint32_t ONE = 0x3C003C00u, ME = 0x03000300u, MO = 0x00C000C0u;
  u4 e = {(l8 & ME) | ONE, (l4 & ME) | ONE, (x & ME) | ONE, (r4 & ME) | ONE};
  u4 o = {(l4 & MO) | ONE, (x & MO) | ONE, (r4 & MO) | ONE, (r8 & MO) | ONE};
  const h8 one = {1, 1, 1, 1, 1, 1, 1, 1};
  be = __builtin_bit_cast(h8, e) - one;
  bo = __builtin_bit_cast(h8, o) - one;
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

// hi/lo fp16 split of two products x0*y0, x1*y1 (one A-operand register):
// hi = the fp32 product truncated to fp16, lo = rn16(exact product - hi), so
// hi + lo carries ~21 significant bits.  hi comes from an intrinsic the
// compiler cannot re-derive: were the register's hi and the hi subtracted for
// lo rounded in two different ways, lo would carry their difference, a whole
// fp16 ulp, as error.
__device__ __forceinline__ void split_mul2(float x0, float y0, float x1, float y1, h8 &hi,
                                           h8 &lo, int k) {
  const auto h = __builtin_amdgcn_cvt_pkrtz(x0 * y0, x1 * y1);
  hi[k] = (_Float16)h[0];
  hi[k + 1] = (_Float16)h[1];
  lo[k] = (_Float16)__builtin_fmaf(x0, y0, -(float)h[0]);
  lo[k + 1] = (_Float16)__builtin_fmaf(x1, y1, -(float)h[1]);
}

}  // namespace

// grid: (n_split, H, B); block: one wave.  Split `split` covers tokens
// [split * tps, min(n_main, (split + 1) * tps)).
// LDS of the kernel.  Separate objects, so the compiler can tell that writes
// to the small arrays never touch the stage buffer being filled by DMA.
struct Lds {
  Stage *st;           // [2]
  float (*p)[kBT];     // [4][kBT] probabilities of the block, per query head
  float *bias;         // [16]: sum q z per A row
  float *zt;           // [16]: sum p z per A row
  float *alpha;        // [4]
  float (*q)[kD];      // [4][kD] (window role)
};

// Matrix-core role: split `split` covers the fully quantized tokens
// [split * tps, min(n_main, (split + 1) * tps)) in blocks of 128.
template <int NREP>
__device__ __forceinline__ void block_role(const DecodeArgs &a, int64_t n_main, int tps,
                                           int split, const Lds &L) {
  static_assert(NREP == 1 || NREP == 2 || NREP == 4, "query heads per KV head");
  constexpr int GA = 16 / NREP;       // key groups per A operand
  Stage *sm_st = L.st;
  float (*sm_p)[kBT] = L.p;
  float *sm_bias = L.bias;
  float *sm_zt = L.zt;
  float *sm_alpha = L.alpha;

  const int lane = threadIdx.x;
  const int i = lane & 15;
  const int kg = lane >> 4;
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
      for (int j = 0; j < 8; ++j) qa[ks][j] = h2f(q[c0 + j]);
    }
  }

  // The key-side A operand is q * s_k * 2^ek, with ek kept so that the
  // largest |q| times the block's largest key scale stays below 2^14 (no fp16
  // overflow for any fp16 input range).  qa carries the current 2^ek.
  float qmax = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) qmax = fmaxf(qmax, fabsf(qa[ks][j]));
  qmax = row_max(qmax);
  qmax = fmaxf(qmax, __shfl_xor(qmax, 16));
  qmax = fmaxf(qmax, __shfl_xor(qmax, 32));
  int ek_run = 0;

  const float LOG2E = 1.4426950408889634f;
  const float c_bias = a.sm_scale * LOG2E;                 // 1/sqrt(D) * log2(e)
  const float c_even = 4.0f * c_bias;                      // 1 + c/4 codes
  const float c_odd = 16.0f * c_bias;                      // 1 + c/16 codes

  // The value-side A operand is p * s_v * 2^ev, with the power of two ev set
  // per block from the block's largest value scale so that the fp16 split
  // stays in the normal range (p can be as small as 2^-20 and still matter).
  int ev_run = 0;
  float m_run = -INFINITY;     // running max (log2 units), head h_s
  float l_run = 0.0f;          // this lane's share of the running sum
  float zt = 0.0f;    // value zero-point sum  sum p' z, row (h_v, c_v)
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
    float bz = 0.0f;   // sum q z over this lane's channels
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c0 = 64 * (ks >> 1) + 16 * kg + 8 * (ks & 1);
      const float *sp = st.ks + g_a * kD + c0;
      const float *zp = st.kz + g_a * kD + c0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        split_mul2(qa[ks][r], sp[r], qa[ks][r + 4], sp[r + 4], ah[ks], al[ks], 2 * r);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int j = r + 4 * e;
          bz = fmaf(qa[ks][j], zp[j], bz);
        }
      }
    }
    // scores: even tokens 4 D 2^-ek + sum q z, odd tokens 16 D 2^-ek + sum q z
    // (qa, hence D and bz, carry 2^ek)
    bz = group_sum(bz);
    if (kg == 0) sm_bias[i] = bz;

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
      const f4 bz4 = *(const f4 *)(sm_bias + 4 * kg);
      const float un = __builtin_amdgcn_ldexpf(1.0f, -ek_run);    // undo 2^ek
      float s2[4][2];
      float bmax = -INFINITY;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float zb = bz4[g] * (c_bias * un);
        s2[g][0] = fmaf(dk[g][0][g], c_even * un, zb);
        s2[g][1] = fmaf(dk[g][1][g], c_odd * un, zb);
        s2[g][0] += mk[g][0];
        s2[g][1] += mk[g][1];
        bmax = fmaxf(bmax, fmaxf(s2[g][0], s2[g][1]));
      }
      bmax = row_max(bmax);
      const float m_new = fmaxf(m_run, bmax);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      float lsum = 0.0f;
      const float sc_e = __builtin_amdgcn_ldexpf(1.0f, ev);        // 2^ev
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float p0 = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s2[g][0] - m_new);
        const float p1 = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s2[g][1] - m_new);
        lsum += p0 + p1;
        float2 pp = make_float2(p0 * sc_e, p1 * sc_e);
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
      zt *= ar;
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
          split_mul2(pp[r], sp[r], pp[r + 4], sp[r + 4], vh[d], vl[d], 2 * r);
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const int j = r + 4 * e;
            zt = fmaf(pp[j], zp[j], zt);
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
  zt = group_sum(zt);
  if (kg == 0) {
    sm_zt[i] = zt;
  }
  const float l_head = row_sum(l_run);
  wave_lds_sync();
  const int slot_stride = kD + 2;
  if (v_valid) {
    const f4 z4 = *(const f4 *)(sm_zt + 4 * kg);
    float *dst = a.part + (((int64_t)b * a.Hq + hk * NREP + kg) * a.S_total + split) * slot_stride;
    const float unit = __builtin_amdgcn_ldexpf(1.0f, -ev_run);      // undo 2^ev
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      // even channels: 4 D + sum p z; odd channels: 16 D + sum p z
      float2 o = make_float2(fmaf(4.0f, dv[g][0][g], z4[g]) * unit,
                             fmaf(16.0f, dv[g][1][g], z4[g]) * unit);
      *(float2 *)(dst + 32 * g + 2 * i) = o;
    }
  }
  if (k_valid && i == 0) {
    float *dst = a.part + (((int64_t)b * a.Hq + hk * NREP + h_s) * a.S_total + split) * slot_stride;
    dst[kD] = m_run == -INFINITY ? -INFINITY : m_run * 0.6931471805599453f;
    dst[kD + 1] = l_head;
  }
}

// Window role: the tokens of one slab that the block role does not cover --
// the fp16 window and the quantized tokens past the last full block -- in
// chunks of 64: tokens [n_main + 64 chunk, min(t, n_main + 64 chunk + 64)).
// Everything the chunk needs is copied to LDS with one batch of DMA, then
// each lane scores one token (scalar fp32) and accumulates two channels.
template <int NREP>
__device__ __forceinline__ void window_role(const DecodeArgs &a, int64_t n_main, int chunk,
                                            int slot, const Lds &L) {
  const int j = threadIdx.x;
  const int hk = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t bh = (int64_t)b * a.H + hk;
  const int64_t Ta = n_main + 64 * (int64_t)chunk;
  const int64_t Tb = Ta + 64 < a.t ? Ta + 64 : a.t;
  const int n = (int)(Tb - Ta);
  const int64_t kq_end = a.n_kq < Ta ? Ta : (a.n_kq > Tb ? Tb : a.n_kq);
  const int64_t vq_end = a.n_vq < Ta ? Ta : (a.n_vq > Tb ? Tb : a.n_vq);
  const int n_qk = (int)(kq_end - Ta), n_fk = (int)(Tb - kq_end);   // n_qk in {0, 32, 64}
  const int n_qv = (int)(vq_end - Ta), n_fv = (int)(Tb - vq_end);
  const int nqg = n_qk / kG;
  const int nqv4 = (n_qv + 3) / 4;
  // 16-byte DMA units of each region, in LDS order
  const int u_krow = 0;
  const int u_kc = u_krow + n_fk * 16;
  const int u_ks = u_kc + nqg * 64;
  const int u_kz = u_ks + nqg * 32;
  const int u_vrow = u_kz + nqg * 32;
  const int u_vc = u_vrow + n_fv * 16;
  const int u_vs = u_vc + n_qv * 2;
  const int u_vz = u_vs + 4 * nqv4;
  const int u_end = u_vz + 4 * nqv4;           // <= 2048 units = 32 KB
  char *lds = (char *)L.st;
  for (int base = 0; base < u_end; base += 64) {
    const int u = base + j;
    if (u < u_end) {
      const void *src;
      if (u < u_kc) {
        const int r = u / 16, part = u % 16;
        src = a.k_res + ((bh * a.R + (kq_end + r) % a.R) * kD + part * 8);
      } else if (u < u_ks) {
        const int x = u - u_kc;
        src = a.k_codes + ((bh * (a.cap / kG) + Ta / kG + x / 64) * 256 + (x % 64) * 4);
      } else if (u < u_kz) {
        const int x = u - u_ks;
        src = a.k_scale + ((bh * (a.cap / kG) + Ta / kG + x / 32) * kD + (x % 32) * 4);
      } else if (u < u_vrow) {
        const int x = u - u_kz;
        src = a.k_zero + ((bh * (a.cap / kG) + Ta / kG + x / 32) * kD + (x % 32) * 4);
      } else if (u < u_vc) {
        const int x = u - u_vrow;
        src = a.v_res + ((bh * a.R + (vq_end + x / 16) % a.R) * kD + (x % 16) * 8);
      } else if (u < u_vs) {
        const int x = u - u_vc;
        src = a.v_codes + ((bh * a.cap + Ta + x / 2) * 8 + (x % 2) * 4);
      } else if (u < u_vz) {
        const int x = u - u_vs;
        src = a.v_scale + ((bh * 4 + x / nqv4) * a.cap + Ta + (x % nqv4) * 4);
      } else {
        const int x = u - u_vz;
        src = a.v_zero + ((bh * 4 + x / nqv4) * a.cap + Ta + (x % nqv4) * 4);
      }
      load_lds(src, (lds_void *)(lds + (size_t)base * 16));
    }
  }
  const uint16_t *q = a.q + ((int64_t)b * a.Hq + hk * NREP) * kD;
  for (int e = j; e < NREP * kD; e += 64) L.q[e / kD][e % kD] = h2f(q[e]);
  wait_staged();
  wave_lds_sync();

  const float LOG2E = 1.4426950408889634f;
  // ---- scores: lane j scores token Ta + j for every head
  float sc[NREP];
#pragma unroll
  for (int h = 0; h < NREP; ++h) sc[h] = 0.0f;
  if (j < n) {
    const int64_t tau = Ta + j;
    if (tau < kq_end) {
      const int gi = j / kG;
      const int e = (int)(tau % kG);
      const uint32_t *kc = (const uint32_t *)(lds + (size_t)u_kc * 16) + gi * 256 + e / 16;
      const float *ks = (const float *)(lds + (size_t)u_ks * 16) + gi * kD;
      const float *kz = (const float *)(lds + (size_t)u_kz * 16) + gi * kD;
      const int sh = 2 * (e % 16);
      for (int c = 0; c < kD; c += 4) {
        const f4 s4 = *(const f4 *)(ks + c);
        const f4 z4 = *(const f4 *)(kz + c);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float code = (float)((kc[(c + u) * 2] >> sh) & 3u);
          const float kh = __fadd_rn(__fmul_rn(code, s4[u]), z4[u]);
#pragma unroll
          for (int h = 0; h < NREP; ++h) sc[h] = fmaf(L.q[h][c + u], kh, sc[h]);
        }
      }
    } else {
      const uint16_t *row = (const uint16_t *)(lds + (size_t)u_krow * 16) + (tau - kq_end) * kD;
      for (int c = 0; c < kD; ++c) {
        const float kh = h2f(row[c]);
#pragma unroll
        for (int h = 0; h < NREP; ++h) sc[h] = fmaf(L.q[h][c], kh, sc[h]);
      }
    }
    const float mk = a.mask ? a.mask[(int64_t)b * a.t + tau] : 0.0f;
#pragma unroll
    for (int h = 0; h < NREP; ++h) sc[h] = (sc[h] * a.sm_scale + mk) * LOG2E;
  } else {
#pragma unroll
    for (int h = 0; h < NREP; ++h) sc[h] = -INFINITY;
  }
  // ---- softmax over the chunk, per head
  float mh[NREP], lh[NREP];
#pragma unroll
  for (int h = 0; h < NREP; ++h) {
    float m = row_max(sc[h]);
    m = fmaxf(m, __shfl_xor(m, 16));
    m = fmaxf(m, __shfl_xor(m, 32));
    const float pj = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[h] - m);
    L.p[h][j] = pj;
    mh[h] = m;
    lh[h] = group_sum(row_sum(pj));
  }
  wave_lds_sync();
  // ---- values: lane j owns channels 2j and 2j+1
  float o[NREP][2];
#pragma unroll
  for (int h = 0; h < NREP; ++h) o[h][0] = o[h][1] = 0.0f;
  const int c0 = 2 * j;
  const int gch = c0 / kG;
  const uint32_t *vc = (const uint32_t *)(lds + (size_t)u_vc * 16);
  const float *vs = (const float *)(lds + (size_t)u_vs * 16) + gch * nqv4 * 4;
  const float *vz = (const float *)(lds + (size_t)u_vz * 16) + gch * nqv4 * 4;
  const uint16_t *vrow = (const uint16_t *)(lds + (size_t)u_vrow * 16);
  for (int t = 0; t < n; ++t) {
    float v0, v1;
    if (t < n_qv) {
      const uint32_t w = vc[t * 8 + c0 / 16] >> (2 * (c0 % 16));
      v0 = __fadd_rn(__fmul_rn((float)(w & 3u), vs[t]), vz[t]);
      v1 = __fadd_rn(__fmul_rn((float)((w >> 2) & 3u), vs[t]), vz[t]);
    } else {
      const uint32_t hv = *(const uint32_t *)(vrow + (t - n_qv) * kD + c0);
      v0 = h2f((uint16_t)(hv & 0xFFFFu));
      v1 = h2f((uint16_t)(hv >> 16));
    }
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
      const float pt = L.p[h][t];
      o[h][0] = fmaf(pt, v0, o[h][0]);
      o[h][1] = fmaf(pt, v1, o[h][1]);
    }
  }
#pragma unroll
  for (int h = 0; h < NREP; ++h) {
    float *dst = a.part + (((int64_t)b * a.Hq + hk * NREP + h) * a.S_total + slot) * (kD + 2);
    *(float2 *)(dst + c0) = make_float2(o[h][0], o[h][1]);
    if (j == 0) {
      dst[kD] = mh[h] == -INFINITY ? -INFINITY : mh[h] * 0.6931471805599453f;
      dst[kD + 1] = lh[h];
    }
  }
}

// grid: (n_window + n_split, H, B); block: one wave.  Workgroups
// [0, n_window) take the window role (dispatched first, so they overlap the
// longer block role), the rest the block role.
template <int NREP>
__global__ void __launch_bounds__(64)
decode_matrix_kernel(DecodeArgs a, int64_t n_main, int tps, int n_split, int n_window) {
  __shared__ Stage sm_st[2];
  __shared__ __attribute__((aligned(16))) float sm_p[4][kBT];
  __shared__ __attribute__((aligned(16))) float sm_bias[16];
  __shared__ __attribute__((aligned(16))) float sm_zt[16];
  __shared__ __attribute__((aligned(16))) float sm_alpha[4];
  __shared__ __attribute__((aligned(16))) float sm_q[4][kD];
  const Lds L{sm_st, sm_p, sm_bias, sm_zt, sm_alpha, sm_q};
  const int x = blockIdx.x;
  if (x < n_window)
    window_role<NREP>(a, n_main, x, n_split + x, L);
  else
    block_role<NREP>(a, n_main, tps, x - n_window, L);
}

bool decode_matrix_supported(const DecodeArgs &a) {
  return a.kb == 2 && a.vb == 2 && a.G == kG && a.D == kD &&
         (a.n_rep == 1 || a.n_rep == 2 || a.n_rep == 4);
}

int decode_matrix_window_chunks(const DecodeArgs &a, int64_t n_main) {
  return (int)((a.t - n_main + 63) / 64);
}

hipError_t launch_decode_matrix(const DecodeArgs &a, int64_t n_main, int tokens_per_split,
                                int n_splits, hipStream_t s) {
  if (!decode_matrix_supported(a) || n_main % kBT != 0 || tokens_per_split % kBT != 0 ||
      n_main > a.n_vq)
    return hipErrorInvalidValue;
  const int n_window = decode_matrix_window_chunks(a, n_main);
  if (n_splits + n_window <= 0) return hipSuccess;
  if (n_splits + n_window > a.S_total) return hipErrorInvalidValue;
  dim3 grid((unsigned)(n_window + n_splits), (unsigned)a.H, (unsigned)a.B);
  switch (a.n_rep) {
    case 1:
      hipLaunchKernelGGL(decode_matrix_kernel<1>, grid, dim3(64), 0, s, a, n_main,
                         tokens_per_split, n_splits, n_window);
      break;
    case 2:
      hipLaunchKernelGGL(decode_matrix_kernel<2>, grid, dim3(64), 0, s, a, n_main,
                         tokens_per_split, n_splits, n_window);
      break;
    default:
      hipLaunchKernelGGL(decode_matrix_kernel<4>, grid, dim3(64), 0, s, a, n_main,
                         tokens_per_split, n_splits, n_window);
      break;
  }
  return hipGetLastError();
}

}  // namespace kivi
