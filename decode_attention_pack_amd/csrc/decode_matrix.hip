// decode_matrix.hip -- matrix-core (MFMA) decode attention over the packed
// KIVI cache, for 2-bit keys and values, group 32, head_dim 128 and 1, 2 or 4
// query heads per KV head.
//
// Method source: web page "Literature audit -- Group 2 (KV-cache compression
// primary sources)", section "1. KIVI -- kivi2024", list "Core algorithm
// (implementation-grade)", item 5: scores q.deq(K)^T over the quantized keys,
// softmax, then P.deq(V) over the quantized values, plus the fp16 window.
//
// One launch does the whole call.  A workgroup of eight waves (one per CU,
// each wave with LDS of its own) takes a share of one (batch row, KV head)
// slab; its waves draw the share's work items from a counter in LDS:
//  * window chunks: the fp16 window and the quantized tokens past the last
//    whole block, 32 tokens each, scalar fp32 (drawn first);
//  * blocks: tokens whose key AND value are both quantized, 128 at a time,
//    on the matrix cores.
// Waves that issue faster (the oldest on a SIMD) take more items, so the
// share ends at about the same time on every wave.  Each wave writes a
// partial (acc[128], m, l) per query head for its blocks and one per window
// chunk; the combine kernel merges them with the log-sum-exp rule.
//
// Algebra.  With a key group's scale s and zero z (per channel c, 32 tokens),
//   q . K_tau = sum_c (q_c s_c) code_{c,tau} + sum_c q_c z_c,
// and for values (scale/zero per token tau and 32-channel group),
//   sum_tau p_tau V_{tau,c} = sum_tau (p_tau s_tau) code_{tau,c} + sum_tau p_tau z_tau.
// The first sums are dense contractions with small-integer codes, done on the
// matrix cores as fp16 x fp16 -> fp32 products.  The codes are exact fp16
// values; the fp32 factors (q s) and (p s) are split into an fp16 high part
// and an fp16 low part, each multiplied in its own MFMA, which keeps about 21
// significant bits.  The zero-point sums are plain fp32 dot products.
//
// Operand delivery.  The 2-bit codes are packed along tokens for keys and
// along channels for values, i.e. along the axis that is NOT contracted.  The
// gfx950 LDS transpose read (ds_read_b64_tr_b4) turns 16 rows of 64 bits into
// 16 columns of 4-bit nibbles across a 16-lane group, which puts a pair of
// codes per nibble exactly where the MFMA B operand wants it: a lane then
// holds, for one token pair (keys) or one channel pair (values), the codes of
// 16 consecutive contraction indices.  A nibble masked down to one code is an
// FP4 (E2M1) number of value code/2, and the gfx950 packed FP4 -> FP16
// conversion with scale 2 turns two such nibbles into two exact fp16 codes in
// one instruction.
//
// Memory pipeline.  A block's key part (codes, scales, zeros: 8 KB) and value
// part (8 KB) have one LDS buffer each per wave, filled by global->LDS DMA.
// The next block's key part is requested as soon as the current one has been
// read into registers, and likewise for the value part, so each DMA overlaps
// the other half's arithmetic.  With ~19 KB of LDS per wave, the eight waves
// (two per SIMD) of one workgroup fill a CU.
#include <math.h>

#include <type_traits>

#include "kivi_internal.hpp"
#include "lane_ops.hpp"

namespace kivi {

namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef int i2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kD = 128;
constexpr int kG = 32;
constexpr int kBT = 128;       // tokens per block (block role)
constexpr int kWT = 32;        // tokens per chunk (window role)
// A record of the packed store at this shape (KB-bit keys, VB-bit values, G
// 32, head_dim 128): byte offsets of its sections and its size, with fp32
// scales or (S16) fp16 scales; and the DMA instructions that copy the key or
// the value part of a block (codes 4 or 8 KB, scales 2 or 1 KB, zeros 1 KB).
template <bool S16, int KB = 2, int VB = KB>
struct Rec {
  static_assert((KB == 2 || KB == 4) && (VB == 2 || VB == 4), "2- or 4-bit codes");
  static constexpr int scale_bytes = S16 ? 1024 : 2048;
  static constexpr int kc = 0, ks = 2048 * KB;   // codes: 128 tokens x 128 channels
  static constexpr int kz = ks + scale_bytes;
  static constexpr int vc = kz + 1024;
  static constexpr int vs = vc + 2048 * VB;
  static constexpr int vz = vs + scale_bytes;
  static constexpr int bytes = vz + 1024;
  static constexpr int sb = S16 ? 2 : 4;    // bytes per scale
  // DMA instructions of the key and value codes, and of the key and value parts
  static constexpr int kncode = 2 * KB, vncode = 2 * VB;
  static constexpr int kdma = kncode + scale_bytes / 1024 + 1;
  static constexpr int vdma = vncode + scale_bytes / 1024 + 1;
};
constexpr int kPRow = 132;     // floats per probability row in LDS (16-byte pad)

// A block's key part and value part in LDS: codes as they sit in the
// record, the scale and zero rows rotated (see rot_chunk, zrot_off).  fp16
// scales fill the first half of ks / vs, rotated like the zeros.  The
// window role stages up to 8 KB in each (32 fp16 rows), hence the padding.
// The 4-bit stages hold twice the codes and are used by the block role only.
template <int BITS>
struct alignas(16) KStageT {
  uint32_t kc[512 * BITS];   // 4 key groups x 128 channels x BITS words
  float ks[512];             // [4 groups][128 channels]
  uint16_t kz[512];          // [4 groups][128 channels], fp16
  uint32_t pad[BITS == 2 ? 256 : 0];
};
template <int BITS>
struct alignas(16) VStageT {
  uint32_t vc[512 * BITS];   // 128 tokens x 4 BITS words
  float vs[512];             // [4 channel groups][128 tokens]
  uint16_t vz[512];          // [4 channel groups][128 tokens], fp16
  uint32_t pad[BITS == 2 ? 256 : 0];
};
using KStage = KStageT<2>;
using VStage = VStageT<2>;


// Global->LDS copies (16 or 4 bytes per lane; lane l's bytes land at LDS
// offset 16 l (4 l) from `l`).  They are written as inline assembly with the
// LDS address in M0, so that the compiler does not track them: it cannot
// tell which LDS buffer a copy fills, and would make every LDS read wait
// for all copies in flight, including those filling the other buffer.  The
// kernel waits for them itself (wait_vm), counting every vector-memory
// operation it issues.  The instructions have no result registers.  Each
// starts with five wait states, which the hardware needs between a VALU
// write of an SGPR (the readfirstlane of the base address) and a
// vector-memory read of it, and between an M0 write and an LDS DMA; the
// compiler inserts them for its own instructions but cannot see into
// inline assembly.
//   dma16:   per-lane 64-bit source address
//   dma16o:  uniform base + per-lane 32-bit byte offset (the base stays in
//            scalar registers)
//   dma16nt_m0: the same with the nontemporal hint and the LDS destination
//            given as a scalar LDS address, for the record stream: each
//            record is read once per call, and streaming it past the caches
//            measured ~13% more HBM bandwidth (6.6 against 5.85 TB/s for a
//            plain read of the records)
//   dma4o_m0: 4 bytes per lane, uniform base + offset
__device__ __forceinline__ uint32_t lds_m0(lds_void *l) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)l);
}
// A wave-uniform address, moved to scalar registers.
__device__ __forceinline__ const void *uniform_ptr(const void *p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void dma16(const void *g, lds_void *l) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds_m0(l))
               : "memory");
}
__device__ __forceinline__ void dma16o(const void *base, uint32_t off, lds_void *l) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "{m0}"(lds_m0(l))
               : "memory");
}
// The same copies with the LDS destination given as a wave-uniform LDS byte
// address (a scalar value, so that no per-copy move from vector registers
// or address-space check is needed).
__device__ __forceinline__ void dma16nt_m0(const void *base, uint32_t off, uint32_t m0) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(off), "s"(uniform_ptr(base)),
               "{m0}"(m0)
               : "memory");
}
__device__ __forceinline__ void dma4o_m0(const void *base, uint32_t off, uint32_t m0) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "{m0}"(m0)
               : "memory");
}
// LDS byte address of an LDS object reached through a generic pointer.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(lds_void *)p;
}

// Rows of 128 floats (a key group's scales or zeros over channels, a value
// channel group's scales or zeros over tokens) are stored in LDS rotated:
// 16-byte chunk k of row r sits at chunk (k + r) % 32.  Lanes that read the
// same columns of different rows then hit different LDS banks.
__device__ __forceinline__ int rot_chunk(int r, int k) { return (k + r) & 31; }
// float offset, within a block of four rows, of columns [c, c + 4) of row r
__device__ __forceinline__ int rot_off(int r, int c) { return r * 128 + rot_chunk(r, c >> 2) * 4; }
// Rows of 128 fp16 zeros (256 bytes) are rotated the same way over their 16
// chunks: the half offset of columns [c, c + 8) (c a multiple of 8) of row r.
__device__ __forceinline__ int zrot_off(int r, int c) { return r * 128 + (((c >> 3) + r) & 15) * 8; }

// Eight consecutive scales of a rotated row in LDS, as floats: columns [c, c
// + 8) of row r (c a multiple of 8) of fp32 rows (rot_off) or fp16 rows
// (zrot_off, widened exactly).
template <bool S16>
__device__ __forceinline__ void scales8(const float *rows, int r, int c, float (&sv)[8]) {
  if constexpr (S16) {
    const h8 s8 = *(const h8 *)((const uint16_t *)rows + zrot_off(r, c));
#pragma unroll
    for (int e = 0; e < 8; ++e) sv[e] = (float)s8[e];
  } else {
    const f4 s0 = *(const f4 *)(rows + rot_off(r, c));
    const f4 s1 = *(const f4 *)(rows + rot_off(r, c + 4));
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sv[e] = s0[e];
      sv[e + 4] = s1[e];
    }
  }
}

// The scale a group stores (KIVI item 1): s, or s rounded to the nearest
// binary16 value in the fp16-scale layout (the codes are chosen for it).
template <bool S16>
__device__ __forceinline__ float rec_scale(float s) {
  if constexpr (S16) return h2f(f2h_bits(s));
  return s;
}

// Per-lane byte offsets of the block DMA.  One DMA instruction fills two
// rotated rows of 128 floats (lanes 0-31 row 2i, lanes 32-63 row 2i + 1):
// lane l writes LDS chunk l % 32 of its row, so it reads source chunk
// (l % 32 - row) % 32.  One instruction fills the four rotated rows of 128
// fp16 zeros (16 lanes per row) the same way.
// lin: lane * 16 (unrotated runs); rot[i]: scale rows 2i, 2i + 1; zrot: the
// zero rows.
struct DmaOffsets {
  uint32_t lin;
  uint32_t rot[2];
  uint32_t zrot;
  __device__ DmaOffsets(int lane) : lin((uint32_t)lane * 16u) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = 2 * i + (lane >> 5);
      rot[i] = (uint32_t)(lane >> 5) * 512u + (uint32_t)((lane - row) & 31) * 16u;
    }
    const int zr = lane >> 4;
    zrot = (uint32_t)zr * 256u + (uint32_t)(((lane & 15) - zr) & 15) * 16u;
  }
};

// The value codes of a block sit in LDS with the 16-byte units of each token
// row (VB of them) permuted: unit h of row r at unit h ^ f(r), f(r) = (r /
// (16 / VB)) % VB.  The transposed reads of 16 consecutive rows then hit
// distinct banks (rows are 8 or 16 words apart, so unpermuted they meet in
// 8 or 4 bank groups).  The permutation is its own inverse: the copy that
// fills LDS unit l of a 1 KB piece reads unit vcode_unit(l) of the source,
// and the unit that holds source unit (r, h) is at LDS unit (r, h ^ f(r)).
template <int VB>
__host__ __device__ constexpr uint32_t vcode_unit(uint32_t l) {
  return l ^ ((l >> 4) & (uint32_t)(VB - 1));
}

// Per-lane source offsets of every copy of a block's key part and value
// part, counted from the start of the record (section offset included), so
// that all copies of a part share one scalar base address -- the record --
// and no per-copy address arithmetic runs.  Set once per wave.
template <bool S16, int KB = 2, int VB = KB>
struct PartOffsets {
  using RC = Rec<S16, KB, VB>;
  static constexpr int NK = RC::kdma, NV = RC::vdma, NCK = RC::kncode, NCV = RC::vncode;
  uint32_t k[NK], v[NV];
  __device__ explicit PartOffsets(const DmaOffsets &o) {
#pragma unroll
    for (int i = 0; i < NCK; ++i) k[i] = RC::kc + i * 1024 + o.lin;
#pragma unroll
    for (int i = 0; i < NCV; ++i) v[i] = RC::vc + i * 1024 + vcode_unit<VB>(o.lin >> 4) * 16u;
    if constexpr (S16) {
      k[NCK] = RC::ks + o.zrot;
      v[NCV] = RC::vs + o.zrot;
    } else {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        k[NCK + i] = RC::ks + i * 1024 + o.rot[i];
        v[NCV + i] = RC::vs + i * 1024 + o.rot[i];
      }
    }
    k[NK - 1] = RC::kz + o.zrot;
    v[NV - 1] = RC::vz + o.zrot;
  }
};

// Start of record `blk` (tokens [128 blk, 128 blk + 128)) of slab bh.
// A paged cache (PAGED) finds it through the page table: record h of page
// pt[b nrec + blk], the page index clamped into the pool.  The paged form is
// a separate instantiation so that the contiguous one keeps its registers.
template <bool PAGED, bool S16, int KB = 2, int VB = KB>
__device__ __forceinline__ const uint8_t *record_of(const DecodeArgs &a, int64_t bh, int64_t blk) {
  constexpr int64_t RB = Rec<S16, KB, VB>::bytes;
  if constexpr (!PAGED) {
    return a.L.blocks + (bh * a.L.nrec + blk) * RB;
  } else {
    const uint32_t b = (uint32_t)bh / (uint32_t)a.H, h = (uint32_t)bh - b * (uint32_t)a.H;
    int64_t p = a.L.pt[(int64_t)b * a.L.nrec + blk];
    p = p < 0 ? 0 : (p >= a.L.n_pages ? a.L.n_pages - 1 : p);
    return a.L.blocks + (p * a.H + h) * RB;
  }
}

// Key part of block `blk` (tokens [128 blk, 128 blk + 128)) of slab bh:
// Rec<S16, KB, VB>::kdma DMA instructions, plus 2 for the mask when there is
// one.  s, mask_s: LDS byte addresses of the wave's KStageT and mask buffer.
template <bool MASKED, bool PAGED, bool S16, int KB = 2, int VB = KB>
__device__ __forceinline__ void stage_keys(const DecodeArgs &a, int64_t bh, int64_t blk,
                                           uint32_t s, uint32_t mask_s,
                                           const PartOffsets<S16, KB, VB> &o, int lane) {
  using KS = KStageT<KB>;
  constexpr int NC = PartOffsets<S16, KB, VB>::NCK;
  const void *rec = uniform_ptr(record_of<PAGED, S16, KB, VB>(a, bh, blk));
  constexpr uint32_t kc = offsetof(KS, kc), ks = offsetof(KS, ks), kz = offsetof(KS, kz);
#pragma unroll
  for (int i = 0; i < NC; ++i) dma16nt_m0(rec, o.k[i], s + kc + i * 1024);
  if constexpr (S16) {
    dma16nt_m0(rec, o.k[NC], s + ks);   // four rows of 128 fp16 scales
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16nt_m0(rec, o.k[NC + i], s + ks + i * 1024);
  }
  dma16nt_m0(rec, o.k[PartOffsets<S16, KB, VB>::NK - 1], s + kz);
  if (MASKED) {
    // dword copies: a mask row need not be 16-byte aligned
    const float *m = a.mask + (bh / a.H) * a.t + blk * kBT;
    dma4o_m0(m, (uint32_t)lane * 4u, mask_s);
    dma4o_m0(m + 64, (uint32_t)lane * 4u, mask_s + 256);
  }
}

// Value part of block `blk`: Rec<S16, KB, VB>::vdma DMA instructions.
// s: LDS byte address of the wave's VStageT.
template <bool PAGED, bool S16, int KB = 2, int VB = KB>
__device__ __forceinline__ void stage_values(const DecodeArgs &a, int64_t bh, int64_t blk,
                                             uint32_t s, const PartOffsets<S16, KB, VB> &o) {
  using VS = VStageT<VB>;
  constexpr int NC = PartOffsets<S16, KB, VB>::NCV;
  const void *rec = uniform_ptr(record_of<PAGED, S16, KB, VB>(a, bh, blk));
  constexpr uint32_t vc = offsetof(VS, vc), vs = offsetof(VS, vs), vz = offsetof(VS, vz);
#pragma unroll
  for (int i = 0; i < NC; ++i) dma16nt_m0(rec, o.v[i], s + vc + i * 1024);
  if constexpr (S16) {
    dma16nt_m0(rec, o.v[NC], s + vs);
  } else {
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16nt_m0(rec, o.v[NC + i], s + vs + i * 1024);
  }
  dma16nt_m0(rec, o.v[PartOffsets<S16, KB, VB>::NV - 1], s + vz);
}

// Selected attention (mode 2): the stored scores of block `blk` for the
// NREP query heads of KV head hk (rows of 128 fp32 at a.scores + (b Hq +
// hk NREP + h) cap + 128 blk) into the wave's key buffer ([NREP][128]):
// ceil(NREP / 2) copies of 1 KB, lane l taking 16 bytes of row l / 32 (the
// last row again past NREP rows).
template <int NREP>
__device__ __forceinline__ void stage_scores(const DecodeArgs &a, int b, int hk, int64_t blk,
                                             uint32_t s, int lane) {
#pragma unroll
  for (int c = 0; c < (NREP + 1) / 2; ++c) {
    // base: row 2c (uniform); lanes 32-63 add one row stride for row 2c + 1
    const float *row = a.scores + ((int64_t)b * a.Hq + hk * NREP + 2 * c) * a.cap + blk * kBT;
    const uint32_t second = 2 * c + 1 < NREP && lane >= 32 ? 1u : 0u;
    dma16nt_m0(row, second * (uint32_t)a.cap * 4u + (uint32_t)(lane & 31) * 16u, s + c * 1024);
  }
}
// DMA instructions of stage_scores.
template <int NREP>
constexpr int kScoreDma = (NREP + 1) / 2;

// LDS transpose read, issued as inline assembly: the compiler's builtin for it
// carries no information on which LDS object it reads, so the compiler would
// wait for every DMA in flight (into either buffer) before it.  Its result is
// only valid after wait_regs() on it.
__device__ __forceinline__ i2 tr4(const uint32_t *p) {
  i2 r;
  const uint32_t addr = (uint32_t)(uintptr_t)(lds_void *)p;
  asm volatile("ds_read_b64_tr_b4 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

// The four 16-byte pieces of q a lane uses (byte offsets 0, 16, 128, 144 from
// p in LDS), read as inline assembly for the same reason as tr4, and waited
// for before returning.
__device__ __forceinline__ void q_reads(const uint16_t *p, uint4 (&w)[4]) {
  const uint32_t addr = (uint32_t)(uintptr_t)(lds_void *)p;
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:16\n\t"
      "ds_read_b128 %2, %4 offset:128\n\t"
      "ds_read_b128 %3, %4 offset:144\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(w[0]), "=&v"(w[1]), "=&v"(w[2]), "=&v"(w[3])
      : "v"(addr)
      : "memory");
}

// Wait for this wave's LDS reads, including those whose results are in
// x[0..7] (so that their buffer may be refilled after this point).
__device__ __forceinline__ void wait_lds8(float (&x)[8]) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                 "+v"(x[6]), "+v"(x[7])::"memory");
}

// Wait for this wave's LDS reads, including the transpose reads whose
// results are in x[0..N).
template <int N>
__device__ __forceinline__ void wait_regs(i2 (&x)[N]) {
  static_assert(N == 8 || N == 16, "8 or 16 transposed reads");
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                 "+v"(x[6]), "+v"(x[7])::"memory");
  if constexpr (N == 16)
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]),
                   "+v"(x[14]), "+v"(x[15])::"memory");
}

// B operands from one transposed dword holding nibbles 0..7 (two codes
// each): element n of `be` is the low code of nibble n, element n of `bo`
// its high code, as exact fp16 integers 0..3.
__device__ __forceinline__ void codes_to_b(uint32_t x, h8 &be, h8 &bo) {
  const uint32_t lo = x & 0x33333333u;
  const uint32_t hi = (x >> 2) & 0x33333333u;
  const h2v e0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 2.0f, 0);
  const h2v e1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 2.0f, 1);
  const h2v e2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 2.0f, 2);
  const h2v e3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(lo, 2.0f, 3);
  const h2v o0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 2.0f, 0);
  const h2v o1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 2.0f, 1);
  const h2v o2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 2.0f, 2);
  const h2v o3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(hi, 2.0f, 3);
  be = (h8){e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
  bo = (h8){o0[0], o0[1], o1[0], o1[1], o2[0], o2[1], o3[0], o3[1]};
}

// B operand from one transposed dword holding nibbles 0..7, one 4-bit code
// each.  A byte 0..15 read as FP8 E4M3 is code * 2^-9, and the gfx950 packed
// FP8 -> FP16 conversion with scale 2^9 returns the exact fp16 code, two per
// instruction.  The bytes of x & 0x0F0F0F0F are nibbles 0, 2, 4, 6 and those
// of (x >> 4) & 0x0F0F0F0F nibbles 1, 3, 5, 7, so element e of the operand
// is the code of nibble perm4(e); the A operand is built in the same order
// (the contraction index order within one MFMA is free).
__device__ __forceinline__ h8 codes4_to_b(uint32_t x) {
  const uint32_t ev = x & 0x0F0F0F0Fu;
  const uint32_t od = (x >> 4) & 0x0F0F0F0Fu;
  const h2v e0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ev, 512.0f, false);
  const h2v e1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ev, 512.0f, true);
  const h2v o0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(od, 512.0f, false);
  const h2v o1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(od, 512.0f, true);
  return (h8){e0[0], e0[1], e1[0], e1[1], o0[0], o0[1], o1[0], o1[1]};
}
__host__ __device__ constexpr int perm4(int e) { return e < 4 ? 2 * e : 2 * (e - 4) + 1; }
// Contraction index of element e of a B operand built from 8 nibbles.
template <int BITS>
__host__ __device__ constexpr int k_order(int e) { return BITS == 2 ? e : perm4(e); }

__device__ __forceinline__ f4 mfma(h8 a, h8 b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The workgroup is a single wave, whose LDS accesses complete in order, so
// sharing data through LDS between its lanes needs only the wave's own LDS
// operations to finish -- not the memory fence of a workgroup barrier, which
// would also wait for the DMA in flight.
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Wait until at most N of this wave's vector-memory operations (DMA
// included) are outstanding; they complete in issue order.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// hi/lo fp16 split of two products x0*y0, x1*y1 into elements k, k+1:
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

// LDS of the kernel.  Separate objects, so the compiler can tell that LDS
// accesses of the arithmetic never touch a buffer being filled by DMA.
struct Lds {
  KStage *ks;          // key part of the block (window role: its key staging)
  VStage *vs;          // value part (window role: its value staging)
  float (*p)[kPRow];   // [4][kPRow] probabilities of the block (window role: q)
  float *mask;         // [128] mask of the block (window role: probabilities)
  float *bias;         // [16] per A row: sum q z (keys), then sum p z (values)
  float *alpha;        // [4]
};

// The workgroup's waves take their work -- window chunks first, then blocks
// -- from a counter in LDS: item = the counter's value before the wave's
// add.  Faster waves take more items, which evens out the differences in
// issue share between the waves of a CU.  Lane 0 adds; every lane gets the
// item.
__device__ __forceinline__ int draw_item(int *ctr, int lane) {
  int v = 0;
  if (lane == 0) v = atomicAdd(ctr, 1);
  return __builtin_amdgcn_readfirstlane(v);
}

// The blocks of one workgroup: block index j (0 <= j < nb) stands for block
// b0 + (j + rot) % nb of the slab; the counter's item n_skip + j is block j.
// Block indices within a slab fit 32 bits (capacity < 2^26 tokens).
struct BlockShare {
  int b0, nb, rot;
  int n_skip;
  int *ctr;
  // block of the slab that index j (0 <= j < nb, rot < nb) stands for
  __device__ __forceinline__ int block(int j) const {
    const int x = j + rot;
    return b0 + (x >= nb ? x - nb : x);
  }
};

// Matrix-core role: blocks of the workgroup's share (tokens whose key and
// value are both quantized, 128 per block), starting with block `first` and
// continuing with the blocks the wave draws, accumulated into one partial
// per query head, left in the wave's probability buffer: row h holds acc[128]
// of head h, then m (natural-log units) and l.
// MODE 1 (scores): only the key half; the score q . K / sqrt(D) + mask of
// every token of the blocks goes to a.scores[(b Hq + hq) cap + tau] (no
// softmax, no values, no partial).
// MODE 2 (selected attention): the key half is replaced by the block's
// stored scores (copied into the key buffer), -inf for the tokens the row's
// selection rule (a.sel) does not take; then the softmax and values as in
// MODE 0.  The mask is part of the stored scores.
// KB / VB 4 (4-bit keys / values, attention only): a transposed read holds
// one code per nibble, so a key tile of 16 columns is 16 consecutive tokens
// (2-bit: 16 token pairs, split into even and odd tiles) and a value tile 16
// consecutive channels.  Index e of the score and accumulator pairs below is
// then that half of the key group or of the channel group instead of the
// token or channel parity.
template <int NREP, bool MASKED, bool PAGED, bool S16, int MODE, int KB = 2, int VB = KB>
__device__ __forceinline__ void block_role(const DecodeArgs &a, const BlockShare &sh,
                                           int64_t first, int hk, int b, const Lds &L,
                                           KStageT<KB> *__restrict__ kbuf,
                                           VStageT<VB> *__restrict__ vbuf, int mslot = 0) {
  static_assert(NREP == 1 || NREP == 2 || NREP == 4, "query heads per KV head");
  static_assert(MODE != 2 || !MASKED, "selected attention takes the mask from the scores");
  static_assert((KB == 2 && VB == 2) || MODE == 0, "4-bit codes: attention only");
  constexpr int GA = 16 / NREP;       // key groups per A operand
  using RC = Rec<S16, KB, VB>;
  // token of score pair element e of key group g held by lane i
  auto tok = [](int g, int e, int i) { return KB == 2 ? 32 * g + 2 * i + e : 32 * g + 16 * e + i; };
  // copies of a block's key part (MODE 2: its scores) and value part
  constexpr int KDMA = MODE == 2 ? kScoreDma<NREP> : RC::kdma + (MASKED ? 2 : 0);
  constexpr int VDMA = MODE == 1 ? 0 : RC::vdma;

  const int lane = threadIdx.x & 63;
  const int i = lane & 15;
  const int kg = lane >> 4;
  const int64_t bh = (int64_t)b * a.H + hk;
  // LDS byte addresses of the wave's staging buffers, as scalar values
  const uint32_t k_lds = __builtin_amdgcn_readfirstlane(lds_addr(kbuf));
  const uint32_t v_lds = __builtin_amdgcn_readfirstlane(lds_addr(vbuf));
  const uint32_t mask_lds = __builtin_amdgcn_readfirstlane(lds_addr(L.mask));
  if (first >= sh.nb) {
    // no block for this wave: an empty partial (m = -inf)
    if (MODE != 1 && lane < NREP) *(float2 *)&L.p[lane][kD] = make_float2(-INFINITY, 0.0f);
    if (MODE == 1 && a.rmax && lane < NREP)
      a.rmax[((int64_t)b * a.Hq + hk * NREP + lane) * a.rmax_n + mslot] = -INFINITY;
    return;
  }

  // --- roles of this lane
  // key A operand: row m = i is (head h_a, key group g_a)
  const int h_a = min(i / GA, NREP - 1);
  const int g_a = (i % GA) & 3;
  // value A operand: row m = i is (head h_v, channel group c_v)
  const int h_v = min(i / 4, NREP - 1);
  const int c_v = i & 3;
  // score / output lanes: rows 4 kg .. 4 kg + 3 of the MFMA result
  const bool k_valid = (NREP == 4) || (NREP == 2 && (kg & 1) == 0) || (NREP == 1 && kg == 0);
  const int h_s = (kg * NREP) / 4;               // head of the scores this lane holds
  const bool v_valid = kg < NREP;                // head of the outputs this lane holds = kg

  // q of the NREP heads (NREP rows of 256 bytes, contiguous) is copied into
  // the probability buffer by the first DMA, ahead of the first block's
  // copies; the copies complete in order, so waiting for q alone lets the
  // block stream in meanwhile.  Lanes past the q rows re-read the last 16
  // bytes.
  const PartOffsets<S16, KB, VB> dmo{DmaOffsets(lane)};
  const uint16_t *q_lds = (const uint16_t *)&L.p[0][0];
  int64_t cur = sh.block((int)first);   // the block being processed
  if constexpr (MODE != 2)
    dma16o(a.q + ((int64_t)b * a.Hq + hk * NREP) * kD, (uint32_t)min(lane, NREP * 16 - 1) * 16u,
           (lds_void *)&L.p[0][0]);
  if constexpr (MODE == 2) {
    stage_scores<NREP>(a, b, hk, cur, k_lds, lane);
  } else {
    stage_keys<MASKED, PAGED, S16, KB, VB>(a, bh, cur, k_lds, mask_lds, dmo, lane);
  }
  if constexpr (MODE != 1) stage_values<PAGED, S16, KB, VB>(a, bh, cur, v_lds, dmo);
  if constexpr (MODE != 2) wait_vm<KDMA + VDMA>();   // q
  // the row's selection rule for the scores this lane holds (head h_s)
  SelectRow selr{};
  if constexpr (MODE == 2) selr = a.sel[(int64_t)b * a.Hq + hk * NREP + h_s];

  // q of head h_a at this lane's 32 key channels c0(ks) + j, with
  // c0(ks) = 64 (ks / 2) + 16 kg + 8 (ks % 2)
  float qa[4][8];
  if constexpr (MODE != 2) {
    uint4 qw[4];
    q_reads(q_lds + h_a * kD + 16 * kg, qw);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t ww[4] = {qw[ks].x, qw[ks].y, qw[ks].z, qw[ks].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qa[ks][2 * j] = h2f((uint16_t)(ww[j] & 0xffffu));
        qa[ks][2 * j + 1] = h2f((uint16_t)(ww[j] >> 16));
      }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) qa[ks][j] = 0.0f;
  }
  // The key A operand is q * s_k * 2^ek with one exponent ek for the whole
  // workgroup.  A key scale is (max - min) / 3 of fp16 values, so it is below
  // 2^16; with max |q| < 2^e, every product q s 2^ek stays below 2^14 for
  // ek = -2 - e, whatever the block -- no fp16 overflow for any fp16 input.
  // Products small enough to fall into the fp16 subnormal range keep an
  // absolute error below 2^-25 2^-ek, far under the attention tolerance.
  float qmax = 0.0f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int j = 0; j < 8; ++j) qmax = fmaxf(qmax, fabsf(qa[ks][j]));
  qmax = group_max(row_max(qmax));
  const int ek = __builtin_amdgcn_readfirstlane(-2 - __builtin_amdgcn_frexp_expf(qmax));
  {
    const float f = __builtin_amdgcn_ldexpf(1.0f, ek);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) qa[ks][j] *= f;
  }

  const float LOG2E = 1.4426950408889634f;
  const float c_bias = a.sm_scale * LOG2E;    // scores in log2 units

  // The value A operand is p * s_v, unscaled: p <= 1 and a value scale of
  // fp16 values is below 2^16, so it never overflows fp16.  zt (sum p z)
  // stays in fp32.
  float m_run = -INFINITY;     // running max (log2 units), head h_s
  float l_run = 0.0f;          // this lane's share of the running sum
  float zt = 0.0f;             // sum p z, value A row (h_v, c_v)
  f4 dv[4][2];
#pragma unroll
  for (int g = 0; g < 4; ++g) dv[g][0] = dv[g][1] = (f4){0, 0, 0, 0};

  // MODE 1: the scores of the previous block (head h_s, tokens 32 g + 2 i +
  // e), kept in registers and stored while the next block is processed.
  float sp[4][2] = {};
  int64_t prev = -1;
  float smax = -INFINITY;   // MODE 1: the largest score this lane stored
  auto store_prev = [&]() __attribute__((always_inline)) {
    if (prev >= 0 && k_valid) {
      float *dst = a.scores + ((int64_t)b * a.Hq + hk * NREP + h_s) * a.cap + prev * kBT + 2 * i;
#pragma unroll
      for (int g = 0; g < 4; ++g) *(float2 *)(dst + 32 * g) = make_float2(sp[g][0], sp[g][1]);
    }
  };

  // One block (block cur), whose key part has arrived.  With a next block
  // (block nxt), its key part and then its value part are requested as soon
  // as this block's key part and value part have been read into registers.
  auto block = [&](auto next_tag, int64_t nxt) __attribute__((always_inline)) {
    constexpr bool has_next = decltype(next_tag)::value;
    float s2[4][2];   // this lane's scores in log2 units (MODE 1: natural)
    if constexpr (MODE == 2) {
    // ================= stored scores =================
    const float *sc_l = (const float *)kbuf;   // [NREP][128]
    float sv[8];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float2 v = *(const float2 *)(sc_l + h_s * kBT + 32 * g + 2 * i);
      sv[2 * g] = v.x;
      sv[2 * g + 1] = v.y;
    }
    wait_lds8(sv);   // read before the buffer is refilled
    if constexpr (has_next) stage_scores<NREP>(a, b, hk, nxt, k_lds, lane);
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float v = sv[2 * g + e];
        const int64_t tau = cur * kBT + 32 * g + 2 * i + e;
        s2[g][e] = k_valid && select_takes(selr, v, tau) ? v * LOG2E : -INFINITY;
      }
    } else {
    if constexpr (MODE == 1) store_prev();
    // ================= key half =================
    const KStageT<KB> &kst = *kbuf;
    // 2-bit: [group g][64-channel half rho]; 4-bit: [g][rho][16-token half u]
    constexpr int NXK = KB == 2 ? 8 : 16;
    i2 xk[NXK];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int rho = 0; rho < 2; ++rho) {
        if constexpr (KB == 2) {
          xk[2 * g + rho] = tr4(kst.kc + g * 256 + (64 * rho + 16 * kg + i) * 2);
        } else {
#pragma unroll
          for (int u = 0; u < 2; ++u)
            xk[4 * g + 2 * rho + u] = tr4(kst.kc + g * 512 + (64 * rho + 16 * kg + i) * 4 + 2 * u);
        }
      }
    float mk[4][2];
    constexpr float kMaskUnit = MODE == 1 ? 1.0f : 1.4426950408889634f;   // natural or log2
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (MASKED) {
        if constexpr (KB == 2) {
          const float2 m2 = *(const float2 *)(L.mask + 32 * g + 2 * i);
          mk[g][0] = m2.x * kMaskUnit;
          mk[g][1] = m2.y * kMaskUnit;
        } else {
          mk[g][0] = L.mask[tok(g, 0, i)] * kMaskUnit;
          mk[g][1] = L.mask[tok(g, 1, i)] * kMaskUnit;
        }
      } else {
        mk[g][0] = mk[g][1] = 0.0f;
      }
    }
    // A = hi/lo(q s) for rows (h_a, g_a); bias = q . z
    h8 ah[4], al[4];
    float bz = 0.0f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c0 = 64 * (ks >> 1) + 16 * kg + 8 * (ks & 1);
      float sv[8];
      scales8<S16>(kst.ks, g_a, c0, sv);
      const h8 zv = *(const h8 *)(kst.kz + zrot_off(g_a, c0));
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        // element j of the operands holds channel c0 + k_order(j)
        const int j0 = k_order<KB>(j), j1 = k_order<KB>(j + 1);
        split_mul2(qa[ks][j0], sv[j0], qa[ks][j1], sv[j1], ah[ks], al[ks], j);
        bz = fmaf(qa[ks][j], (float)zv[j], bz);
        bz = fmaf(qa[ks][j + 1], (float)zv[j + 1], bz);
      }
    }
    // every read of the key part has completed: request the next one
    wait_regs(xk);
    if constexpr (has_next)
      stage_keys<MASKED, PAGED, S16, KB, VB>(a, bh, nxt, k_lds, mask_lds, dmo, lane);

    bz = group_sum(bz);
    if (kg == 0) L.bias[i] = bz;

    f4 dk[4][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      dk[g][0] = dk[g][1] = (f4){0, 0, 0, 0};
#pragma unroll
      for (int rho = 0; rho < 2; ++rho) {
        if constexpr (KB == 2) {
          const i2 x = xk[2 * g + rho];
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            h8 be, bo;
            codes_to_b((uint32_t)x[d], be, bo);
            const int ks = 2 * rho + d;
            dk[g][0] = mfma(ah[ks], be, dk[g][0]);
            dk[g][1] = mfma(ah[ks], bo, dk[g][1]);
            dk[g][0] = mfma(al[ks], be, dk[g][0]);
            dk[g][1] = mfma(al[ks], bo, dk[g][1]);
          }
        } else {
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const i2 x = xk[4 * g + 2 * rho + u];
#pragma unroll
            for (int d = 0; d < 2; ++d) {
              const h8 bq = codes4_to_b((uint32_t)x[d]);
              const int ks = 2 * rho + d;
              dk[g][u] = mfma(ah[ks], bq, dk[g][u]);
              dk[g][u] = mfma(al[ks], bq, dk[g][u]);
            }
          }
        }
      }
    }
    wave_lds_sync();

    // scores (even / odd token of each pair), head h_s
    if (k_valid) {
      const f4 bz4 = *(const f4 *)(L.bias + 4 * kg);
      // undo 2^ek; log2 units, or natural ones for the stored scores
      const float cs = (MODE == 1 ? a.sm_scale : c_bias) * __builtin_amdgcn_ldexpf(1.0f, -ek);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        s2[g][0] = fmaf(dk[g][0][g] + bz4[g], cs, mk[g][0]);
        s2[g][1] = fmaf(dk[g][1][g] + bz4[g], cs, mk[g][1]);
      }
    }
    if constexpr (MODE == 1) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        sp[g][0] = s2[g][0];
        sp[g][1] = s2[g][1];
        smax = fmaxf(smax, fmaxf(s2[g][0], s2[g][1]));
      }
      prev = cur;
      return;
    }
    }   // key half

    // online softmax, head h_s
    if (k_valid) {
      float bmax = -INFINITY;
#pragma unroll
      for (int g = 0; g < 4; ++g) bmax = fmaxf(bmax, fmaxf(s2[g][0], s2[g][1]));
      bmax = row_max(bmax);
      const float m_new = fmaxf(m_run, bmax);
      const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      float lsum = 0.0f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float p0 = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s2[g][0] - m_new);
        const float p1 = m_new == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s2[g][1] - m_new);
        lsum += p0 + p1;
        if constexpr (KB == 2) {
          *(float2 *)(&L.p[h_s][32 * g + 2 * i]) = make_float2(p0, p1);
        } else {
          L.p[h_s][tok(g, 0, i)] = p0;
          L.p[h_s][tok(g, 1, i)] = p1;
        }
      }
      l_run = fmaf(l_run, alpha, lsum);
      m_run = m_new;
      if (i == 0) L.alpha[h_s] = alpha;
    }

    // ================= value half =================
    if constexpr (has_next)
      wait_vm<KDMA>();               // value part of this block in; the next key part may fly
    else
      wait_vm<0>();
    wave_lds_sync();
    const VStageT<VB> &vst = *vbuf;
    // 2-bit: [16-token half u][channel group g]; 4-bit: [u][16-channel unit w]
    constexpr int NXV = VB == 2 ? 8 : 16;
    i2 xv[NXV];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if constexpr (VB == 2) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          xv[4 * u + g] = tr4(vst.vc + (32 * kg + 16 * u + i) * 8 +
                              4 * ((g >> 1) ^ ((i >> 3) & 1)) + 2 * (g & 1));
      } else {
#pragma unroll
        for (int w = 0; w < 8; ++w)
          xv[8 * u + w] = tr4(vst.vc + (32 * kg + 16 * u + i) * 16 +
                              4 * ((w >> 1) ^ ((i >> 2) & 3)) + 2 * (w & 1));
      }
    }
    {
      // accumulators follow the running maximum
      const float av = v_valid ? L.alpha[kg] : 1.0f;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        dv[g][0][g] *= av;
        dv[g][1][g] *= av;
      }
      zt *= L.alpha[h_v];
    }
    // A = hi/lo(p s) for rows (h_v, c_v); zt += p . z
    h8 vh[2][2], vl[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        const int t0 = 32 * kg + 16 * u + 8 * d;
        const f4 p0 = *(const f4 *)(&L.p[h_v][t0]);
        const f4 p1 = *(const f4 *)(&L.p[h_v][t0 + 4]);
        float sv[8];
        scales8<S16>(vst.vs, c_v, t0, sv);
        const h8 zv = *(const h8 *)(vst.vz + zrot_off(c_v, t0));
        const float pv[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const int j0 = k_order<VB>(j), j1 = k_order<VB>(j + 1);
          split_mul2(pv[j0], sv[j0], pv[j1], sv[j1], vh[u][d], vl[u][d], j);
          zt = fmaf(pv[j], (float)zv[j], zt);
          zt = fmaf(pv[j + 1], (float)zv[j + 1], zt);
        }
      }
    }
    // every read of the value part has completed: request the next one
    wait_regs(xv);
    if constexpr (has_next) stage_values<PAGED, S16, KB, VB>(a, bh, nxt, v_lds, dmo);

    // dv[g][e]: channels 32 g + 2 j + e (2-bit) or 32 g + 16 e + j (4-bit)
    // of column j
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if constexpr (VB == 2) {
          const i2 x = xv[4 * u + g];
#pragma unroll
          for (int d = 0; d < 2; ++d) {
            h8 be, bo;
            codes_to_b((uint32_t)x[d], be, bo);
            dv[g][0] = mfma(vh[u][d], be, dv[g][0]);
            dv[g][1] = mfma(vh[u][d], bo, dv[g][1]);
            dv[g][0] = mfma(vl[u][d], be, dv[g][0]);
            dv[g][1] = mfma(vl[u][d], bo, dv[g][1]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const i2 x = xv[8 * u + 2 * g + e];
#pragma unroll
            for (int d = 0; d < 2; ++d) {
              const h8 bq = codes4_to_b((uint32_t)x[d]);
              dv[g][e] = mfma(vh[u][d], bq, dv[g][e]);
              dv[g][e] = mfma(vl[u][d], bq, dv[g][e]);
            }
          }
        }
      }
    }
  };
  // The next block is drawn once this block's key part is in; the draw is an
  // LDS atomic, so its wait passes over the copies in flight.  (MODE 1 waits
  // for everything: the score stores are vector-memory operations too.)
  for (;;) {
    if constexpr (MODE == 1)
      wait_vm<0>();
    else
      wait_vm<VDMA>();   // key part of this block in
    const int64_t nxt = draw_item(sh.ctr, lane) - sh.n_skip;
    if (nxt >= sh.nb) break;
    const int64_t nb2 = sh.block((int)nxt);
    block(std::true_type{}, nb2);
    cur = nb2;
  }
  block(std::false_type{}, 0);
  if constexpr (MODE == 1) {
    store_prev();
    // the wave's largest score of head h_s: the 16 lanes of its row
    const float hm = row_max(smax);
    if (a.rmax && k_valid && i == 0)
      a.rmax[((int64_t)b * a.Hq + hk * NREP + h_s) * a.rmax_n + mslot] = hm;
    return;
  }

  // ---- the wave's partial (acc[128], m, l) of each query head, into its
  // probability buffer (rows of kPRow floats), for the workgroup's merge
  zt = group_sum(zt);
  wave_lds_sync();
  if (kg == 0) L.bias[i] = zt;
  const float l_head = row_sum(l_run);
  wave_lds_sync();
  if (v_valid) {
    const f4 z4 = *(const f4 *)(L.bias + 4 * kg);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if constexpr (VB == 2) {
        *(float2 *)&L.p[kg][32 * g + 2 * i] =
            make_float2(dv[g][0][g] + z4[g], dv[g][1][g] + z4[g]);
      } else {
        L.p[kg][32 * g + i] = dv[g][0][g] + z4[g];
        L.p[kg][32 * g + 16 + i] = dv[g][1][g] + z4[g];
      }
    }
  }
  if (k_valid && i == 0)
    *(float2 *)&L.p[h_s][kD] =
        make_float2(m_run == -INFINITY ? -INFINITY : m_run * 0.6931471805599453f, l_head);
}

// Window role: tokens [Ta, Tb) = [n_main + 32 chunk, min(t, n_main + 32 chunk + 32))
// of one slab -- fp16 window tokens and quantized tokens past the last whole
// block.  The chunk's key data goes to the key buffer and its value data to
// the value buffer, in one batch of DMA (window_issue); then each lane
// scores one token over half of the channels (scalar fp32) and accumulates
// two output channels (window_role).

// Where a window chunk's data lies.
struct WinChunk {
  int64_t bh, Ta, Tb, vq_end, t_pop, wslot;
  int n, n_qv, n_fv, nqvs, nqv8, lt, u_vs, u_vz, u_vrow;
  bool kq, kq_now, pop_here, new_here;
  const uint8_t *rec;
};

template <bool PAGED, bool S16, int KB, int VB>
__device__ __forceinline__ WinChunk win_chunk(const DecodeArgs &a, const RowSpan &rs,
                                              int64_t n_main, int chunk, int hk, int b) {
  WinChunk c;
  c.bh = (int64_t)b * a.H + hk;
  c.Ta = n_main + (int64_t)kWT * chunk;
  c.Tb = c.Ta + kWT < rs.t ? c.Ta + kWT : rs.t;
  c.n = (int)(c.Tb - c.Ta);
  // keys: Ta and n_kq are multiples of 32, so the chunk is one whole
  // quantized key group or consists of fp16 window rows
  c.kq = c.Ta < rs.n_kq;
  // A fused step whose token completes a key block quantizes keys [t - R, t)
  // in this launch: each of those chunks stages its 32 fp16 rows and turns
  // them into its key group (kq_now).
  c.kq_now = rs.t_new >= 0 && rs.t % a.R == 0 && c.Ta >= rs.t - a.R;
  // values: [Ta, vq_end) quantized, [vq_end, Tb) fp16
  c.vq_end = rs.n_vq < c.Ta ? c.Ta : (rs.n_vq > c.Tb ? c.Tb : rs.n_vq);
  c.n_qv = (int)(c.vq_end - c.Ta);
  c.n_fv = (int)(c.Tb - c.vq_end);
  c.nqv8 = (c.n_qv + 7) / 8;    // 16-byte units of fp16 zeros per channel group
  // 16-byte units of scales per channel group (fp32, or fp16 like the zeros)
  c.nqvs = S16 ? c.nqv8 : (c.n_qv + 3) / 4;
  // the chunk lies in one record (Ta is a multiple of 32), at token lt of it
  c.rec = record_of<PAGED, S16, KB, VB>(a, c.bh, c.Ta / kBT);
  c.lt = (int)(c.Ta % kBT);
  // value buffer: codes (VB units per token), scales (4 channel groups x
  // nqvs units), fp16 zeros (4 x nqv8 units), then fp16 rows (16 units each)
  c.u_vs = c.n_qv * VB;
  c.u_vz = c.u_vs + 4 * c.nqvs;
  c.u_vrow = c.u_vz + 4 * c.nqv8;
  // Fused decode step: the value that leaves the window with this token
  // (t_pop = t_new - R, the last quantized value) and the new token's slot.
  c.t_pop = rs.t_new >= a.R ? rs.t_new - a.R : -1;
  c.pop_here = c.t_pop >= c.Ta && c.t_pop < c.vq_end;
  c.new_here = rs.t_new >= c.Ta && rs.t_new < c.Tb;
  c.wslot = rs.t_new >= 0 ? rs.t_new % a.R : 0;
  return c;
}

// What window_issue reads into registers: the fused step's popped value
// and new key / value (lane j: channels 2j, 2j + 1), and q (lane j: channels
// 2j, 2j + 1 of each head).
template <int NREP>
struct WinLoads {
  uint32_t popped, nv, nk;
  uint32_t q[NREP];
};

// Units (16 bytes) of a staged key group in the window role's key buffer:
// codes (32 KB units: channel c at words KB c ..), then scales (32 fp32 or
// 16 fp16 units), then zeros (16).
template <bool S16, int KB>
struct WinKeyUnits {
  static constexpr int scales = 32 * KB, zeros = scales + (S16 ? 16 : 32), end = zeros + 16;
};

// The loads of one window chunk, issued and not waited for.  MODE 1 (scores)
// stages no values; MODE 2 (selected attention) no keys and no q.
template <int NREP, bool PAGED, bool S16, int MODE, int KB, int VB>
__device__ __forceinline__ WinLoads<NREP> window_issue(const DecodeArgs &a, const RowSpan &rs,
                                                       int64_t n_main, int chunk, int hk, int b,
                                                       const Lds &L) {
  using RC = Rec<S16, KB, VB>;
  using KU = WinKeyUnits<S16, KB>;
  const int j = threadIdx.x & 63;
  const WinChunk c = win_chunk<PAGED, S16, KB, VB>(a, rs, n_main, chunk, hk, b);
  const int64_t bh = c.bh, Ta = c.Ta, vq_end = c.vq_end;
  const int n = c.n, nqvs = c.nqvs, nqv8 = c.nqv8, lt = c.lt;
  const bool kq = c.kq, kq_now = c.kq_now;
  const uint8_t *rec = c.rec;
  // ---- DMA, in 16-byte units.  Key buffer: a key group (WinKeyUnits), or
  // n fp16 rows (16 units each) -- at most 512 units = 8 KB.
  char *kl = (char *)L.ks;
  const int ku_end = MODE == 2 ? 0 : (kq && !kq_now ? KU::end : n * 16);
  for (int base = 0; base < ku_end; base += 64) {
    const int u = base + j;
    if (u < ku_end) {
      const void *src;
      if (kq && !kq_now) {
        const int lg = lt / kG;    // key group within the record
        if (u < KU::scales)
          src = rec + RC::kc + lg * (512 * KB) + u * 16;
        else if (u < KU::zeros)
          src = rec + RC::ks + lg * (kD * RC::sb) + (u - KU::scales) * 16;
        else
          src = rec + RC::kz + lg * 256 + (u - KU::zeros) * 16;
      } else {
        // row r = u / 16 of the chunk; its 16-byte unit k is stored at unit
        // (k + r) % 16 of the row's LDS slot, so that lanes reading the same
        // unit of different rows hit different banks
        const int64_t tok = Ta + u / 16;
        const int k = ((u & 15) - (u >> 4)) & 15;
        src = tok == rs.t_new ? a.k_new + (bh * kD + k * 8)
                             : a.k_res + ((bh * a.R + tok % a.R) * kD + k * 8);
      }
      dma16(src, (lds_void *)(kl + (size_t)base * 16));
    }
  }
  // value buffer (at most 512 units)
  char *vl = (char *)L.vs;
  const int u_vs = c.u_vs, u_vz = c.u_vz, u_vrow = c.u_vrow;
  const int vu_end = MODE == 1 ? 0 : u_vrow + c.n_fv * 16;
  for (int base = 0; base < vu_end; base += 64) {
    const int u = base + j;
    if (u < vu_end) {
      const void *src;
      if (u < u_vs) {
        src = rec + RC::vc + (lt + u / VB) * (16 * VB) + (u % VB) * 16;
      } else if (u < u_vz) {
        const int x = u - u_vs;
        src = rec + RC::vs + ((x / nqvs) * kBT + lt) * RC::sb + (x % nqvs) * 16;
      } else if (u < u_vrow) {
        const int x = u - u_vz;
        src = rec + RC::vz + ((x / nqv8) * kBT + lt) * 2 + (x % nqv8) * 16;
      } else {
        const int x = u - u_vrow;
        const int64_t tok = vq_end + x / 16;
        src = tok == rs.t_new ? a.v_new + (bh * kD + (x % 16) * 8)
                             : a.v_res + ((bh * a.R + tok % a.R) * kD + (x % 16) * 8);
      }
      dma16(src, (lds_void *)(vl + (size_t)base * 16));
    }
  }
  WinLoads<NREP> ld;
  ld.popped = ld.nv = ld.nk = 0u;
  uint16_t *slot_v = const_cast<uint16_t *>(a.v_res) + (bh * a.R + c.wslot) * kD + 2 * j;
  if (c.pop_here) ld.popped = *(const uint32_t *)slot_v;
  if (c.pop_here || c.new_here) ld.nv = *(const uint32_t *)(a.v_new + bh * kD + 2 * j);
  if (c.new_here) ld.nk = *(const uint32_t *)(a.k_new + bh * kD + 2 * j);
  const uint16_t *q = a.q + ((int64_t)b * a.Hq + hk * NREP) * kD;
#pragma unroll
  for (int h = 0; h < NREP; ++h) ld.q[h] = MODE == 2 ? 0u : *(const uint32_t *)(q + h * kD + 2 * j);
  return ld;
}

// MODE 1 (scores): the scores of the chunk's tokens go to a.scores (natural
// units, mask included); nothing else.  MODE 2 (selected attention): the
// chunk's scores come from a.scores, -inf where the row's selection rule
// does not take the token.
template <int NREP, bool MASKED, bool PAGED, bool S16, int MODE, int KB, int VB>
__device__ __forceinline__ void window_role(const DecodeArgs &a, const RowSpan &rs, int64_t n_main,
                                            int chunk, int slot, int hk, int b, const Lds &L,
                                            const WinLoads<NREP> &ld) {
  using RC = Rec<S16, KB, VB>;
  using KU = WinKeyUnits<S16, KB>;
  constexpr int VW = 4 * VB;              // code words per value token
  constexpr int KCPW = 32 / KB, VCPW = 32 / VB;   // codes per word
  constexpr uint32_t KCM = (1u << KB) - 1u, VCM = (1u << VB) - 1u;
  const int j = threadIdx.x & 63;
  const WinChunk c = win_chunk<PAGED, S16, KB, VB>(a, rs, n_main, chunk, hk, b);
  const int64_t bh = c.bh, Ta = c.Ta, t_pop = c.t_pop;
  const int n = c.n, n_qv = c.n_qv, nqvs = c.nqvs, nqv8 = c.nqv8;
  const int u_vs = c.u_vs, u_vz = c.u_vz, u_vrow = c.u_vrow;
  const bool kq = c.kq, kq_now = c.kq_now, pop_here = c.pop_here, new_here = c.new_here;
  char *kl = (char *)L.ks;
  char *vl = (char *)L.vs;
  uint16_t *slot_v = const_cast<uint16_t *>(a.v_res) + (bh * a.R + c.wslot) * kD + 2 * j;
  const uint32_t popped = ld.popped, nv = ld.nv, nk = ld.nk;
  // the chunk's record (it lies in one), where a fused step's cache writes go
  uint8_t *recw = const_cast<uint8_t *>(c.rec);
  const int64_t wslot = c.wslot;
  // q of the NREP heads, kept in the probability buffer (unused by this role)
  float(*q_s)[kPRow] = L.p;
#pragma unroll
  for (int h = 0; h < NREP; ++h) {
    q_s[h][2 * j] = h2f((uint16_t)(ld.q[h] & 0xFFFFu));
    q_s[h][2 * j + 1] = h2f((uint16_t)(ld.q[h] >> 16));
  }
  wait_vm<0>();
  if (pop_here) {
    // KIVI item 3 on the popped value: 16 lanes per 32-channel group, the
    // bit-exact quantizer (IEEE division, round half to even).  Its codes,
    // scales and zeros replace what the DMA brought for that row (not yet
    // written) and go to the cache.
    const float x0 = h2f((uint16_t)(popped & 0xFFFFu)), x1 = h2f((uint16_t)(popped >> 16));
    float mn = first_min(x0, x1), mx = first_max(x0, x1);   // channel 2j comes first
    lanes_first_min_max(mn, mx, j, 16);
    const float sc = rec_scale<S16>(group_scale(mn, mx, VB));
    // lanes of one code word: VCPW / 2 (two channels per lane)
    constexpr int LW = VCPW / 2;
    uint32_t w = (quant_code(x0, mn, sc, VB) | (quant_code(x1, mn, sc, VB) << VB))
                 << (2 * VB * (j & (LW - 1)));
#pragma unroll
    for (int o = 1; o < LW; o <<= 1) w |= __shfl_xor(w, o);
    const int xr = (int)(t_pop - Ta);
    const int gch = j >> 4;
    if ((j & (LW - 1)) == 0) {
      ((uint32_t *)vl)[xr * VW + j / LW] = w;
      ((uint32_t *)(recw + RC::vc) + (t_pop % kBT) * VW)[j / LW] = w;
    }
    if ((j & 15) == 0) {
      const uint16_t zh = f2h_bits(mn);
      if constexpr (S16) {
        const uint16_t sh = f2h_bits(sc);
        ((uint16_t *)(vl + (size_t)u_vs * 16))[gch * nqvs * 8 + xr] = sh;
        ((uint16_t *)(recw + RC::vs))[gch * kBT + t_pop % kBT] = sh;
      } else {
        ((float *)(vl + (size_t)u_vs * 16))[gch * nqvs * 4 + xr] = sc;
        ((float *)(recw + RC::vs))[gch * kBT + t_pop % kBT] = sc;
      }
      ((uint16_t *)(vl + (size_t)u_vz * 16))[gch * nqv8 * 8 + xr] = zh;
      ((uint16_t *)(recw + RC::vz))[gch * kBT + t_pop % kBT] = zh;
    }
    // the slot now takes the new value (this lane read its old contents above)
    *(uint32_t *)slot_v = nv;
  }
  if (new_here) {
    if (t_pop < 0) *(uint32_t *)slot_v = nv;   // no value left the window: the slot is free
    *(uint32_t *)(const_cast<uint16_t *>(a.k_res) + (bh * a.R + wslot) * kD + 2 * j) = nk;
  }
  if (kq_now) {
    // KIVI item 2 on this chunk's key group (32 tokens; n == 32): lane j
    // takes channels 2j and 2j + 1 over the staged rows -- min/max, then the
    // codes, with the quantizer of the append path.  The codes, scales and
    // zeros replace the rows in LDS in the layout of a staged key group and
    // go to the cache.
    // word j of row r (channels 2j, 2j + 1), in the rows' rotated layout
    const uint32_t *kw = (const uint32_t *)kl;
    auto row_word = [&](int r) { return kw[r * 64 + ((((j >> 2) + r) & 15) << 2) + (j & 3)]; };
    float mn0, mx0, mn1, mx1;
    {
      const uint32_t w = row_word(0);
      mn0 = mx0 = h2f((uint16_t)(w & 0xFFFFu));
      mn1 = mx1 = h2f((uint16_t)(w >> 16));
    }
    for (int r = 1; r < kWT; ++r) {
      const uint32_t w = row_word(r);
      const float x0 = h2f((uint16_t)(w & 0xFFFFu)), x1 = h2f((uint16_t)(w >> 16));
      mn0 = x0 < mn0 ? x0 : mn0;
      mx0 = x0 > mx0 ? x0 : mx0;
      mn1 = x1 < mn1 ? x1 : mn1;
      mx1 = x1 > mx1 ? x1 : mx1;
    }
    const float sc0 = rec_scale<S16>(group_scale(mn0, mx0, KB));
    const float sc1 = rec_scale<S16>(group_scale(mn1, mx1, KB));
    // channel 2j: words 0 .. KB - 1; channel 2j + 1: words KB .. 2 KB - 1
    uint32_t cw[2 * KB];
#pragma unroll
    for (int k = 0; k < 2 * KB; ++k) cw[k] = 0u;
    for (int r = 0; r < kWT; ++r) {
      const uint32_t w = row_word(r);
      const int sh = KB * (r % KCPW), hw = r / KCPW;
      cw[hw] |= quant_code(h2f((uint16_t)(w & 0xFFFFu)), mn0, sc0, KB) << sh;
      cw[KB + hw] |= quant_code(h2f((uint16_t)(w >> 16)), mn1, sc1, KB) << sh;
    }
    wave_lds_sync();   // every lane's row reads are done before the rows are overwritten
    // codes: KB words per channel, channels 2j and 2j + 1 at words 2 KB j ..
    uint4 c4[KB / 2];
#pragma unroll
    for (int k = 0; k < KB / 2; ++k) {
      c4[k] = make_uint4(cw[4 * k], cw[4 * k + 1], cw[4 * k + 2], cw[4 * k + 3]);
      *(uint4 *)((uint32_t *)kl + 2 * KB * j + 4 * k) = c4[k];
    }
    const uint32_t z2 = (uint32_t)f2h_bits(mn0) | ((uint32_t)f2h_bits(mn1) << 16);
    const int64_t grp = Ta / kG;
    const int lg = (int)(grp % (kBT / kG));   // the group within the record
    if constexpr (S16) {
      const uint32_t s2 = (uint32_t)f2h_bits(sc0) | ((uint32_t)f2h_bits(sc1) << 16);
      *((uint32_t *)(kl + KU::scales * 16) + j) = s2;
      *(uint32_t *)((uint16_t *)(recw + RC::ks) + lg * kD + 2 * j) = s2;
    } else {
      *(float2 *)((float *)(kl + KU::scales * 16) + 2 * j) = make_float2(sc0, sc1);
      *(float2 *)((float *)(recw + RC::ks) + lg * kD + 2 * j) = make_float2(sc0, sc1);
    }
    *((uint32_t *)(kl + KU::zeros * 16) + j) = z2;
#pragma unroll
    for (int k = 0; k < KB / 2; ++k)
      *(uint4 *)((uint32_t *)(recw + RC::kc) + (lg * kD + 2 * j) * KB + 4 * k) = c4[k];
    *(uint32_t *)((uint16_t *)(recw + RC::kz) + lg * kD + 2 * j) = z2;
  }
  wave_lds_sync();

  const float LOG2E = 1.4426950408889634f;
  // ---- scores: lane j scores token Ta + (j & 31) over channels [64 hf, 64 hf + 64)
  const int tj = j & 31, hf = j >> 5;
  float sc[NREP];
#pragma unroll
  for (int h = 0; h < NREP; ++h) sc[h] = 0.0f;
  if (MODE != 2 && tj < n) {
    // 16-byte LDS reads throughout: the key group's words, scales and zeros
    // and q are the same for all lanes of a half (broadcasts); channels are
    // summed in increasing order
    if (kq) {
      const uint32_t *kc = (const uint32_t *)kl;   // channel c: words KB c ..
      const char *ks = kl + KU::scales * 16;
      const uint16_t *kz = (const uint16_t *)(kl + KU::zeros * 16);
      const int sh = KB * (tj % KCPW);
      const bool hi = tj >= 16;
#pragma unroll 4
      for (int c = 64 * hf; c < 64 * hf + 64; c += 4) {
        uint32_t cw[4];
        if constexpr (KB == 2) {
          const uint4 wa = *(const uint4 *)(kc + 2 * c);
          const uint4 wb = *(const uint4 *)(kc + 2 * c + 4);
          cw[0] = hi ? wa.y : wa.x;
          cw[1] = hi ? wa.w : wa.z;
          cw[2] = hi ? wb.y : wb.x;
          cw[3] = hi ? wb.w : wb.z;
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) cw[u] = kc[4 * (c + u) + tj / KCPW];
        }
        f4 s4;
        if constexpr (S16) {
          const uint2 ss = *(const uint2 *)((const uint16_t *)ks + c);
          s4 = (f4){h2f((uint16_t)(ss.x & 0xFFFFu)), h2f((uint16_t)(ss.x >> 16)),
                    h2f((uint16_t)(ss.y & 0xFFFFu)), h2f((uint16_t)(ss.y >> 16))};
        } else {
          s4 = *(const f4 *)((const float *)ks + c);
        }
        const uint2 zz = *(const uint2 *)(kz + c);
        const float z4[4] = {h2f((uint16_t)(zz.x & 0xFFFFu)), h2f((uint16_t)(zz.x >> 16)),
                             h2f((uint16_t)(zz.y & 0xFFFFu)), h2f((uint16_t)(zz.y >> 16))};
        f4 q4[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) q4[h] = *(const f4 *)&q_s[h][c];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float code = (float)((cw[u] >> sh) & KCM);
          const float kh = code * s4[u] + z4[u];
#pragma unroll
          for (int h = 0; h < NREP; ++h) sc[h] = fmaf(q4[h][u], kh, sc[h]);
        }
      }
    } else {
      // row tj, units 8 hf .. 8 hf + 7 (8 channels each), rotated by tj
      const uint4 *row = (const uint4 *)kl + tj * 16;
#pragma unroll
      for (int k = 8 * hf; k < 8 * hf + 8; ++k) {
        const uint4 w = row[(k + tj) & 15];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
        const int c = 8 * k;
        f4 qa[NREP], qb[NREP];
#pragma unroll
        for (int h = 0; h < NREP; ++h) {
          qa[h] = *(const f4 *)&q_s[h][c];
          qb[h] = *(const f4 *)&q_s[h][c + 4];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t x = ww[e / 2];
          const float kh = h2f((uint16_t)(e % 2 ? x >> 16 : x & 0xFFFFu));
#pragma unroll
          for (int h = 0; h < NREP; ++h) sc[h] = fmaf(e < 4 ? qa[h][e] : qb[h][e - 4], kh, sc[h]);
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < NREP; ++h) sc[h] += __shfl_xor(sc[h], 32);
  if constexpr (MODE == 1) {
    // the scores, natural units, from the lanes of the first half (the
    // second half holds the same); with rmax, the chunk's largest score of
    // each head goes to entry `slot` of the head's row
    const float mk = MASKED && tj < n ? a.mask[(int64_t)b * a.t + Ta + tj] : 0.0f;
#pragma unroll
    for (int h = 0; h < NREP; ++h) {
      const float v = tj < n ? sc[h] * a.sm_scale + mk : -INFINITY;
      const int64_t row = (int64_t)b * a.Hq + hk * NREP + h;
      if (tj < n && hf == 0) a.scores[row * a.cap + Ta + tj] = v;
      if (a.rmax) {
        const float cm = group_max(row_max(v));
        if (j == 0) a.rmax[row * a.rmax_n + slot] = cm;
      }
    }
    return;
  }
  if (tj < n) {
    if constexpr (MODE == 2) {
      // the stored scores (mask included), -inf where the rule does not take
      // the token
#pragma unroll
      for (int h = 0; h < NREP; ++h) {
        const int64_t r = (int64_t)b * a.Hq + hk * NREP + h;
        const float v = a.scores[r * a.cap + Ta + tj];
        sc[h] = select_takes(a.sel[r], v, Ta + tj) ? v * LOG2E : -INFINITY;
      }
    } else {
      const float mk = MASKED ? a.mask[(int64_t)b * a.t + Ta + tj] : 0.0f;
#pragma unroll
      for (int h = 0; h < NREP; ++h) sc[h] = (sc[h] * a.sm_scale + mk) * LOG2E;
    }
  } else {
#pragma unroll
    for (int h = 0; h < NREP; ++h) sc[h] = -INFINITY;
  }
  // ---- softmax over the chunk, per head (lanes j and j ^ 32 hold the same token)
  float *p_s = L.mask;    // [NREP][32]
  float mh[NREP], lh[NREP];
#pragma unroll
  for (int h = 0; h < NREP; ++h) {
    float m = row_max(sc[h]);
    m = fmaxf(m, __shfl_xor(m, 16));
    const float pj = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(sc[h] - m);
    if (hf == 0) p_s[h * kWT + tj] = pj;
    mh[h] = m;
    const float l = row_sum(pj);
    lh[h] = l + __shfl_xor(l, 16);
  }
  wave_lds_sync();
  // ---- values: lane j owns channels 2j and 2j+1
  float o[NREP][2];
#pragma unroll
  for (int h = 0; h < NREP; ++h) o[h][0] = o[h][1] = 0.0f;
  const int c0 = 2 * j;
  const int gch = c0 / kG;
  const uint32_t *vc = (const uint32_t *)vl;
  // the group's scales: nqvs units (4 fp32 or 8 fp16 scales each)
  const char *vsc = vl + (size_t)u_vs * 16 + (size_t)gch * nqvs * 16;
  const uint16_t *vz = (const uint16_t *)(vl + (size_t)u_vz * 16) + gch * nqv8 * 8;
  const uint16_t *vrow = (const uint16_t *)(vl + (size_t)u_vrow * 16);
  // four tokens per step: their probabilities, scales and zeros in 16- and
  // 8-byte reads (p_s is 0 for tokens past n, whose values are not read)
  for (int t0 = 0; t0 < n; t0 += 4) {
    f4 p4[NREP];
#pragma unroll
    for (int h = 0; h < NREP; ++h) p4[h] = *(const f4 *)(p_s + h * kWT + t0);
    f4 s4 = {0.0f, 0.0f, 0.0f, 0.0f};
    uint2 z2 = make_uint2(0u, 0u);
    if (t0 < n_qv) {
      if constexpr (S16) {
        const uint2 ss = *(const uint2 *)((const uint16_t *)vsc + t0);
        s4 = (f4){h2f((uint16_t)(ss.x & 0xFFFFu)), h2f((uint16_t)(ss.x >> 16)),
                  h2f((uint16_t)(ss.y & 0xFFFFu)), h2f((uint16_t)(ss.y >> 16))};
      } else {
        s4 = *(const f4 *)((const float *)vsc + t0);
      }
      z2 = *(const uint2 *)(vz + t0);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = t0 + u;
      float v0 = 0.0f, v1 = 0.0f;
      if (t < n_qv) {
        const uint32_t w = vc[t * VW + c0 / VCPW] >> (VB * (c0 % VCPW));
        const uint32_t zw = u < 2 ? z2.x : z2.y;
        const float zt = h2f((uint16_t)(u % 2 ? zw >> 16 : zw & 0xFFFFu));
        v0 = (float)(w & VCM) * s4[u] + zt;
        v1 = (float)((w >> VB) & VCM) * s4[u] + zt;
      } else if (t < n) {
        const uint32_t hv = *(const uint32_t *)(vrow + (t - n_qv) * kD + c0);
        v0 = h2f((uint16_t)(hv & 0xFFFFu));
        v1 = h2f((uint16_t)(hv >> 16));
      }
#pragma unroll
      for (int h = 0; h < NREP; ++h) {
        o[h][0] = fmaf(p4[h][u], v0, o[h][0]);
        o[h][1] = fmaf(p4[h][u], v1, o[h][1]);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < NREP; ++h) {
    float *dst = a.part + (((int64_t)b * a.Hq + hk * NREP + h) * a.S_total + slot) * (kD + 4);
    *(float2 *)(dst + c0) = make_float2(o[h][0], o[h][1]);
    if (j == 0)
      *(float2 *)(dst + kD) =
          make_float2(mh[h] == -INFINITY ? -INFINITY : mh[h] * 0.6931471805599453f, lh[h]);
  }
}

// grid: n_groups workgroups of W waves per slab, n_groups * B * H in all
// (W = 8: one workgroup per CU; the masked variant, whose registers allow
// one wave per SIMD, W = 4).  Workgroup s of slab sl is lin = s (B H) +
// (sl + s) % (B H), so consecutive workgroups belong to different slabs and
// every slab's workgroups spread over the XCDs.  Its share: blocks
// [s nblk / n_groups, (s + 1) nblk / n_groups) and window chunks s, s +
// n_groups, ...; its waves draw the chunks first, then the blocks, from the
// counter in LDS, so waves that run faster take more of them.  Partial
// slots: s for the workgroup's blocks (its waves' partials merged in LDS),
// n_groups + x for window chunk x.  A slab with a single workgroup merges
// them into out in the same launch.
// Ragged batch (RAGGED): each row has its own token count rows.t[b] and
// its own number of workgroups per KV head, planned on the host in
// proportion to its work; workgroup lin serves share u = lin % n_shares of
// KV head lin / n_shares, and rows.share[u] names the row, the share's
// index s among the row's workgroups and their number.  n_main, n_groups
// and n_window then follow per row (n_groups argument = n_shares).
// The masked variant holds the block's mask in registers as well; it may
// use more than half the register file rather than spill, since a spill
// reload inside the block loop would wait for every DMA in flight.
// MODE 1 (scores) and MODE 2 (selected attention): see block_role; MODE 1
// writes no partials.
// KB or VB 4 (4-bit keys or values: attention and the fused step of a
// uniform batch): six waves (four masked) so that their 11 KB stages fit
// the LDS.
template <int NREP, bool MASKED, bool RAGGED, bool PAGED, bool S16, int MODE, int KB = 2,
          int VB = KB>
__global__ void __launch_bounds__(MASKED ? 256 : (KB == 2 && VB == 2 ? 512 : 384))
    __attribute__((amdgpu_waves_per_eu(MASKED ? 1 : 2)))
    decode_matrix_kernel(DecodeArgs a, int64_t n_main_all, int n_groups_all, int n_window_all,
                         MatrixRowArg<RAGGED> rows) {
  static_assert((KB == 2 && VB == 2) || MODE == 0, "4-bit codes: attention only");
  static_assert(KB == VB || (!RAGGED && !PAGED), "mixed widths: a uniform contiguous cache");
  constexpr int W = MASKED ? 4 : (KB == 2 && VB == 2 ? 8 : 6);
  __shared__ KStageT<KB> sm_k[W];
  __shared__ VStageT<VB> sm_v[W];
  __shared__ __attribute__((aligned(16))) float sm_p[W][4][kPRow];
  __shared__ __attribute__((aligned(16))) float sm_mask[W][kBT];
  __shared__ __attribute__((aligned(16))) float sm_bias[W][16];
  __shared__ __attribute__((aligned(16))) float sm_alpha[W][4];
  __shared__ int sm_ctr;
  // wave-uniform, so that the wave's LDS addresses stay scalar
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  // (the window role addresses the stages as bytes: at most 8 KB of rows)
  const Lds L{reinterpret_cast<KStage *>(&sm_k[w]), reinterpret_cast<VStage *>(&sm_v[w]), sm_p[w],
              sm_mask[w], sm_bias[w], sm_alpha[w]};
  const uint32_t lin = blockIdx.x;
  uint32_t s, sl;
  int hk, b, n_groups, n_window;
  int64_t n_main;
  RowSpan rs;
  if constexpr (RAGGED) {
    const uint32_t n_shares = (uint32_t)n_groups_all;
    const uint32_t u = lin % n_shares;
    const uint32_t e = rows.share[u];
    hk = (int)(lin / n_shares);
    b = (int)(e & 255u);
    s = (e >> 8) & 4095u;
    n_groups = (int)(e >> 20);
    sl = (uint32_t)b * (uint32_t)a.H + (uint32_t)hk;
    rs = row_span(rows.t[b], a.R, a.t_new >= 0);
    n_main = matrix_main(rs, a.R);
    n_window = matrix_window_chunks(rs.t, n_main);
  } else {
    const uint32_t n_slabs = (uint32_t)a.B * (uint32_t)a.H;
    s = lin / n_slabs;
    sl = (lin % n_slabs + n_slabs - s % n_slabs) % n_slabs;
    hk = (int)(sl % (uint32_t)a.H);
    b = (int)(sl / (uint32_t)a.H);
    n_groups = n_groups_all;
    n_window = n_window_all;
    n_main = n_main_all;
    rs.t = a.t;
    rs.n_kq = a.n_kq;
    rs.n_vq = a.n_vq;
    rs.t_new = a.t_new;
  }
  const int64_t nblk = n_main / kBT;
  BlockShare sh;
  sh.b0 = (int)((int64_t)s * nblk / n_groups);
  sh.nb = (int)(((int64_t)s + 1) * nblk / n_groups - sh.b0);
  // The blocks are visited from a starting block that a hash picks,
  // wrapping around.  Every slab's records sit a multiple of the capacity
  // apart, so workgroups walking their shares in lock-step from the first
  // block hit HBM channels in step for some capacities (13% slower at 257 x
  // 128 tokens); scattered starting points break that up.  The order only
  // changes the rounding order of the online softmax.
  sh.rot = sh.nb > 0 ? (int)((((sl * 2654435761u) ^ (s * 2246822519u)) >> 8) % (uint32_t)sh.nb) : 0;
  sh.n_skip = (int)s < n_window ? (n_window - 1 - (int)s) / n_groups + 1 : 0;
  sh.ctr = &sm_ctr;
  if (threadIdx.x == 0) sm_ctr = 0;
  __syncthreads();
  int item = draw_item(&sm_ctr, lane);
  while (item < sh.n_skip) {
    const int x = (int)s + item * n_groups;
    const WinLoads<NREP> ld =
        window_issue<NREP, PAGED, S16, MODE, KB, VB>(a, rs, n_main, x, hk, b, L);
    window_role<NREP, MASKED, PAGED, S16, MODE, KB, VB>(a, rs, n_main, x,
                                                        MODE == 1 ? n_groups * W + x
                                                                  : n_groups + x,
                                                        hk, b, L,
                                                      ld);
    wave_lds_sync();   // the LDS reads of the chunk are done
    item = draw_item(&sm_ctr, lane);
  }
  block_role<NREP, MASKED, PAGED, S16, MODE, KB, VB>(a, sh, item - sh.n_skip, hk, b, L, &sm_k[w],
                                                   &sm_v[w], (int)s * W + w);
  if constexpr (MODE == 1) return;   // the scores are stored; no partials

  // The W partials of the workgroup's waves, merged with the log-sum-exp
  // rule into partial slot s of the slab: thread e takes channel e % 128 of
  // head e / 128.  Partials with m = -inf (no block, or every score -inf)
  // add nothing.
  __syncthreads();
  for (int e = threadIdx.x; e < NREP * kD; e += 64 * W) {
    const int h = e / kD, c = e % kD;
    float M = -INFINITY, Ls = 0.0f, acc = 0.0f;
#pragma unroll
    for (int v = 0; v < W; ++v) {
      const float mv = sm_p[v][h][kD];
      if (mv == -INFINITY) continue;
      const float lv = sm_p[v][h][kD + 1], av = sm_p[v][h][c];
      if (mv > M) {
        const float f = __expf(M - mv);   // 0 while M is -inf
        acc = fmaf(acc, f, av);
        Ls = fmaf(Ls, f, lv);
        M = mv;
      } else {
        const float f = __expf(mv - M);
        acc = fmaf(av, f, acc);
        Ls = fmaf(lv, f, Ls);
      }
    }
    float *dst = a.part + (((int64_t)b * a.Hq + hk * NREP + h) * a.S_total + s) * (kD + 4);
    dst[c] = acc;
    if (c == 0) *(float2 *)(dst + kD) = make_float2(M, Ls);
  }

  // A slab with one workgroup: it merges its slot and the window chunks'
  // slots (all written by its own waves) into out itself, and no combine
  // launch follows.  With more, the combine kernel merges the slots.
  if (n_groups > 1) return;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's slot stores are done
  __syncthreads();
  const int S = n_groups + n_window;   // slots of this slab; a.S_total is their stride
  for (int e = threadIdx.x; e < NREP * kD; e += 64 * W) {
    const int h = e / kD, c = e % kD;
    const int64_t row = (int64_t)b * a.Hq + hk * NREP + h;
    const float *pr = a.part + row * a.S_total * (int64_t)(kD + 4);
    float M = -INFINITY, Ls = 0.0f, acc = 0.0f;
    for (int s0 = 0; s0 < S; s0 += 16) {
      float mv[16], lv[16], av[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const float *ps = pr + (int64_t)min(s0 + u, S - 1) * (kD + 4);   // in bounds
        const float2 ml = *(const float2 *)(ps + kD);
        mv[u] = s0 + u < S ? ml.x : -INFINITY;
        lv[u] = ml.y;
        av[u] = ps[c];
      }
      float cm = mv[0];
#pragma unroll
      for (int u = 1; u < 16; ++u) cm = fmaxf(cm, mv[u]);
      if (cm == -INFINITY) continue;
      if (cm > M) {
        const float f = __expf(M - cm);   // 0 while M is -inf
        acc *= f;
        Ls *= f;
        M = cm;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (mv[u] == -INFINITY) continue;
        const float f = __expf(mv[u] - M);
        acc = fmaf(av[u], f, acc);
        Ls = fmaf(lv[u], f, Ls);
      }
    }
    const float inv = Ls > 0.0f ? 1.0f / Ls : 0.0f;
    a.out[row * kD + c] = acc * inv;
  }
}

template <bool S16, int KB = 2, int VB = KB>
static bool layout_is(const Layout &L) {
  using RC = Rec<S16, KB, VB>;
  return L.sb == RC::sb && L.rec == RC::bytes && L.kc == RC::kc && L.ks == RC::ks &&
         L.kz == RC::kz && L.vc == RC::vc && L.vs == RC::vs && L.vz == RC::vz;
}

bool decode_matrix_supported(const DecodeArgs &a) {
  // records of the 2-bit / G 32 / head_dim 128 shape (fp32 or fp16 scales),
  // copied 16 bytes at a time like the window rows and q
  return a.kb == 2 && a.vb == 2 && a.G == kG && a.D == kD &&
         (a.n_rep == 1 || a.n_rep == 2 || a.n_rep == 4) &&
         (layout_is<false>(a.L) || layout_is<true>(a.L)) && ((uintptr_t)a.L.blocks & 15) == 0 &&
         ((uintptr_t)a.k_res & 15) == 0 && ((uintptr_t)a.v_res & 15) == 0 &&
         ((uintptr_t)a.q & 15) == 0;
}

template <int KB, int VB>
static bool layout_is_any(const Layout &L) {
  return layout_is<false, KB, VB>(L) || layout_is<true, KB, VB>(L);
}

bool decode_matrix4_supported(const DecodeArgs &a, bool ragged) {
  // records of the G 32 / head_dim 128 shape with 4-bit keys and values (any
  // batch, contiguous or paged) or with one of the two 4-bit (a uniform
  // batch in a contiguous cache), fp32 or fp16 scales, copied 16 bytes at a
  // time like the window rows and q
  const bool both = a.kb == 4 && a.vb == 4 && layout_is_any<4, 4>(a.L);
  const bool mixed = (a.kb == 2 && a.vb == 4 && layout_is_any<2, 4>(a.L)) ||
                     (a.kb == 4 && a.vb == 2 && layout_is_any<4, 2>(a.L));
  return (both || (mixed && !ragged && a.L.pt == nullptr)) && a.G == kG && a.D == kD &&
         (a.n_rep == 1 || a.n_rep == 2 || a.n_rep == 4) &&
         ((uintptr_t)a.L.blocks & 15) == 0 && ((uintptr_t)a.k_res & 15) == 0 &&
         ((uintptr_t)a.v_res & 15) == 0 && ((uintptr_t)a.q & 15) == 0;
}

int decode_matrix_window_chunks(const DecodeArgs &a, int64_t n_main) {
  return matrix_window_chunks(a.t, n_main);
}

int decode_matrix_waves(const DecodeArgs &a) {
  return a.mask ? 4 : (a.kb == 4 || a.vb == 4 ? 6 : 8);
}

template <int NREP, bool RAGGED, bool PAGED, bool S16, int MODE = 0, int B4 = 2>
static void launch_rep(const DecodeArgs &a, dim3 grid, hipStream_t s, int64_t n_main,
                       int n_groups, int n_window, const MatrixRowArg<RAGGED> &rows) {
  // selected attention takes the mask from the stored scores
  if (a.mask && MODE != 2)
    hipLaunchKernelGGL((decode_matrix_kernel<NREP, MODE != 2, RAGGED, PAGED, S16, MODE, B4, B4>),
                       grid, dim3(256), 0, s, a, n_main, n_groups, n_window, rows);
  else
    hipLaunchKernelGGL((decode_matrix_kernel<NREP, false, RAGGED, PAGED, S16, MODE, B4, B4>), grid,
                       dim3(B4 == 2 ? 512 : 384), 0, s, a, n_main, n_groups, n_window, rows);
}

// B4: the code width of keys and values alike (2, or 4 for attention)
template <bool RAGGED, bool PAGED, bool S16, int MODE, int B4 = 2>
static void launch_layout(const DecodeArgs &a, dim3 grid, hipStream_t s, int64_t n_main,
                          int n_groups, int n_window, const MatrixRowArg<RAGGED> &rows) {
  switch (a.n_rep) {
    case 1:
      launch_rep<1, RAGGED, PAGED, S16, MODE, B4>(a, grid, s, n_main, n_groups, n_window, rows);
      break;
    case 2:
      launch_rep<2, RAGGED, PAGED, S16, MODE, B4>(a, grid, s, n_main, n_groups, n_window, rows);
      break;
    default:
      launch_rep<4, RAGGED, PAGED, S16, MODE, B4>(a, grid, s, n_main, n_groups, n_window, rows);
      break;
  }
}

// 4-bit keys, values or both: a uniform batch in a contiguous cache,
// attention (and the fused step) only.
template <int NREP, bool S16, int KB, int VB>
static void launch_rep4(const DecodeArgs &a, dim3 grid, hipStream_t s, int64_t n_main,
                        int n_groups, int n_window) {
  if (a.mask)
    hipLaunchKernelGGL((decode_matrix_kernel<NREP, true, false, false, S16, 0, KB, VB>), grid,
                       dim3(256), 0, s, a, n_main, n_groups, n_window, NoRows{});
  else
    hipLaunchKernelGGL((decode_matrix_kernel<NREP, false, false, false, S16, 0, KB, VB>), grid,
                       dim3(384), 0, s, a, n_main, n_groups, n_window, NoRows{});
}

template <bool S16, int KB, int VB>
static void launch_reps4(const DecodeArgs &a, dim3 grid, hipStream_t s, int64_t n_main,
                         int n_groups, int n_window) {
  switch (a.n_rep) {
    case 1: launch_rep4<1, S16, KB, VB>(a, grid, s, n_main, n_groups, n_window); break;
    case 2: launch_rep4<2, S16, KB, VB>(a, grid, s, n_main, n_groups, n_window); break;
    default: launch_rep4<4, S16, KB, VB>(a, grid, s, n_main, n_groups, n_window); break;
  }
}

template <bool S16>
static void launch_widths4(const DecodeArgs &a, dim3 grid, hipStream_t s, int64_t n_main,
                           int n_groups, int n_window) {
  if (a.kb == 4 && a.vb == 4)
    launch_reps4<S16, 4, 4>(a, grid, s, n_main, n_groups, n_window);
  else if (a.kb == 2)
    launch_reps4<S16, 2, 4>(a, grid, s, n_main, n_groups, n_window);
  else
    launch_reps4<S16, 4, 2>(a, grid, s, n_main, n_groups, n_window);
}

template <bool RAGGED, int MODE = 0>
static void launch_reps(const DecodeArgs &a, dim3 grid, hipStream_t s, int64_t n_main,
                        int n_groups, int n_window, const MatrixRowArg<RAGGED> &rows) {
  const bool s16 = a.L.sb == 2;
  if constexpr (MODE == 0) {
    // 4-bit keys and values: any batch, contiguous or paged
    if (a.kb == 4 && a.vb == 4) {
      if (a.L.pt && s16)
        launch_layout<RAGGED, true, true, 0, 4>(a, grid, s, n_main, n_groups, n_window, rows);
      else if (a.L.pt)
        launch_layout<RAGGED, true, false, 0, 4>(a, grid, s, n_main, n_groups, n_window, rows);
      else if (s16)
        launch_layout<RAGGED, false, true, 0, 4>(a, grid, s, n_main, n_groups, n_window, rows);
      else
        launch_layout<RAGGED, false, false, 0, 4>(a, grid, s, n_main, n_groups, n_window, rows);
      return;
    }
  }
  if (a.L.pt) {
    if (s16)
      launch_layout<RAGGED, true, true, MODE>(a, grid, s, n_main, n_groups, n_window, rows);
    else
      launch_layout<RAGGED, true, false, MODE>(a, grid, s, n_main, n_groups, n_window, rows);
  } else {
    if (s16)
      launch_layout<RAGGED, false, true, MODE>(a, grid, s, n_main, n_groups, n_window, rows);
    else
      launch_layout<RAGGED, false, false, MODE>(a, grid, s, n_main, n_groups, n_window, rows);
  }
}

hipError_t launch_decode_matrix(const DecodeArgs &a, int64_t n_main, int n_groups,
                                hipStream_t s) {
  const bool four = decode_matrix4_supported(a, false);
  if (!(four || decode_matrix_supported(a)) || a.t <= 0 || n_main < 0 || n_main % kBT != 0 ||
      n_main > a.n_vq || n_groups <= 0)
    return hipErrorInvalidValue;
  // the window role's key staging assumes whole key groups below n_kq
  if (a.n_kq % kG != 0) return hipErrorInvalidValue;
  // a fused step appends token t - 1 and keeps the value it pushes out of the
  // window (token t - 1 - R) out of the block role, whose workgroups read
  // quantized values from the cache; when the token completes a key block,
  // the window role quantizes keys [t - R, t), which lie above n_main
  if (a.t_new >= 0) {
    if (a.t_new != a.t - 1 || !a.k_new || !a.v_new) return hipErrorInvalidValue;
    if (a.t_new >= a.R && n_main > a.t_new - a.R) return hipErrorInvalidValue;
    if (a.t % a.R == 0 && n_main > a.t - a.R) return hipErrorInvalidValue;
  }
  const int n_window = decode_matrix_window_chunks(a, n_main);
  if ((int64_t)n_groups + n_window > a.S_total) return hipErrorInvalidValue;
  const int64_t n_wg = (int64_t)n_groups * a.H * a.B;
  if (n_wg > ((int64_t)1 << 25)) return hipErrorInvalidValue;   // 32-bit workgroup ids
  const bool mixed = four && a.kb != a.vb;
  if (mixed && a.L.sb == 2)
    launch_widths4<true>(a, dim3((unsigned)n_wg), s, n_main, n_groups, n_window);
  else if (mixed)
    launch_widths4<false>(a, dim3((unsigned)n_wg), s, n_main, n_groups, n_window);
  else
    launch_reps<false>(a, dim3((unsigned)n_wg), s, n_main, n_groups, n_window, NoRows{});
  return hipGetLastError();
}

// The selection workload on the matrix cores: the scores of every token
// (MODE 1; a.scores [B][Hq][cap]) and the attention over the selected ones
// (MODE 2; a.sel, partial slots as launch_decode_matrix).  Same plan as
// launch_decode_matrix; no fused step.
static hipError_t check_select_matrix(const DecodeArgs &a, int64_t n_main, int n_groups) {
  if (!decode_matrix_supported(a) || a.t <= 0 || n_main < 0 || n_main % kBT != 0 ||
      n_main > a.n_vq || n_groups <= 0 || a.t_new >= 0 || a.n_kq % kG != 0)
    return hipErrorInvalidValue;
  // score rows are copied 16 bytes at a time
  if (!a.scores || ((uintptr_t)a.scores & 15) != 0 || a.cap % 4 != 0 || a.cap > ((int64_t)1 << 26))
    return hipErrorInvalidValue;
  if ((int64_t)n_groups * a.H * a.B > ((int64_t)1 << 25)) return hipErrorInvalidValue;
  return hipSuccess;
}

hipError_t launch_scores_matrix(const DecodeArgs &a, int64_t n_main, int n_groups,
                                hipStream_t s) {
  const hipError_t e = check_select_matrix(a, n_main, n_groups);
  if (e != hipSuccess) return e;
  const int n_window = decode_matrix_window_chunks(a, n_main);
  // one largest-score entry per wave of every workgroup and per window chunk
  if (a.rmax && a.rmax_n != n_groups * decode_matrix_waves(a) + n_window)
    return hipErrorInvalidValue;
  const int64_t n_wg = (int64_t)n_groups * a.H * a.B;
  launch_reps<false, 1>(a, dim3((unsigned)n_wg), s, n_main, n_groups, n_window, NoRows{});
  return hipGetLastError();
}

hipError_t launch_selected_matrix(const DecodeArgs &a, int64_t n_main, int n_groups,
                                  hipStream_t s) {
  const hipError_t e = check_select_matrix(a, n_main, n_groups);
  if (e != hipSuccess) return e;
  if (!a.sel || !a.part) return hipErrorInvalidValue;
  const int n_window = decode_matrix_window_chunks(a, n_main);
  if ((int64_t)n_groups + n_window > a.S_total) return hipErrorInvalidValue;
  const int64_t n_wg = (int64_t)n_groups * a.H * a.B;
  launch_reps<false, 2>(a, dim3((unsigned)n_wg), s, n_main, n_groups, n_window, NoRows{});
  return hipGetLastError();
}

hipError_t launch_decode_matrix_rows(const DecodeArgs &a, const MatrixRows &rows, int n_shares,
                                     hipStream_t s) {
  if (!(decode_matrix_supported(a) || decode_matrix4_supported(a, true)) || a.B > kMaxRows ||
      n_shares <= 0 || n_shares > kMaxRows)
    return hipErrorInvalidValue;
  if (a.t_new >= 0 && (!a.k_new || !a.v_new)) return hipErrorInvalidValue;
  // every share names a row of the batch and a valid index among the row's
  // workgroups, and every row's slots fit the partial stride
  for (int u = 0; u < n_shares; ++u) {
    const uint32_t e = rows.share[u];
    const int b = (int)(e & 255u), si = (int)((e >> 8) & 4095u), n = (int)(e >> 20);
    if (b >= a.B || n <= 0 || si >= n) return hipErrorInvalidValue;
    const int64_t t = rows.t[b];
    if (t < (a.t_new >= 0 ? 1 : 0) || t > a.cap || t > a.t) return hipErrorInvalidValue;
    const RowSpan rs = row_span(t, a.R, a.t_new >= 0);
    const int64_t nm = matrix_main(rs, a.R);
    if ((int64_t)n + matrix_window_chunks(t, nm) > a.S_total) return hipErrorInvalidValue;
  }
  const int64_t n_wg = (int64_t)n_shares * a.H;
  launch_reps<true>(a, dim3((unsigned)n_wg), s, 0, n_shares, 0, rows);
  return hipGetLastError();
}

}  // namespace kivi
