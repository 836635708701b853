// pack.hip -- KIVI quantize-and-pack kernels for keys and values, and the
// fp16 window copy used by append.
//
// Method source: web page "Literature audit -- Group 2 (KV-cache compression
// primary sources)", section "1. KIVI -- kivi2024", list "Core algorithm
// (implementation-grade)", items 1-4.
#include "kivi_internal.hpp"

namespace kivi {

// KIVI item 2 for key group g (tokens g G .. g G + G - 1) of channel c of
// slab bh.  Two passes over the group's tokens (min/max, then codes) keep
// the code free of per-thread arrays; the second pass hits the caches.
__device__ __forceinline__ void quantize_key_group(const TokenSource &src, int64_t bh, int64_t g,
                                                   int c, const Layout &L) {
  const int G = L.G, bits = L.kb;
  const int64_t tau0 = g * G;
  const int per = 32 / bits;
  const int words = G / per;
  float mn = h2f(src.row(bh, tau0)[c]);
  float mx = mn;
  for (int i = 1; i < G; ++i) {
    const float x = h2f(src.row(bh, tau0 + i)[c]);
    mn = x < mn ? x : mn;
    mx = x > mx ? x : mx;
  }
  const float s = stored_scale(group_scale(mn, mx, bits), L);
  uint32_t *dst = L.key_codes(bh, g, c);
  for (int w = 0; w < words; ++w) {
    uint32_t word = 0;
    for (int e = 0; e < per; ++e) {
      const float x = h2f(src.row(bh, tau0 + w * per + e)[c]);
      word |= quant_code(x, mn, s, bits) << (bits * e);
    }
    dst[w] = word;
  }
  L.put_key_scale(bh, g, c, s);
  *L.key_zero(bh, g, c) = f2h_bits(mn);
}

// KIVI item 2: one thread per (channel, key group).  A key group is G
// consecutive tokens of one channel; its codes are packed along tokens.
__global__ void __launch_bounds__(128)
key_groups_kernel(TokenSource src, int64_t g_first, Layout L) {
  const int64_t bh = blockIdx.y;
  const int64_t g = g_first + blockIdx.x;
  for (int c = threadIdx.x; c < L.D; c += blockDim.x) quantize_key_group(src, bh, g, c, L);
}

// KIVI item 3: one thread per (token, value group).  A value group is G
// consecutive channels of one token; its codes are packed along channels.
__global__ void __launch_bounds__(256)
value_rows_kernel(TokenSource src, int64_t tau_first, int64_t n_rows, Layout L) {
  const int64_t bh = blockIdx.y;
  const int64_t r = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
  if (r >= n_rows) return;
  const int G = L.G, D = L.D, bits = L.vb;
  const int64_t tau = tau_first + r;
  const int per = 32 / bits;
  const int n_groups = D / G;
  const uint16_t *row = src.row(bh, tau);
  uint32_t *dst = L.value_codes(bh, tau);
  for (int g = threadIdx.x >> 6; g < n_groups; g += 4) {
    float mn = h2f(row[g * G]);
    float mx = mn;
    for (int i = 1; i < G; ++i) {
      const float x = h2f(row[g * G + i]);
      mn = x < mn ? x : mn;
      mx = x > mx ? x : mx;
    }
    const float s = stored_scale(group_scale(mn, mx, bits), L);
    for (int w = 0; w < G / per; ++w) {
      uint32_t word = 0;
      for (int e = 0; e < per; ++e)
        word |= quant_code(h2f(row[g * G + w * per + e]), mn, s, bits) << (bits * e);
      dst[(g * G) / per + w] = word;
    }
    L.put_value_scale(bh, tau, g, s);
    *L.value_zero(bh, tau, g) = f2h_bits(mn);
  }
}

// Copy rows of the new keys / values into their window slots.
__global__ void __launch_bounds__(256)
write_window_kernel(const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
                    uint16_t *__restrict__ k_res, uint16_t *__restrict__ v_res, int64_t t0,
                    int64_t n_new, int64_t k_from, int64_t v_from, int R, int D) {
  const int64_t bh = blockIdx.y;
  const int64_t t1 = t0 + n_new;
  const int64_t lo = k_from < v_from ? k_from : v_from;
  const int64_t first = lo > t0 ? lo : t0;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t tau = first + idx / D;
  const int c = (int)(idx % D);
  if (tau >= t1) return;
  const int64_t srow = (bh * n_new + (tau - t0)) * D + c;
  const int64_t drow = (bh * R + tau % R) * D + c;
  if (tau >= k_from) k_res[drow] = k_new[srow];
  if (tau >= v_from) v_res[drow] = v_new[srow];
}

// KIVI item 2, fast path for whole groups of a contiguous fp16 input (the
// pack entry point): one wave per (key group, slab).  Lane l reads channels
// [l D/64, (l + 1) D/64) of the group's G token rows straight from memory --
// each load instruction of the wave covers one whole row -- then reduces and
// packs them.  The code words of adjacent channels are adjacent in the
// record, so the wave stores one contiguous run of 16-byte stores.
// grid: (n_groups, BH); block: 64 threads.
template <int G, int D, int BITS>
__global__ void __launch_bounds__(64)
key_tiles_kernel(const uint16_t *__restrict__ x, int64_t T_in, int64_t g_first, Layout L) {
  constexpr int CPT = D / 64;                       // channels per thread
  static_assert(CPT == 1 || CPT == 2 || CPT == 4, "head_dim 64, 128 or 256");
  const int64_t bh = blockIdx.y;
  const int64_t g = blockIdx.x;                     // group within the input
  const int c0 = threadIdx.x * CPT;
  const uint16_t *src = x + (bh * T_in + g * G) * (int64_t)D + c0;
  float v[CPT][G];
  if constexpr (CPT == 1) {
    uint16_t w[G];
#pragma unroll
    for (int i = 0; i < G; ++i) w[i] = src[i * D];
#pragma unroll
    for (int i = 0; i < G; ++i) v[0][i] = h2f(w[i]);
  } else if constexpr (CPT == 2) {
    uint32_t w[G];
#pragma unroll
    for (int i = 0; i < G; ++i) w[i] = *(const uint32_t *)(src + i * D);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      v[0][i] = h2f((uint16_t)(w[i] & 0xffffu));
      v[1][i] = h2f((uint16_t)(w[i] >> 16));
    }
  } else {
    uint2 w[G];
#pragma unroll
    for (int i = 0; i < G; ++i) w[i] = *(const uint2 *)(src + i * D);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      v[0][i] = h2f((uint16_t)(w[i].x & 0xffffu));
      v[1][i] = h2f((uint16_t)(w[i].x >> 16));
      v[2][i] = h2f((uint16_t)(w[i].y & 0xffffu));
      v[3][i] = h2f((uint16_t)(w[i].y >> 16));
    }
  }
  constexpr int per = 32 / BITS;
  constexpr int words = G / per;
  const int64_t gd = g_first + g;                   // destination group
  uint32_t out[CPT * words];
  float sv[CPT];
  uint16_t zv[CPT];
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    float mn, mx;
    group_first_min_max(v[k], mn, mx);
    const float s = stored_scale(group_scale(mn, mx, BITS), L);
    const float r = __builtin_amdgcn_rcpf(s);
    uint32_t c[G];
    quant_codes_r(v[k], mn, s, r, BITS, c);
#pragma unroll
    for (int w = 0; w < words; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < per; ++e) word |= c[w * per + e] << (BITS * e);
      out[k * words + w] = word;
    }
    sv[k] = s;
    zv[k] = f2h_bits(mn);
  }
  uint32_t *dst = L.key_codes(bh, gd, c0);
  if constexpr ((CPT * words) % 4 == 0) {
    // the lane's run starts at a multiple of 16 bytes of a record
#pragma unroll
    for (int w = 0; w < CPT * words; w += 4)
      *(uint4 *)(dst + w) = make_uint4(out[w], out[w + 1], out[w + 2], out[w + 3]);
  } else {
#pragma unroll
    for (int w = 0; w < CPT * words; ++w) dst[w] = out[w];
  }
  uint16_t *dz = L.key_zero(bh, gd, c0);
#pragma unroll
  for (int k = 0; k < CPT; ++k) {
    L.put_key_scale(bh, gd, c0 + k, sv[k]);
    dz[k] = zv[k];
  }
}

// KIVI item 3, fast path for a contiguous fp16 input: one workgroup per 64
// tokens of one slab, which lie in one record (the first destination token
// is a multiple of 64).  Thread (group g, token t) reads its G channels
// straight from memory with 16-byte loads, then reduces and packs them, so
// for each group the 64 scales / zeros of the tile are one contiguous run;
// the code rows of the tile are staged in LDS and stored as one contiguous
// run of 16-byte stores.  grid: (ceil(n_rows / 64), BH); block: 256.
template <int D, int G, int BITS>
__global__ void __launch_bounds__(256)
value_tiles_kernel(const uint16_t *__restrict__ x, int64_t T_in, int64_t n_rows,
                   int64_t tau_first, Layout L) {
  const int64_t bh = blockIdx.y;
  const int64_t r0 = (int64_t)blockIdx.x * 64;
  const int rows = (int)(n_rows - r0 < 64 ? n_rows - r0 : 64);
  const int t = threadIdx.x & 63;
  constexpr int per = 32 / BITS;
  constexpr int n_groups = D / G;
  constexpr int kWords = D / per;                   // code words per token row
  __shared__ __attribute__((aligned(16))) uint32_t out_s[64 * kWords];
  for (int g = threadIdx.x >> 6; g < n_groups; g += 4) {
    if (t >= rows) continue;
    // the group's G channels of token t, straight from memory
    uint16_t v16[G];
    const uint16_t *src = x + (bh * T_in + r0 + t) * (int64_t)D + g * G;
#pragma unroll
    for (int k = 0; k < G / 8; ++k)
      *(uint4 *)(v16 + 8 * k) = *(const uint4 *)(src + 8 * k);
    float v[G];
#pragma unroll
    for (int i = 0; i < G; ++i) v[i] = h2f(v16[i]);
    float mn, mx;
    group_first_min_max(v, mn, mx);
    const float s = stored_scale(group_scale(mn, mx, BITS), L);
    const float r = __builtin_amdgcn_rcpf(s);
    const int64_t tau = tau_first + r0 + t;
    uint32_t *dst = out_s + t * kWords + (g * G) / per;
    // (a branch per value: the branch-free form doubles this kernel's
    // registers, and its occupancy matters more than the branches)
#pragma unroll
    for (int w = 0; w < G / per; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < per; ++e)
        word |= quant_code_r(v[w * per + e], mn, s, r, BITS) << (BITS * e);
      dst[w] = word;
    }
    L.put_value_scale(bh, tau, g, s);
    *L.value_zero(bh, tau, g) = f2h_bits(mn);
  }
  __syncthreads();
  // the tile's rows are consecutive tokens of one record: one contiguous run
  uint32_t *run = L.value_codes(bh, tau_first + r0);
  for (int i = threadIdx.x; i < rows * kWords / 4; i += 256)
    *(uint4 *)(run + 4 * i) = *(const uint4 *)(out_s + 4 * i);
}

bool pack_tiles_supported(int D, int G, int bits) {
  const int per = 32 / bits;
  if (!(D == 64 || D == 128 || D == 256)) return false;
  const int cpl = D / 64;
  if ((G & (G - 1)) != 0 || G < 16 || G < cpl || per < cpl || D % G != 0) return false;
  return G * D * 2 <= 16384 && G <= 64;
}

hipError_t launch_key_tiles(const uint16_t *x, int64_t T_in, int64_t n_rows, int64_t g_first,
                            int64_t BH, const Layout &L, hipStream_t s) {
  const int G = L.G, D = L.D, bits = L.kb;
  const int64_t n_groups = n_rows / G;
  if (n_groups <= 0 || BH <= 0) return hipSuccess;
  if (!pack_tiles_supported(D, G, bits) || n_rows % G != 0 || n_rows > T_in)
    return hipErrorInvalidValue;
  dim3 grid((unsigned)n_groups, (unsigned)BH);
#define KIVI_KT(GG, DD)                                                                        \
  if (G == GG && D == DD) {                                                                     \
    if (bits == 2)                                                                              \
      hipLaunchKernelGGL((key_tiles_kernel<GG, DD, 2>), grid, dim3(64), 0, s, x, T_in,        \
                         g_first, L);                                                           \
    else                                                                                        \
      hipLaunchKernelGGL((key_tiles_kernel<GG, DD, 4>), grid, dim3(64), 0, s, x, T_in,        \
                         g_first, L);                                                           \
    return hipGetLastError();                                                                   \
  }
  KIVI_KT(16, 64) KIVI_KT(32, 64) KIVI_KT(64, 64)
  KIVI_KT(16, 128) KIVI_KT(32, 128) KIVI_KT(64, 128)
  KIVI_KT(16, 256) KIVI_KT(32, 256)
#undef KIVI_KT
  return hipErrorInvalidValue;
}

hipError_t launch_value_tokens(const uint16_t *x, int64_t T_in, int64_t n_rows, int64_t tau_first,
                               int64_t BH, const Layout &L, hipStream_t s) {
  const int G = L.G, D = L.D, bits = L.vb;
  if (n_rows <= 0 || BH <= 0) return hipSuccess;
  if (!pack_tiles_supported(D, G, bits) || n_rows > T_in) return hipErrorInvalidValue;
  if (tau_first % 64 != 0) {
    // the tile kernel needs its 64 tokens in one record; any other
    // destination takes the per-row kernel
    TokenSource src{nullptr, x, tau_first, T_in, 1, D};
    return launch_value_rows(src, tau_first, n_rows, BH, L, s);
  }
  dim3 grid((unsigned)((n_rows + 63) / 64), (unsigned)BH);
#define KIVI_VT(DD, GG)                                                                         \
  if (D == DD && G == GG) {                                                                     \
    if (bits == 2)                                                                              \
      hipLaunchKernelGGL((value_tiles_kernel<DD, GG, 2>), grid, dim3(256), 0, s, x, T_in,      \
                         n_rows, tau_first, L);                                                 \
    else                                                                                        \
      hipLaunchKernelGGL((value_tiles_kernel<DD, GG, 4>), grid, dim3(256), 0, s, x, T_in,      \
                         n_rows, tau_first, L);                                                 \
    return hipGetLastError();                                                                   \
  }
  KIVI_VT(64, 16) KIVI_VT(64, 32) KIVI_VT(64, 64)
  KIVI_VT(128, 16) KIVI_VT(128, 32) KIVI_VT(128, 64)
  KIVI_VT(256, 16) KIVI_VT(256, 32) KIVI_VT(256, 64)
#undef KIVI_VT
  return hipErrorInvalidValue;
}

// One decode step of append (one new token per slab), fused: quantize the
// value that leaves the window (KIVI item 3; token t0 - R, when t0 >= R),
// then put the new value -- and the new key, unless it completes a key block
// -- into slot t0 % R (KIVI item 4).  Block: D threads rounded up to a wave,
// thread c owns channel c.  Group min/max and the packing of codes into
// words are lane reductions, so G and 32 / bits must be powers of two no
// larger than a wave.
__device__ __forceinline__ void append_one_slab(const uint16_t *__restrict__ k_new,
                                                const uint16_t *__restrict__ v_new,
                                                uint16_t *__restrict__ k_res,
                                                uint16_t *__restrict__ v_res, int64_t bh,
                                                int64_t t0, int R, bool key_to_window,
                                                const Layout &L) {
  const int c = threadIdx.x;
  const int D = L.D, G = L.G, bits = L.vb;
  const bool on = c < D;
  const int64_t slot = (bh * R + t0 % R) * D + c;
  if (t0 >= R) {
    // every lane of a group takes part in the reductions; lanes past D hold
    // a copy of channel 0 of their group's wave and write nothing
    const float x = h2f(v_res[on ? slot : (bh * R + t0 % R) * D]);
    float mn = x, mx = x;
    lanes_first_min_max(mn, mx, c, G);
    const float sc = stored_scale(group_scale(mn, mx, bits), L);
    const int per = 32 / bits;
    uint32_t w = quant_code(x, mn, sc, bits) << (bits * (c % per));
    for (int o = 1; o < per; o <<= 1) w |= __shfl_xor(w, o);
    const int64_t tau = t0 - R;
    if (on && c % per == 0) L.value_codes(bh, tau)[c / per] = w;
    if (on && c % G == 0) {
      L.put_value_scale(bh, tau, c / G, sc);
      *L.value_zero(bh, tau, c / G) = f2h_bits(mn);
    }
  }
  if (on) {
    v_res[slot] = v_new[bh * D + c];
    if (key_to_window) k_res[slot] = k_new[bh * D + c];
  }
}

// grid: BH; every slab appends token t0.
__global__ void __launch_bounds__(256)
append_one_kernel(const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
                  uint16_t *__restrict__ k_res, uint16_t *__restrict__ v_res, int64_t t0,
                  int R, bool key_to_window, Layout L) {
  append_one_slab(k_new, v_new, k_res, v_res, blockIdx.x, t0, R, key_to_window, L);
}

// A decode step of a ragged batch: slab bh (row b = bh / H) appends token t0
// = rows.n[b].  When that token completes a key block (t0 + 1 a multiple of
// R), thread c then quantizes channel c of the block's key groups (KIVI
// item 2) from the window slots and the new key, which never enters the
// window.  grid: BH.
__global__ void __launch_bounds__(256)
append_one_rows_kernel(const uint16_t *__restrict__ k_new, const uint16_t *__restrict__ v_new,
                       uint16_t *__restrict__ k_res, uint16_t *__restrict__ v_res, int H, int R,
                       Layout L, RowCounts rows) {
  const int64_t bh = blockIdx.x;
  const int64_t t0 = rows.n[bh / H];
  const bool completes = (t0 + 1) % R == 0;
  append_one_slab(k_new, v_new, k_res, v_res, bh, t0, R, !completes, L);
  if (completes && (int)threadIdx.x < L.D) {
    const TokenSource src{k_res, k_new, t0, 1, R, L.D};
    for (int64_t g = (t0 + 1 - R) / L.G; g < (t0 + 1) / L.G; ++g)
      quantize_key_group(src, bh, g, threadIdx.x, L);
  }
}

hipError_t launch_append_one(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_res,
                             uint16_t *v_res, int64_t t0, int64_t BH, int R, bool key_to_window,
                             const Layout &L, hipStream_t s) {
  if (!append_one_supported(L.D, L.G, L.vb) || BH <= 0) return hipErrorInvalidValue;
  const int threads = (L.D + 63) / 64 * 64;
  hipLaunchKernelGGL(append_one_kernel, dim3((unsigned)BH), dim3(threads), 0, s, k_new, v_new,
                     k_res, v_res, t0, R, key_to_window, L);
  return hipGetLastError();
}

hipError_t launch_append_one_rows(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_res,
                                  uint16_t *v_res, int64_t BH, int H, int R,
                                  const RowCounts &rows, const Layout &L, hipStream_t s) {
  if (!append_one_supported(L.D, L.G, L.vb) || BH <= 0 || H <= 0 || BH % H != 0 ||
      BH / H > kMaxRows || R % L.G != 0)
    return hipErrorInvalidValue;
  for (int64_t b = 0; b < BH / H; ++b)
    if (rows.n[b] < 0 || rows.n[b] >= L.nrec * kRecTokens) return hipErrorInvalidValue;
  const int threads = (L.D + 63) / 64 * 64;
  hipLaunchKernelGGL(append_one_rows_kernel, dim3((unsigned)BH), dim3(threads), 0, s, k_new,
                     v_new, k_res, v_res, H, R, L, rows);
  return hipGetLastError();
}

hipError_t launch_key_groups(const TokenSource &src, int64_t g_first, int64_t n_groups,
                             int64_t BH, const Layout &L, hipStream_t s) {
  if (n_groups <= 0 || BH <= 0) return hipSuccess;
  dim3 grid((unsigned)n_groups, (unsigned)BH);
  hipLaunchKernelGGL(key_groups_kernel, grid, dim3(128), 0, s, src, g_first, L);
  return hipGetLastError();
}

hipError_t launch_value_rows(const TokenSource &src, int64_t tau_first, int64_t n_rows,
                             int64_t BH, const Layout &L, hipStream_t s) {
  if (n_rows <= 0 || BH <= 0) return hipSuccess;
  dim3 grid((unsigned)((n_rows + 63) / 64), (unsigned)BH);
  hipLaunchKernelGGL(value_rows_kernel, grid, dim3(256), 0, s, src, tau_first, n_rows, L);
  return hipGetLastError();
}

hipError_t launch_write_window(const uint16_t *k_new, const uint16_t *v_new, uint16_t *k_res,
                               uint16_t *v_res, int64_t t0, int64_t n_new, int64_t k_from,
                               int64_t v_from, int64_t BH, int R, int D, hipStream_t s) {
  const int64_t t1 = t0 + n_new;
  int64_t lo = k_from < v_from ? k_from : v_from;
  if (lo < t0) lo = t0;
  const int64_t n = (t1 - lo) * D;
  if (n <= 0 || BH <= 0) return hipSuccess;
  dim3 grid((unsigned)((n + 255) / 256), (unsigned)BH);
  hipLaunchKernelGGL(write_window_kernel, grid, dim3(256), 0, s, k_new, v_new, k_res, v_res, t0,
                     n_new, k_from, v_from, R, D);
  return hipGetLastError();
}

}  // namespace kivi
