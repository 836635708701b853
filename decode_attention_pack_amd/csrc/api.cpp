// api.cpp -- the C ABI of libkivi.so: argument validation, planning of the
// decode split, and kernel dispatch.  Declarations and the storage contract
// are in include/kivi.h.
//
// Method source: web page "Literature audit -- Group 2 (KV-cache compression
// primary sources)", section "1. KIVI -- kivi2024", list "Core algorithm
// (implementation-grade)", items 1-5.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "../../include/kivi.h"
#include "kivi_internal.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return KIVI_OK;
  return fail(KIVI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool bits_ok(int bits) { return bits == 2 || bits == 4; }

// Shape rules shared by every entry point.
int check_shape(int32_t D, int32_t bits, int32_t G, const char *who) {
  if (!bits_ok(bits)) return fail(KIVI_ERR_INVALID_ARG, "%s: bits must be 2 or 4 (got %d)", who, bits);
  if (G <= 0 || G % (32 / bits) != 0 || kivi::kRecTokens % G != 0)
    return fail(KIVI_ERR_INVALID_ARG, "%s: group %d must divide %d and be a multiple of %d", who, G,
                kivi::kRecTokens, 32 / bits);
  if (D <= 0 || D > 256 || D % G != 0)
    return fail(KIVI_ERR_INVALID_ARG, "%s: head_dim %d must be a multiple of group %d, at most 256",
                who, D, G);
  return KIVI_OK;
}

// Slabs (batch rows x heads) index the second grid dimension of the pack and
// append kernels, whose limit is 65535 workgroups.
constexpr int64_t kMaxSlabs = 65535;

int check_cache(const kivi_cache *c, const char *who) {
  if (!c) return fail(KIVI_ERR_INVALID_ARG, "%s: cache is NULL", who);
  if (c->batch <= 0 || c->n_kv_heads <= 0)
    return fail(KIVI_ERR_INVALID_ARG, "%s: batch and n_kv_heads must be positive", who);
  if ((int64_t)c->batch * c->n_kv_heads > kMaxSlabs)
    return fail(KIVI_ERR_INVALID_ARG, "%s: batch x n_kv_heads = %lld passes %lld", who,
                (long long)c->batch * c->n_kv_heads, (long long)kMaxSlabs);
  int rc = check_shape(c->head_dim, c->k_bits, c->group, who);
  if (rc) return rc;
  rc = check_shape(c->head_dim, c->v_bits, c->group, who);
  if (rc) return rc;
  if (c->residual <= 0 || c->residual % c->group != 0)
    return fail(KIVI_ERR_INVALID_ARG, "%s: residual %d must be a positive multiple of group %d", who,
                c->residual, c->group);
  if (c->capacity <= 0 || c->capacity % c->residual != 0 || c->capacity % kivi::kRecTokens != 0)
    return fail(KIVI_ERR_INVALID_ARG,
                "%s: capacity %lld must be a positive multiple of residual %d and of %d", who,
                (long long)c->capacity, c->residual, kivi::kRecTokens);
  if (c->row_tokens) {
    if (c->batch > kivi::kMaxRows)
      return fail(KIVI_ERR_INVALID_ARG, "%s: a ragged batch holds at most %d rows (batch %d)", who,
                  kivi::kMaxRows, c->batch);
    for (int32_t b = 0; b < c->batch; ++b)
      if (c->row_tokens[b] < 0 || c->row_tokens[b] > c->capacity)
        return fail(KIVI_ERR_INVALID_ARG, "%s: row_tokens[%d] = %lld outside [0, capacity]", who,
                    b, (long long)c->row_tokens[b]);
  } else if (c->n_tokens < 0 || c->n_tokens > c->capacity) {
    return fail(KIVI_ERR_INVALID_ARG, "%s: n_tokens %lld outside [0, capacity]", who,
                (long long)c->n_tokens);
  }
  if (!c->blocks || !c->k_res || !c->v_res)
    return fail(KIVI_ERR_INVALID_ARG, "%s: a cache array pointer is NULL", who);
  if (c->scale_fp16 != 0 && c->scale_fp16 != 1)
    return fail(KIVI_ERR_INVALID_ARG, "%s: scale_fp16 must be 0 or 1 (got %d)", who, c->scale_fp16);
  if (c->page_table) {
    if (((uintptr_t)c->page_table & 3) != 0)
      return fail(KIVI_ERR_INVALID_ARG, "%s: page_table must be 4-byte aligned", who);
    if (c->n_pages <= 0 || c->n_pages > ((int64_t)1 << 40) / c->n_kv_heads)
      return fail(KIVI_ERR_INVALID_ARG, "%s: n_pages %lld outside [1, 2^40 / n_kv_heads]", who,
                  (long long)c->n_pages);
  }
  if (((uintptr_t)c->blocks & 15) != 0 || ((uintptr_t)c->k_res & 15) != 0 ||
      ((uintptr_t)c->v_res & 15) != 0)
    return fail(KIVI_ERR_INVALID_ARG, "%s: blocks, k_res and v_res must be 16-byte aligned", who);
  return KIVI_OK;
}

kivi::Layout layout_of(const kivi_cache *c) {
  kivi::Layout L = kivi::make_layout(c->blocks, c->head_dim, c->k_bits, c->v_bits, c->group,
                                     c->capacity, c->scale_fp16 != 0);
  L.pt = c->page_table;
  L.n_pages = c->n_pages;
  L.H = c->n_kv_heads;
  return L;
}

// Token counts of the rows of a checked cache: per row (ragged) or n_tokens
// for every row.
struct Rows {
  bool ragged = false;
  int64_t t_max = 0, t_sum = 0;
  kivi::RowCounts n{};
};
Rows rows_of(const kivi_cache *c) {
  Rows r;
  r.ragged = c->row_tokens != nullptr;
  if (!r.ragged) {
    r.t_max = c->n_tokens;
    r.t_sum = c->n_tokens * c->batch;
    return r;
  }
  for (int32_t b = 0; b < c->batch; ++b) {
    const int64_t t = c->row_tokens[b];
    r.n.n[b] = (int32_t)t;
    r.t_max = t > r.t_max ? t : r.t_max;
    r.t_sum += t;
  }
  return r;
}

// After a call that changed a ragged cache's counts: n_tokens = the longest row.
void set_longest(kivi_cache *c) {
  int64_t m = 0;
  for (int32_t b = 0; b < c->batch; ++b) m = c->row_tokens[b] > m ? c->row_tokens[b] : m;
  c->n_tokens = m;
}

// Row b of a cache alone, as a uniform cache of batch 1 holding t tokens.
kivi_cache row_view(const kivi_cache *c, int32_t b, int64_t t) {
  kivi_cache v = *c;
  const size_t rb = kivi::make_layout(nullptr, c->head_dim, c->k_bits, c->v_bits, c->group, 0,
                                      c->scale_fp16 != 0)
                        .rec;
  const int64_t slabs = (int64_t)b * c->n_kv_heads;
  v.batch = 1;
  v.n_tokens = t;
  v.row_tokens = nullptr;
  if (c->page_table)   // the same page pool; the row's line of the table
    v.page_table = c->page_table + (int64_t)b * (c->capacity / kivi::kRecTokens);
  else
    v.blocks = c->blocks + slabs * (c->capacity / kivi::kRecTokens) * (int64_t)rb;
  v.k_res = c->k_res + slabs * c->residual * c->head_dim;
  v.v_res = c->v_res + slabs * c->residual * c->head_dim;
  return v;
}

int check_pack(const kivi_cache *dst, const void *x, int64_t T, int64_t off, bool keys,
               const char *who) {
  int rc = check_cache(dst, who);
  if (rc) return rc;
  if (T < 0 || off < 0) return fail(KIVI_ERR_INVALID_ARG, "%s: T and offset must be >= 0", who);
  if (keys && (T % dst->group != 0 || off % dst->group != 0))
    return fail(KIVI_ERR_INVALID_ARG, "%s: T (%lld) and offset (%lld) must be multiples of group %d",
                who, (long long)T, (long long)off, dst->group);
  if (off + T > dst->capacity)
    return fail(KIVI_ERR_CAPACITY, "%s: tokens [%lld, %lld) pass capacity %lld", who,
                (long long)off, (long long)(off + T), (long long)dst->capacity);
  if (T > 0 && !x) return fail(KIVI_ERR_INVALID_ARG, "%s: NULL input", who);
  return KIVI_OK;
}

int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

constexpr int kGenericMinSplit = 256;
constexpr int kMatrixBlock = 128;   // tokens per block of the matrix-core kernel
constexpr int kVectorStep = 128;    // tokens per step of the vector kernel's four waves
// Vector kernel: workgroups to aim for.  Three waves per SIMD hold 768
// workgroups at once; fewer, longer splits measure faster than twice as
// many short ones (less per-split set-up and merge work).
constexpr int kVectorWorkgroups = 2048;
constexpr int kTargetWorkgroups = 4096;   // scalar kernel
// Compute units of the current device (the matrix kernel plans one
// workgroup per CU); 256 when it cannot be queried.
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

struct Plan {
  bool matrix = false;
  int64_t n_main = 0;           // tokens [0, n_main) in the matrix kernel's block role
  int n_groups_matrix = 0;      // matrix-kernel workgroups per slab
  int n_window = 0;             // 32-token chunks of [n_main, t) in its window role
  bool vector = false;          // vector kernel instead of the scalar one
  int tps_generic = 0;          // vector / scalar kernel (shapes the matrix kernel does not cover)
  int n_split_generic = 0;
  int S_total = 0;
  bool combine = true;          // a combine launch follows
  // ragged batch, matrix kernel: the workgroup shares (per KV head) and the
  // slots each row's combine merges (0: the row's single workgroup wrote it)
  int n_shares = 0;
  kivi::MatrixRows mrows{};
  kivi::RowCounts slots{};
};

int head_chunks(int n_rep) { return (n_rep + 7) / 8; }

int64_t ceil_div(int64_t x, int64_t y) { return (x + y - 1) / y; }

// Matrix-kernel plan of a ragged batch, about one workgroup per CU in all:
// every row starts with one workgroup per KV head, and the others go one at
// a time to the row with the most work per workgroup, a row taking at most
// one per `waves` items (blocks and window chunks).  Work counts a window
// chunk (32 tokens, scalar arithmetic and a load it waits for) as two
// 128-token blocks, about what it costs a wave.  With tps_req, a workgroup
// per tps_req tokens of a row.
int plan_matrix_rows(const kivi_cache *c, const Rows &r, int32_t tps_req, int waves, bool fused,
                     Plan &p, const char *who) {
  const int B = c->batch, R = c->residual;
  int64_t work[kivi::kMaxRows], cap[kivi::kMaxRows], groups[kivi::kMaxRows];
  int nwin[kivi::kMaxRows];
  for (int b = 0; b < B; ++b) {
    const int64_t t = r.n.n[b] + (fused ? 1 : 0);
    p.mrows.t[b] = (int32_t)t;
    const kivi::RowSpan rs = kivi::row_span(t, R, fused);
    const int64_t nm = kivi::matrix_main(rs, R);
    nwin[b] = kivi::matrix_window_chunks(t, nm);
    work[b] = nm / kMatrixBlock + 2 * nwin[b];
    cap[b] = max64(1, ceil_div(nm / kMatrixBlock + nwin[b], waves));
    if (tps_req > 0) {
      const int64_t tps = ceil_div(tps_req, kMatrixBlock) * kMatrixBlock;
      groups[b] = max64(1, ceil_div(nm, tps));
    }
  }
  int64_t used = 0;
  if (tps_req == 0) {
    const int64_t target = std::min<int64_t>(
        kivi::kMaxRows,
        max64(B, (int64_t)device_cus() * (c->k_bits == 4 || c->v_bits == 4 ? 1 : 8 / waves) /
                     c->n_kv_heads));
    for (int b = 0; b < B; ++b) groups[b] = 1;
    used = B;
    while (used < target) {
      int best = -1;
      for (int b = 0; b < B; ++b)
        if (groups[b] < cap[b] &&
            (best < 0 || work[b] * groups[best] > work[best] * groups[b]))
          best = b;
      if (best < 0) break;
      ++groups[best];
      ++used;
    }
  } else {
    for (int b = 0; b < B; ++b) used += groups[b];
    if (used > kivi::kMaxRows)
      return fail(KIVI_ERR_INVALID_ARG,
                  "%s: tokens_per_split %d gives %lld workgroups per KV head for a ragged batch; "
                  "at most %d", who, tps_req, (long long)used, kivi::kMaxRows);
  }
  int u = 0;
  p.S_total = 1;
  p.combine = false;
  for (int b = 0; b < B; ++b) {
    for (int64_t g = 0; g < groups[b]; ++g)
      p.mrows.share[u++] = (uint32_t)b | ((uint32_t)g << 8) | ((uint32_t)groups[b] << 20);
    const int S = (int)groups[b] + nwin[b];
    p.S_total = std::max(p.S_total, S);
    p.slots.n[b] = groups[b] > 1 ? S : 0;
    p.combine = p.combine || groups[b] > 1;
  }
  p.n_shares = u;
  return KIVI_OK;
}

// Whether the matrix kernel takes this call: the 2-bit shapes it handles
// (any batch), and 4-bit ones of a uniform batch -- by default where several
// query heads share a KV head (the vector kernel reads the cache once per
// pair of query heads), and with one from three blocks per wave of a
// workgroup on (the vector kernel is faster on shorter rows; measured on B64
// x 32 heads at 2049 tokens, 15 blocks: 138 against 177 us; on B8 x 32 heads
// at 4065 tokens, 30 blocks: 55 against 46 us).
bool matrix_wanted(const kivi::DecodeArgs &a, int32_t path, bool ragged) {
  if (!(path == KIVI_PATH_AUTO || path == KIVI_PATH_MATRIX) || a.t <= 0) return false;
  if (kivi::decode_matrix_supported(a)) return true;
  if (!kivi::decode_matrix4_supported(a, ragged)) return false;
  if (path == KIVI_PATH_MATRIX || a.n_rep >= 2) return true;
  const int64_t blocks =
      kivi::matrix_main(kivi::row_span(a.t, a.R, a.t_new >= 0), a.R) / kMatrixBlock;
  return blocks >= 3 * kivi::decode_matrix_waves(a);
}

// Split plan.  Deterministic in (shape, token counts, options).
int make_plan(const kivi_cache *c, int32_t Hq, int32_t tps_req, int32_t path,
              const kivi::DecodeArgs &a, const Rows &r, Plan &p, const char *who) {
  const int64_t t = a.t;
  const int n_rep = Hq / c->n_kv_heads;
  const int64_t units = (int64_t)c->batch * c->n_kv_heads;
  p.matrix = matrix_wanted(a, path, r.ragged);
  if (p.matrix && r.ragged)
    return plan_matrix_rows(c, r, tps_req, kivi::decode_matrix_waves(a), a.t_new >= 0, p, who);
  if (p.matrix) {
    p.n_main = kivi::matrix_main(kivi::row_span(t, a.R, a.t_new >= 0), a.R);
    p.n_window = kivi::decode_matrix_window_chunks(a, p.n_main);
    const int64_t blocks = p.n_main / kMatrixBlock;
    const int waves = kivi::decode_matrix_waves(a);
    int64_t groups;
    if (tps_req == 0) {
      // one workgroup per CU (two for the four-wave masked variant of 2-bit
      // codes), no more than the blocks and window chunks keep busy
      const int64_t per_cu = a.kb == 4 || a.vb == 4 ? 1 : 8 / waves;
      const int64_t target = max64(1, device_cus() * per_cu / units);
      groups = std::min(target, max64(1, ceil_div(blocks + p.n_window, waves)));
    } else {
      // a workgroup per tps_req tokens (rounded up to whole blocks)
      const int64_t tps = ceil_div(tps_req, kMatrixBlock) * kMatrixBlock;
      groups = max64(1, ceil_div(p.n_main, tps));
    }
    p.n_groups_matrix = (int)groups;
    // one partial slot per workgroup, then one per window chunk
    p.S_total = (int)(groups + p.n_window);
    // a slab with a single workgroup writes its output itself
    p.combine = groups > 1;
    return KIVI_OK;
  }
  p.vector = (path == KIVI_PATH_AUTO || path == KIVI_PATH_VECTOR) &&
             kivi::decode_vector_supported(a);
  // a ragged batch sizes its splits by the mean row; rows shorter than the
  // longest leave their last splits empty
  const int64_t t_eff = r.ragged ? ceil_div(r.t_sum, c->batch) : t;
  int64_t tps = tps_req;
  if (tps == 0 && p.vector) {
    // whole 4-group steps (one group per wave), about kVectorWorkgroups
    // workgroups (a workgroup per two query heads of a slab)
    const int64_t vunits = units * (n_rep == 1 ? 1 : n_rep / 2);
    const int64_t splits = max64(1, kVectorWorkgroups / vunits);
    tps = max64(1, ((t_eff + splits - 1) / splits + kVectorStep - 1) / kVectorStep) * kVectorStep;
  } else if (tps == 0) {
    const int64_t gunits = units * head_chunks(n_rep);
    const int64_t splits = max64(1, kTargetWorkgroups / gunits);
    tps = ((t_eff + splits - 1) / splits + kGenericMinSplit - 1) / kGenericMinSplit *
          kGenericMinSplit;
    tps = max64(tps, kGenericMinSplit);
  }
  p.tps_generic = (int)tps;
  p.n_split_generic = (int)max64(1, (t + tps - 1) / tps);
  p.S_total = p.n_split_generic;
  // a single vector-kernel split writes the output itself
  p.combine = !(p.vector && p.n_split_generic == 1);
  return KIVI_OK;
}

// Upper bound on partial slots for any n_tokens <= capacity.
int64_t max_slots(const kivi_cache *c, int32_t tps_req) {
  // the matrix kernel's window is at most one block + R tokens long
  const int64_t n_window = (kMatrixBlock + (int64_t)c->residual + 31) / 32 + 1;
  const int64_t blocks = ceil_div(c->capacity, kMatrixBlock);
  if (tps_req == 0) {
    // matrix kernel: at most ceil((blocks + window) / waves) workgroups of at
    // most 8 waves; the other kernels split at least 128 tokens at a time
    return blocks + 2 * n_window + 8 + 1;
  }
  // matrix kernel: one workgroup of at most 8 waves per tps_req tokens
  // (rounded up to whole blocks); the other kernels: one slot per split
  const int64_t m = 8 * ceil_div(c->capacity, ceil_div(tps_req, kMatrixBlock) * kMatrixBlock);
  const int64_t g = ceil_div(c->capacity, tps_req);
  return std::max(m, g) + 8 + n_window + 1;
}



}  // namespace

extern "C" {

const char *kivi_status_string(int status) {
  switch (status) {
    case KIVI_OK: return "ok";
    case KIVI_ERR_INVALID_ARG: return "invalid argument";
    case KIVI_ERR_CAPACITY: return "capacity exceeded";
    case KIVI_ERR_WORKSPACE: return "workspace too small";
    case KIVI_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char *kivi_last_error(void) { return g_last_error.c_str(); }

size_t kivi_record_bytes(int32_t head_dim, int32_t k_bits, int32_t v_bits, int32_t group) {
  return kivi_record_bytes_ex(head_dim, k_bits, v_bits, group, 0);
}

size_t kivi_record_bytes_ex(int32_t head_dim, int32_t k_bits, int32_t v_bits, int32_t group,
                            int32_t scale_fp16) {
  if (head_dim <= 0 || head_dim > 256 || (scale_fp16 != 0 && scale_fp16 != 1)) return 0;
  return (size_t)kivi::make_layout(nullptr, head_dim, k_bits, v_bits, group, 0, scale_fp16 != 0)
      .rec;
}

int kivi_pack_keys(const kivi_cache *dst, const void *k_fp16, int64_t T, int64_t dst_token_offset,
                   void *stream) {
  int rc = check_pack(dst, k_fp16, T, dst_token_offset, true, "kivi_pack_keys");
  if (rc) return rc;
  if (T == 0) return KIVI_OK;
  const kivi::Layout L = layout_of(dst);
  const int64_t BH = (int64_t)dst->batch * dst->n_kv_heads;
  const int G = dst->group, D = dst->head_dim;
  if (kivi::pack_tiles_supported(D, G, dst->k_bits))
    return hip_status(kivi::launch_key_tiles((const uint16_t *)k_fp16, T, T, dst_token_offset / G,
                                             BH, L, (hipStream_t)stream),
                      "kivi_pack_keys");
  kivi::TokenSource src{nullptr, (const uint16_t *)k_fp16, dst_token_offset, T, 1, D};
  return hip_status(kivi::launch_key_groups(src, dst_token_offset / G, T / G, BH, L,
                                            (hipStream_t)stream),
                    "kivi_pack_keys");
}

int kivi_pack_values(const kivi_cache *dst, const void *v_fp16, int64_t T,
                     int64_t dst_token_offset, void *stream) {
  int rc = check_pack(dst, v_fp16, T, dst_token_offset, false, "kivi_pack_values");
  if (rc) return rc;
  if (T == 0) return KIVI_OK;
  const kivi::Layout L = layout_of(dst);
  const int64_t BH = (int64_t)dst->batch * dst->n_kv_heads;
  const int G = dst->group, D = dst->head_dim;
  if (kivi::pack_tiles_supported(D, G, dst->v_bits))
    return hip_status(kivi::launch_value_tokens((const uint16_t *)v_fp16, T, T, dst_token_offset,
                                                BH, L, (hipStream_t)stream),
                      "kivi_pack_values");
  kivi::TokenSource src{nullptr, (const uint16_t *)v_fp16, dst_token_offset, T, 1, D};
  return hip_status(kivi::launch_value_rows(src, dst_token_offset, T, BH, L, (hipStream_t)stream),
                    "kivi_pack_values");
}

}  // extern "C"

namespace {

int append_uniform(kivi_cache *c, const void *k_new_fp16, const void *v_new_fp16, int64_t n_new,
                   void *stream);

// kivi_append on a ragged batch: every row takes n_new tokens at its own
// length.  A single token per row (the decode step) is one launch; longer
// appends run row by row, each row alone as a cache of batch 1.
int append_rows(kivi_cache *c, const void *k_new_fp16, const void *v_new_fp16, int64_t n_new,
                void *stream) {
  const Rows r = rows_of(c);
  if (r.t_max + n_new > c->capacity)
    return fail(KIVI_ERR_CAPACITY, "kivi_append: a row of %lld + %lld tokens passes capacity %lld",
                (long long)r.t_max, (long long)n_new, (long long)c->capacity);
  int rc;
  if (n_new == 1 && kivi::append_one_supported(c->head_dim, c->group, c->v_bits)) {
    rc = hip_status(kivi::launch_append_one_rows((const uint16_t *)k_new_fp16,
                                                 (const uint16_t *)v_new_fp16, c->k_res, c->v_res,
                                                 (int64_t)c->batch * c->n_kv_heads,
                                                 c->n_kv_heads, c->residual, r.n, layout_of(c),
                                                 (hipStream_t)stream),
                    "kivi_append (rows)");
    if (rc) return rc;
  } else {
    const int64_t per_row = (int64_t)c->n_kv_heads * n_new * c->head_dim;   // fp16 elements
    for (int32_t b = 0; b < c->batch; ++b) {
      kivi_cache v = row_view(c, b, c->row_tokens[b]);
      rc = append_uniform(&v, (const uint16_t *)k_new_fp16 + b * per_row,
                          (const uint16_t *)v_new_fp16 + b * per_row, n_new, stream);
      if (rc) return rc;
    }
  }
  for (int32_t b = 0; b < c->batch; ++b) c->row_tokens[b] += n_new;
  set_longest(c);
  return KIVI_OK;
}

}  // namespace

extern "C" {

int kivi_append(kivi_cache *c, const void *k_new_fp16, const void *v_new_fp16, int64_t n_new,
                void *stream) {
  int rc = check_cache(c, "kivi_append");
  if (rc) return rc;
  if (n_new < 0) return fail(KIVI_ERR_INVALID_ARG, "kivi_append: n_new must be >= 0");
  if (n_new == 0) return KIVI_OK;
  if (!k_new_fp16 || !v_new_fp16) return fail(KIVI_ERR_INVALID_ARG, "kivi_append: NULL input");
  if (c->row_tokens) return append_rows(c, k_new_fp16, v_new_fp16, n_new, stream);
  if (c->n_tokens + n_new > c->capacity)
    return fail(KIVI_ERR_CAPACITY, "kivi_append: %lld + %lld tokens pass capacity %lld",
                (long long)c->n_tokens, (long long)n_new, (long long)c->capacity);
  return append_uniform(c, k_new_fp16, v_new_fp16, n_new, stream);
}

int kivi_append_row(kivi_cache *c, int32_t b, const void *k_new_fp16, const void *v_new_fp16,
                    int64_t n_new, void *stream) {
  const char *who = "kivi_append_row";
  int rc = check_cache(c, who);
  if (rc) return rc;
  if (!c->row_tokens)
    return fail(KIVI_ERR_INVALID_ARG, "%s: the cache has no row_tokens (not a ragged batch)", who);
  if (b < 0 || b >= c->batch)
    return fail(KIVI_ERR_INVALID_ARG, "%s: row %d outside [0, %d)", who, b, c->batch);
  if (n_new < 0) return fail(KIVI_ERR_INVALID_ARG, "%s: n_new must be >= 0", who);
  if (n_new == 0) return KIVI_OK;
  if (!k_new_fp16 || !v_new_fp16) return fail(KIVI_ERR_INVALID_ARG, "%s: NULL input", who);
  if (c->row_tokens[b] + n_new > c->capacity)
    return fail(KIVI_ERR_CAPACITY, "%s: %lld + %lld tokens pass capacity %lld", who,
                (long long)c->row_tokens[b], (long long)n_new, (long long)c->capacity);
  kivi_cache v = row_view(c, b, c->row_tokens[b]);
  rc = append_uniform(&v, k_new_fp16, v_new_fp16, n_new, stream);
  if (rc) return rc;
  c->row_tokens[b] = v.n_tokens;
  set_longest(c);
  return KIVI_OK;
}

}  // extern "C"

namespace {

// kivi_append on a checked uniform cache with room for the n_new > 0 tokens.
int append_uniform(kivi_cache *c, const void *k_new_fp16, const void *v_new_fp16, int64_t n_new,
                   void *stream) {
  int rc;
  hipStream_t s = (hipStream_t)stream;
  const kivi::Layout L = layout_of(c);
  const int64_t R = c->residual, G = c->group, D = c->head_dim;
  const int64_t BH = (int64_t)c->batch * c->n_kv_heads;
  const int64_t t0 = c->n_tokens, t1 = t0 + n_new;
  const int64_t vq0 = max64(0, t0 - R), vq1 = max64(0, t1 - R);
  const int64_t kq0 = t0 - t0 % R, kq1 = t1 - t1 % R;
  if (n_new == 1 && kivi::append_one_supported((int)D, (int)G, c->v_bits)) {
    // decode step: one fused kernel, plus the key block when this token completes one
    rc = hip_status(kivi::launch_append_one((const uint16_t *)k_new_fp16,
                                            (const uint16_t *)v_new_fp16, c->k_res, c->v_res, t0,
                                            BH, (int)R, kq1 == kq0, L, s),
                    "kivi_append (step)");
    if (rc) return rc;
    if (kq1 > kq0) {
      kivi::TokenSource ksrc{c->k_res, (const uint16_t *)k_new_fp16, t0, 1, (int32_t)R,
                             (int32_t)D};
      rc = hip_status(kivi::launch_key_groups(ksrc, kq0 / G, (kq1 - kq0) / G, BH, L, s),
                      "kivi_append (keys)");
      if (rc) return rc;
    }
    c->n_tokens = t1;
    return KIVI_OK;
  }
  if (t0 == 0 && kivi::pack_tiles_supported((int)D, (int)G, c->v_bits) &&
      kivi::pack_tiles_supported((int)D, (int)G, c->k_bits)) {
    // prefill into an empty cache: every quantized token comes from the input
    rc = hip_status(kivi::launch_value_tokens((const uint16_t *)v_new_fp16, n_new, vq1, 0, BH, L,
                                              s),
                    "kivi_append (values)");
    if (rc) return rc;
    rc = hip_status(kivi::launch_key_tiles((const uint16_t *)k_new_fp16, n_new, kq1, 0, BH, L, s),
                    "kivi_append (keys)");
    if (rc) return rc;
    rc = hip_status(kivi::launch_write_window((const uint16_t *)k_new_fp16,
                                              (const uint16_t *)v_new_fp16, c->k_res, c->v_res,
                                              t0, n_new, kq1, vq1, BH, (int)R, (int)D, s),
                    "kivi_append (window)");
    if (rc) return rc;
    c->n_tokens = t1;
    return KIVI_OK;
  }
  // 1. values leaving the window (read old slots before they are reused)
  kivi::TokenSource vsrc{c->v_res, (const uint16_t *)v_new_fp16, t0, n_new, (int32_t)R,
                         (int32_t)D};
  rc = hip_status(kivi::launch_value_rows(vsrc, vq0, vq1 - vq0, BH, L, s),
                  "kivi_append (values)");
  if (rc) return rc;
  // 2. complete R-blocks of keys
  kivi::TokenSource ksrc{c->k_res, (const uint16_t *)k_new_fp16, t0, n_new, (int32_t)R,
                         (int32_t)D};
  rc = hip_status(kivi::launch_key_groups(ksrc, kq0 / G, (kq1 - kq0) / G, BH, L, s),
                  "kivi_append (keys)");
  if (rc) return rc;
  // 3. the new tokens that stay in fp16 take their slots
  rc = hip_status(kivi::launch_write_window((const uint16_t *)k_new_fp16,
                                            (const uint16_t *)v_new_fp16, c->k_res, c->v_res, t0,
                                            n_new, max64(kq1, t0), max64(vq1, t0), BH, (int)R,
                                            (int)D, s),
                  "kivi_append (window)");
  if (rc) return rc;
  c->n_tokens = t1;
  return KIVI_OK;
}

}  // namespace

extern "C" {

size_t kivi_decode_attn_workspace_bytes_ex(const kivi_cache *c, int32_t n_q_heads,
                                           int32_t tokens_per_split, int32_t path) {
  if (check_cache(c, "kivi_decode_attn_workspace_bytes")) return 0;
  if (n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0) return 0;
  if (tokens_per_split < 0 || tokens_per_split % 64 != 0) return 0;
  if (path < KIVI_PATH_AUTO || path > KIVI_PATH_VECTOR) return 0;
  // partial slots: acc[D], m, l, padded to D + 4 floats (16-byte rows)
  return (size_t)c->batch * n_q_heads * max_slots(c, tokens_per_split) * (c->head_dim + 4) *
         sizeof(float);
}

size_t kivi_decode_attn_workspace_bytes(const kivi_cache *c, int32_t n_q_heads) {
  return kivi_decode_attn_workspace_bytes_ex(c, n_q_heads, 0, KIVI_PATH_AUTO);
}

}  // extern "C"

namespace {

// Validation, planning and launch of an attention call.  With k_new and v_new
// set, the launch is a fused decode step: it also appends token c->n_tokens
// (the caller has checked that the matrix kernel takes the shape, and the
// capacity) and attends over c->n_tokens + 1 tokens; the caller advances
// n_tokens on success.
// Partial slots of the no-allocation entry point: one array per GPU, held
// from the first load of the library until the process ends.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this GPU's `scratch`, looked up once per device with
// that device current.  The array's name in host code is a host-side
// stand-in, never a device address.
int scratch_address(void **out, const char *who) {
  constexpr int kMaxDevices = 64;
  static std::mutex m;
  static void *ptrs[kMaxDevices] = {nullptr};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, who);
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KIVI_ERR_INVALID_ARG, "%s: device %d outside [0, %d)", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(m);
  if (!ptrs[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(KIVI_ERR_HIP, "%s: address of the scratch array: %s", who,
                  hipGetErrorString(e));
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return KIVI_OK;
}

// With use_scratch, the partials go to this GPU's scratch array (workspace
// and workspace_bytes are ignored) and the call fails with
// KIVI_ERR_WORKSPACE when this call's plan needs more than kScratchBytes.
int decode_call(const kivi_cache *c, const void *q_fp16, int32_t n_q_heads, const float *mask,
                float *out, void *workspace, size_t workspace_bytes, int32_t tokens_per_split,
                int32_t path, void *stream, const void *k_new, const void *v_new,
                const char *who, bool use_scratch = false) {
  int rc = check_cache(c, who);
  if (rc) return rc;
  if (n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0)
    return fail(KIVI_ERR_INVALID_ARG, "%s: n_q_heads %d must be a positive multiple of n_kv_heads %d",
                who, n_q_heads, c->n_kv_heads);
  if (!q_fp16 || !out) return fail(KIVI_ERR_INVALID_ARG, "%s: NULL q or out", who);
  if (tokens_per_split < 0 || tokens_per_split % 64 != 0)
    return fail(KIVI_ERR_INVALID_ARG, "%s: tokens_per_split %d must be 0 or a positive multiple of 64",
                who, tokens_per_split);
  if (path < KIVI_PATH_AUTO || path > KIVI_PATH_VECTOR)
    return fail(KIVI_ERR_INVALID_ARG, "%s: unknown path %d", who, path);
  if (!use_scratch) {
    const size_t need =
        kivi_decode_attn_workspace_bytes_ex(c, n_q_heads, tokens_per_split, path);
    if (!workspace || workspace_bytes < need)
      return fail(KIVI_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who,
                  workspace_bytes, need);
  }

  kivi::DecodeArgs a{};
  a.L = layout_of(c);
  a.k_res = c->k_res;
  a.v_res = c->v_res;
  a.q = (const uint16_t *)q_fp16;
  a.mask = mask;
  a.part = (float *)workspace;
  a.out = out;
  a.B = c->batch;
  a.H = c->n_kv_heads;
  a.D = c->head_dim;
  a.kb = c->k_bits;
  a.vb = c->v_bits;
  a.G = c->group;
  a.R = c->residual;
  a.Hq = n_q_heads;
  a.n_rep = n_q_heads / c->n_kv_heads;
  a.cap = c->capacity;
  const bool fused = k_new != nullptr;
  // a ragged batch: the kernels take each row's count from the launch's
  // tables; a.t is the longest row (the mask's row stride)
  const Rows r = rows_of(c);
  a.t = r.t_max + (fused ? 1 : 0);
  a.k_new = (const uint16_t *)k_new;
  a.v_new = (const uint16_t *)v_new;
  a.t_new = fused ? a.t - 1 : -1;
  a.n_kq = a.t - a.t % a.R;
  a.n_vq = max64(0, a.t - a.R);
  a.sm_scale = 1.0f / sqrtf((float)a.D);

  if (path == KIVI_PATH_MATRIX && !kivi::decode_matrix_supported(a) &&
      !kivi::decode_matrix4_supported(a, r.ragged))
    return fail(KIVI_ERR_INVALID_ARG, "%s: the matrix-core kernel does not handle this shape", who);
  if (path == KIVI_PATH_VECTOR && !kivi::decode_vector_supported(a))
    return fail(KIVI_ERR_INVALID_ARG, "%s: the vector kernel does not handle this shape", who);
  Plan p;
  rc = make_plan(c, n_q_heads, tokens_per_split, path, a, r, p, who);
  if (rc) return rc;
  if (fused && !p.matrix)
    return fail(KIVI_ERR_INVALID_ARG, "%s: internal: fused step without the matrix kernel", who);
  if (p.S_total > max_slots(c, tokens_per_split))
    return fail(KIVI_ERR_WORKSPACE, "%s: internal split plan exceeds the workspace bound", who);
  a.S_total = p.S_total;
  if (use_scratch) {
    // every slot a merge reads is written by this call: nothing in the array
    // must start at zero
    const size_t need =
        (size_t)c->batch * n_q_heads * p.S_total * (c->head_dim + 4) * sizeof(float);
    if (need > kScratchBytes)
      return fail(KIVI_ERR_WORKSPACE,
                  "%s: %zu bytes of partial results needed, the scratch array holds %zu", who,
                  need, kScratchBytes);
    void *sp = nullptr;
    rc = scratch_address(&sp, who);
    if (rc) return rc;
    a.part = (float *)sp;
  }
  hipStream_t s = (hipStream_t)stream;
  const kivi::RowCounts *rows = r.ragged ? &r.n : nullptr;
  if (p.matrix && r.ragged)
    rc = hip_status(kivi::launch_decode_matrix_rows(a, p.mrows, p.n_shares, s),
                    "kivi_decode_attn (matrix)");
  else if (p.matrix)
    rc = hip_status(kivi::launch_decode_matrix(a, p.n_main, p.n_groups_matrix, s),
                    "kivi_decode_attn (matrix)");
  else if (p.vector)
    rc = hip_status(kivi::launch_decode_vector(a, p.tps_generic, p.n_split_generic, s, rows),
                    "kivi_decode_attn (vector)");
  else
    rc = hip_status(
        kivi::launch_decode_generic(a, 0, p.tps_generic, p.n_split_generic, 0, s, rows),
        "kivi_decode_attn (scalar)");
  if (rc || !p.combine) return rc;
  return hip_status(kivi::launch_combine(a, s, p.matrix && r.ragged ? &p.slots : nullptr),
                    "kivi_decode_attn (combine)");
}

}  // namespace

extern "C" {

int kivi_decode_attn_ex(const kivi_cache *c, const void *q_fp16, int32_t n_q_heads,
                        const float *mask, float *out, void *workspace, size_t workspace_bytes,
                        int32_t tokens_per_split, int32_t path, void *stream) {
  return decode_call(c, q_fp16, n_q_heads, mask, out, workspace, workspace_bytes,
                     tokens_per_split, path, stream, nullptr, nullptr, "kivi_decode_attn");
}

int kivi_decode_attn_noalloc(const kivi_cache *c, const void *q_fp16, int32_t n_q_heads,
                             const float *mask, float *out, void *stream) {
  return decode_call(c, q_fp16, n_q_heads, mask, out, nullptr, 0, 0, KIVI_PATH_AUTO, stream,
                     nullptr, nullptr, "kivi_decode_attn_noalloc", true);
}

int kivi_decode_attn(const kivi_cache *c, const void *q_fp16, int32_t n_q_heads, const float *mask,
                     float *out, void *workspace, size_t workspace_bytes, void *stream) {
  return kivi_decode_attn_ex(c, q_fp16, n_q_heads, mask, out, workspace, workspace_bytes, 0,
                             KIVI_PATH_AUTO, stream);
}

int kivi_decode_step(kivi_cache *c, const void *k_new_fp16, const void *v_new_fp16,
                     const void *q_fp16, int32_t n_q_heads, const float *mask, float *out,
                     void *workspace, size_t workspace_bytes, void *stream) {
  const char *who = "kivi_decode_step";
  int rc = check_cache(c, who);
  if (rc) return rc;
  if (!k_new_fp16 || !v_new_fp16 || !q_fp16 || !out)
    return fail(KIVI_ERR_INVALID_ARG, "%s: NULL k_new, v_new, q or out", who);
  if (n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0)
    return fail(KIVI_ERR_INVALID_ARG, "%s: n_q_heads %d must be a positive multiple of n_kv_heads %d",
                who, n_q_heads, c->n_kv_heads);
  if (rows_of(c).t_max + 1 > c->capacity)
    return fail(KIVI_ERR_CAPACITY, "%s: the cache is full (%lld tokens)", who,
                (long long)c->capacity);
  // the workspace is checked before anything runs, so that a failing call
  // leaves the cache as it was
  const size_t need = kivi_decode_attn_workspace_bytes_ex(c, n_q_heads, 0, KIVI_PATH_AUTO);
  if (!workspace || workspace_bytes < need)
    return fail(KIVI_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", who, workspace_bytes,
                need);
  kivi::DecodeArgs probe{};
  probe.L = layout_of(c);
  probe.k_res = c->k_res;
  probe.v_res = c->v_res;
  probe.kb = c->k_bits;
  probe.vb = c->v_bits;
  probe.G = c->group;
  probe.D = c->head_dim;
  probe.n_rep = n_q_heads / c->n_kv_heads;
  probe.cap = c->capacity;
  probe.q = (const uint16_t *)q_fp16;
  probe.mask = mask;
  probe.R = c->residual;
  probe.t = rows_of(c).t_max + 1;
  probe.t_new = probe.t - 1;
  const bool fused = matrix_wanted(probe, KIVI_PATH_AUTO, c->row_tokens != nullptr) &&
                     ((uintptr_t)k_new_fp16 & 15) == 0 && ((uintptr_t)v_new_fp16 & 15) == 0;
  if (!fused) {
    // a shape the matrix kernel does not take: the append, then the
    // attention call
    rc = kivi_append(c, k_new_fp16, v_new_fp16, 1, stream);
    if (rc) return rc;
    return kivi_decode_attn_ex(c, q_fp16, n_q_heads, mask, out, workspace, workspace_bytes, 0,
                               KIVI_PATH_AUTO, stream);
  }
  rc = decode_call(c, q_fp16, n_q_heads, mask, out, workspace, workspace_bytes, 0, KIVI_PATH_AUTO,
                   stream, k_new_fp16, v_new_fp16, who);
  if (rc) return rc;
  if (c->row_tokens) {
    for (int32_t b = 0; b < c->batch; ++b) c->row_tokens[b] += 1;
    set_longest(c);
  } else {
    c->n_tokens += 1;
  }
  return KIVI_OK;
}

}  // extern "C"

namespace {

// Byte offsets of the sections of kivi_select_attn's workspace: the scores
// [B][Hq][cap] f32, the per-row selection rules, the partial slots of the
// attention over the selected tokens (as kivi_decode_attn's); each section
// 256-byte aligned.
struct SelectWorkspace {
  size_t scores, rows, part, total;
};
SelectWorkspace select_workspace(const kivi_cache *c, int32_t n_q_heads) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  SelectWorkspace w;
  const size_t rows = (size_t)c->batch * n_q_heads;
  w.scores = 0;
  w.rows = up(rows * c->capacity * sizeof(float));
  w.part = w.rows + up(rows * sizeof(kivi::SelectRow));
  w.total = w.part + up(rows * (size_t)max_slots(c, 0) * (c->head_dim + 4) * sizeof(float));
  return w;
}

}  // namespace

extern "C" {

size_t kivi_select_attn_workspace_bytes(const kivi_cache *c, int32_t n_q_heads) {
  if (check_cache(c, "kivi_select_attn_workspace_bytes")) return 0;
  if (n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0) return 0;
  return select_workspace(c, n_q_heads).total;
}

int kivi_select_attn(const kivi_cache *c, const void *q_fp16, int32_t n_q_heads,
                     const float *mask, float tau, float *out, int32_t *n_selected,
                     uint32_t *sel_mask, void *workspace, size_t workspace_bytes, void *stream) {
  const char *who = "kivi_select_attn";
  int rc = check_cache(c, who);
  if (rc) return rc;
  if (c->row_tokens)
    return fail(KIVI_ERR_INVALID_ARG, "%s: ragged batches are not supported", who);
  if (n_q_heads <= 0 || n_q_heads % c->n_kv_heads != 0)
    return fail(KIVI_ERR_INVALID_ARG, "%s: n_q_heads %d must be a positive multiple of n_kv_heads %d",
                who, n_q_heads, c->n_kv_heads);
  if (!q_fp16 || !out) return fail(KIVI_ERR_INVALID_ARG, "%s: NULL q or out", who);
  if (!(tau > 0.0f && tau <= 1.0f))
    return fail(KIVI_ERR_INVALID_ARG, "%s: tau %g outside (0, 1]", who, (double)tau);
  if (c->n_tokens >= ((int64_t)1 << 27))
    return fail(KIVI_ERR_INVALID_ARG, "%s: at most 2^27 - 1 tokens", who);
  const SelectWorkspace ws = select_workspace(c, n_q_heads);
  if (!workspace || workspace_bytes < ws.total || ((uintptr_t)workspace & 255) != 0)
    return fail(KIVI_ERR_WORKSPACE, "%s: workspace of %zu bytes (256-byte aligned), %zu needed",
                who, workspace_bytes, ws.total);
  kivi::DecodeArgs a{};
  a.L = layout_of(c);
  a.k_res = c->k_res;
  a.v_res = c->v_res;
  a.q = (const uint16_t *)q_fp16;
  a.mask = mask;
  a.out = out;
  a.B = c->batch;
  a.H = c->n_kv_heads;
  a.D = c->head_dim;
  a.kb = c->k_bits;
  a.vb = c->v_bits;
  a.G = c->group;
  a.R = c->residual;
  a.Hq = n_q_heads;
  a.n_rep = n_q_heads / c->n_kv_heads;
  a.cap = c->capacity;
  a.t = c->n_tokens;
  a.t_new = -1;
  a.n_kq = a.t - a.t % a.R;
  a.n_vq = max64(0, a.t - a.R);
  a.sm_scale = 1.0f / sqrtf((float)a.D);
  char *w = (char *)workspace;
  a.scores = (float *)(w + ws.scores);
  kivi::SelectRow *rows = (kivi::SelectRow *)(w + ws.rows);
  a.sel = rows;
  a.part = (float *)(w + ws.part);
  hipStream_t s = (hipStream_t)stream;
  // the matrix kernel where it takes the shape (its scores mode, then its
  // selected-attention mode), else the vector kernel, else the scalar one,
  // both to score the tokens and to attend over the selected ones; plans as
  // kivi_decode_attn makes them.  The selected attention reads the mask
  // from the stored scores, so the matrix kernel's is planned unmasked.
  const bool mat = a.t > 0 && kivi::decode_matrix_supported(a);
  const bool vec = !mat && kivi::decode_vector_supported(a);
  Plan p;
  const Rows r = rows_of(c);
  {
    kivi::DecodeArgs ap = a;
    if (mat) ap.mask = nullptr;
    rc = make_plan(c, n_q_heads, 0,
                   mat ? KIVI_PATH_MATRIX : (vec ? KIVI_PATH_VECTOR : KIVI_PATH_GENERIC), ap, r, p,
                   who);
  }
  if (rc) return rc;
  a.S_total = p.S_total;
  if (mat) {
    // 1. scores (masked: the four-wave variant's plan)
    Plan ps = p;
    if (a.mask) {
      rc = make_plan(c, n_q_heads, 0, KIVI_PATH_MATRIX, a, r, ps, who);
      if (rc) return rc;
    }
    // with each wave's largest score per row in the partial-slot section
    // (read by the selection before the attention writes its partials there)
    kivi::DecodeArgs as = a;
    as.rmax = a.part;
    as.rmax_n = ps.n_groups_matrix * kivi::decode_matrix_waves(a) +
                kivi::decode_matrix_window_chunks(a, ps.n_main);
    rc = hip_status(kivi::launch_scores_matrix(as, ps.n_main, ps.n_groups_matrix, s),
                    "kivi_select_attn (scores)");
    if (rc) return rc;
    // 2. the selection of every row
    rc = hip_status(kivi::launch_select_rows(as, tau, rows, n_selected, sel_mask, s),
                    "kivi_select_attn (select)");
    if (rc) return rc;
    // 3. attention over the selected tokens, then the merge of the workgroups
    rc = hip_status(kivi::launch_selected_matrix(a, p.n_main, p.n_groups_matrix, s),
                    "kivi_select_attn (attention)");
    if (rc || !p.combine) return rc;
    return hip_status(kivi::launch_combine(a, s), "kivi_select_attn (combine)");
  }
  // 1. scores of every token (KIVI item 5's scores); the vector kernel takes
  // all heads of a KV head in one workgroup when there are 4 or 8
  if (a.t > 0) {
    const int64_t units = (int64_t)c->batch * c->n_kv_heads;
    const bool whole = a.n_rep == 1 || a.n_rep == 4 || a.n_rep == 8;
    const int step = vec ? kVectorStep : kGenericMinSplit;
    const int64_t target = vec ? kVectorWorkgroups / (units * (whole ? 1 : a.n_rep / 2))
                               : kTargetWorkgroups / (units * head_chunks(a.n_rep));
    const int64_t tps = max64(1, ceil_div(ceil_div(a.t, max64(1, target)), step)) * step;
    const int n_split = (int)ceil_div(a.t, tps);
    rc = hip_status(vec ? kivi::launch_scores_vector(a, (int)tps, n_split, s)
                        : kivi::launch_scores_generic(a, (int)tps, n_split, s),
                    "kivi_select_attn (scores)");
    if (rc) return rc;
  }
  // 2. the selection of every row
  rc = hip_status(kivi::launch_select_rows(a, tau, rows, n_selected, sel_mask, s),
                  "kivi_select_attn (select)");
  if (rc) return rc;
  // 3. attention over the selected tokens, then the merge of the splits
  rc = hip_status(vec ? kivi::launch_selected_vector(a, p.tps_generic, p.n_split_generic, s)
                      : kivi::launch_selected_generic(a, p.tps_generic, p.n_split_generic, s),
                  "kivi_select_attn (attention)");
  if (rc || !p.combine) return rc;
  return hip_status(kivi::launch_combine(a, s), "kivi_select_attn (combine)");
}

}  // extern "C"

