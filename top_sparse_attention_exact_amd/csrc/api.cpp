// Host side of the C ABI declared in include/atopk.h: argument validation,
// workspace layout and kernel dispatch.  Nothing here allocates, frees or
// synchronises; every argument is checked before the first HIP call, so the
// error paths run (and are tested) without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <cstring>
#include <new>

#include "atopk.h"
#include "launch.h"

using namespace atopk;

// ---- stage events (measurement aid) -------------------------------------------

namespace {
thread_local void* const* t_stage_events = nullptr;
thread_local int t_stage_cap = 0;
thread_local int t_stage_marks = 0;
}  // namespace

void atopk::stage_mark(hipStream_t s) {
  if (t_stage_events != nullptr && t_stage_marks < t_stage_cap)
    (void)hipEventRecord(static_cast<hipEvent_t>(t_stage_events[t_stage_marks]), s);
  ++t_stage_marks;
}

namespace {

constexpr int64_t kMaxN = (int64_t)1 << 31;  // indices are int32
constexpr int64_t kMaxCand = (int64_t)1 << 20;
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace carving: successive 256-byte aligned regions.
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  }
};

int64_t pow2_ceil(int64_t v) {
  int64_t p = 1;
  while (p < v) p <<= 1;
  return p;
}

// ---- device check (cached per device) ---------------------------------------

std::atomic<int> g_arch_ok[64];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATOPK_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    int c = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return ATOPK_OK;
    if (c == 2) return ATOPK_ERR_UNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATOPK_ERR_HIP;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev >= 0 && dev < 64) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? ATOPK_OK : ATOPK_ERR_UNSUPPORTED;
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATOPK_OK : ATOPK_ERR_HIP; }

// ---- exact -----------------------------------------------------------------------

int validate_exact(int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k) {
  if (m < 0 || n < 1 || ldx < n || k < 1 || k > n) return ATOPK_ERR_SHAPE;
  if (dtype != ATOPK_F32 && dtype != ATOPK_BF16) return ATOPK_ERR_UNSUPPORTED;
  if (n >= kMaxN || k > ATOPK_MAX_K) return ATOPK_ERR_UNSUPPORTED;
  return ATOPK_OK;
}

// ---- wide fp32 rows ------------------------------------------------------------------

struct WideLayout {
  WidePlan plan;
  size_t vals, thr, need, cand, rowthr, row_cnt, row_keys;
  size_t total;
};

WideLayout wide_layout(int dtype, int64_t m, int64_t n, int64_t k, int64_t b, int64_t kb, bool exact,
                       bool final_exact) {
  WideLayout L{};
  L.plan = plan_wide(dtype, m, n, k, b, kb, exact, final_exact);
  if (!L.plan.ok) return L;
  const WidePlan& p = L.plan;
  Carve c;
  L.vals = c.take(p.vals_bytes);
  L.thr = c.take(exact ? 0 : p.bucket_bytes);
  L.need = c.take(exact ? 0 : p.bucket_bytes);
  L.cand = c.take(p.cand_bytes);
  L.rowthr = c.take(exact ? p.bucket_bytes : 0);
  L.row_cnt = c.take(exact ? p.bucket_bytes : 0);
  L.row_keys = c.take(p.row_bytes);
  L.total = c.off;
  return L;
}

// Large k on fp32 rows goes to the two-pass path (k <= 64 has the row kernel).
bool wide_exact(int dtype, int64_t m, int64_t n, int64_t k) {
  return k > 64 && plan_wide(dtype, m, n, k, 0, 0, true, true).ok;
}

// fp32 rows whose exact top-k the sampled one-read route takes ahead of the
// certified route: rows of 2^14 elements or more, where one read with a cheap
// filter and a final that ranks the collected keys directly (split over up
// to four workgroups per row) beat the certified stage 1's 64-bit key queues
// and its rescan (64 x 128256, k = 256: 45 -> 33 us; 256 x 262144, k = 470:
// 91 -> 70 us; 128 x 2653751, k = 100: 356 -> 281 us).  Below that the row
// is too short for the sample's strata.
bool wide_sampled_exact(int dtype, int64_t m, int64_t n, int64_t k) {
  if (k <= 64 || n < ((int64_t)1 << 14)) return false;
  const WidePlan p = plan_wide(dtype, m, n, k, 0, 0, true, true);
  return p.ok && p.sampled;
}

// fp32 rows with k_b > 4 go to the two-pass path.
bool wide_bucketed(int dtype, int64_t m, int64_t n, int64_t k, int64_t b, int64_t kb, int final_exact) {
  return kb > 4 && plan_wide(dtype, m, n, k, b, kb, false, final_exact != 0).ok;
}

int run_wide(const WideLayout& L, const void* x, int64_t m, int64_t n, int64_t ldx, int64_t k, bool exact,
             bool final_exact, void* out_vals, int32_t* out_idx, void* ws, hipStream_t s) {
  uint8_t* w = static_cast<uint8_t*>(ws);
  WideBuffers B{};
  B.vals = reinterpret_cast<float*>(w + L.vals);
  B.thr = reinterpret_cast<float*>(w + L.thr);
  B.need = reinterpret_cast<int*>(w + L.need);
  B.cand = reinterpret_cast<uint64_t*>(w + L.cand);
  B.rowthr = reinterpret_cast<float*>(w + L.rowthr);
  B.row_cnt = reinterpret_cast<int*>(w + L.row_cnt);
  B.row_keys = reinterpret_cast<uint64_t*>(w + L.row_keys);
  return hip_status(launch_wide(L.plan, static_cast<const float*>(x), m, n, ldx, k, exact, final_exact, B, out_vals,
                                out_idx, s));
}

// Certified exact route (defined with the bucketed path below).
struct CertPlan {
  bool ok = false;
  int64_t b = 0, kb = 0;
};
CertPlan plan_certified(int dtype, int64_t m, int64_t n, int64_t k);
size_t certified_ws_bytes(int dtype, int64_t m, int64_t n, const CertPlan& c);
int run_certified(const CertPlan& c, const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k,
                  void* out_vals, int32_t* out_idx, void* ws, hipStream_t s);

size_t exact_ws_bytes(int dtype, int64_t m, int64_t n, int64_t k) {
  if (row_small_exact_ok(dtype, m, n, k)) return 0;
  if (wide_sampled_exact(dtype, m, n, k)) return wide_layout(dtype, m, n, k, 0, 0, true, true).total;
  const CertPlan cert = plan_certified(dtype, m, n, k);
  if (cert.ok) return certified_ws_bytes(dtype, m, n, cert);
  if (wide_exact(dtype, m, n, k)) return wide_layout(dtype, m, n, k, 0, 0, true, true).total;
  const ExactPlan p = plan_exact(dtype, m, n, k);
  if (p.splits <= 1) return 0;
  Carve c;
  c.take((size_t)m * p.splits * k * 8);
  return c.off;
}

bool rows_aligned(const void* x, int64_t ldx, int64_t es) {
  return ((reinterpret_cast<uintptr_t>(x) | (uintptr_t)(ldx * es)) & 15) == 0;
}

int run_exact(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, void* out_vals,
              int32_t* out_idx, void* ws, hipStream_t s) {
  const int64_t es = dtype == ATOPK_F32 ? 4 : 2;
  if (row_exact_ok(dtype, m, n, k, rows_aligned(x, ldx, es)))
    return hip_status(launch_row_exact(x, dtype, m, n, ldx, k, out_vals, out_idx, s));
  if (row_small_exact_ok(dtype, m, n, k))
    return hip_status(launch_row_small_exact(x, dtype, m, n, ldx, k, out_vals, out_idx, s));
  if (wide_sampled_exact(dtype, m, n, k))
    return run_wide(wide_layout(dtype, m, n, k, 0, 0, true, true), x, m, n, ldx, k, true, true, out_vals, out_idx, ws,
                    s);
  const CertPlan cert = plan_certified(dtype, m, n, k);
  if (cert.ok) return run_certified(cert, x, dtype, m, n, ldx, k, out_vals, out_idx, ws, s);
  if (wide_exact(dtype, m, n, k))
    return run_wide(wide_layout(dtype, m, n, k, 0, 0, true, true), x, m, n, ldx, k, true, true, out_vals, out_idx, ws,
                    s);
  const ExactPlan p = plan_exact(dtype, m, n, k);
  if (p.splits <= 1) return hip_status(launch_exact(p, x, dtype, m, n, ldx, k, nullptr, x, dtype, ldx, out_vals, out_idx, s));
  uint64_t* part = static_cast<uint64_t*>(ws);
  hipError_t e = launch_exact(p, x, dtype, m, n, ldx, k, part, x, dtype, ldx, nullptr, nullptr, s);
  if (e != hipSuccess) return ATOPK_ERR_HIP;
  const int64_t n2 = (int64_t)p.splits * k;
  const ExactPlan p2 = plan_exact(IN_KEY64, m, n2, k);
  return hip_status(launch_exact(p2, part, IN_KEY64, m, n2, n2, k, nullptr, x, dtype, ldx, out_vals, out_idx, s));
}

// ---- bucketed --------------------------------------------------------------------

bool exact_route(int64_t k, int64_t b, int64_t kb) { return b == 1 && kb == k; }

// Elements (and the int32 indices) must sit at addresses that are multiples
// of their size.
bool elems_misaligned(const void* x, const void* out_vals, const int32_t* out_idx, int dtype) {
  const uintptr_t es = dtype == ATOPK_F32 ? 4 : 2;
  return ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(out_vals)) & (es - 1)) != 0 ||
         (reinterpret_cast<uintptr_t>(out_idx) & 3) != 0;
}

int validate_bucketed(int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b, int64_t kb) {
  if (m < 0 || n < 1 || ldx < n || k < 1 || k > n) return ATOPK_ERR_SHAPE;
  if (b < 1 || b > n || kb < 1 || kb > n / b || b * kb < k) return ATOPK_ERR_PARAM;
  if (dtype != ATOPK_F32 && dtype != ATOPK_BF16) return ATOPK_ERR_UNSUPPORTED;
  if (n >= kMaxN || k > ATOPK_MAX_K) return ATOPK_ERR_UNSUPPORTED;
  if (exact_route(k, b, kb)) return ATOPK_OK;
  if (kb > ATOPK_MAX_KB || b * kb > kMaxCand) return ATOPK_ERR_UNSUPPORTED;
  return ATOPK_OK;
}

struct BucketLayout {
  BucketPlan plan;
  size_t lists_off, lists_bytes;
  size_t cand_off, cand_bytes;  // merged candidates when the final stage runs on the exact path
  size_t total;
};

int64_t kb_slots_host(int64_t kb) { return pow2_ceil(kb); }

BucketLayout bucket_layout(int dtype, int64_t m, int64_t n, int64_t b, int64_t kb, int final_exact, bool aligned) {
  BucketLayout L{};
  L.plan = plan_bucketed(dtype, m, n, b, kb, aligned);
  Carve c;
  L.lists_bytes = (size_t)m * L.plan.lists_per_row * b * kb_slots_host(kb) * 8;
  L.lists_off = c.take(L.lists_bytes);
  L.cand_bytes = (final_exact && b * kb > kFinishMaxCand) ? (size_t)m * b * kb * 8 : 0;
  L.cand_off = c.take(L.cand_bytes);
  L.total = c.off;
  return L;
}

size_t bucketed_ws_bytes(int dtype, int64_t m, int64_t n, int64_t k, int64_t b, int64_t kb, int final_exact) {
  if (exact_route(k, b, kb)) return exact_ws_bytes(dtype, m, n, k);
  if (wide_bucketed(dtype, m, n, k, b, kb, final_exact))
    return wide_layout(dtype, m, n, k, b, kb, false, final_exact != 0).total;
  // The plan depends on the data pointer's alignment; report the larger need.
  return std::max(bucket_layout(dtype, m, n, b, kb, final_exact, true).total,
                  bucket_layout(dtype, m, n, b, kb, final_exact, false).total);
}

int run_bucketed(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b, int64_t kb,
                 int final_exact, void* out_vals, int32_t* out_idx, void* ws, hipStream_t s) {
  if (exact_route(k, b, kb)) return run_exact(x, dtype, m, n, ldx, k, out_vals, out_idx, ws, s);
  const int64_t es = dtype == ATOPK_F32 ? 4 : 2;
  const bool aligned = rows_aligned(x, ldx, es);
  if (row_bucket_ok(dtype, m, n, b, kb, aligned))
    return hip_status(launch_row_bucket(x, dtype, m, n, ldx, k, b, kb, final_exact, out_vals, out_idx, s));
  if (wide_bucketed(dtype, m, n, k, b, kb, final_exact))
    return run_wide(wide_layout(dtype, m, n, k, b, kb, false, final_exact != 0), x, m, n, ldx, k, false,
                    final_exact != 0, out_vals, out_idx, ws, s);
  const BucketLayout L = bucket_layout(dtype, m, n, b, kb, final_exact, aligned);
  uint8_t* w = static_cast<uint8_t*>(ws);
  uint64_t* lists = reinterpret_cast<uint64_t*>(w + L.lists_off);
  uint64_t* cand = L.cand_bytes ? reinterpret_cast<uint64_t*>(w + L.cand_off) : nullptr;
  bool direct = false;
  if (launch_bucket_stage1(L.plan, x, dtype, m, n, ldx, b, kb, lists, s, k, final_exact, out_vals, out_idx,
                           cand ? nullptr : &direct) != hipSuccess)
    return ATOPK_ERR_HIP;
  if (direct) return ATOPK_OK;
  if (launch_bucket_finish(lists, L.plan.lists_per_row, m, n, b, kb, k, final_exact, x, dtype, ldx, out_vals, out_idx,
                           cand, s) != hipSuccess)
    return ATOPK_ERR_HIP;
  if (cand) {
    const int64_t nc = b * kb;
    const ExactPlan p2 = plan_exact(IN_KEY64, m, nc, k);
    return hip_status(launch_exact(p2, cand, IN_KEY64, m, nc, nc, k, nullptr, x, dtype, ldx, out_vals, out_idx, s));
  }
  return ATOPK_OK;
}

// ---- certified exact: bucketed stage 1, then the finish's rescan ------------------

// Expected number of buckets that receive at least kb of the k largest
// values of an iid row (each lands in one of b buckets with probability 1/b).
double saturated_buckets(int64_t k, int64_t b, int64_t kb) {
  const double p = 1.0 / (double)b;
  double term = std::pow(1.0 - p, (double)k);  // P(X = 0), X ~ Bin(k, p)
  double cdf = 0.0;
  for (int64_t j = 0; j < kb && j <= k; ++j) {
    cdf += term;
    term *= (double)(k - j) / (double)(j + 1) * p / (1.0 - p);
  }
  return (double)b * std::max(0.0, 1.0 - cdf);
}

// k_b = 4 and the smallest power-of-two b whose expected number of buckets
// to rescan stays below 1/4 per row and whose expected rescan (that number
// times a bucket's length) stays below 2048 elements; failing the second,
// the largest b that meets the first.  b * k_b <= 8192 keeps the candidates
// in LDS.  Rows far from iid only rescan more buckets, or take the finish's
// full-row fallback: the result is exact either way.
CertPlan plan_certified(int dtype, int64_t m, int64_t n, int64_t k) {
  CertPlan c;
  if (m < 1 || (dtype != ATOPK_F32 && dtype != ATOPK_BF16)) return c;
  const int64_t kb = 4;
  for (int64_t b = std::max<int64_t>(2, pow2_ceil((k + kb - 1) / kb)); b * kb <= kFinishMaxCand; b *= 2) {
    if (b > n || kb > n / b) break;
    const double e = saturated_buckets(k, b, kb);
    if (e <= 0.25) {
      c.ok = true;
      c.b = b;
      c.kb = kb;
      if (e * (double)((n + b - 1) / b) <= 2048.0) break;
    }
  }
  return c;
}

size_t certified_ws_bytes(int dtype, int64_t m, int64_t n, const CertPlan& c) {
  return bucket_layout(dtype, m, n, c.b, c.kb, 1, true).total;
}

int run_certified(const CertPlan& c, const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k,
                  void* out_vals, int32_t* out_idx, void* ws, hipStream_t s) {
  const BucketLayout L = bucket_layout(dtype, m, n, c.b, c.kb, 1, true);
  uint64_t* lists = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(ws) + L.lists_off);
  if (launch_bucket_stage1(L.plan, x, dtype, m, n, ldx, c.b, c.kb, lists, s) != hipSuccess) return ATOPK_ERR_HIP;
  return hip_status(launch_bucket_finish(lists, L.plan.lists_per_row, m, n, c.b, c.kb, k, kFinishCertified, x, dtype,
                                         ldx, out_vals, out_idx, nullptr, s));
}

// ---- decode --------------------------------------------------------------------------

int validate_decode(int64_t batch, int64_t hq, int64_t hkv, int64_t ctx, int64_t ctx_stride, int64_t d, int64_t k_sel,
                    int64_t b, int64_t kb) {
  if (batch < 0 || hq < 1 || hkv < 1 || hq % hkv != 0 || ctx < 1 || ctx_stride < ctx || d < 1 || k_sel < 1 ||
      k_sel > ctx)
    return ATOPK_ERR_SHAPE;
  if (b < 1 || b > ctx || kb < 1 || kb > ctx / b || b * kb < k_sel) return ATOPK_ERR_PARAM;
  if (d != 128 || hq / hkv > 8 || ctx >= kMaxN || k_sel > ATOPK_MAX_K) return ATOPK_ERR_UNSUPPORTED;
  if (!exact_route(k_sel, b, kb) && (kb > ATOPK_MAX_KB || b * kb > kMaxCand)) return ATOPK_ERR_UNSUPPORTED;
  return ATOPK_OK;
}

struct DecodeLayout {
  DecodePlan plan;
  bool certified;                                          // exact Top-K from a fused bucketed pass
  int64_t cb, ckb;                                         // its (b, kb)
  int cmode;                                               // rescan on the matrix cores (1) or dot products (2)
  size_t partial_off;                                      // fused path
  size_t scores_off, vals_off, idx_off, sel_ws_off;        // separate passes; scores_off also the certified fallback rows
  size_t sel_ws_bytes;
  size_t total;
};

// The exact Top-K of a decode as a fused bucketed pass plus the finish's
// certification: k_b = 8 and the smallest b the fused kernels take whose
// expected number of flagged buckets (on iid scores) stays at most one per
// head and whose expected rescan (that number times a bucket's length) stays
// at most 1024 keys.  No score is written: the finish recomputes a flagged
// bucket's scores with the scoring kernel's arithmetic (matrix cores for
// query-head groups, mode 1; 16-lane dot products otherwise, mode 2).
bool plan_decode_certified(int64_t batch, int64_t hq, int64_t hkv, int64_t ctx, int64_t k_sel, int64_t* b_out,
                           int64_t* kb_out, int* mode) {
  const bool groups = hq / hkv >= 2;
  const int64_t kb = 8;
  for (int64_t b = std::max<int64_t>(2, pow2_ceil((k_sel + kb - 1) / kb)); b * kb <= kFinishMaxCand; b *= 2) {
    if (b > ctx || kb > ctx / b) break;
    if (!plan_decode(batch, hq, hkv, ctx, k_sel, b, kb).fused) break;
    const double e = saturated_buckets(k_sel, b, kb);
    if (e <= 1.0 && e * (double)((ctx + b - 1) / b) <= 1024.0) {
      *b_out = b;
      *kb_out = kb;
      *mode = groups ? 1 : 2;
      return true;
    }
  }
  return false;
}

DecodeLayout decode_layout(int64_t batch, int64_t hq, int64_t hkv, int64_t ctx, int64_t k_sel, int64_t b, int64_t kb) {
  DecodeLayout L{};
  L.certified =
      exact_route(k_sel, b, kb) && plan_decode_certified(batch, hq, hkv, ctx, k_sel, &L.cb, &L.ckb, &L.cmode);
  L.plan = L.certified ? plan_decode(batch, hq, hkv, ctx, k_sel, L.cb, L.ckb) : plan_decode(batch, hq, hkv, ctx, k_sel, b, kb);
  Carve c;
  if (L.certified) {
    L.partial_off = c.take(L.plan.partial_bytes);
    L.scores_off = c.take((size_t)batch * hq * ctx * 4);
  } else if (L.plan.fused) {
    L.partial_off = c.take(L.plan.partial_bytes);
  } else {
    const int64_t rows = batch * hq;
    L.scores_off = c.take((size_t)rows * ctx * 4);
    L.vals_off = c.take((size_t)rows * k_sel * 4);
    L.idx_off = c.take((size_t)rows * k_sel * 4);
    L.sel_ws_bytes = bucketed_ws_bytes(ATOPK_F32, rows, ctx, k_sel, b, kb, 1);
    L.sel_ws_off = c.take(L.sel_ws_bytes);
  }
  L.total = c.off;
  return L;
}

int check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return ATOPK_OK;
  if (ws == nullptr || ws_bytes < need) return ATOPK_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0) return ATOPK_ERR_WORKSPACE;
  return ATOPK_OK;
}

template <typename F>
int guarded(F&& f) {
  try {
    return f();
  } catch (...) {
    return ATOPK_ERR_HIP;
  }
}

int validate_rerank(int64_t batch, int64_t hq, int64_t hkv, int64_t ctx, int64_t ctx_stride, int64_t d, int64_t k_sel,
                    int64_t ncand, int64_t cand_stride, int64_t window) {
  if (batch < 0 || hq < 1 || hkv < 1 || hq % hkv != 0 || ctx < 1 || ctx_stride < ctx || d < 1 || k_sel < 1 ||
      ncand < 0 || cand_stride < ncand)
    return ATOPK_ERR_SHAPE;
  if (window < 1 || window > ctx) return ATOPK_ERR_PARAM;
  if (d != 128 || ctx > kRerankMaxCtx || ncand + window > kRerankMaxCand || k_sel > ATOPK_MAX_K)
    return ATOPK_ERR_UNSUPPORTED;
  return ATOPK_OK;
}

int validate_assignment(int dtype, int64_t n, int64_t k, int64_t b, int64_t kb, int final_exact, int assignment) {
  if (assignment != ATOPK_INTERLEAVED && assignment != ATOPK_CONTIGUOUS) return ATOPK_ERR_PARAM;
  if (assignment == ATOPK_CONTIGUOUS && !exact_route(k, b, kb) && !row_contig_ok(n, b, kb, final_exact))
    return ATOPK_ERR_UNSUPPORTED;
  (void)dtype;
  return ATOPK_OK;
}

}  // namespace

extern "C" {

const char* atopk_status_str(int status) {
  switch (status) {
    case ATOPK_OK: return "ok";
    case ATOPK_ERR_NULL: return "a required pointer is NULL";
    case ATOPK_ERR_SHAPE: return "invalid shape (sizes, leading dimension, k)";
    case ATOPK_ERR_PARAM: return "invalid bucket parameters (b, k_b, b*k_b >= k)";
    case ATOPK_ERR_UNSUPPORTED: return "unsupported dtype, size, alignment or device (gfx950 only)";
    case ATOPK_ERR_WORKSPACE: return "workspace missing, too small or not 256-byte aligned";
    case ATOPK_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int atopk_version(void) { return 10000 * 0 + 100 * 2 + 0; }

int atopk_stage_events(void* const* events, int count) {
  if (count < 0 || (count > 0 && events == nullptr)) return ATOPK_ERR_PARAM;
  t_stage_events = count > 0 ? events : nullptr;
  t_stage_cap = count;
  t_stage_marks = 0;
  return ATOPK_OK;
}

int atopk_stage_count(void) { return t_stage_marks; }

int atopk_exact_workspace(int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, size_t* ws_bytes) {
  return guarded([&] {
    if (ws_bytes == nullptr) return (int)ATOPK_ERR_NULL;
    int st = validate_exact(dtype, m, n, ldx, k);
    if (st) return st;
    *ws_bytes = m == 0 ? 0 : exact_ws_bytes(dtype, m, n, k);
    return (int)ATOPK_OK;
  });
}

int atopk_exact(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, void* out_vals,
                int32_t* out_idx, void* ws, size_t ws_bytes, void* stream) {
  return guarded([&] {
    int st = validate_exact(dtype, m, n, ldx, k);
    if (st) return st;
    if (m == 0) return (int)ATOPK_OK;
    if (!x || !out_vals || !out_idx) return (int)ATOPK_ERR_NULL;
    if (elems_misaligned(x, out_vals, out_idx, dtype)) return (int)ATOPK_ERR_PARAM;
    st = check_ws(ws, ws_bytes, exact_ws_bytes(dtype, m, n, k));
    if (st) return st;
    st = check_device();
    if (st) return st;
    return run_exact(x, dtype, m, n, ldx, k, out_vals, out_idx, ws, static_cast<hipStream_t>(stream));
  });
}

int atopk_bucketed_workspace(int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b, int64_t kb,
                             int final_exact, size_t* ws_bytes) {
  return guarded([&] {
    if (ws_bytes == nullptr) return (int)ATOPK_ERR_NULL;
    int st = validate_bucketed(dtype, m, n, ldx, k, b, kb);
    if (st) return st;
    *ws_bytes = m == 0 ? 0 : bucketed_ws_bytes(dtype, m, n, k, b, kb, final_exact);
    return (int)ATOPK_OK;
  });
}

int atopk_bucketed_ex_workspace(int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b, int64_t kb,
                                int final_exact, int assignment, size_t* ws_bytes) {
  return guarded([&] {
    if (ws_bytes == nullptr) return (int)ATOPK_ERR_NULL;
    int st = validate_bucketed(dtype, m, n, ldx, k, b, kb);
    if (st) return st;
    st = validate_assignment(dtype, n, k, b, kb, final_exact, assignment);
    if (st) return st;
    const bool contig = assignment == ATOPK_CONTIGUOUS && !exact_route(k, b, kb);
    *ws_bytes = (m == 0 || contig) ? 0 : bucketed_ws_bytes(dtype, m, n, k, b, kb, final_exact);
    return (int)ATOPK_OK;
  });
}

int atopk_bucketed_ex(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b, int64_t kb,
                      int final_exact, int assignment, void* out_vals, int32_t* out_idx, void* ws, size_t ws_bytes,
                      void* stream) {
  return guarded([&] {
    int st = validate_bucketed(dtype, m, n, ldx, k, b, kb);
    if (st) return st;
    st = validate_assignment(dtype, n, k, b, kb, final_exact, assignment);
    if (st) return st;
    if (m == 0) return (int)ATOPK_OK;
    if (!x || !out_vals || !out_idx) return (int)ATOPK_ERR_NULL;
    if (elems_misaligned(x, out_vals, out_idx, dtype)) return (int)ATOPK_ERR_PARAM;
    const bool contig = assignment == ATOPK_CONTIGUOUS && !exact_route(k, b, kb);
    st = check_ws(ws, ws_bytes, contig ? 0 : bucketed_ws_bytes(dtype, m, n, k, b, kb, final_exact));
    if (st) return st;
    st = check_device();
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (contig) {
      const int64_t es = dtype == ATOPK_F32 ? 4 : 2;
      return hip_status(launch_row_contig(x, dtype, m, n, ldx, k, b, kb, final_exact, rows_aligned(x, ldx, es),
                                          out_vals, out_idx, s));
    }
    return run_bucketed(x, dtype, m, n, ldx, k, b, kb, final_exact, out_vals, out_idx, ws, s);
  });
}

int atopk_bucketed(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b, int64_t kb,
                   int final_exact, void* out_vals, int32_t* out_idx, void* ws, size_t ws_bytes, void* stream) {
  return guarded([&] {
    int st = validate_bucketed(dtype, m, n, ldx, k, b, kb);
    if (st) return st;
    if (m == 0) return (int)ATOPK_OK;
    if (!x || !out_vals || !out_idx) return (int)ATOPK_ERR_NULL;
    if (elems_misaligned(x, out_vals, out_idx, dtype)) return (int)ATOPK_ERR_PARAM;
    st = check_ws(ws, ws_bytes, bucketed_ws_bytes(dtype, m, n, k, b, kb, final_exact));
    if (st) return st;
    st = check_device();
    if (st) return st;
    return run_bucketed(x, dtype, m, n, ldx, k, b, kb, final_exact, out_vals, out_idx, ws,
                        static_cast<hipStream_t>(stream));
  });
}

int atopk_sparse_attn_decode_workspace(int64_t batch, int64_t hq, int64_t hkv, int64_t ctx, int64_t d, int64_t k_sel,
                                       int64_t b, int64_t kb, size_t* ws_bytes) {
  return guarded([&] {
    if (ws_bytes == nullptr) return (int)ATOPK_ERR_NULL;
    int st = validate_decode(batch, hq, hkv, ctx, ctx, d, k_sel, b, kb);
    if (st) return st;
    *ws_bytes = batch == 0 ? 0 : decode_layout(batch, hq, hkv, ctx, k_sel, b, kb).total;
    return (int)ATOPK_OK;
  });
}

int atopk_sparse_attn_decode(const void* q, const void* K, const void* V, int64_t batch, int64_t hq, int64_t hkv,
                             int64_t ctx, int64_t ctx_stride, int64_t d, float scale, int64_t k_sel, int64_t b,
                             int64_t kb, void* out, int32_t* sel_idx, float* scores, void* ws, size_t ws_bytes,
                             void* stream) {
  return guarded([&] {
    int st = validate_decode(batch, hq, hkv, ctx, ctx_stride, d, k_sel, b, kb);
    if (st) return st;
    if (batch == 0) return (int)ATOPK_OK;
    if (!q || !K || !V || !out) return (int)ATOPK_ERR_NULL;
    if (((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(K) | reinterpret_cast<uintptr_t>(V)) & 15) != 0)
      return (int)ATOPK_ERR_UNSUPPORTED;
    const DecodeLayout L = decode_layout(batch, hq, hkv, ctx, k_sel, b, kb);
    st = check_ws(ws, ws_bytes, L.total);
    if (st) return st;
    st = check_device();
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* w = static_cast<uint8_t*>(ws);
    const uint16_t* q16 = static_cast<const uint16_t*>(q);
    const uint16_t* k16 = static_cast<const uint16_t*>(K);
    const uint16_t* v16 = static_cast<const uint16_t*>(V);
    if (L.certified) {
      float* buf = scores ? scores : reinterpret_cast<float*>(w + L.scores_off);
      return hip_status(launch_decode_fused(L.plan, q16, k16, v16, batch, hq, hkv, ctx, ctx_stride, scale, k_sel, L.cb,
                                            L.ckb, reinterpret_cast<uint64_t*>(w + L.partial_off),
                                            static_cast<uint16_t*>(out), sel_idx, scores, L.cmode, buf, s));
    }
    if (L.plan.fused) {
      return hip_status(launch_decode_fused(L.plan, q16, k16, v16, batch, hq, hkv, ctx, ctx_stride, scale, k_sel, b,
                                            kb, reinterpret_cast<uint64_t*>(w + L.partial_off),
                                            static_cast<uint16_t*>(out), sel_idx, scores, 0, nullptr, s));
    }
    float* sc = scores ? scores : reinterpret_cast<float*>(w + L.scores_off);
    float* vals = reinterpret_cast<float*>(w + L.vals_off);
    int32_t* idx = sel_idx ? sel_idx : reinterpret_cast<int32_t*>(w + L.idx_off);
    const int64_t rows = batch * hq;
    if (launch_decode_scores(q16, k16, batch, hq, hkv, ctx, ctx_stride, scale, sc, s) != hipSuccess)
      return (int)ATOPK_ERR_HIP;
    st = run_bucketed(sc, ATOPK_F32, rows, ctx, ctx, k_sel, b, kb, 1, vals, idx, w + L.sel_ws_off, s);
    if (st) return st;
    return hip_status(launch_sparse_softmax_v(vals, idx, v16, batch, hq, hkv, ctx_stride, k_sel,
                                              static_cast<uint16_t*>(out), s));
  });
}

int atopk_sparse_attn_rerank_workspace(int64_t batch, int64_t hq, int64_t hkv, int64_t ctx, int64_t ncand,
                                       int64_t window, size_t* ws_bytes) {
  return guarded([&] {
    if (ws_bytes == nullptr) return (int)ATOPK_ERR_NULL;
    int st = validate_rerank(batch, hq, hkv, ctx, ctx, 128, 1, ncand, ncand, window);
    if (st) return st;
    *ws_bytes = batch == 0 ? 0 : rerank_ws_bytes(batch, hq, ncand, window);
    return (int)ATOPK_OK;
  });
}

int atopk_sparse_attn_rerank(const void* q, const void* K, const void* V, int64_t batch, int64_t hq, int64_t hkv,
                             int64_t ctx, int64_t ctx_stride, int64_t d, float scale, const int32_t* cand,
                             int64_t ncand, int64_t cand_stride, int64_t window, int64_t k_sel, void* out,
                             int32_t* sel_idx, float* scores, void* ws, size_t ws_bytes, void* stream) {
  return guarded([&] {
    int st = validate_rerank(batch, hq, hkv, ctx, ctx_stride, d, k_sel, ncand, cand_stride, window);
    if (st) return st;
    if (batch == 0) return (int)ATOPK_OK;
    if (!q || !K || !V || !out || (ncand > 0 && !cand)) return (int)ATOPK_ERR_NULL;
    if (((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(K) | reinterpret_cast<uintptr_t>(V)) & 15) != 0)
      return (int)ATOPK_ERR_UNSUPPORTED;
    st = check_ws(ws, ws_bytes, rerank_ws_bytes(batch, hq, ncand, window));
    if (st) return st;
    st = check_device();
    if (st) return st;
    return hip_status(launch_rerank(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(K),
                                    static_cast<const uint16_t*>(V), batch, hq, hkv, ctx, ctx_stride, scale, cand,
                                    ncand, cand_stride, window, k_sel, static_cast<uint16_t*>(out), sel_idx, scores, ws,
                                    static_cast<hipStream_t>(stream)));
  });
}

}  // extern "C"
