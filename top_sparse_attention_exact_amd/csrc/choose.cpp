// (b, k_b) chooser for the bucketed top-k, and the recall model it uses.
//
// "Approximate Top-k for Increased Parallelism" (Pith review page):
//  * "What carries the argument": Eq. (1) gives the expected recall of the
//    two-stage bucketed top-k when the top values fall uniformly over the b
//    interleaved buckets;
//  * "Core claim" and "If this is right": the recall and cost models let a
//    practitioner pick (b, k_b) for a target trade-off without rerunning the
//    downstream task; the design rule is more buckets with k_b = 1 when k is
//    small against n, and a small k_b > 1 with b * k_b near k when k is a
//    sizeable fraction of n;
//  * major comment 3: the page's runtime figure picks the better of its
//    kernel's two modes per configuration by measurement.
//
// Here the recall is the finite-n form of Eq. (1) (exact for an iid row of
// distinct values: a hypergeometric in place of the binomial, averaged over
// the two bucket sizes when b does not divide n).  The chooser keeps, for
// every k_b in {1, 2, 4, 8, 16}, the smallest power-of-two b whose expected
// recall meets the target and the next larger one, adds the exact top-k
// (recall 1), times every candidate on the caller's rows through the public
// entry points, and returns the fastest.  Host code only; no kernel of its
// own.
#include <hip/hip_runtime.h>

#include <cmath>
#include <vector>

#include "atopk.h"

namespace {

constexpr int64_t kChooseMaxCand = 8192;  // b * k_b of a candidate: the final stage stays in LDS
constexpr int kChooseReps = 3;

double log_fact(double v) {
  int sign = 0;
  return lgamma_r(v + 1.0, &sign);
}

double log_comb(int64_t a, int64_t c) {
  if (c < 0 || c > a) return -INFINITY;
  return log_fact((double)a) - log_fact((double)c) - log_fact((double)(a - c));
}

// P(X <= x) for X ~ Hypergeometric(population pop, successes succ, draws).
double hyper_cdf(int64_t x, int64_t pop, int64_t succ, int64_t draws) {
  const int64_t lo = std::max<int64_t>(0, draws - (pop - succ));
  const int64_t hi = std::min(std::min(x, succ), draws);
  const double total = log_comb(pop, draws);
  double s = 0.0;
  for (int64_t j = lo; j <= hi; ++j) s += std::exp(log_comb(succ, j) + log_comb(pop - succ, draws - j) - total);
  return std::min(1.0, s);
}

// The i-th largest value (i = 0 the largest) survives stage 1 iff fewer than
// k_b of the i larger values share its bucket; they are a uniform i-subset
// of the other n - 1 positions, s - 1 of which lie in its bucket of size s.
double finite_recall(int64_t n, int64_t k, int64_t b, int64_t kb) {
  const int64_t lo = n / b, big = n % b;
  double acc = 0.0;
  for (int part = 0; part < 2; ++part) {
    const int64_t s = part == 0 ? lo + 1 : lo;
    const int64_t cnt = part == 0 ? big : b - big;
    if (cnt == 0 || s == 0) continue;
    const double w = (double)(cnt * s) / (double)n;
    double sum = 0.0;
    for (int64_t i = 0; i < k; ++i) sum += hyper_cdf(kb - 1, n - 1, s - 1, i);
    acc += w * sum;
  }
  return acc / (double)k;
}

int validate_model(int64_t n, int64_t k, int64_t b, int64_t kb) {
  if (n < 1 || k < 1 || k > n) return ATOPK_ERR_SHAPE;
  if (b < 1 || b > n || kb < 1 || kb > n / b || b * kb < k) return ATOPK_ERR_PARAM;
  return ATOPK_OK;
}

struct Cand {
  int64_t b, kb;
  double recall;
};

std::vector<Cand> candidates(int64_t n, int64_t k, double min_recall) {
  std::vector<Cand> out;
  out.push_back({1, k, 1.0});  // exact top-k
  for (int64_t kb = 1; kb <= ATOPK_MAX_KB; kb *= 2) {
    int64_t b = 1;
    while (b * kb < k) b *= 2;
    if (b == 1) continue;  // b = 1 is the exact route
    int found = 0;
    for (; b * kb <= kChooseMaxCand && b <= n && kb <= n / b && found < 2; b *= 2) {
      const double r = finite_recall(n, k, b, kb);
      if (found > 0 || r >= min_recall) {
        out.push_back({b, kb, r});
        ++found;
      }
    }
  }
  return out;
}

int validate_choose(int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, double min_recall) {
  if (!(min_recall >= 0.0 && min_recall <= 1.0)) return ATOPK_ERR_PARAM;
  size_t ws = 0;
  return atopk_exact_workspace(dtype, m, n, ldx, k, &ws);
}

int choose_ws(int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, double min_recall, size_t* need) {
  *need = 0;
  for (const Cand& c : candidates(n, k, min_recall)) {
    size_t ws = 0;
    const int st = atopk_bucketed_workspace(dtype, m, n, ldx, k, c.b, c.kb, 1, &ws);
    if (st == ATOPK_ERR_UNSUPPORTED) continue;
    if (st != ATOPK_OK) return st;
    *need = std::max(*need, ws);
  }
  return ATOPK_OK;
}

}  // namespace

extern "C" {

int atopk_expected_recall(int64_t n, int64_t k, int64_t b, int64_t kb, double* recall) {
  if (recall == nullptr) return ATOPK_ERR_NULL;
  const int st = validate_model(n, k, b, kb);
  if (st) return st;
  *recall = finite_recall(n, k, b, kb);
  return ATOPK_OK;
}

int atopk_choose_workspace(int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, double min_recall,
                           size_t* ws_bytes) {
  if (ws_bytes == nullptr) return ATOPK_ERR_NULL;
  const int st = validate_choose(dtype, m, n, ldx, k, min_recall);
  if (st) return st;
  return choose_ws(dtype, m, n, ldx, k, min_recall, ws_bytes);
}

int atopk_choose(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, double min_recall,
                 void* out_vals, int32_t* out_idx, void* ws, size_t ws_bytes, void* stream, int64_t* b_out,
                 int64_t* kb_out, double* recall_out, float* us_out) {
  if (b_out == nullptr || kb_out == nullptr) return ATOPK_ERR_NULL;
  int st = validate_choose(dtype, m, n, ldx, k, min_recall);
  if (st) return st;
  if (m == 0) {
    *b_out = 1;
    *kb_out = k;
    if (recall_out) *recall_out = 1.0;
    if (us_out) *us_out = 0.0f;
    return ATOPK_OK;
  }
  if (!x || !out_vals || !out_idx) return ATOPK_ERR_NULL;
  size_t need = 0;
  st = choose_ws(dtype, m, n, ldx, k, min_recall, &need);
  if (st) return st;
  if (need > 0 && (ws == nullptr || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % 256 != 0))
    return ATOPK_ERR_WORKSPACE;

  std::vector<Cand> cs;
  for (const Cand& c : candidates(n, k, min_recall)) {
    size_t w = 0;
    if (atopk_bucketed_workspace(dtype, m, n, ldx, k, c.b, c.kb, 1, &w) == ATOPK_OK) cs.push_back(c);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  std::vector<hipEvent_t> ev(2 * cs.size(), nullptr);
  for (auto& e : ev) {
    if (hipEventCreate(&e) != hipSuccess) {
      st = ATOPK_ERR_HIP;
      break;
    }
  }
  for (size_t i = 0; st == ATOPK_OK && i < cs.size(); ++i) {
    const Cand& c = cs[i];
    auto run = [&] { return atopk_bucketed(x, dtype, m, n, ldx, k, c.b, c.kb, 1, out_vals, out_idx, ws, ws_bytes, stream); };
    st = run();  // warm-up
    if (st == ATOPK_OK && hipEventRecord(ev[2 * i], s) != hipSuccess) st = ATOPK_ERR_HIP;
    for (int r = 0; st == ATOPK_OK && r < kChooseReps; ++r) st = run();
    if (st == ATOPK_OK && hipEventRecord(ev[2 * i + 1], s) != hipSuccess) st = ATOPK_ERR_HIP;
  }
  size_t best = 0;
  float best_ms = INFINITY;
  if (st == ATOPK_OK && hipEventSynchronize(ev.back()) != hipSuccess) st = ATOPK_ERR_HIP;
  for (size_t i = 0; st == ATOPK_OK && i < cs.size(); ++i) {
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, ev[2 * i], ev[2 * i + 1]) != hipSuccess) {
      st = ATOPK_ERR_HIP;
      break;
    }
    if (ms < best_ms) {
      best_ms = ms;
      best = i;
    }
  }
  for (auto& e : ev)
    if (e) (void)hipEventDestroy(e);
  if (st) return st;
  const Cand& c = cs[best];
  st = atopk_bucketed(x, dtype, m, n, ldx, k, c.b, c.kb, 1, out_vals, out_idx, ws, ws_bytes, stream);
  if (st) return st;
  *b_out = c.b;
  *kb_out = c.kb;
  if (recall_out) *recall_out = c.recall;
  if (us_out) *us_out = best_ms * 1000.0f / kChooseReps;
  return ATOPK_OK;
}

}  // extern "C"
