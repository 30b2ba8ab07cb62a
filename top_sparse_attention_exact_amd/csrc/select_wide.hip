// Wide fp32 rows with large k_b (bucketed) or large k (exact).
//
// Bucketed ("Approximate Top-k for Increased Parallelism", Pith review page,
// "What carries the argument") with k_b up to 16, and exact top-k with k up
// to 8192 (same page, "The reading").  A register queue of (value, index)
// keys per bucket costs far too much at k_b = 16, so the work is split into
// two streaming passes over the rows:
//
//  1. values pass: a workgroup owns a group of 64 buckets of one row; its
//     waves take consecutive chunks of sweeps (a sweep is b consecutive
//     elements, one per bucket), each lane keeping the KB largest VALUES of
//     its bucket (one v_max_f32 and KB-1 v_med3_f32 per element).  The waves
//     then merge their lists through LDS.  Bucketed: T_r = the k_b-th
//     largest value of bucket r, and need_r = how many of the bucket's top
//     k_b equal T_r.  Exact: the top KB values of every bucket go out, and a
//     per-row step takes T = the k-th largest of those b * KB values: they
//     are b * KB >= k distinct elements of the row, so at least k elements
//     reach T and the row's k-th largest value is >= T.
//  2. collect pass, same layout: bucketed, a lane sees its bucket in index
//     order and keeps (as keys) every element > T_r plus the first need_r
//     elements == T_r of its chunk -- the ties the pages' radix select
//     collects separately (Figure 12) -- and the waves merge their key
//     queues, leaving each bucket's exact top-k_b; exact, every element
//     >= T goes to the row's key list.
//  3. final (skipped by stage-1-only calls): the exact top-k of the
//     candidates (radix select on the keys), a counting sort on the value,
//     and the output; with few rows up to four workgroups per row split the
//     sort by value.  If the exact collection overflowed (rows made of few
//     distinct values) the workgroup runs a full radix select over its row
//     instead.
#include <algorithm>
#include <cmath>

#include "common.h"
#include "launch.h"

namespace atopk {

namespace {

constexpr int kWideKB = 16;     // widest value network (k_b <= 16)
constexpr int kWideU = 16;      // sweeps in flight per lane
constexpr int kMaxChunks = 8;   // waves (chunks) per streaming workgroup
constexpr int kRowCap = 32768;  // exact-mode candidate keys per row
constexpr int kFinT = 1024;
constexpr int kFinP = 8;                // keys per thread in the final sort
constexpr int kFinMax = kFinT * kFinP;  // 8192 candidates in LDS
constexpr int kExactP = kRowCap / kFinT;  // collected keys per thread in the exact final
constexpr int kFinParts = 4;             // most final workgroups per row
constexpr int64_t kFinCUs = 256;         // compute units the final fills
constexpr int kExactB = 1024;           // bucketing that bounds the exact k-th value
constexpr int kFlush = 256;             // per-wave key buffer of the exact collect

// Insert x into a descending list of KB floats (max / med3 network).
template <int KB>
__device__ __forceinline__ void fnet_insert(float (&q)[KB], float x) {
#pragma unroll
  for (int j = KB - 1; j >= 1; --j) q[j] = __builtin_amdgcn_fmed3f(q[j - 1], q[j], x);
  q[0] = fmaxf(q[0], x);
}

// A streaming workgroup: (row, group of 64 buckets); wave w takes sweeps
// [w * spc, (w + 1) * spc).  Workgroups go round-robin to the 8 XCDs, so
// when the rows split evenly the map puts all groups of a row -- the
// workgroups that read the same sweeps -- on one XCD.  `rev` walks the
// workgroups in reverse launch order: the collect passes then start on the
// data the values pass read last, which is still in the Infinity Cache.
constexpr int kXcds = 8;

struct Unit {
  int row, r, s0, s1, full;
};

__device__ __forceinline__ Unit unit_of(int n, int b, int groups, int spc, bool rev) {
  Unit u;
  const int bid = rev ? (int)(gridDim.x - 1 - blockIdx.x) : (int)blockIdx.x;
  const int rows = (int)gridDim.x / groups;
  int grp;
  if (rows % kXcds == 0) {
    const int slot = bid / kXcds;
    u.row = bid % kXcds + kXcds * (slot / groups);
    grp = slot % groups;
  } else {
    u.row = bid / groups;
    grp = bid - u.row * groups;
  }
  u.r = grp * kWave + lane_id();
  const int nsweeps = (n + b - 1) / b;
  u.s0 = min((int)(threadIdx.x / kWave) * spc, nsweeps);
  u.s1 = min(u.s0 + spc, nsweeps);
  u.full = min(u.s1, n / b);  // sweeps in which every bucket has an element
  return u;
}

// Merge the sorted KB-lists of the workgroup's nw waves into wave 0 (a tree
// through `lds`, which holds nw/2 * KB * 64 elements; nw a power of two).
template <int KB, typename K>
__device__ __forceinline__ void tree_merge(K (&q)[KB], K* lds, int nw) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  for (int half = nw / 2; half >= 1; half /= 2) {
    if (wave >= half && wave < 2 * half) {
#pragma unroll
      for (int j = 0; j < KB; ++j) lds[((wave - half) * KB + j) * kWave + lane] = q[j];
    }
    __syncthreads();
    if (wave < half) {
      K c[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) c[j] = lds[(wave * KB + j) * kWave + lane];
      queue_merge<KB>(q, c);
    }
    __syncthreads();
  }
}

// 1. values pass.  Bucketed: thr / need per (row, bucket).  Exact: the top
//    KB values per bucket to vals[(row * KB + j) * b + r].
template <int KB>
__global__ __launch_bounds__(kWave * kMaxChunks) void wide_values_kernel(const float* __restrict__ x, int64_t ldx,
                                                                        int n, int b, int kb, int groups, int spc,
                                                                        int exact_mode, float* __restrict__ thr,
                                                                        int* __restrict__ need,
                                                                        float* __restrict__ vals) {
  __shared__ float lds[kMaxChunks / 2 * KB * kWave];
  const Unit u = unit_of(n, b, groups, spc, false);
  const float* xr = x + (int64_t)u.row * ldx + u.r;
  float q[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) q[j] = -INFINITY;
  int s = u.s0;
  for (; s + kWideU <= u.full; s += kWideU) {
    float w[kWideU];
#pragma unroll
    for (int v = 0; v < kWideU; ++v) w[v] = xr[(int64_t)(s + v) * b];
#pragma unroll
    for (int v = 0; v < kWideU; ++v) fnet_insert<KB>(q, w[v]);
  }
  for (; s < u.s1; ++s)
    if ((int64_t)s * b + u.r < n) fnet_insert<KB>(q, xr[(int64_t)s * b]);
  tree_merge<KB>(q, lds, blockDim.x / kWave);
  if (threadIdx.x >= kWave) return;
  if (exact_mode) {
#pragma unroll
    for (int j = 0; j < KB; ++j) vals[((int64_t)u.row * KB + j) * b + u.r] = q[j];
    return;
  }
  float t = q[0];
#pragma unroll
  for (int j = 0; j < KB; ++j)
    if (j == kb - 1) t = q[j];
  int gt = 0;
#pragma unroll
  for (int j = 0; j < KB; ++j) gt += (j < kb && q[j] > t) ? 1 : 0;
  thr[(int64_t)u.row * b + u.r] = t;
  need[(int64_t)u.row * b + u.r] = kb - gt;
}

// 1b. exact threshold: one workgroup per row, thread per bucket (b = 1024).
//     rowthr[row] = the k-th largest of the row's b * KB bucket tops.
__global__ __launch_bounds__(kExactB) void wide_exact_threshold_kernel(const float* __restrict__ vals, int k,
                                                                      float* __restrict__ rowthr,
                                                                      int* __restrict__ row_cnt) {
  constexpr int KB = kWideKB;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t ctl[4];
  const int row = blockIdx.x;
  uint32_t o[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j)
    o[j] = ord_f32(__float_as_uint(vals[((int64_t)row * KB + j) * kExactB + threadIdx.x]));
  int rem;
  const uint32_t v = block_radix_kth32<kExactB>(
      k, hist, ctl,
      [&](uint32_t mask, uint32_t prefix, int shift) {
#pragma unroll
        for (int j = 0; j < KB; ++j) hist_add_grouped(hist, (o[j] >> shift) & 255u, (o[j] & mask) == prefix);
      },
      &rem);
  if (threadIdx.x == 0) {
    rowthr[row] = __uint_as_float(bits_from_ord(v));
    row_cnt[row] = 0;
  }
}

// 2a. bucketed collect.  A lane's kept keys number at most k_b (the bucket
//     holds exactly k_b - need_r elements above T_r); they are appended to
//     the lane's LDS slots, sorted into a queue after the sweep, and the
//     merged queue of the waves is the bucket's exact top-k_b.
//     final_exact: keys to cand[(row * b + r) * kb + j]; otherwise the
//     bucket-major output itself.
template <int KB>
__global__ __launch_bounds__(kWave * kMaxChunks) void wide_collect_bucket_kernel(
    const float* __restrict__ x, int64_t ldx, int n, int b, int kb, int groups, int spc, int final_exact,
    const float* __restrict__ thr, const int* __restrict__ need, uint64_t* __restrict__ cand,
    float* __restrict__ out_vals, int32_t* __restrict__ out_idx) {
  __shared__ uint64_t lds[kMaxChunks * KB * kWave];  // kept keys, then the merge tree
  const Unit u = unit_of(n, b, groups, spc, true);
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const float* xr = x + (int64_t)u.row * ldx + u.r;
  const int64_t rb = (int64_t)u.row * b + u.r;
  const float th = thr[rb];
  int left = need[rb];
  int cnt = 0;
  uint64_t* mine = lds + wave * KB * kWave + lane;  // slot j at mine[j * 64]
  auto see = [&](float v, int s) {
    if (v >= th && (v > th || left > 0)) {
      left -= v > th ? 0 : 1;
      if (cnt < KB)
        mine[cnt * kWave] = make_key(ord_f32(__float_as_uint(v)), (uint32_t)s * (uint32_t)b + (uint32_t)u.r);
      ++cnt;
    }
  };
  int s = u.s0;
  for (; s + kWideU <= u.full; s += kWideU) {
    float w[kWideU];
#pragma unroll
    for (int v = 0; v < kWideU; ++v) w[v] = xr[(int64_t)(s + v) * b];
#pragma unroll
    for (int v = 0; v < kWideU; ++v) see(w[v], s + v);
  }
  for (; s < u.s1; ++s)
    if ((int64_t)s * b + u.r < n) see(xr[(int64_t)s * b], s);
  uint64_t q[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) q[j] = 0;
  cnt = min(cnt, KB);
  for (int j = 0; j < cnt; ++j) queue_insert<KB>(q, mine[j * kWave]);
  __syncthreads();  // the slots are reused by the merge
  tree_merge<KB>(q, lds, blockDim.x / kWave);
  if (threadIdx.x >= kWave) return;
  if (final_exact) {
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if (j < kb) cand[rb * kb + j] = q[j];
    return;
  }
  const uint32_t* xb = reinterpret_cast<const uint32_t*>(x + (int64_t)u.row * ldx);
#pragma unroll
  for (int j = 0; j < KB; ++j) {
    if (j < kb) {
      uint32_t idx = key_idx(q[j]);
      idx = idx < (uint32_t)n ? idx : 0u;  // only reachable with NaN inputs
      out_idx[rb * kb + j] = (int32_t)idx;
      reinterpret_cast<uint32_t*>(out_vals)[rb * kb + j] = xb[idx];
    }
  }
}

// 2b. exact collect: element >= T -> the row's key list (kRowCap entries;
//     the count keeps growing past the cap).  Keys gather in a per-wave LDS
//     buffer; a full buffer is flushed with one atomic of its own, and the
//     last keys of all the workgroup's waves with one atomic between them
//     (per-wave atomics on the row's one counter serialise: they doubled the
//     pass).
__global__ __launch_bounds__(kWave * kMaxChunks) void wide_collect_exact_kernel(
    const float* __restrict__ x, int64_t ldx, int n, int b, int groups, int spc, const float* __restrict__ rowthr,
    int* __restrict__ row_cnt, uint64_t* __restrict__ row_keys) {
  __shared__ uint64_t wbuf[kMaxChunks][kFlush];
  __shared__ uint32_t wg_off[kMaxChunks];
  __shared__ uint32_t wg_base;
  const Unit u = unit_of(n, b, groups, spc, true);
  const int wave = threadIdx.x / kWave;
  uint64_t* buf = wbuf[wave];
  const int lane = lane_id();
  const float* xr = x + (int64_t)u.row * ldx + u.r;
  const float th = rowthr[u.row];
  uint64_t* out = row_keys + (int64_t)u.row * kRowCap;
  int fill = 0;  // wave-uniform
  auto flush = [&]() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int base = 0;
    if (lane == 0) base = atomicAdd(&row_cnt[u.row], fill);
    base = (int)wave_lane0((uint32_t)base);
    for (int j = lane; j < fill; j += kWave)
      if (base + j < kRowCap) out[base + j] = buf[j];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    fill = 0;
  };
  auto see = [&](bool keep, float v, int s) {
    const uint64_t m = __ballot(keep);
    if (m) {
      if (keep)
        buf[fill + (int)lanes_below(m)] =
            make_key(ord_f32(__float_as_uint(v)), (uint32_t)s * (uint32_t)b + (uint32_t)u.r);
      fill += __popcll(m);
      if (fill > kFlush - kWave) flush();
    }
  };
  // sweeps [s0, fe) hold an element of every bucket; the rest may not
  const int fe = u.full > u.s0 ? u.full : u.s0;
  int s = u.s0;
  // groups of kWideU sweeps through two register sets: the next group's
  // loads are in flight while a group is filtered
  const int ng = (fe - s) / kWideU;
  float wa[kWideU], wb[kWideU];
  auto load = [&](float (&w)[kWideU], int s0) {
#pragma unroll
    for (int v = 0; v < kWideU; ++v) w[v] = xr[(int64_t)(s0 + v) * b];
  };
  auto filt = [&](const float (&w)[kWideU], int s0) {
#pragma unroll
    for (int v = 0; v < kWideU; ++v) see(w[v] >= th, w[v], s0 + v);
  };
  if (ng > 0) {
    int g = 0;
    load(wa, s);
    for (; g + 2 < ng; g += 2) {
      load(wb, s + (g + 1) * kWideU);
      filt(wa, s + g * kWideU);
      load(wa, s + (g + 2) * kWideU);
      filt(wb, s + (g + 1) * kWideU);
    }
    if (g + 1 < ng) {
      load(wb, s + (g + 1) * kWideU);
      filt(wa, s + g * kWideU);
      filt(wb, s + (g + 1) * kWideU);
    } else {
      filt(wa, s + g * kWideU);
    }
    s += ng * kWideU;
  }
  for (; s < u.s1; ++s) {
    const bool in = (int64_t)s * b + u.r < n;
    const float v = in ? xr[(int64_t)s * b] : -INFINITY;
    see(in && v >= th, v, s);
  }
  // the waves' last keys: offsets inside the workgroup, one atomic in all
  if (lane == 0) wg_off[wave] = (uint32_t)fill;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t tot = 0;
    for (int w2 = 0; w2 < (int)(blockDim.x / kWave); ++w2) {
      const uint32_t c = wg_off[w2];
      wg_off[w2] = tot;
      tot += c;
    }
    wg_base = tot ? (uint32_t)atomicAdd(&row_cnt[u.row], (int)tot) : 0u;
  }
  __syncthreads();
  const int base = (int)(wg_base + wg_off[wave]);
  for (int j = lane; j < fill; j += kWave)
    if (base + j < kRowCap) out[base + j] = buf[j];
}

// Bitonic sort (descending) of T*P keys held P per thread, key index
// tid*P + p.  Strides below P stay in registers, strides below 64*P move
// across lanes, larger ones go through `lds` (T*P keys, index p*T + tid so
// that a wave's accesses are consecutive).
template <int P, int S>
__device__ __forceinline__ void sort_step_regs(uint64_t (&key)[P], int tid, int size) {
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if ((p & S) == 0) {
      const bool desc = ((tid * P + p) & size) == 0;
      const uint64_t a = key[p], c = key[p + S];
      key[p] = desc ? kmax(a, c) : kmin(a, c);
      key[p + S] = desc ? kmin(a, c) : kmax(a, c);
    }
  }
}

template <int T, int P>
__device__ void block_sort_desc_regs(uint64_t (&key)[P], uint64_t* lds) {
  static_assert(P == 8, "the register strides below are written for P = 8");
  const int tid = threadIdx.x;
  const int lane = lane_id();
  for (int size = 2; size <= T * P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride == 4) {
        sort_step_regs<P, 4>(key, tid, size);
      } else if (stride == 2) {
        sort_step_regs<P, 2>(key, tid, size);
      } else if (stride == 1) {
        sort_step_regs<P, 1>(key, tid, size);
      } else if (stride < kWave * P) {
        const int ls = stride / P;
        const bool lower = (lane & ls) == 0;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const bool desc = ((tid * P + p) & size) == 0;
          const uint64_t o = shfl_xor_u64(key[p], ls);
          key[p] = (lower == desc) ? kmax(key[p], o) : kmin(key[p], o);
        }
      } else {
        const int ts = stride / P;
        const bool lower = (tid & ts) == 0;
#pragma unroll
        for (int p = 0; p < P; ++p) lds[p * T + tid] = key[p];
        __syncthreads();
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const bool desc = ((tid * P + p) & size) == 0;
          const uint64_t o = lds[p * T + (tid ^ ts)];
          key[p] = (lower == desc) ? kmax(key[p], o) : kmin(key[p], o);
        }
        __syncthreads();
      }
    }
  }
}

// Sorted output of part `part` of `parts` of a row's cnt unique nonzero
// keys (global memory, cnt <= kFinT * PIN): the keys of rank r < k whose
// rank falls in this part, written as values (bit copies of the row) and
// indices.  The parts of a row run in separate workgroups that each read
// every key and split the work by value.
//
// Counting sort on the value over equi-depth bins.  Each key's distance
// below the largest, hi - ord, maps monotonically onto x in [0, kCoarse]
// (an fp32 conversion and a product, both monotone).  Coarse bin floor(x):
// a histogram and its scan give every coarse bin its place in the order,
// and part q takes the coarse bins that start in [q * kk / parts,
// (q + 1) * kk / parts), kk = min(cnt, k) (bins starting at kk or later
// hold no rank below k).  Its keys are compacted, every coarse bin is cut
// into as many fine bins as it holds keys, the fractional part of x (exact:
// x - floor(x) loses no bits) picks the fine bin, and a scan and a scatter
// group the keys by fine bin -- about one key per bin, even when a few
// outliers stretch the range.  A key's rank is its fine bin's start plus
// the larger keys in its bin.
//
// Returns false, having written nothing, when the part holds more than
// kFinMax keys or a fine bin more than kBinRank (heavy ties); [*r0, *r1)
// is then the part's rank range, which the caller fills another way.
// `cand` holds kFinMax keys, `bins` kFinMax words, `red` kFinRed.
constexpr int kBinRank = 256;
constexpr int kCoarse = 1024;  // one coarse bin per thread of the final
constexpr int kCoarseSub = 4;
constexpr int kFinRed = 128 + (2 + kCoarseSub) * kCoarse;  // words of `red`

// Bitonic sort (out of line: it needs its own registers): cand[0..cnt)
// descending, kFinMax entries (zeros past cnt).
__device__ __noinline__ void block_sort_desc_bitonic(uint64_t* cand, int cnt) {
  const int t = threadIdx.x;
  uint64_t key[kFinP];
#pragma unroll
  for (int p = 0; p < kFinP; ++p) {
    const int i = t * kFinP + p;
    key[p] = i < cnt ? cand[i] : 0;
  }
  __syncthreads();
  block_sort_desc_regs<kFinT, kFinP>(key, cand);
#pragma unroll
  for (int p = 0; p < kFinP; ++p) cand[t * kFinP + p] = key[p];
  __syncthreads();
}

// Output entry r of the sorted row from its key.
__device__ __forceinline__ void write_ranked(uint64_t key, int r, const float* __restrict__ xr, int n,
                                             float* __restrict__ out_vals, int32_t* __restrict__ out_idx) {
  uint32_t idx = key_idx(key);
  idx = idx < (uint32_t)n ? idx : 0u;  // only reachable with NaN inputs
  out_idx[r] = (int32_t)idx;
  // the order key gives the value back, except the sign of a zero
  const uint32_t o = key_ord(key);
  reinterpret_cast<uint32_t*>(out_vals)[r] =
      o == 0x80000000u ? reinterpret_cast<const uint32_t*>(xr)[idx] : bits_from_ord(o);
}

template <int PIN>
__device__ __forceinline__ bool sort_part_and_write(const uint64_t* __restrict__ src, int cnt, int k, int part,
                                                    int parts, const float* __restrict__ xr, int n,
                                                    float* __restrict__ out_vals, int32_t* __restrict__ out_idx,
                                                    uint64_t* cand, uint32_t* bins, uint32_t* red, int* r0, int* r1) {
  constexpr int T = kFinT, P = kFinP;
  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = t / kWave;
  // the coarse counts (kCoarseSub copies: lane l counts into copy
  // l mod kCoarseSub, so that the lanes of a wave whose keys crowd a few
  // coarse bins hit more addresses), then their sums and exclusive scan
  static_assert(kCoarse == T, "one coarse bin per thread");
  uint32_t* coarse = red + 128;
  uint32_t* coarse_sub = coarse + 2 * kCoarse;
  // key p of thread t is entry p * T + t: at one p a wave reads 64 entries
  // in a row, which hold keys of different ranks, so the histogram atomics
  // of one instruction spread over many bins.  Slots past np stay unused.
  const int np = (cnt + T - 1) / T;
  uint64_t key[PIN];
#pragma unroll
  for (int p = 0; p < PIN; ++p) key[p] = p < np && p * T + t < cnt ? src[p * T + t] : 0;
  auto valid = [&](int p) { return p < np && p * T + t < cnt; };
  uint32_t lo = 0xffffffffu, hi = 0;
#pragma unroll
  for (int p = 0; p < PIN; ++p) {
    if (valid(p)) {
      lo = min(lo, key_ord(key[p]));
      hi = max(hi, key_ord(key[p]));
    }
  }
  lo = wave_reduce_dpp(lo, [](uint32_t x, uint32_t y) { return min(x, y); });
  hi = wave_reduce_dpp(hi, [](uint32_t x, uint32_t y) { return max(x, y); });
  if (lane == 0) {
    red[wave] = lo;
    red[16 + wave] = hi;
  }
  for (int j = t; j < kFinMax; j += T) bins[j] = 0;
  for (int j = t; j < kCoarse * kCoarseSub; j += T) coarse_sub[j] = 0;
  if (t == 0) {
    red[32] = 0;  // a fine bin above kBinRank
    red[33] = 0;  // the part's keys compacted so far
  }
  __syncthreads();
  lo = red[0];
  hi = red[16];
  for (int w = 1; w < T / kWave; ++w) {
    lo = min(lo, red[w]);
    hi = max(hi, red[16 + w]);
  }
  const float scale = (float)kCoarse / ((float)(hi - lo) + 1.0f);
  auto pos_of = [&](uint64_t kv) { return (float)(hi - key_ord(kv)) * scale; };
  auto coarse_of = [&](float xv) { return min((uint32_t)xv, (uint32_t)kCoarse - 1); };
  uint32_t* my_sub = coarse_sub + (lane % kCoarseSub) * kCoarse;
#pragma unroll
  for (int p = 0; p < PIN; ++p)
    if (p < np) hist_add(my_sub, coarse_of(pos_of(key[p])), valid(p));
  __syncthreads();
  const int kk = min(cnt, k);
  // coarse bin t: its count (the copies summed), then the exclusive scan
  uint32_t cc = 0;
#pragma unroll
  for (int u = 0; u < kCoarseSub; ++u) cc += coarse_sub[u * kCoarse + t];
  const uint32_t cincl = (uint32_t)wave_incl_scan((int)cc);
  if (lane == kWave - 1) red[40 + wave] = cincl;
  __syncthreads();
  uint32_t cstart = cincl - cc;
  for (int w = 0; w < wave; ++w) cstart += red[40 + w];
  coarse[t] = cc;
  coarse[kCoarse + t] = cstart;
  {
    // this part's coarse bins: those starting in [cut0, cut1)
    const uint32_t cut0 = (uint32_t)((int64_t)part * kk / parts);
    const uint32_t cut1 = (uint32_t)((int64_t)(part + 1) * kk / parts);
    const uint64_t m0 = __ballot(cstart < cut0), m1 = __ballot(cstart < cut1);
    if (lane == 0) {
      red[64 + wave] = (uint32_t)__popcll(m0);
      red[80 + wave] = (uint32_t)__popcll(m1);
    }
  }
  __syncthreads();
  uint32_t c0 = 0, c1 = 0;
  for (int w = 0; w < T / kWave; ++w) {
    c0 += red[64 + w];
    c1 += red[80 + w];
  }
  const int start0 = c0 < (uint32_t)kCoarse ? (int)coarse[kCoarse + c0] : cnt;  // the part's first rank
  const int count = (c1 < (uint32_t)kCoarse ? (int)coarse[kCoarse + c1] : cnt) - start0;
  *r0 = start0;
  *r1 = start0 + count;
  if (count > kFinMax) return false;
  // the part's keys to cand[0..count), one atomic per wave
  uint32_t mine = 0, wave_keys = 0;
#pragma unroll
  for (int p = 0; p < PIN; ++p) {
    if (p < np) {
      const uint32_t c = coarse_of(pos_of(key[p]));
      const bool in = valid(p) && c >= c0 && c < c1;
      mine |= in ? 1u << p : 0u;
      wave_keys += (uint32_t)__popcll(__ballot(in));
    }
  }
  uint32_t at = 0;
  if (lane == 0 && wave_keys > 0) at = atomicAdd(&red[33], wave_keys);
  at = wave_lane0(at);
#pragma unroll
  for (int p = 0; p < PIN; ++p) {
    if (p < np) {
      const bool in = (mine >> p) & 1u;
      const uint64_t m = __ballot(in);
      if (in) cand[at + lanes_below(m)] = key[p];
      at += (uint32_t)__popcll(m);
    }
  }
  __syncthreads();
  // fine bins, numbered from the part's first rank
  uint64_t own[P];
  uint32_t bin[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int j = p * T + t;
    own[p] = j < count ? cand[j] : 0;
    const float xv = pos_of(own[p]);
    const uint32_t c = coarse_of(xv);
    const uint32_t cn = coarse[c];  // >= 1 for a key of the part: it was counted there
    const uint32_t f = (uint32_t)((xv - (float)c) * (float)cn);
    bin[p] = j < count ? coarse[kCoarse + c] - (uint32_t)start0 + min(f, cn - 1) : 0u;
    hist_add(bins, bin[p], j < count);
  }
  __syncthreads();
  // exclusive scan over the bins; thread t owns bins [t*P, t*P + P)
  uint32_t c[P];
  uint32_t sum = 0, big = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    c[p] = bins[t * P + p];
    sum += c[p];
    big |= c[p] > (uint32_t)kBinRank ? 1u : 0u;
  }
  const uint32_t incl = (uint32_t)wave_incl_scan((int)sum);
  if (lane == kWave - 1) red[40 + wave] = incl;
  if (big) red[32] = 1;
  __syncthreads();
  uint32_t before = incl - sum;
  for (int w = 0; w < wave; ++w) before += red[40 + w];
  if (red[32] != 0) return false;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    bins[t * P + p] = before;  // start of the bin: the scatter cursor
    before += c[p];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p * T + t < count) cand[atomicAdd(&bins[bin[p]], 1u)] = own[p];
  __syncthreads();
  // bins[j] is now the end of bin j
  uint32_t rank[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    rank[p] = 0;
    if (p * T + t < count) {
      const int s0 = bin[p] == 0 ? 0 : (int)bins[bin[p] - 1];
      const int e = (int)bins[bin[p]];
      int r = s0;
      int i = s0;
      for (; i + 4 <= e; i += 4) {
        const uint64_t a0 = cand[i], a1 = cand[i + 1], a2 = cand[i + 2], a3 = cand[i + 3];
        r += (a0 > own[p]) + (a1 > own[p]) + (a2 > own[p]) + (a3 > own[p]);
      }
      for (; i < e; ++i) r += cand[i] > own[p];
      rank[p] = (uint32_t)r;
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (p * T + t < count) cand[rank[p]] = own[p];
  __syncthreads();
  for (int i = t; i < count && start0 + i < k; i += T) write_ranked(cand[i], start0 + i, xr, n, out_vals, out_idx);
  return true;
}

// Full-row exact top-k of an fp32 row (the fallback for rows whose
// collection overflowed); leaves the k keys in cand[0..k).
__device__ __noinline__ void row_radix_topk(const float* __restrict__ xr, int n, int k, uint64_t* cand,
                                            uint32_t* hist, uint32_t* ctl) {
  const uint32_t* xb = reinterpret_cast<const uint32_t*>(xr);
  block_row_topk<kFinT>([&](int i) { return ord_f32(xb[i]); }, n, k, cand, hist, ctl);
}

// The final's other route (out of line: rows of heavy ties, a part above
// kFinMax keys, an overflowed or failed exact collection): the row's exact
// top-k keys into cand by a radix select, a bitonic sort, and the ranks in
// [r0, r1) below k written out.
__device__ __noinline__ void final_by_select(int exact_mode, const float* __restrict__ xr, int n, int k, int b,
                                             int kb, const uint64_t* __restrict__ bucket_keys,
                                             const uint64_t* __restrict__ keys, int cnt, uint64_t* cand,
                                             uint32_t* bins, uint32_t* red, int r0, int r1,
                                             float* __restrict__ ov, int32_t* __restrict__ oi) {
  constexpr int T = kFinT;
  const int t = threadIdx.x;
  uint32_t* hist = bins;
  uint32_t* ctl = bins + 256;
  __syncthreads();  // the caller's last reads of cand, bins and red are done
  int have;
  if (!exact_mode) {
    cnt = b * kb;  // <= kFinMax (the plan checks it)
    for (int i = t; i < cnt; i += T) cand[i] = bucket_keys[i];
    __syncthreads();
    if (cnt > k) {
      const uint64_t kth = block_kth_key<T>(cand, cnt, k, hist, ctl);
      cnt = block_compact_ge<T, kFinMax / T>(cand, cnt, kth, ctl);
    }
    have = cnt;
  } else if (cnt > kRowCap || cnt < k) {  // overflow, or a sampled threshold above the k-th
    row_radix_topk(xr, n, k, cand, hist, ctl);
    have = k;
  } else {
    // k <= cnt <= kRowCap unique keys, all loaded once (kExactP per thread,
    // key i in thread i mod T): the k-th largest order word v by a radix
    // select; the k - rem keys above it are in, and of the keys equal to it
    // the rem with the largest index words (the lowest indices), found by a
    // second select on those words when more than rem tie
    // (loops over the register slots stop at np = the slots in use; the
    // leading bytes every kept key shares skip their radix passes)
    const int np = (cnt + T - 1) / T;
    uint64_t kk[kExactP];
#pragma unroll
    for (int p = 0; p < kExactP; ++p) kk[p] = p < np && t + p * T < cnt ? keys[t + p * T] : 0;
    auto valid = [&](int p) { return t + p * T < cnt; };
    uint32_t wa = 0xffffffffu, wo = 0;
#pragma unroll
    for (int p = 0; p < kExactP; ++p) {
      if (p < np && valid(p)) {
        wa &= key_ord(kk[p]);
        wo |= key_ord(kk[p]);
      }
    }
    wa = wave_reduce_dpp(wa, [](uint32_t a, uint32_t c) { return a & c; });
    wo = wave_reduce_dpp(wo, [](uint32_t a, uint32_t c) { return a | c; });
    if (lane_id() == 0) {
      red[2 * (t / kWave)] = wa;
      red[2 * (t / kWave) + 1] = wo;
    }
    __syncthreads();
    wa = 0xffffffffu;
    wo = 0;
    for (int w2 = 0; w2 < T / kWave; ++w2) {
      wa &= red[2 * w2];
      wo |= red[2 * w2 + 1];
    }
    __syncthreads();
    const int common = (wa ^ wo) == 0 ? 3 : min(3, __builtin_clz(wa ^ wo) / 8);
    const uint32_t lead = common > 0 ? wa & (0xffffffffu << (32 - 8 * common)) : 0u;
    int rem;
    const uint32_t v = block_radix_kth32<T>(
        k, hist, ctl,
        [&](uint32_t mask, uint32_t prefix, int shift) {
#pragma unroll
          for (int p = 0; p < kExactP; ++p) {
            if (p < np) {
              const uint32_t o = key_ord(kk[p]);
              hist_add_grouped(hist, (o >> shift) & 255u, valid(p) && (o & mask) == prefix);
            }
          }
        },
        &rem, common, lead);
    int ties = 0;
#pragma unroll
    for (int p = 0; p < kExactP; ++p) ties += (p < np && valid(p) && key_ord(kk[p]) == v) ? 1 : 0;
    ties = wave_sum(ties);
    if (lane_id() == 0) red[t / kWave] = (uint32_t)ties;
    __syncthreads();
    ties = 0;
    for (int w2 = 0; w2 < T / kWave; ++w2) ties += (int)red[w2];
    __syncthreads();
    uint32_t v2 = 0;  // keys equal to v with an index word >= v2 are in
    if (ties > rem) {
      int rem2;
      v2 = block_radix_kth32<T>(
          rem, hist, ctl,
          [&](uint32_t mask, uint32_t prefix, int shift) {
#pragma unroll
            for (int p = 0; p < kExactP; ++p) {
              if (p < np) {
                const uint32_t lo = (uint32_t)kk[p];
                hist_add(hist, (lo >> shift) & 255u, valid(p) && key_ord(kk[p]) == v && (lo & mask) == prefix);
              }
            }
          },
          &rem2);
    }
    if (t == 0) ctl[4] = 0;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kExactP; ++p) {
      if (p >= np) continue;
      const uint32_t o = key_ord(kk[p]);
      const bool keep = valid(p) && (o > v || (o == v && (uint32_t)kk[p] >= v2));
      const uint64_t m = __ballot(keep);
      if (m) {
        uint32_t pos = 0;
        if (lane_id() == 0) pos = atomicAdd(&ctl[4], (uint32_t)__popcll(m));
        pos = wave_lane0(pos);
        if (keep) cand[pos + lanes_below(m)] = kk[p];
      }
    }
    __syncthreads();
    const int kept = min((int)ctl[4], kFinMax);
    __syncthreads();
    have = kept;
  }
  block_sort_desc_bitonic(cand, have);
  for (int i = r0 + t; i < r1 && i < k; i += T) write_ranked(cand[i], i, xr, n, ov, oi);
}

// 3. final: `parts` workgroups per row (workgroup part * rows + row), each
//    writing the ranks of its share of the values.  exact_mode: the
//    collected keys (up to PIN = kExactP register slots per thread, fewer
//    when the row kept fewer keys); else the b * kb <= kFinMax bucket
//    candidates (PIN = kFinP).
template <int PIN>
__global__ __launch_bounds__(kFinT) void wide_final_kernel(const float* __restrict__ x, int64_t ldx, int n, int b,
                                                          int kb, int k, int exact_mode,
                                                          const uint64_t* __restrict__ bucket_cand,
                                                          const int* __restrict__ row_cnt,
                                                          const uint64_t* __restrict__ row_keys,
                                                          float* __restrict__ out_vals, int32_t* __restrict__ out_idx,
                                                          int parts) {
  __shared__ uint64_t cand[kFinMax];
  __shared__ uint32_t bins[kFinMax];
  __shared__ uint32_t red[kFinRed];
  const int m = (int)gridDim.x / parts;
  const int row = (int)blockIdx.x % m;  // the parts of a row on different XCDs
  const int part = (int)blockIdx.x / m;
  const float* xr = x + (int64_t)row * ldx;
  float* ov = out_vals + (int64_t)row * k;
  int32_t* oi = out_idx + (int64_t)row * k;
  const uint64_t* bucket_keys = bucket_cand + (int64_t)row * b * kb;
  const uint64_t* keys = row_keys + (int64_t)row * kRowCap;
  const int cnt = exact_mode ? row_cnt[row] : b * kb;
  int r0 = (int)((int64_t)part * k / parts), r1 = (int)((int64_t)(part + 1) * k / parts);
  bool done = false;
  // the fewest register slots that hold the row's keys: the sort's loops
  // over the slots are unrolled, so unused slots still cost time
  auto sort = [&](auto pin_c) {
    constexpr int P = decltype(pin_c)::value;
    return sort_part_and_write<P>(exact_mode ? keys : bucket_keys, cnt, k, part, parts, xr, n, ov, oi, cand, bins,
                                  red, &r0, &r1);
  };
  if (!exact_mode) {
    done = sort(std::integral_constant<int, PIN>{});
  } else if (cnt <= kRowCap && cnt >= k) {
    if (PIN > kFinP && cnt <= kFinP * kFinT)
      done = sort(std::integral_constant<int, kFinP>{});
    else if (PIN > 2 * kFinP && cnt <= 2 * kFinP * kFinT)
      done = sort(std::integral_constant<int, 2 * kFinP>{});
    else
      done = sort(std::integral_constant<int, PIN>{});
  }
  if (!done) final_by_select(exact_mode, xr, n, k, b, kb, bucket_keys, keys, cnt, cand, bins, red, r0, r1, ov, oi);
}

constexpr int kBufferWord3 = 0x00020000;  // buffer resource flags word (raw 32-bit loads)

// Orders a wave's LDS accesses around cross-lane exchanges (the wave's LDS
// operations complete in order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---- exact top-k in one read: sampled threshold, contiguous collect ---------
//
// The row's k-th largest key bounds what must be collected; a threshold at
// or below it, close to it, comes from a sample: stratum t of the row (n /
// 1024 elements) gives one 16-element chunk at a pseudo-random offset, so
// every element of the strata has the same chance to be drawn, whatever the
// row's structure.  The threshold is the r-th largest of the maxima of the
// 4096 groups of four consecutive samples, rounded down to a multiple of 256
// order steps -- at most the r-th largest sample, since r groups hold a
// sample at or above it -- with r above the sample's expected count of
// top-k elements by a wide margin, so that the row almost surely holds k
// elements at or above it.  The collect
// then keeps every element at or above it in one contiguous read, and the
// final takes the exact top-k of the kept keys -- or, when fewer than k were
// kept (the margin failed) or the list overflowed, a full-row exact select.
// The sample decides the cost, never the result.
constexpr int kSampleT = 1024;    // strata (threads) per row
constexpr int kSampleChunk = 16;  // elements per sample chunk
constexpr int kCrT = 512;         // collect workgroup
constexpr int kCrU = 16;          // loads per lane per step
constexpr int kCrStep = kCrT * kCrU;

__device__ __forceinline__ uint32_t mix32(uint32_t v) {  // an integer hash (xorshift-multiply rounds)
  v ^= v >> 16;
  v *= 0x7feb352du;
  v ^= v >> 15;
  v *= 0x846ca68bu;
  v ^= v >> 16;
  return v;
}

// The r-th largest of the T * G order words o[] (G per thread, r <= T * G)
// with its low 8 bits cleared: a lower bound of it, at most 255 order steps
// below, from two 12-bit radix passes (bits 31..20, then bits 19..8 of the
// words that match the first digit) -- half the passes of a full 8-bit
// select.  hist: 4096 words, ctl: 2 + T / 64 words.
template <int T, int G>
__device__ uint32_t block_kth32_floor(const uint32_t (&o)[G], int r, uint32_t* hist, uint32_t* ctl) {
  constexpr int NB = 4096, Q = NB / T;  // bins per thread
  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = t / kWave;
  uint32_t prefix = 0, mask = 0;
  int rem = r;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int shift = pass == 0 ? 20 : 8;
    for (int i = t; i < NB; i += T) hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const uint32_t d = (o[j] >> shift) & 0xfffu;
      if (pass == 0)
        hist_add_grouped(hist, d, true);  // the leading digit crowds a few bins
      else
        hist_add(hist, d, (o[j] & mask) == prefix);
    }
    __syncthreads();
    // thread t owns the Q bins below NB - Q t, high digits first
    uint32_t h[Q];
    int sum = 0;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      h[q] = hist[NB - 1 - Q * t - q];
      sum += (int)h[q];
    }
    const int incl = wave_incl_scan(sum);
    if (lane == kWave - 1) ctl[2 + wave] = (uint32_t)incl;
    __syncthreads();
    int acc = incl - sum;
    for (int w = 0; w < wave; ++w) acc += (int)ctl[2 + w];
    if (acc < rem && rem <= acc + sum) {
      int d = -1;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        if (d < 0) {
          if (acc + (int)h[q] >= rem)
            d = NB - 1 - Q * t - q;
          else
            acc += (int)h[q];
        }
      }
      ctl[0] = (uint32_t)d;
      ctl[1] = (uint32_t)(rem - acc);
    }
    __syncthreads();
    prefix |= ctl[0] << shift;
    mask |= 0xfffu << shift;
    rem = (int)ctl[1];
  }
  return prefix;
}

__global__ __launch_bounds__(kSampleT) void wide_sample_kernel(const float* __restrict__ x, int64_t ldx, int n,
                                                              int r_sel, float* __restrict__ rowthr,
                                                              int* __restrict__ row_cnt) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t ctl[2 + kSampleT / kWave];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int st = n / kSampleT;  // stratum length, >= kSampleChunk
  const uint32_t slots = (uint32_t)(st / kSampleChunk);
  const int off = (int)(mix32((uint32_t)row * kSampleT + (uint32_t)t + 0x9e3779b9u) % slots) * kSampleChunk;
  const uint32_t* xs = reinterpret_cast<const uint32_t*>(x + (int64_t)row * ldx) + (int64_t)t * st + off;
  constexpr int G = kSampleChunk / 4;
  uint32_t o[G];
#pragma unroll
  for (int j = 0; j < G; ++j)
    o[j] = max(max(ord_f32(xs[4 * j]), ord_f32(xs[4 * j + 1])), max(ord_f32(xs[4 * j + 2]), ord_f32(xs[4 * j + 3])));
  const uint32_t v = block_kth32_floor<kSampleT, G>(o, r_sel, hist, ctl);
  if (t == 0) {
    rowthr[row] = __uint_as_float(bits_from_ord(v));
    row_cnt[row] = 0;
  }
}

// Collect: workgroup (row, c) -- the chunks of a row on different XCDs --
// reads steps [c * spc, (c + 1) * spc) of the row (step s: elements s *
// kCrStep + u * kCrT + t) in order, two steps of loads in flight behind the
// one it filters.  An element at or above the row's threshold goes to the
// wave's LDS buffer; a buffer past its mark moves to the workgroup's LDS list
// (one LDS atomic), and at the end the list goes to the row's key list with
// one atomic on the row's counter per workgroup.  (Atomics on one global
// counter from many workgroups are slow here -- they serialise across the
// XCDs -- so none are taken while the loads stream.)  Keys beyond the list's
// capacity go to the row's list directly, with an atomic of their own.
constexpr int kCrMark = 192;                 // move a wave's buffer above this many keys
constexpr int kCrBuf = kCrMark + kWave;      // + one instruction's worth
constexpr int kCrList = 6144;                // keys per workgroup list (48 KiB)
__global__ __launch_bounds__(kCrT) void wide_collect_row_kernel(const float* __restrict__ x, int64_t ldx, int n,
                                                               int chunks, int spc, const float* __restrict__ rowthr,
                                                               int* __restrict__ row_cnt,
                                                               uint64_t* __restrict__ row_keys) {
  constexpr int W = kCrT / kWave;
  __shared__ uint64_t wbuf[W][kCrBuf];
  __shared__ uint64_t wg_list[kCrList];
  __shared__ uint32_t wg_n;
  __shared__ uint32_t wg_base;
  const int row = (int)blockIdx.x / chunks;
  const int c = (int)blockIdx.x % chunks;
  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  uint64_t* buf = wbuf[wave];
  const float* xrow = x + (int64_t)row * ldx;
  const float th = rowthr[row];
  uint64_t* out = row_keys + (int64_t)row * kRowCap;
  const int nsteps_row = (n + kCrStep - 1) / kCrStep;
  const int full_steps = n / kCrStep;
  const int s_begin = c * spc;
  const int ns = max(0, min(nsteps_row, s_begin + spc) - s_begin);
  auto phys = [&](int i) { return s_begin + i; };
  if (t == 0) wg_n = 0;
  __syncthreads();
  int fill = 0;  // wave-uniform
  // the wave's buffer to the workgroup list; what does not fit goes to the
  // row's list
  auto move = [&]() {
    wave_sync_lds();
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&wg_n, (uint32_t)fill);
    base = wave_lane0(base);
    const int fit = (int)min((uint32_t)fill, base < (uint32_t)kCrList ? (uint32_t)kCrList - base : 0u);
    for (int j = lane; j < fit; j += kWave) wg_list[base + j] = buf[j];
    if (fit < fill) {
      int gb = 0;
      if (lane == 0) gb = atomicAdd(&row_cnt[row], fill - fit);
      gb = (int)wave_lane0((uint32_t)gb);
      for (int j = fit + lane; j < fill; j += kWave)
        if (gb + j - fit < kRowCap) out[gb + j - fit] = buf[j];
    }
    wave_sync_lds();
    fill = 0;
  };
  auto see = [&](bool keep, float v, uint32_t idx) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(keep);
    if (m) {
      if (keep) buf[fill + (int)lanes_below(m)] = make_key(ord_f32(__float_as_uint(v)), idx);
      fill += __popcll(m);
      if (fill > kCrMark) move();
    }
  };
  float wa[kCrU], wb[kCrU], wc[kCrU];
  auto load = [&](float (&w)[kCrU], int i) {
    const int s = phys(i);
    if (s < full_steps) {
      const float* p = xrow + (int64_t)s * kCrStep + t;
#pragma unroll
      for (int u = 0; u < kCrU; ++u) w[u] = p[u * kCrT];
    } else {
#pragma unroll
      for (int u = 0; u < kCrU; ++u) {
        const int64_t e = (int64_t)s * kCrStep + u * kCrT + t;
        w[u] = e < n ? xrow[e] : 0.0f;
      }
    }
  };
  auto filt = [&](const float (&w)[kCrU], int i) {
    const int s = phys(i);
    const uint32_t i0 = (uint32_t)s * kCrStep + (uint32_t)t;
    if (s < full_steps) {
#pragma unroll
      for (int u = 0; u < kCrU; ++u) see(w[u] >= th, w[u], i0 + (uint32_t)(u * kCrT));
    } else {
#pragma unroll
      for (int u = 0; u < kCrU; ++u) {
        const uint32_t e = i0 + (uint32_t)(u * kCrT);
        see(e < (uint32_t)n && w[u] >= th, w[u], e);
      }
    }
  };
  // step i sits in buffer i mod 3; steps i + 1 and i + 2 load while it is
  // filtered
  if (ns > 0) load(wa, 0);
  if (ns > 1) load(wb, 1);
  for (int i = 0; i < ns; i += 3) {
    if (i + 2 < ns) load(wc, i + 2);
    filt(wa, i);
    if (i + 1 < ns) {
      if (i + 3 < ns) load(wa, i + 3);
      filt(wb, i + 1);
    }
    if (i + 2 < ns) {
      if (i + 4 < ns) load(wb, i + 4);
      filt(wc, i + 2);
    }
  }
  if (fill > 0) move();
  __syncthreads();
  const int tot = (int)min(wg_n, (uint32_t)kCrList);
  if (t == 0) wg_base = tot ? (uint32_t)atomicAdd(&row_cnt[row], tot) : 0u;
  __syncthreads();
  const int base = (int)wg_base;
  for (int j = t; j < tot; j += kCrT)
    if (base + j < kRowCap) out[base + j] = wg_list[j];
}

// ---- one-pass stage 1 (bucketed, b a multiple of 64, k_b <= 16) ----------
//
// A workgroup owns 64 consecutive buckets of one row over the whole row --
// lane l is bucket 64 * g + l -- and its 8 waves take interleaved batches of
// sweeps, so every element of a bucket passes through the workgroup that
// owns it.  Per bucket, in LDS:
//  - a window [lo, lo + span] of order keys: of the bucket's 256 first
//    samples each wave keeps the four largest of its 32, and lo is the k_b-th
//    largest of those 32 (k_b elements of the bucket reach it, so its k_b-th
//    largest does too); the window's top sits half its width above the
//    largest sample, where the bucket's k_b-th largest often lies;
//  - a histogram of the window (64 bins, two 16-bit counts per word);
//  - thr, the highest bin whose count together with the bins above reaches
//    k_b, refreshed at a few points of the stream.  Counts only grow, so thr
//    never passes the bin of the bucket's final k_b-th largest key, and the
//    bins below thr can never matter again: elements below them are dropped
//    without being counted;
//  - a log of (key, index) for every element at or above thr when it
//    arrives.  An element of the bucket's exact top-k_b has a key >= the
//    final k_b-th, so its bin is >= every thr the stream ever saw: it is
//    logged.
// A lane tests each of its elements against one float (the lower edge of
// its bucket's threshold bin); the few that pass go through a per-wave LDS
// ring, and the histogram and log updates run on full 64-element chunks of
// it.  At the end the keys of the log in bins >= the final thr (the k_b-th
// largest's bin: fewer than k_b keys above it, all of it logged) are ranked
// and the first k_b kept, sorted.  A bucket whose log overflowed or whose
// threshold bin holds more keys than a wave ranks at once is redone by one
// wave with a full scan of the bucket, so the result is exact for any input.
// Each lane keeps two batches of loads in flight behind the one it works on.
constexpr int kOpW = 8;    // waves per 64 buckets
constexpr int kOpU = 16;   // sweeps per wave and batch (loads per lane per batch)
constexpr int kOpNB = 64;  // histogram bins per bucket: lane l of a tick owns bin l
constexpr int kOpHW = kOpNB / 2 + 1;  // histogram words per bucket (padded row)
constexpr int kOpCap = 120;           // logged keys per bucket
constexpr int kOpQ = 128;             // per-wave ring of staged elements

struct OnepassShared {
  uint32_t hist[kWave][kOpHW];
  uint64_t logk[kWave][kOpCap];  // the first samples' value lists merge here before any key is logged
  alignas(16) uint64_t ring[kOpW][kOpQ];  // staged (value bits, sweep, bucket); candidates of the end phase
  uint32_t logn[kWave];
  int thr[kWave];
  uint32_t lo[kWave], span[kWave];
  int sh[kWave];
};

// Exact top-16 keys of bucket r of the row (elements r, r + b, ...), sorted,
// by one wave: per-lane key queues over a strided scan, merged across lanes.
// Lane j returns entry j.
__device__ __noinline__ uint64_t wave_bucket_top16(const float* __restrict__ xrow, int n, int b, int r) {
  const int lane = lane_id();
  const uint32_t* xb = reinterpret_cast<const uint32_t*>(xrow);
  uint64_t q[kWideKB];
#pragma unroll
  for (int j = 0; j < kWideKB; ++j) q[j] = 0;
  for (int64_t i = (int64_t)r + (int64_t)lane * b; i < n; i += (int64_t)kWave * b)
    queue_insert<kWideKB>(q, make_key(ord_f32(xb[i]), (uint32_t)i));
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    uint64_t other[kWideKB];
#pragma unroll
    for (int j = 0; j < kWideKB; ++j) other[j] = shfl_xor_u64(q[j], o);
    queue_merge<kWideKB>(q, other);
  }
  uint64_t mine = 0;
#pragma unroll
  for (int j = 0; j < kWideKB; ++j)
    if (j == lane) mine = q[j];
  return mine;
}

// Inclusive prefix sum over the 64 lanes with DPP: row shifts build each
// row's prefix, then row broadcasts carry the totals of the rows below.
__device__ __forceinline__ int wave_prefix_dpp(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2 and 3
  return v;
}

// A workgroup-scope relaxed load of an LDS word other waves may be updating.
template <typename U>
__device__ __forceinline__ U lds_load_relaxed(const U* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}


__global__ __launch_bounds__(kOpW * kWave) void wide_onepass_kernel(const float* __restrict__ x, int64_t ldx, int n,
                                                                    int b, int kb, int groups, int final_exact,
                                                                    uint64_t* __restrict__ cand,
                                                                    float* __restrict__ out_vals,
                                                                    int32_t* __restrict__ out_idx) {
  constexpr int NB = kWave;  // buckets per workgroup
  constexpr int NW = kOpW;   // waves
  constexpr int T = NW * kWave;
  __shared__ OnepassShared S;
  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(t / kWave);
  const int sw = wave;  // the wave takes sweeps sw + W * (U * bt + u)
  // consecutive workgroups go to different XCDs: taking the row from the low
  // part of the index spreads every bucket group over the XCDs, so that no
  // XCD's L2 channels see only one column slice of the sweeps
  const int mrows = (int)(gridDim.x / groups);
  const int row = (int)blockIdx.x % mrows;
  const int g = (int)blockIdx.x / mrows;
  const int lb = lane;        // this lane's bucket in the group
  const int r = g * NB + lb;  // ... in the row
  const float* xrow = x + (int64_t)row * ldx;
  const float* xr = xrow + r;
  const int nsw = (n + b - 1) / b;  // sweeps; the last may be partial
  const int nbatch = (nsw + kOpW * kOpU - 1) / (kOpW * kOpU);

  for (int i = t; i < NB * kOpHW; i += T) (&S.hist[0][0])[i] = 0;
  if (t < NB) {
    S.logn[t] = 0;
    S.thr[t] = 0;
  }

  // batch bt of the stream is batch (bt + rot) mod nbatch of the row:
  // workgroups start at different offsets, so the ones in flight together
  // read addresses spread over the rows instead of one offset of every row
  // (which crowds a few HBM channels); any order sees every element once
  const int rot = (int)(blockIdx.x % (unsigned)nbatch);
  auto phys = [&](int bt) { return bt + rot < nbatch ? bt + rot : bt + rot - nbatch; };
  auto sweep_of = [&](int bt, int u) { return sw + kOpW * (kOpU * phys(bt) + u); };
  // A batch below the row's first partial sweep is full: every lane has an
  // element in each of its sweeps, so a load is a buffer load at the lane's
  // byte offset in a resource over the sweep (scalar address arithmetic
  // only), and no element needs a liveness test.  In the others a sweep past
  // the lane's last element is read at that element instead (every load is
  // unconditional) and masked afterwards.
  const int full_sweeps = n / b;
  auto full = [&](int bt) { return kOpW * kOpU * (phys(bt) + 1) <= full_sweeps; };
  const int last = (n - 1 - r) / b;  // the lane's last sweep
  auto live = [&](int s) { return s <= last; };
  float wa[kOpU], wb[kOpU], wc[kOpU];
  auto load = [&](float (&w)[kOpU], int bt) {
    if (full(bt)) {
#pragma unroll
      for (int u = 0; u < kOpU; ++u) {
        const __amdgpu_buffer_rsrc_t sweep_rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(xrow + (int64_t)sweep_of(bt, u) * b), (short)0, b * 4, kBufferWord3);
        w[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sweep_rs, r * 4, 0, 0));
      }
    } else {
#pragma unroll
      for (int u = 0; u < kOpU; ++u) w[u] = xr[(int64_t)min(sweep_of(bt, u), last) * b];
    }
  };
  load(wa, 0);
  if (nbatch > 1) load(wb, 1);
  if (nbatch > 2) load(wc, 2);  // in flight while the window is computed

  // the window, from each bucket's first two batches (256 samples): every
  // lane keeps the four largest of its 32, the waves' lists merge into the
  // first wave (top 16), and lo is the k_b-th largest of the merged list --
  // k_b distinct elements of the bucket reach it
  {
    float q4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    const bool full0 = full(0), full1 = nbatch > 1 && full(1);
#pragma unroll
    for (int u = 0; u < kOpU; ++u) fnet_insert<4>(q4, (full0 || live(sweep_of(0, u))) ? wa[u] : -INFINITY);
#pragma unroll
    for (int u = 0; u < kOpU; ++u)
      fnet_insert<4>(q4, (full1 || (nbatch > 1 && live(sweep_of(1, u)))) ? wb[u] : -INFINITY);
    float q[kWideKB];
#pragma unroll
    for (int j = 0; j < kWideKB; ++j) q[j] = j < 4 ? q4[j] : -INFINITY;
    float* mbuf = reinterpret_cast<float*>(&S.logk[0][0]);
    for (int half = kOpW / 2; half >= 1; half /= 2) {
      if (sw >= half && sw < 2 * half) {
#pragma unroll
        for (int j = 0; j < kWideKB; ++j) mbuf[((sw - half) * kWideKB + j) * kWave + lane] = q[j];
      }
      __syncthreads();
      if (sw < half) {
        float c[kWideKB];
#pragma unroll
        for (int j = 0; j < kWideKB; ++j) c[j] = mbuf[(sw * kWideKB + j) * kWave + lane];
        queue_merge<kWideKB>(q, c);
      }
      __syncthreads();
    }
    if (sw == 0) {
      float lo_v = q[0];
#pragma unroll
      for (int j = 0; j < kWideKB; ++j)
        if (j == kb - 1) lo_v = q[j];
      const uint32_t lo = ord_f32(__float_as_uint(lo_v));
      const uint32_t width = ord_f32(__float_as_uint(q[0])) - lo;
      const uint32_t span = (uint32_t)min((uint64_t)width + width / 2, (uint64_t)(0xffffffffu - lo));
      int sh = 0;
      while ((span >> sh) >= (uint32_t)kOpNB) ++sh;
      S.lo[lb] = lo;
      S.span[lb] = span;
      S.sh[lb] = sh;
    }
  }
  __syncthreads();
  const uint32_t my_lo = S.lo[lb];
  const int my_sh = S.sh[lb];
  float fthr = __uint_as_float(bits_from_ord(my_lo));  // lower edge of the threshold bin

  // staged elements: ring entries head .. tail (wave-uniform counters)
  int head = 0, tail = 0;
  uint64_t* ring = S.ring[wave];
  auto drain = [&](int cnt) {  // the oldest cnt (<= 64) staged elements
    wave_sync_lds();
    if (lane < cnt) {
      const uint64_t e = ring[(head + lane) & (kOpQ - 1)];
      const uint32_t o = ord_f32((uint32_t)e);
      const int s = (int)((e >> 32) & 0xffffu);
      const int bl = (int)(e >> 48);
      const int bin = (int)(min(o - S.lo[bl], S.span[bl]) >> S.sh[bl]);
      atomicAdd(&S.hist[bl][bin >> 1], 1u << ((bin & 1) << 4));
      if (bin >= lds_load_relaxed(&S.thr[bl])) {
        const uint32_t slot = atomicAdd(&S.logn[bl], 1u);
        if (slot < (uint32_t)kOpCap) S.logk[bl][slot] = make_key(o, (uint32_t)(s * b + g * NB + bl));
      }
    }
    head += cnt;
    wave_sync_lds();
  };
  // a staged element: value bits, then (sweep | bucket << 16)
  auto stage = [&](bool pass, float v, uint32_t hi) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(pass);
    if (m) {
      if (pass) {
        const uint32_t pos =
            __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)tail));
        uint32_t* e = reinterpret_cast<uint32_t*>(ring + (pos & (kOpQ - 1)));
        e[0] = __float_as_uint(v);
        e[1] = hi;
      }
      tail += __popcll(m);
      if (tail - head >= kWave) drain(kWave);
    }
  };
  auto process = [&](const float (&w)[kOpU], int bt) {
    const uint32_t hi0 = (uint32_t)sweep_of(bt, 0) | ((uint32_t)lb << 16);
    if (full(bt)) {
#pragma unroll
      for (int u = 0; u < kOpU; ++u) stage(w[u] >= fthr, w[u], hi0 + (uint32_t)(kOpW * u));
    } else {
#pragma unroll
      for (int u = 0; u < kOpU; ++u)
        stage(live(sweep_of(bt, u)) && w[u] >= fthr, w[u], hi0 + (uint32_t)(kOpW * u));
    }
  };
  // threshold bins from the histograms: wave w refreshes buckets w, w + NW,
  // ...  Only the last refresh waits for every wave's counts.  Before it a
  // wave reads counts other waves are still adding to: they are lower bounds
  // of the counts so far, so the bin it finds is at or below the one the
  // full counts give -- still never above the bin of the bucket's final k_b-th
  // largest key, which is all the filter and the log rely on
  constexpr int kQ = NB / NW;
  auto tick = [&](bool last_tick) {
    if (tail > head) drain(tail - head);
    if (last_tick) lds_barrier();
    // lane l holds bin 63 - l, so a prefix sum over the lanes is the count
    // of keys in the bins from 63 - l up; the first lane reaching k_b names
    // the threshold bin
    const int bin = kOpNB - 1 - lane;
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      const int rb = wave + NW * q;
      const int c = (int)((lds_load_relaxed(&S.hist[rb][bin >> 1]) >> ((bin & 1) << 4)) & 0xffffu);
      const uint64_t reach = __builtin_amdgcn_ballot_w64(wave_prefix_dpp(c) >= kb);
      if (reach != 0 && lane == 0)
        __hip_atomic_store(&S.thr[rb], kOpNB - 1 - (int)__builtin_ctzll(reach), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (last_tick) {
      lds_barrier();
    } else {
      wave_sync_lds();
    }
    fthr = __uint_as_float(bits_from_ord(my_lo + ((uint32_t)lds_load_relaxed(&S.thr[lb]) << my_sh)));
  };
  // refreshes after 3, 4, 6, 8, 12, 16, 24, ... batches and the last one
  // (after the first two the counted keys are the samples at or above lo,
  // exactly k_b of which reach it: the bin could not move yet)
  auto ticks_after = [&](int bt) {
    const int c = bt + 1, c3 = c / 3;
    return bt == nbatch - 1 || (c >= 3 && ((c & (c - 1)) == 0 || (c == 3 * c3 && (c3 & (c3 - 1)) == 0)));
  };

  // batch bt sits in buffer bt mod 3; the loads of bt + 1 and bt + 2 are in
  // flight while it is worked on
  for (int bt = 0; bt < nbatch; bt += 3) {
    if (bt > 0 && bt + 2 < nbatch) load(wc, bt + 2);
    process(wa, bt);
    if (ticks_after(bt)) tick(bt == nbatch - 1);
    if (bt + 1 < nbatch) {
      if (bt + 3 < nbatch) load(wa, bt + 3);
      process(wb, bt + 1);
      if (ticks_after(bt + 1)) tick(bt + 1 == nbatch - 1);
    }
    if (bt + 2 < nbatch) {
      if (bt + 4 < nbatch) load(wb, bt + 4);
      process(wc, bt + 2);
      if (ticks_after(bt + 2)) tick(bt + 2 == nbatch - 1);
    }
  }
  // the tick after the last batch left every bucket's final threshold bin

  // each bucket's exact top-k_b, wave w taking buckets w, w + NW, ...  Lane
  // l holds bucket l's final parameters; the candidates of consecutive
  // buckets go to alternate halves of the wave's ring (no wait between
  // buckets), and the results are stored together at the end (a store in
  // flight would otherwise hold up the next bucket's LDS reads)
  const int p_nl = (int)S.logn[lane];
  const int p_thr = S.thr[lane];
  const int p_span = (int)S.span[lane];
  uint64_t res[kQ];
  int rk[kQ];
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    const int rb = wave + NW * q;
    const int nl = __builtin_amdgcn_readlane(p_nl, rb);
    const int B = __builtin_amdgcn_readlane(p_thr, rb);
    const uint32_t blo = (uint32_t)__builtin_amdgcn_readlane((int)my_lo, rb);
    const uint32_t bspan = (uint32_t)__builtin_amdgcn_readlane(p_span, rb);
    const int bsh = __builtin_amdgcn_readlane(my_sh, rb);
    uint64_t* cb = ring + (q & 1) * kWave;
    int cnt = 0;
    if (nl <= kOpCap) {
      for (int i0 = 0; i0 < nl; i0 += kWave) {
        const int i = i0 + lane;
        const uint64_t key = i < nl ? S.logk[rb][i] : 0;
        const bool keep = i < nl && (int)(min(key_ord(key) - blo, bspan) >> bsh) >= B;
        const uint64_t m = __ballot(keep);
        const int slot = cnt + (int)lanes_below(m);
        if (keep && slot < kWave) cb[slot] = key;
        cnt += __popcll(m);
      }
    }
    const bool ok = nl <= kOpCap && cnt >= kb && cnt <= kWave;
    // zero keys pad the candidates to a multiple of 4 (a zero key is above none)
    if (ok && lane >= cnt && lane < ((cnt + 3) & ~3)) cb[lane] = 0;
    wave_sync_lds();
    uint64_t mine = 0;
    int rank = kWave;
    if (ok) {
      // rank of each candidate among the candidates (lane = candidate), the
      // others read as LDS broadcasts four at a time
      mine = lane < cnt ? cb[lane] : 0;
      rank = 0;
      for (int j = 0; j < cnt; j += 4) {
        const ulonglong2 p0 = *reinterpret_cast<const ulonglong2*>(cb + j);
        const ulonglong2 p1 = *reinterpret_cast<const ulonglong2*>(cb + j + 2);
        rank += (p0.x > mine ? 1 : 0) + (p0.y > mine ? 1 : 0) + (p1.x > mine ? 1 : 0) + (p1.y > mine ? 1 : 0);
      }
      if (lane >= cnt) rank = kWave;
    } else {
      mine = wave_bucket_top16(xrow, n, b, g * NB + rb);
      rank = lane;
    }
    res[q] = mine;
    rk[q] = rank;
  }
#pragma unroll
  for (int q = 0; q < kQ; ++q) {
    if (rk[q] < kb) {
      const int64_t slot = ((int64_t)row * b + g * NB + wave + NW * q) * kb + rk[q];
      if (final_exact) {
        cand[slot] = res[q];
      } else {
        uint32_t idx = key_idx(res[q]);
        idx = idx < (uint32_t)n ? idx : 0u;  // only reachable with NaN inputs
        const uint32_t o = key_ord(res[q]);
        out_idx[slot] = (int32_t)idx;
        reinterpret_cast<uint32_t*>(out_vals)[slot] =
            o == 0x80000000u ? reinterpret_cast<const uint32_t*>(xrow)[idx] : bits_from_ord(o);
      }
    }
  }
}

}  // namespace

WidePlan plan_wide(int dtype, int64_t m, int64_t n, int64_t k, int64_t b, int64_t kb, bool exact, bool final_exact) {
  WidePlan p{};
  if (exact) {
    b = kExactB;
    kb = kWideKB;
  }
  p.b = b;
  p.kb = kb;
  p.kbn = kb <= 8 ? 8 : kWideKB;
  const bool shape_ok = exact ? (k <= kFinMax && n >= (int64_t)kExactB * kWideKB)
                              : (kb >= 1 && kb <= kWideKB && n / b >= kb && (!final_exact || b * kb <= kFinMax));
  p.ok = dtype == IN_F32 && m >= 1 && b % kWave == 0 && b >= kWave && b <= 65536 && n <= INT32_MAX && shape_ok;
  if (!p.ok) return p;
  const int64_t nsweeps = (n + b - 1) / b;
  p.groups = b / kWave;
  // waves per workgroup = chunks of sweeps: a power of two up to kMaxChunks,
  // each chunk at least 4 * KB sweeps long
  int nc = kMaxChunks;
  while (nc > 1 && nsweeps / nc < 4 * p.kbn) nc /= 2;
  p.nchunks = nc;
  p.sweeps_per_chunk = (int)((nsweeps + nc - 1) / nc);
  p.blocks = m * p.groups;
  // final: one 1024-thread workgroup holds a CU; with fewer rows than CUs a
  // row's sort is split over up to kFinParts workgroups
  p.final_parts = (int)std::max<int64_t>(1, std::min<int64_t>(kFinParts, kFinCUs / m));
  if (exact) {
    // one read when the list the sampled threshold is expected to keep fits
    // well inside the row's list: r = the sample's expected count of top-k
    // elements plus six of its standard deviations (the chunks make the
    // count lumpier than independent draws) plus 16
    const double S = (double)kSampleT * kSampleChunk;
    const double rate = (double)k * S / (double)n;
    const double r = std::min(S / 4, std::ceil(rate + 6.0 * std::sqrt(rate)) + 16.0);
    p.sample_r = (int)r;
    p.sampled = n / kSampleT >= kSampleChunk && r * (double)n / S <= 0.75 * kRowCap;
    const int64_t nsteps_row = (n + kCrStep - 1) / kCrStep;
    // collect workgroups: about 512 in all, and chunks of at most 512 KiB
    // (128 rows of 2653751 elements: 4 chunks per row took 289 us, 21 took
    // 268 us; 256 KiB chunks on 64 rows of 2^20 were slower than 512 KiB)
    int64_t chunks = std::min<int64_t>(
        std::max<int64_t>({(int64_t)1, (512 + m - 1) / m, (n * 4 + (512 << 10) - 1) / (512 << 10)}), nsteps_row);
    const int64_t spc = (nsteps_row + chunks - 1) / chunks;
    p.steps_per_chunk = (int)spc;
    p.row_chunks = (int)((nsteps_row + spc - 1) / spc);
  }
  p.vals_bytes = exact && !p.sampled ? (size_t)m * kWideKB * b * 4 : 0;
  p.bucket_bytes = exact ? (size_t)m * 4 : (size_t)m * b * 4;
  p.cand_bytes = (!exact && final_exact) ? (size_t)m * b * kb * 8 : 0;
  p.row_bytes = exact ? (size_t)m * kRowCap * 8 : 0;
  return p;
}

hipError_t launch_wide(const WidePlan& p, const float* x, int64_t m, int64_t n, int64_t ldx, int64_t k, bool exact,
                       bool final_exact, const WideBuffers& w, void* out_vals, int32_t* out_idx, hipStream_t s) {
  const int b = (int)p.b, kb = (int)p.kb;
  const dim3 grid((unsigned)p.blocks), block((unsigned)(kWave * p.nchunks));
  const int fparts = p.final_parts;
  // bucketed rows whose buckets hold at most 65535 elements (16-bit
  // histogram counts): one pass over the input
  if (!exact && (n + b - 1) / b <= 65535) {
    ATOPK_LAUNCH(wide_onepass_kernel, grid, dim3(kOpW * kWave), 0, s, x, ldx, (int)n, b, kb, (int)p.groups,
                 final_exact ? 1 : 0, w.cand, static_cast<float*>(out_vals), out_idx);
    if (final_exact)
      ATOPK_LAUNCH(wide_final_kernel<kFinP>, dim3((unsigned)(m * fparts)), dim3(kFinT), 0, s, x, ldx, (int)n, b, kb,
                   (int)k, 0, w.cand, w.row_cnt, w.row_keys, static_cast<float*>(out_vals), out_idx, fparts);
    return hipGetLastError();
  }
  if (exact && p.sampled) {
    ATOPK_LAUNCH(wide_sample_kernel, dim3((unsigned)m), dim3(kSampleT), 0, s, x, ldx, (int)n, p.sample_r, w.rowthr,
                 w.row_cnt);
    ATOPK_LAUNCH(wide_collect_row_kernel, dim3((unsigned)(m * p.row_chunks)), dim3(kCrT), 0, s, x, ldx, (int)n,
                 p.row_chunks, p.steps_per_chunk, w.rowthr, w.row_cnt, w.row_keys);
    ATOPK_LAUNCH(wide_final_kernel<kExactP>, dim3((unsigned)(m * fparts)), dim3(kFinT), 0, s, x, ldx, (int)n, b, kb,
                 (int)k, 1,
                 w.cand, w.row_cnt, w.row_keys, static_cast<float*>(out_vals), out_idx, fparts);
    return hipGetLastError();
  }
  if (p.kbn == 8)
    ATOPK_LAUNCH(wide_values_kernel<8>, grid, block, 0, s, x, ldx, (int)n, b, kb, (int)p.groups,
                       p.sweeps_per_chunk, exact ? 1 : 0, w.thr, w.need, w.vals);
  else
    ATOPK_LAUNCH(wide_values_kernel<kWideKB>, grid, block, 0, s, x, ldx, (int)n, b, kb, (int)p.groups,
                       p.sweeps_per_chunk, exact ? 1 : 0, w.thr, w.need, w.vals);
  if (exact) {
    ATOPK_LAUNCH(wide_exact_threshold_kernel, dim3((unsigned)m), dim3(kExactB), 0, s, w.vals, (int)k, w.rowthr,
                       w.row_cnt);
    ATOPK_LAUNCH(wide_collect_exact_kernel, grid, block, 0, s, x, ldx, (int)n, b, (int)p.groups,
                       p.sweeps_per_chunk, w.rowthr, w.row_cnt, w.row_keys);
  } else if (p.kbn == 8) {
    ATOPK_LAUNCH(wide_collect_bucket_kernel<8>, grid, block, 0, s, x, ldx, (int)n, b, kb, (int)p.groups,
                       p.sweeps_per_chunk, final_exact ? 1 : 0, w.thr, w.need, w.cand,
                       static_cast<float*>(out_vals), out_idx);
  } else {
    ATOPK_LAUNCH(wide_collect_bucket_kernel<kWideKB>, grid, block, 0, s, x, ldx, (int)n, b, kb, (int)p.groups,
                       p.sweeps_per_chunk, final_exact ? 1 : 0, w.thr, w.need, w.cand,
                       static_cast<float*>(out_vals), out_idx);
  }
  if (exact)
    ATOPK_LAUNCH(wide_final_kernel<kExactP>, dim3((unsigned)(m * fparts)), dim3(kFinT), 0, s, x, ldx, (int)n, b, kb,
                 (int)k, 1, w.cand, w.row_cnt, w.row_keys, static_cast<float*>(out_vals), out_idx, fparts);
  else if (final_exact)
    ATOPK_LAUNCH(wide_final_kernel<kFinP>, dim3((unsigned)(m * fparts)), dim3(kFinT), 0, s, x, ldx, (int)n, b, kb,
                 (int)k, 0, w.cand, w.row_cnt, w.row_keys, static_cast<float*>(out_vals), out_idx, fparts);
  return hipGetLastError();
}

}  // namespace atopk
