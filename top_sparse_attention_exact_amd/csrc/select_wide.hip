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
//  3. final, one workgroup per row (skipped by stage-1-only calls): the
//     exact top-k of the candidates (radix select on the keys), a counting
//     sort on the value, and the output.  If the exact collection overflowed
//     (rows made of few distinct values) the workgroup runs a full radix
//     select over its row instead.
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

// Sort cand[0..cnt) (LDS, cnt <= kFinMax, unique nonzero keys) descending.
// Counting sort on the value over equi-depth bins (bin 0 = largest values;
// see below), a scan and a scatter; then every key's place is its bin's
// start plus the number of larger keys in its bin.  A bin above kBinRank
// keys (heavy ties) sends the whole set to the bitonic sort.  `bins` holds
// kFinMax words, `red` 64 + 2 * kCoarse.
constexpr int kBinRank = 256;
constexpr int kCoarse = 256;

__device__ bool block_sort_desc_binned(uint64_t* cand, int cnt, uint32_t* bins, uint32_t* red) {
  constexpr int T = kFinT, P = kFinP;
  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = t / kWave;
  uint64_t key[P];
  uint32_t lo = 0xffffffffu, hi = 0;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int i = t * P + p;
    key[p] = i < cnt ? cand[i] : 0;
    if (i < cnt) {
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
  if (t == 0) red[32] = 0;  // a bin above kBinRank
  __syncthreads();
  lo = red[0];
  hi = red[16];
  for (int w = 1; w < T / kWave; ++w) {
    lo = min(lo, red[w]);
    hi = max(hi, red[16 + w]);
  }
  const uint64_t span = (uint64_t)(hi - lo) + 1;
  // Equi-depth bins: a coarse histogram (kCoarse bins evenly over the
  // order-key range), then each coarse bin is cut into as many fine bins as
  // it holds keys, evenly over its own range -- about one key per fine bin
  // even when a few outliers stretch the range.  red[64 ..) holds the coarse
  // counts, then their exclusive scan.
  uint32_t* coarse = red + 64;
  for (int j = t; j < kCoarse; j += T) coarse[j] = 0;
  __syncthreads();
  uint32_t cb[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    cb[p] = (uint32_t)(((uint64_t)(hi - key_ord(key[p])) * kCoarse) / span);
    hist_add(coarse, cb[p], t * P + p < cnt);
  }
  __syncthreads();
  if (t < kWave) {  // lane l scans coarse bins [4l, 4l + 4)
    uint32_t c4[4], s4 = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      c4[j] = coarse[4 * t + j];
      s4 += c4[j];
    }
    uint32_t run = (uint32_t)wave_incl_scan((int)s4) - s4;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      coarse[kCoarse + 4 * t + j] = run;  // start of coarse bin j
      run += c4[j];
    }
  }
  __syncthreads();
  uint32_t bin[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const uint64_t rel = hi - key_ord(key[p]);
    const uint32_t c = cb[p];
    // coarse bin c covers rel in [ceil(c * span / K), ceil((c + 1) * span / K))
    const uint64_t c_lo = (c * span + kCoarse - 1) / kCoarse;
    const uint64_t c_hi = ((c + 1) * span + kCoarse - 1) / kCoarse;
    const uint32_t cn = coarse[c];
    // a monotone map of rel inside the coarse bin (the rank step below only
    // needs the bins in value order), in fp32: rel - c_lo and the bin width
    // stay below 2^24 + 1, so both convert exactly
    const uint32_t f =
        (uint32_t)((float)(uint32_t)(rel - c_lo) * (float)cn / (float)(uint32_t)max<uint64_t>(c_hi - c_lo, 1));
    bin[p] = coarse[kCoarse + c] + min(f, cn > 0 ? cn - 1 : 0u);
    hist_add(bins, bin[p], t * P + p < cnt);
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
  if (red[32] != 0) return false;  // cand untouched
#pragma unroll
  for (int p = 0; p < P; ++p) {
    bins[t * P + p] = before;  // start of the bin: the scatter cursor
    before += c[p];
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (t * P + p < cnt) cand[atomicAdd(&bins[bin[p]], 1u)] = key[p];
  __syncthreads();
  // bins[j] is now the end of bin j
  uint32_t rank[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    rank[p] = 0;
    if (t * P + p < cnt) {
      const int s0 = bin[p] == 0 ? 0 : (int)bins[bin[p] - 1];
      const int e = (int)bins[bin[p]];
      int r = s0;
      int i = s0;
      for (; i + 4 <= e; i += 4) {
        const uint64_t a0 = cand[i], a1 = cand[i + 1], a2 = cand[i + 2], a3 = cand[i + 3];
        r += (a0 > key[p]) + (a1 > key[p]) + (a2 > key[p]) + (a3 > key[p]);
      }
      for (; i < e; ++i) r += cand[i] > key[p];
      rank[p] = (uint32_t)r;
    }
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (t * P + p < cnt) cand[rank[p]] = key[p];
  __syncthreads();
  return true;
}

// Bitonic fallback (out of line: it needs its own registers).
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

// Sort cand[0..cnt) and write the first k as values (bit copies of the row)
// and indices.
__device__ void sort_and_write(uint64_t* cand, int cnt, int k, const float* __restrict__ xr, int n,
                               float* __restrict__ out_vals, int32_t* __restrict__ out_idx, uint32_t* bins,
                               uint32_t* red) {
  if (!block_sort_desc_binned(cand, cnt, bins, red)) block_sort_desc_bitonic(cand, cnt);
  for (int i = threadIdx.x; i < k; i += kFinT) {
    uint32_t idx = key_idx(cand[i]);
    idx = idx < (uint32_t)n ? idx : 0u;  // only reachable with NaN inputs
    out_idx[i] = (int32_t)idx;
    // the order key gives the value back, except the sign of a zero
    const uint32_t o = key_ord(cand[i]);
    reinterpret_cast<uint32_t*>(out_vals)[i] =
        o == 0x80000000u ? reinterpret_cast<const uint32_t*>(xr)[idx] : bits_from_ord(o);
  }
}

// Full-row exact top-k of an fp32 row (the fallback for rows whose
// collection overflowed); leaves the k keys in cand[0..k).
__device__ __noinline__ void row_radix_topk(const float* __restrict__ xr, int n, int k, uint64_t* cand,
                                            uint32_t* hist, uint32_t* ctl) {
  const uint32_t* xb = reinterpret_cast<const uint32_t*>(xr);
  block_row_topk<kFinT>([&](int i) { return ord_f32(xb[i]); }, n, k, cand, hist, ctl);
}

// 3. final: one workgroup per row.  exact_mode: the collected keys; else
//    the b * kb bucket candidates.
__global__ __launch_bounds__(kFinT) void wide_final_kernel(const float* __restrict__ x, int64_t ldx, int n, int b,
                                                          int kb, int k, int exact_mode,
                                                          const uint64_t* __restrict__ bucket_cand,
                                                          const int* __restrict__ row_cnt,
                                                          const uint64_t* __restrict__ row_keys,
                                                          float* __restrict__ out_vals, int32_t* __restrict__ out_idx) {
  constexpr int T = kFinT;
  __shared__ uint64_t cand[kFinMax];
  __shared__ uint32_t bins[kFinMax];
  __shared__ uint32_t red[64 + 2 * kCoarse];
  uint32_t* hist = bins;  // the radix selects run before the sort
  uint32_t* ctl = bins + 256;
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const float* xr = x + (int64_t)row * ldx;
  float* ov = out_vals + (int64_t)row * k;
  int32_t* oi = out_idx + (int64_t)row * k;
  if (exact_mode) {
    const int cnt = row_cnt[row];
    if (cnt > kRowCap) {
      row_radix_topk(xr, n, k, cand, hist, ctl);
      sort_and_write(cand, k, k, xr, n, ov, oi, bins, red);
      return;
    }
    // cnt >= k unique keys: the k-th largest, then exactly k survive
    const uint64_t* keys = row_keys + (int64_t)row * kRowCap;
    const uint64_t kth = block_kth_key<T>(keys, cnt, k, hist, ctl);
    if (t == 0) ctl[4] = 0;
    __syncthreads();
    for (int i0 = 0; i0 < cnt; i0 += T) {
      const int i = i0 + t;
      const uint64_t key = i < cnt ? keys[i] : 0;
      const bool keep = key != 0 && key >= kth;
      const uint64_t m = __ballot(keep);
      if (m) {
        uint32_t pos = 0;
        if (lane_id() == 0) pos = atomicAdd(&ctl[4], (uint32_t)__popcll(m));
        pos = wave_lane0(pos);
        const uint32_t slot = pos + lanes_below(m);
        if (keep && slot < (uint32_t)kFinMax) cand[slot] = key;
      }
    }
    __syncthreads();
    const int kept = min((int)ctl[4], kFinMax);
    __syncthreads();
    sort_and_write(cand, kept, k, xr, n, ov, oi, bins, red);
    return;
  }
  int cnt = b * kb;
  for (int i = t; i < cnt; i += T) cand[i] = bucket_cand[(int64_t)row * cnt + i];
  __syncthreads();
  if (cnt > k) {
    const uint64_t kth = block_kth_key<T>(cand, cnt, k, hist, ctl);
    cnt = block_compact_ge<T, kFinMax / T>(cand, cnt, kth, ctl);
  }
  sort_and_write(cand, cnt, k, xr, n, ov, oi, bins, red);
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
  p.vals_bytes = exact ? (size_t)m * kWideKB * b * 4 : 0;
  p.bucket_bytes = exact ? (size_t)m * 4 : (size_t)m * b * 4;
  p.cand_bytes = (!exact && final_exact) ? (size_t)m * b * kb * 8 : 0;
  p.row_bytes = exact ? (size_t)m * kRowCap * 8 : 0;
  return p;
}

hipError_t launch_wide(const WidePlan& p, const float* x, int64_t m, int64_t n, int64_t ldx, int64_t k, bool exact,
                       bool final_exact, const WideBuffers& w, void* out_vals, int32_t* out_idx, hipStream_t s) {
  const int b = (int)p.b, kb = (int)p.kb;
  const dim3 grid((unsigned)p.blocks), block((unsigned)(kWave * p.nchunks));
  if (p.kbn == 8)
    hipLaunchKernelGGL(wide_values_kernel<8>, grid, block, 0, s, x, ldx, (int)n, b, kb, (int)p.groups,
                       p.sweeps_per_chunk, exact ? 1 : 0, w.thr, w.need, w.vals);
  else
    hipLaunchKernelGGL(wide_values_kernel<kWideKB>, grid, block, 0, s, x, ldx, (int)n, b, kb, (int)p.groups,
                       p.sweeps_per_chunk, exact ? 1 : 0, w.thr, w.need, w.vals);
  if (exact) {
    hipLaunchKernelGGL(wide_exact_threshold_kernel, dim3((unsigned)m), dim3(kExactB), 0, s, w.vals, (int)k, w.rowthr,
                       w.row_cnt);
    hipLaunchKernelGGL(wide_collect_exact_kernel, grid, block, 0, s, x, ldx, (int)n, b, (int)p.groups,
                       p.sweeps_per_chunk, w.rowthr, w.row_cnt, w.row_keys);
  } else if (p.kbn == 8) {
    hipLaunchKernelGGL(wide_collect_bucket_kernel<8>, grid, block, 0, s, x, ldx, (int)n, b, kb, (int)p.groups,
                       p.sweeps_per_chunk, final_exact ? 1 : 0, w.thr, w.need, w.cand,
                       static_cast<float*>(out_vals), out_idx);
  } else {
    hipLaunchKernelGGL(wide_collect_bucket_kernel<kWideKB>, grid, block, 0, s, x, ldx, (int)n, b, kb, (int)p.groups,
                       p.sweeps_per_chunk, final_exact ? 1 : 0, w.thr, w.need, w.cand,
                       static_cast<float*>(out_vals), out_idx);
  }
  if (exact || final_exact)
    hipLaunchKernelGGL(wide_final_kernel, dim3((unsigned)m), dim3(kFinT), 0, s, x, ldx, (int)n, b, kb, (int)k,
                       exact ? 1 : 0, w.cand, w.row_cnt, w.row_keys, static_cast<float*>(out_vals), out_idx);
  return hipGetLastError();
}

}  // namespace atopk
