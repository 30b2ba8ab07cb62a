// Bucketed top-k, stage 1 (exact top-k_b inside each of b interleaved
// buckets) and the merge / final stage.
//
// "Approximate Top-k for Increased Parallelism" (Pith review page), "What
// carries the argument": position i goes to bucket i mod b, each bucket keeps
// its own k_b best independently of the others, and when more than k
// survivors result, an exact top-k over them follows.  The pages' kernel keeps
// one small priority queue per thread in registers (k_b <= 4); here every
// lane keeps one sorted k_b-queue per element slot of its 16-byte loads, so
// a sweep of the workgroup over T*V consecutive elements (a multiple of b)
// always feeds the same buckets into the same registers.  Queues of lanes
// that share a bucket are merged with cross-lane shuffles, then across the
// waves of the workgroup in LDS, then across workgroups of a row by the
// finish kernel.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace atopk {

namespace {

constexpr int kStage1Threads = 256;
constexpr int kStage1LdsBytes = 32768;
constexpr int kTargetBlocks = 1024;
constexpr int64_t kListBudget = 1 << 17;  // stage-1 list keys per row

// The kernels keep KB = next power of two >= k_b entries per queue; the
// top-k_b of a bucket is the first k_b of its sorted top-KB, so the finish
// kernel reads only those.
int kb_slots(int64_t kb) {
  int v = 1;
  while (v < kb) v <<= 1;
  return v;
}


template <int DT>
struct VecOf {
  static constexpr int V = (DT == IN_F32) ? 4 : 8;   // elements per 16-byte load
  static constexpr int ES = (DT == IN_F32) ? 4 : 2;  // element bytes
};

// fp32 bit pattern of element e of a 16-byte vector.
template <int DT>
__device__ __forceinline__ uint32_t elem_bits(const uint4& w, int e) {
  const uint32_t word[4] = {w.x, w.y, w.z, w.w};
  if constexpr (DT == IN_F32) {
    return word[e];
  } else {
    const uint32_t v = word[e >> 1];
    return (e & 1) ? (v & 0xffff0000u) : (v << 16);
  }
}

template <int DT>
__device__ __forceinline__ uint32_t load_elem_bits(const uint8_t* row, int64_t i) {
  if constexpr (DT == IN_F32) {
    return *reinterpret_cast<const uint32_t*>(row + i * 4);
  } else {
    return (uint32_t)(*reinterpret_cast<const uint16_t*>(row + i * 2)) << 16;
  }
}

template <int DT, int KB>
__device__ __forceinline__ void consume_vec(uint64_t (&q)[VecOf<DT>::V][KB], const uint4& w, uint32_t idx0) {
#pragma unroll
  for (int e = 0; e < VecOf<DT>::V; ++e) queue_insert<KB>(q[e], make_key(ord_f32(elem_bits<DT>(w, e)), idx0 + e));
}

__device__ __forceinline__ void write_result(uint8_t* out_vals, int32_t* out_idx, int64_t o, const uint8_t* xr,
                                             int dt, uint64_t key) {
  const uint32_t idx = key_idx(key);
  out_idx[o] = (int32_t)idx;
  if (dt == IN_F32) {
    reinterpret_cast<uint32_t*>(out_vals)[o] = reinterpret_cast<const uint32_t*>(xr)[idx];
  } else {
    reinterpret_cast<uint16_t*>(out_vals)[o] = reinterpret_cast<const uint16_t*>(xr)[idx];
  }
}

template <int DT, int KB>
// direct != 0 (one split per row, queues merged in LDS): the workgroup
// writes the row's result itself instead of its lists -- direct == 1 the
// bucket-major candidates (slot r * kb + j), direct == 2 the sorted top-k of
// the b * kb <= 64 candidates (one wave sorts them in registers).
__global__ __launch_bounds__(kStage1Threads) void bucket_stage1_kernel(const uint8_t* __restrict__ x, int64_t ld_bytes,
                                                                      int n, int b, int64_t chunk, int lds_merge,
                                                                      int lists_per_row,
                                                                      uint64_t* __restrict__ lists, int direct, int kb,
                                                                      int k, uint8_t* __restrict__ out_vals,
                                                                      int32_t* __restrict__ out_idx) {
  constexpr int T = kStage1Threads;
  constexpr int V = VecOf<DT>::V;
  constexpr int ES = VecOf<DT>::ES;
  constexpr int W = T * V;
  constexpr int U = (V * KB >= 32) ? 1 : 4;  // loads in flight, bounded by queue registers
  constexpr int NW = T / kWave;
  __shared__ uint64_t lds[kStage1LdsBytes / 8];

  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = t / kWave;
  const int row = blockIdx.y;
  const int split = blockIdx.x;
  const uint8_t* xr = x + (int64_t)row * ld_bytes;
  // The row's first `a` elements come before its first 16-byte boundary; the
  // vector loads start there.  Position p of a sweep holds element a + base + p,
  // so its bucket is (a + p) mod b for every sweep (b divides W).
  const int a = min((int)((16u - (uint32_t)(reinterpret_cast<uintptr_t>(xr) & 15u)) & 15u) / ES, n);
  const uint8_t* xv = xr + (int64_t)a * ES;
  const int64_t c0 = (int64_t)split * chunk;
  const int64_t c1 = min((int64_t)(n - a), c0 + chunk);

  uint64_t q[V][KB];
#pragma unroll
  for (int e = 0; e < V; ++e)
#pragma unroll
    for (int j = 0; j < KB; ++j) q[e][j] = 0;

  if (split == 0 && a > 0) {  // head: a partial sweep at base -W, element-wise
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int i = t * V + e - (W - a);
      if (i >= 0) queue_insert<KB>(q[e], make_key(ord_f32(load_elem_bits<DT>(xr, i)), (uint32_t)i));
    }
  }
  int64_t base = c0;
  for (; base + U * W <= c1; base += U * W) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      w[u] = *reinterpret_cast<const uint4*>(xv + (base + (int64_t)u * W + (int64_t)t * V) * ES);
#pragma unroll
    for (int u = 0; u < U; ++u) consume_vec<DT, KB>(q, w[u], (uint32_t)(a + base + (int64_t)u * W + t * V));
  }
  for (; base + W <= c1; base += W) {
    uint4 w = *reinterpret_cast<const uint4*>(xv + (base + (int64_t)t * V) * ES);
    consume_vec<DT, KB>(q, w, (uint32_t)(a + base + t * V));
  }
  if (base < c1) {  // ragged tail: element-wise, bounds-checked
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int64_t v = base + (int64_t)t * V + e;
      if (v < c1) queue_insert<KB>(q[e], make_key(ord_f32(load_elem_bits<DT>(xv, v)), (uint32_t)(a + v)));
    }
  }

  // Slots e and e + half of one lane share a bucket when b <= half.
#pragma unroll
  for (int half = V / 2; half >= 1; half /= 2) {
    if (b <= half) {
#pragma unroll
      for (int e = 0; e < half; ++e) queue_merge<KB>(q[e], q[e + half]);
    }
  }
  // Lanes l and l ^ m share all their buckets when m * V is a multiple of b.
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    if (m * V >= b) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        uint64_t o[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) o[j] = shfl_xor_u64(q[e][j], m);
        queue_merge<KB>(q[e], o);
      }
    }
  }

  // Representatives: one queue per (bucket, copy) left in the workgroup.
  const bool wave_has_all = kWave * V >= b;
  const int ncopies = wave_has_all ? NW : W / b;
  if (lds_merge) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int p = wave * kWave * V + lane * V + e;
      const bool rep = wave_has_all ? (lane * V + e < b) : true;
      const int c = wave_has_all ? wave : p / b;
      const int r = (p + a) % b;
      if (rep) {
#pragma unroll
        for (int j = 0; j < KB; ++j) lds[((int64_t)c * b + r) * KB + j] = q[e][j];
      }
    }
    __syncthreads();
    constexpr int ES_ = VecOf<DT>::ES;
    if (direct == 2) {  // b * kb <= 64 < T: thread r merges bucket r
      uint64_t m[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) m[j] = 0;
      if (t < b) {
#pragma unroll
        for (int j = 0; j < KB; ++j) m[j] = lds[(int64_t)t * KB + j];
        for (int c = 1; c < ncopies; ++c) {
          uint64_t o[KB];
#pragma unroll
          for (int j = 0; j < KB; ++j) o[j] = lds[((int64_t)c * b + t) * KB + j];
          queue_merge<KB>(m, o);
        }
      }
      __syncthreads();
      if (t < b) {
#pragma unroll
        for (int j = 0; j < KB; ++j)
          if (j < kb) lds[t * kb + j] = m[j];
      }
      __syncthreads();
      if (t < kWave) {
        const uint64_t key = wave_sort64_desc(t < b * kb ? lds[t] : 0);
        if (t < k) write_result(out_vals, out_idx, (int64_t)row * k + t, xr, DT, key);
      }
      (void)ES_;
      return;
    }
    for (int r = t; r < b; r += T) {
      uint64_t a[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) a[j] = lds[(int64_t)r * KB + j];
      for (int c = 1; c < ncopies; ++c) {
        uint64_t o[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) o[j] = lds[((int64_t)c * b + r) * KB + j];
        queue_merge<KB>(a, o);
      }
      if (direct == 1) {
        const int64_t nc = (int64_t)b * kb;
#pragma unroll
        for (int j = 0; j < KB; ++j)
          if (j < kb) write_result(out_vals, out_idx, (int64_t)row * nc + (int64_t)r * kb + j, xr, DT, a[j]);
        continue;
      }
      uint64_t* dst = lists + (((int64_t)row * lists_per_row + split) * b + r) * KB;
#pragma unroll
      for (int j = 0; j < KB; ++j) dst[j] = a[j];
    }
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int p = wave * kWave * V + lane * V + e;
      const bool rep = wave_has_all ? (lane * V + e < b) : true;
      const int c = wave_has_all ? wave : p / b;
      const int r = (p + a) % b;
      if (rep) {
        uint64_t* dst = lists + (((int64_t)row * lists_per_row + (int64_t)split * ncopies + c) * b + r) * KB;
#pragma unroll
        for (int j = 0; j < KB; ++j) dst[j] = q[e][j];
      }
    }
  }
}

// Any b: one thread walks one bucket r, r + b, r + 2b, ... of one row
// (neighbouring threads read neighbouring elements), kGenU loads in flight.
constexpr int kGenU = 8;
constexpr int64_t kGenTargetThreads = 256 * 1024;

// Split s of a row covers elements [s * chunk, (s + 1) * chunk), chunk a
// multiple of b, and writes list s of the row.
template <int DT, int KB>
__global__ __launch_bounds__(256) void bucket_generic_kernel(const uint8_t* __restrict__ x, int64_t ld_bytes, int n,
                                                            int b, int64_t chunk, int lists_per_row,
                                                            uint64_t* __restrict__ lists) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  const int row = blockIdx.y;
  const int split = blockIdx.z;
  if (r >= b) return;
  const uint8_t* xr = x + (int64_t)row * ld_bytes;
  const int64_t end = min((int64_t)n, (int64_t)(split + 1) * chunk);
  uint64_t q[KB];
#pragma unroll
  for (int j = 0; j < KB; ++j) q[j] = 0;
  const int64_t step = (int64_t)kGenU * b;
  int64_t i0 = (int64_t)split * chunk + r;
  for (; i0 + (kGenU - 1) * (int64_t)b < end; i0 += step) {
    uint32_t v[kGenU];
#pragma unroll
    for (int u = 0; u < kGenU; ++u) v[u] = load_elem_bits<DT>(xr, i0 + (int64_t)u * b);
#pragma unroll
    for (int u = 0; u < kGenU; ++u) queue_insert<KB>(q, make_key(ord_f32(v[u]), (uint32_t)(i0 + (int64_t)u * b)));
  }
  for (int64_t i = i0; i < end; i += b) queue_insert<KB>(q, make_key(ord_f32(load_elem_bits<DT>(xr, i)), (uint32_t)i));
  uint64_t* dst = lists + (((int64_t)row * lists_per_row + split) * b + r) * KB;
#pragma unroll
  for (int j = 0; j < KB; ++j) dst[j] = q[j];
}


constexpr int kFinishThreads = 1024;

// mode 0: write the stage-1 candidates bucket-major; mode 1: final exact
// top-k in LDS; mode 2: write merged candidate keys to cand_out.
// Order key of element i of a row of dtype dt.
__device__ __forceinline__ uint32_t row_ord(const uint8_t* xr, int dt, int64_t i) {
  return ord_f32(dt == IN_F32 ? reinterpret_cast<const uint32_t*>(xr)[i]
                              : (uint32_t)reinterpret_cast<const uint16_t*>(xr)[i] << 16);
}

__device__ __noinline__ void finish_row_fallback(const uint8_t* xr, int dt, int n, int k, uint64_t* cand,
                                                 uint32_t* hist, uint32_t* ctl) {
  block_row_topk<kFinishThreads>([&](int i) { return row_ord(xr, dt, i); }, n, k, cand, hist, ctl);
}

constexpr int kFlagMax = 256;  // flagged buckets rescanned in LDS; more take the full-row fallback

// Sort keys[0..n_pow2) (LDS) descending, n_pow2 a power of two in [128,
// kFinishMaxCand]: each wave first sorts runs of 64 in registers, storing the
// odd runs ascending, so that every pair of runs is a bitonic sequence; then
// come the bitonic merges of sizes 128 .. n_pow2.  Stages with a stride of 64
// or more run in LDS, one barrier each; the six stages below pair keys inside
// one run of 64, which a wave merges in registers by shuffles (the direction
// is the same for the whole run).  After the merges of one size, the blocks
// of that size alternate descending / ascending, and the last size leaves the
// whole array descending.  Strides are powers of two, so the pair index
// arithmetic is shifts and masks.
template <int T>
__device__ void finish_sort_desc(uint64_t* keys, int n_pow2) {
  constexpr int NW = T / kWave;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  __syncthreads();
  for (int r = wave; r < n_pow2 / kWave; r += NW) {
    const uint64_t v = wave_sort64_desc(keys[r * kWave + lane]);
    keys[r * kWave + ((r & 1) ? kWave - 1 - lane : lane)] = v;
  }
  for (int size = 2 * kWave; size <= n_pow2; size <<= 1) {
    for (int ls = __builtin_ctz((unsigned)size) - 1; (1 << ls) >= kWave; --ls) {
      __syncthreads();
      const int stride = 1 << ls;
      for (int i = tid; i < (n_pow2 >> 1); i += T) {
        const int lo = ((i >> ls) << (ls + 1)) | (i & (stride - 1));
        const int hi = lo + stride;
        const bool desc = (lo & size) == 0;
        const uint64_t a = keys[lo], c = keys[hi];
        if (desc ? (a < c) : (a > c)) {
          keys[lo] = c;
          keys[hi] = a;
        }
      }
    }
    __syncthreads();
    for (int r = wave; r < n_pow2 / kWave; r += NW) {
      uint64_t v = keys[r * kWave + lane];
      const bool desc = ((r * kWave) & size) == 0;
#pragma unroll
      for (int j = kWave / 2; j > 0; j >>= 1) {
        const uint64_t o = shfl_xor_u64(v, j);
        const bool keep_max = ((lane & j) == 0) == desc;
        v = keep_max ? (v > o ? v : o) : (v < o ? v : o);
      }
      keys[r * kWave + lane] = v;
    }
  }
  __syncthreads();
}

// mode 3 (certified exact top-k from the bucket candidates).  With T the
// k-th largest candidate key: a true top-k element e missing from the
// candidates was dropped by its bucket, so that bucket kept k_b keys above
// e, all of them true top-k and hence all in the top-k of the candidates;
// its k_b-th kept key is then >= T.  Rescanning exactly those buckets for
// the keys between T and their k_b-th kept key (all missing elements lie
// there: e beats some candidate of the top-k, so key(e) > T) and taking the
// top-k of the enlarged pool gives the exact top-k.
template <int KB>
__global__ __launch_bounds__(kFinishThreads) void bucket_finish_kernel(const uint64_t* __restrict__ lists, int nl,
                                                                      int b, int k, int mode,
                                                                      int kb, const uint8_t* __restrict__ x, int dt,
                                                                      int64_t ld_bytes, int n, uint8_t* out_vals,
                                                                      int32_t* out_idx, uint64_t* cand_out) {
  constexpr int T = kFinishThreads;
  __shared__ uint64_t cand[kFinishMaxCand];
  __shared__ uint32_t hist[256 * kKthSub];
  __shared__ uint32_t ctl[8];
  __shared__ uint32_t flg_r[kFlagMax];
  __shared__ uint64_t flg_c[kFlagMax];
  const int t = threadIdx.x;
  const int row = blockIdx.x;
  const uint8_t* xr = x + (int64_t)row * ld_bytes;
  const int64_t nc = (int64_t)b * kb;

  // Queue of bucket r merged over lists l0, l0 + P, l0 + 2P, ... < nl, LB
  // loads in flight.
  constexpr int LB = KB >= 8 ? 1 : 8 / KB;
  auto merge_lists = [&](uint64_t (&a)[KB], int r, int l0, int P) {
    const uint64_t* src = lists + ((int64_t)row * nl * b + r) * KB;
#pragma unroll
    for (int j = 0; j < KB; ++j) a[j] = 0;
    int l = l0;
    for (; l + (LB - 1) * P < nl; l += LB * P) {
      uint64_t o[LB][KB];
#pragma unroll
      for (int u = 0; u < LB; ++u)
#pragma unroll
        for (int j = 0; j < KB; ++j) o[u][j] = src[(int64_t)(l + u * P) * b * KB + j];
#pragma unroll
      for (int u = 0; u < LB; ++u) queue_merge<KB>(a, o[u]);
    }
    for (; l < nl; l += P) {
      uint64_t o[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) o[j] = src[(int64_t)l * b * KB + j];
      queue_merge<KB>(a, o);
    }
  };
  // Few buckets, many lists: P = 2^h threads share a bucket, each merges
  // every P-th list, and an LDS tree joins their queues (P * b * KB keys
  // fit in `cand`).
  int P = 1;
  if (KB <= 4 && nl > 1)
    while (2 * P * b <= T && 2 * P <= nl) P *= 2;
  for (int r0 = 0; r0 < b; r0 += T) {
    const int r = P > 1 ? t % b : r0 + t;
    const int p = P > 1 ? t / b : 0;
    uint64_t a[KB];
    if (r < b && p < P) merge_lists(a, r, p, P);
    if (P > 1) {
      if (p < P) {
#pragma unroll
        for (int j = 0; j < KB; ++j) cand[((int64_t)p * b + r) * KB + j] = a[j];
      }
      for (int half = P / 2; half >= 1; half /= 2) {
        __syncthreads();
        if (p < half) {
          uint64_t o[KB];
#pragma unroll
          for (int j = 0; j < KB; ++j) o[j] = cand[((int64_t)(p + half) * b + r) * KB + j];
          queue_merge<KB>(a, o);
#pragma unroll
          for (int j = 0; j < KB; ++j) cand[((int64_t)p * b + r) * KB + j] = a[j];
        }
      }
      __syncthreads();  // every partial is read before `cand` takes the candidates
    }
    if (r >= b || p != 0) continue;
    if (mode == 0) {
#pragma unroll
      for (int j = 0; j < KB; ++j)
        if (j < kb) write_result(out_vals, out_idx, (int64_t)row * nc + (int64_t)r * kb + j, xr, dt, a[j]);
    } else if (mode == 1 || mode == 3) {
#pragma unroll
      for (int j = 0; j < KB; ++j)
        if (j < kb) cand[r * kb + j] = a[j];
    } else {
#pragma unroll
      for (int j = 0; j < KB; ++j)
        if (j < kb) cand_out[(int64_t)row * nc + (int64_t)r * kb + j] = a[j];
    }
  }
  if (mode != 1 && mode != 3) return;
  __syncthreads();
  int cnt = (int)nc;
  if (mode == 3) {
    const int lane = lane_id();
    const uint64_t thr = block_kth_key<T, kKthSub>(cand, cnt, k, hist, ctl);
    if (t == 0) {
      ctl[5] = 0;
      ctl[6] = 0;
    }
    __syncthreads();
    for (int r = t; r < b; r += T) {
      const uint64_t c = cand[r * kb + kb - 1];
      const int size = (n - r + b - 1) / b;
      if (size > kb && c >= thr) {
        const uint32_t f = atomicAdd(&ctl[5], 1u);
        if (f < (uint32_t)kFlagMax) {
          flg_r[f] = (uint32_t)r;
          flg_c[f] = c;
        }
      }
    }
    cnt = block_compact_ge<T, kFinishMaxCand / T>(cand, cnt, thr, ctl);  // k keys, all >= thr
    const int nflag = (int)ctl[5];
    if (nflag > 0) {
      bool overflow = nflag > kFlagMax;
      if (!overflow) {
        // Every thread of the workgroup steps through slot s of the flagged
        // buckets' elements: bucket f = s / S, element r_f + (s % S) * b, with
        // S = ceil(n / b) slots per bucket (the last may be past the row).
        constexpr int U = 4;
        const int64_t S = ((int64_t)n + b - 1) / b;
        const int64_t total = (int64_t)nflag * S;
        for (int64_t s0 = 0; s0 < total; s0 += (int64_t)U * T) {
          uint32_t o[U];
          int64_t ii[U];
          uint64_t cc[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t sl = s0 + (int64_t)u * T + t;
            const int f = sl < total ? (int)(sl / S) : 0;
            ii[u] = sl < total ? (int64_t)flg_r[f] + (sl - (int64_t)f * S) * b : (int64_t)n;
            cc[u] = flg_c[f];
            o[u] = ii[u] < n ? row_ord(xr, dt, ii[u]) : 0u;
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const uint64_t key = make_key(o[u], (uint32_t)ii[u]);
            const bool keep = ii[u] < n && key > thr && key < cc[u];
            const uint64_t msk = __ballot(keep);
            if (msk) {
              uint32_t pos = 0;
              if (lane == 0) pos = atomicAdd(&ctl[6], (uint32_t)__popcll(msk));
              pos = wave_lane0(pos);
              const uint32_t slot = (uint32_t)k + pos + lanes_below(msk);
              if (keep && slot < (uint32_t)kFinishMaxCand) cand[slot] = key;
            }
          }
        }
        __syncthreads();
        const int extra = (int)ctl[6];
        __syncthreads();
        overflow = k + extra > kFinishMaxCand;
        if (!overflow && extra > 0) {
          cnt = k + extra;
          const uint64_t thr2 = block_kth_key<T, kKthSub>(cand, cnt, k, hist, ctl);
          cnt = block_compact_ge<T, kFinishMaxCand / T>(cand, cnt, thr2, ctl);
        }
      }
      if (overflow) {
        finish_row_fallback(xr, dt, n, k, cand, hist, ctl);
        cnt = k;
      }
    }
  } else if (cnt > k) {
    const uint64_t thr = block_kth_key<T, kKthSub>(cand, cnt, k, hist, ctl);
    cnt = block_compact_ge<T, kFinishMaxCand / T>(cand, cnt, thr, ctl);
  }
  if (cnt <= kWave) {  // one wave sorts the (at most 64) keys in registers
    if (t < kWave) {
      const uint64_t key = wave_sort64_desc(t < cnt ? cand[t] : 0);
      if (t < k) write_result(out_vals, out_idx, (int64_t)row * k + t, xr, dt, key);
    }
    return;
  }
  int npow = 1;
  while (npow < k) npow <<= 1;
  for (int i = cnt + t; i < npow; i += T) cand[i] = 0;
  finish_sort_desc<T>(cand, npow);  // npow >= 128 here (k >= cnt > 64)
  for (int j = t; j < k; j += T) write_result(out_vals, out_idx, (int64_t)row * k + j, xr, dt, cand[j]);
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

template <int DT>
hipError_t launch_stage1_dt(const BucketPlan& p, const void* x, int64_t m, int64_t n, int64_t ldx, int64_t b,
                            int64_t kb, uint64_t* lists, hipStream_t s, int64_t k, int final_exact, void* out_vals,
                            int32_t* out_idx, bool* direct_done) {
  const int64_t ld_bytes = ldx * VecOf<DT>::ES;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  if (p.fast) {
    const int V = VecOf<DT>::V;
    const int W = kStage1Threads * V;
    const bool wave_has_all = kWave * V >= b;
    const int ncopies = wave_has_all ? kStage1Threads / kWave : (int)(W / b);
    const int lds_merge = (int64_t)ncopies * b * kb_slots(kb) * 8 <= kStage1LdsBytes;
    int direct = 0;
    if (direct_done != nullptr && p.splits == 1 && lds_merge) {
      if (!final_exact) direct = 1;
      else if (b * kb <= kWave && k <= kWave && k <= b * kb) direct = 2;
    }
    if (direct_done != nullptr) *direct_done = direct != 0;
    uint8_t* ov = static_cast<uint8_t*>(out_vals);
    dim3 grid((unsigned)p.splits, (unsigned)m);
#define ATOPK_S1(KBV)                                                                                          \
  case KBV:                                                                                                    \
    ATOPK_LAUNCH((bucket_stage1_kernel<DT, KBV>), grid, dim3(kStage1Threads), 0, s, xb, ld_bytes, (int)n, \
                       (int)b, p.chunk, lds_merge, p.lists_per_row, lists, direct, (int)kb, (int)k, ov,       \
                       out_idx);                                                                              \
    break;
    switch (kb_slots(kb)) {
      ATOPK_S1(1) ATOPK_S1(2) ATOPK_S1(4) ATOPK_S1(8) ATOPK_S1(16)
      default: return hipErrorInvalidValue;
    }
#undef ATOPK_S1
  } else {
    dim3 grid((unsigned)((b + 255) / 256), (unsigned)m, (unsigned)p.splits);
#define ATOPK_G(KBV)                                                                                       \
  case KBV:                                                                                                \
    ATOPK_LAUNCH((bucket_generic_kernel<DT, KBV>), grid, dim3(256), 0, s, xb, ld_bytes, (int)n, (int)b, \
                       p.chunk, p.lists_per_row, lists);                                                  \
    break;
    switch (kb_slots(kb)) {
      ATOPK_G(1) ATOPK_G(2) ATOPK_G(4) ATOPK_G(8) ATOPK_G(16)
      default: return hipErrorInvalidValue;
    }
#undef ATOPK_G
  }
  return hipGetLastError();
}

}  // namespace

BucketPlan plan_bucketed(int dtype, int64_t m, int64_t n, int64_t b, int64_t kb, bool aligned) {
  BucketPlan p{};
  const int V = dtype == IN_F32 ? 4 : 8;
  const int W = kStage1Threads * V;
  p.threads = kStage1Threads;
  (void)aligned;  // misaligned rows take a scalar head sweep
  p.fast = is_pow2(b) && b <= W && (int64_t)V * kb_slots(kb) <= 64;
  if (!p.fast) {
    // One thread per (bucket, split): enough splits to give the chip about
    // kGenTargetThreads threads, while every thread still walks >= 64
    // elements and the finish merges at most 16 lists per bucket.
    const int64_t row_threads = (b + 255) / 256 * 256;
    int64_t splits = (kGenTargetThreads + row_threads * m - 1) / (row_threads * std::max<int64_t>(m, 1));
    splits = std::min<int64_t>(splits, std::max<int64_t>(1, n / (b * 64)));
    splits = std::max<int64_t>(1, std::min<int64_t>(splits, 16));
    const int64_t per = (n + splits - 1) / splits;
    p.chunk = (per + b - 1) / b * b;
    p.splits = (int)((n + p.chunk - 1) / p.chunk);
    p.lists_per_row = p.splits;
    return p;
  }
  // Long chunks amortise the per-workgroup merge; enough of them fill the chip.
  const int64_t sweeps = (n + W - 1) / W;
  int64_t splits = (kTargetBlocks + m - 1) / (m > 0 ? m : 1);
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, sweeps / 8));
  // The finish reads lists_per_row * b queues per row with one workgroup.
  splits = std::min<int64_t>(splits, std::max<int64_t>(1, kListBudget / (b * kb_slots(kb))));
  splits = std::max<int64_t>(splits, 1);
  const int64_t chunk_sweeps = (sweeps + splits - 1) / splits;
  p.chunk = chunk_sweeps * W;
  p.splits = (int)((n + p.chunk - 1) / p.chunk);
  const bool wave_has_all = (int64_t)kWave * V >= b;
  const int ncopies = wave_has_all ? kStage1Threads / kWave : (int)(W / b);
  const bool lds_merge = (int64_t)ncopies * b * kb_slots(kb) * 8 <= kStage1LdsBytes;
  p.lists_per_row = p.splits * (lds_merge ? 1 : ncopies);
  return p;
}

hipError_t launch_bucket_stage1(const BucketPlan& p, const void* x, int dtype, int64_t m, int64_t n, int64_t ldx,
                                int64_t b, int64_t kb, uint64_t* lists, hipStream_t s, int64_t k, int final_exact,
                                void* out_vals, int32_t* out_idx, bool* direct_done) {
  if (direct_done != nullptr) *direct_done = false;
  if (dtype == IN_F32)
    return launch_stage1_dt<IN_F32>(p, x, m, n, ldx, b, kb, lists, s, k, final_exact, out_vals, out_idx, direct_done);
  return launch_stage1_dt<IN_BF16>(p, x, m, n, ldx, b, kb, lists, s, k, final_exact, out_vals, out_idx, direct_done);
}

hipError_t launch_bucket_finish(const uint64_t* lists, int lists_per_row, int64_t m, int64_t n, int64_t b, int64_t kb,
                                int64_t k, int final_exact, const void* x, int dtype, int64_t ldx, void* out_vals,
                                int32_t* out_idx, uint64_t* cand_out, hipStream_t s) {
  const int64_t es = dtype == IN_F32 ? 4 : 2;
  int mode = 0;
  if (final_exact == kFinishCertified) {
    if (b * kb > kFinishMaxCand || k > b * kb) return hipErrorInvalidValue;
    mode = 3;
  } else if (final_exact) {
    mode = (b * kb <= kFinishMaxCand) ? 1 : 2;
  }
  dim3 grid((unsigned)m);
#define ATOPK_F(KBV)                                                                                               \
  case KBV:                                                                                                        \
    ATOPK_LAUNCH((bucket_finish_kernel<KBV>), grid, dim3(kFinishThreads), 0, s, lists, lists_per_row, (int)b, \
                       (int)k, mode, (int)kb, static_cast<const uint8_t*>(x), dtype, ldx * es, (int)n,             \
                       static_cast<uint8_t*>(out_vals), out_idx, cand_out);                                        \
    break;
  switch (kb_slots(kb)) {
    ATOPK_F(1) ATOPK_F(2) ATOPK_F(4) ATOPK_F(8) ATOPK_F(16)
    default: return hipErrorInvalidValue;
  }
#undef ATOPK_F
  return hipGetLastError();
}

}  // namespace atopk
