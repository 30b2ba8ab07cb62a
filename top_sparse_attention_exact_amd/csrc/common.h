// Device-side building blocks shared by the selection and decode kernels
// (gfx950, wave64).
//
// Ordering.  Every stage compares elements by (value descending, index
// ascending), the tie rule that makes each top-k result unique.  A value is
// mapped to a 32-bit unsigned "order key" whose unsigned order is the
// numeric order, with -0.0 and +0.0 mapped to the same key; a 64-bit key
// packs (order key << 32) | ~index, so one unsigned comparison decides value
// and tie at once.  Key 0 never comes from a real element and marks an empty
// slot.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace atopk {

constexpr int kWave = 64;

// ----------------------------------------------------------------- keys ---

// fp32 bits -> order key.  Positive values get the sign bit set; negative
// values become 0x80000000 - |bits|, so -0.0 lands on the same key as +0.0.
__device__ __forceinline__ uint32_t ord_f32(uint32_t bits) {
  return (bits & 0x80000000u) ? (0x80000000u - (bits & 0x7fffffffu)) : (bits | 0x80000000u);
}

// Inverse of ord_f32 (a key from -0.0 comes back as +0.0).
__device__ __forceinline__ uint32_t bits_from_ord(uint32_t o) {
  return (o & 0x80000000u) ? (o & 0x7fffffffu) : (0x80000000u | (0x80000000u - o));
}

__device__ __forceinline__ uint64_t make_key(uint32_t ord, uint32_t idx) {
  return ((uint64_t)ord << 32) | (uint64_t)(~idx);
}
__device__ __forceinline__ uint32_t key_idx(uint64_t key) { return ~(uint32_t)key; }
__device__ __forceinline__ uint32_t key_ord(uint64_t key) { return (uint32_t)(key >> 32); }
__device__ __forceinline__ float key_value_f32(uint64_t key) { return __uint_as_float(bits_from_ord(key_ord(key))); }

template <typename K>
__device__ __forceinline__ K kmax(K a, K b) { return a > b ? a : b; }
template <typename K>
__device__ __forceinline__ K kmin(K a, K b) { return a < b ? a : b; }

// --------------------------------------------------- register queues ------
//
// A queue is KB keys held in registers, sorted descending.  Inserting x keeps
// the KB largest of queue + {x}: slot j becomes the median of (old q[j-1],
// old q[j], x), i.e. x clamped to [q[j], q[j-1]]; one max/min pair per slot
// and no data-dependent branch.

template <int KB, typename K>
__device__ __forceinline__ void queue_insert(K (&q)[KB], K x) {
#pragma unroll
  for (int j = KB - 1; j >= 1; --j) q[j] = kmax(q[j], kmin(q[j - 1], x));
  q[0] = kmax(q[0], x);
}

// a := top-KB of (a union c), both sorted descending.  max(a_i, c_{KB-1-i})
// holds the KB largest of the union as a bitonic sequence, which a bitonic
// half-cleaner cascade then sorts.  KB must be a power of two.
template <int KB, typename K>
__device__ __forceinline__ void queue_merge(K (&a)[KB], const K (&c)[KB]) {
  K d[KB];
#pragma unroll
  for (int i = 0; i < KB; ++i) d[i] = kmax(a[i], c[KB - 1 - i]);
#pragma unroll
  for (int stride = KB / 2; stride > 0; stride /= 2) {
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      if ((i & stride) == 0) {
        K hi = kmax(d[i], d[i + stride]);
        K lo = kmin(d[i], d[i + stride]);
        d[i] = hi;
        d[i + stride] = lo;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < KB; ++i) a[i] = d[i];
}

// ------------------------------------------------------- wave helpers -----

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = (uint32_t)__shfl_xor((int)lo, m, kWave);
  hi = (uint32_t)__shfl_xor((int)hi, m, kWave);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = (uint32_t)__shfl((int)lo, src, kWave);
  hi = (uint32_t)__shfl((int)hi, src, kWave);
  return ((uint64_t)hi << 32) | lo;
}

// Lane 0's value for the whole wave (a scalar read, no LDS round trip; lane
// 0 must be active).
__device__ __forceinline__ uint32_t wave_lane0(uint32_t v) { return (uint32_t)__builtin_amdgcn_readlane((int)v, 0); }

// Bitwise AND and OR over the wave: DPP inside each row of 16 lanes (two
// quad swaps and two mirrors reach every lane of the row), then the 4 rows.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_dpp(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, true));   // quad_perm 1,0,3,2
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, true));   // quad_perm 2,3,0,1
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, true));  // row_half_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, true));  // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(a, b), op(c, d));
}

// Inclusive prefix sum over the wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    int t = __shfl_up(v, o, kWave);
    if (l >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// ------------------------------------------------------ block helpers -----
//
// All block helpers must be called by every thread of the block.

// Workgroup barrier that orders LDS only.  __syncthreads() also fences
// global memory, which makes every wave wait for its outstanding global
// loads at the barrier; this one leaves prefetched loads in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Sort one key per lane descending across the wave (bitonic, lane = rank).
__device__ __forceinline__ uint64_t wave_sort64_desc(uint64_t key) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t o = shfl_xor_u64(key, stride);
      const bool desc = (lane & size) == 0;
      const bool lower = (lane & stride) == 0;
      key = (lower == desc) ? kmax(key, o) : kmin(key, o);
    }
  }
  return key;
}

// Sort 64*P keys held P per lane (key index lane*P + p) descending, bitonic.
template <int P>
__device__ __forceinline__ void wave_sort_desc(uint64_t (&key)[P]) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= kWave * P; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < P) {
#pragma unroll
        for (int p = 0; p < P; ++p) {
          if ((p & stride) == 0) {
            const bool desc = ((lane * P + p) & size) == 0;
            const uint64_t a = key[p], c = key[p + stride];
            key[p] = desc ? kmax(a, c) : kmin(a, c);
            key[p + stride] = desc ? kmin(a, c) : kmax(a, c);
          }
        }
      } else {
        const int ls = stride / P;
        const bool lower = (lane & ls) == 0;
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const bool desc = ((lane * P + p) & size) == 0;
          const uint64_t o = shfl_xor_u64(key[p], ls);
          key[p] = (lower == desc) ? kmax(key[p], o) : kmin(key[p], o);
        }
      }
    }
  }
}

// Number of keys greater than x in a descending run of 64 keys (0..64).
__device__ __forceinline__ int run_count_greater(const uint64_t* run, uint64_t x) {
  if (run[kWave - 1] > x) return kWave;
  int lo = 0;  // invariant: run[lo - 1] > x (or lo == 0), answer < 64
#pragma unroll
  for (int step = 32; step > 0; step >>= 1)
    if (run[lo + step - 1] > x) lo += step;
  return lo;
}

// a := the 64 largest of two descending 64-runs, a in registers (one key
// per lane) and b in LDS: lane p takes max(a_p, b_{63-p}), a bitonic
// sequence holding the 64 largest, which six half-cleaner steps sort.
__device__ __forceinline__ uint64_t wave_merge_top64(uint64_t a, const uint64_t* b) {
  const int lane = lane_id();
  uint64_t m = kmax(a, b[kWave - 1 - lane]);
#pragma unroll
  for (int stride = kWave / 2; stride > 0; stride >>= 1) {
    const uint64_t o = shfl_xor_u64(m, stride);
    m = (lane & stride) == 0 ? kmax(m, o) : kmin(m, o);
  }
  return m;
}

// Rank of `key` among the 64-key descending runs runs[0..nr) (LDS): its
// place `own_rank` in its own run `own` plus, per other run, the number of
// larger keys -- one binary search per run, all runs advanced in lockstep so
// their LDS reads overlap.
template <int MAXR>
__device__ __forceinline__ int rank_in_runs(const uint64_t* runs, int nr, int own, int own_rank, uint64_t key) {
  int lo[MAXR];
#pragma unroll
  for (int r = 0; r < MAXR; ++r) lo[r] = (r < nr && r != own && runs[r * kWave + kWave - 1] > key) ? kWave : 0;
#pragma unroll
  for (int step = 32; step > 0; step >>= 1) {
#pragma unroll
    for (int r = 0; r < MAXR; ++r) {
      if (r < nr && r != own && lo[r] < kWave) {
        if (runs[r * kWave + lo[r] + step - 1] > key) lo[r] += step;
      }
    }
  }
  int rank = own_rank;
#pragma unroll
  for (int r = 0; r < MAXR; ++r) rank += (r < nr && r != own) ? lo[r] : 0;
  return rank;
}

// Exact top-k of n <= T unique nonzero keys in cand[] (LDS), written in
// descending order through write(rank, key): every wave sorts a run of 64,
// then each key's rank is its place in its run plus, per other run, the
// count of larger keys found by binary search.  `runs` holds 64*ceil(n/64)
// keys and may alias cand.
template <int T, typename Writer>
__device__ void block_sortmerge_final(const uint64_t* cand, uint64_t* runs, int n, int k, Writer&& write) {
  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = t / kWave;
  const int nr = (n + kWave - 1) / kWave;
  uint64_t key = t < n ? cand[t] : 0;
  __syncthreads();
  if (wave < nr) {
    key = wave_sort64_desc(key);
    runs[wave * kWave + lane] = key;
  }
  __syncthreads();
  if (wave < nr && key != 0) {
    const int rank = rank_in_runs<T / kWave>(runs, nr, wave, lane, key);
    if (rank < k) write(rank, key);
  }
}

// hist[bin] += 1 for every active lane with `add`: one LDS atomic per lane.
// Lanes that hit one address serialise inside the LDS unit, which still
// costs less than folding equal bins first: that takes a shuffle, two
// ballots and an LDS round trip per distinct bin, all on the vector and
// scalar units every wave shares (measured at 2048 keys: 6.1 against 3.6 us
// per radix select, the keys of the first digit in a few bins).
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool add) {
  if (add) atomicAdd(&hist[bin], 1u);
}

// The same where most lanes of most waves fall into one or two bins for
// several digits in a row (the largest values of a uniform row): the first
// few distinct bins of the wave take one atomic each (count = lanes in that
// bin), the rest go lane by lane.
__device__ __forceinline__ void hist_add_grouped(uint32_t* hist, uint32_t bin, bool add) {
  uint64_t todo = __ballot(add);
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    if (!todo) return;
    const int leader = __builtin_ctzll(todo);
    const uint32_t lb = __shfl(bin, leader, kWave);
    const uint64_t same = __ballot(add && bin == lb);
    if (lane_id() == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(same));
    add = add && bin != lb;
    todo &= ~same;
  }
  if (add) atomicAdd(&hist[bin], 1u);
}

// The threshold key t such that exactly k of the n unique keys in `keys`
// (LDS) are >= t: radix select, 8-bit digits from the first byte the keys do
// not all share.  Once at most 64 keys share the selected prefix, they are
// gathered into `hist` and one wave ranks them, which ends the select in
// place of the remaining digit passes.  With SUB > 1 lane l counts into copy
// l mod SUB of the histogram, so keys of one digit hit SUB addresses instead
// of one.  `hist` is a 256 * SUB entry LDS array, `ctl` 4 LDS words.
constexpr int kKthSub = 4;  // histogram copies for candidate sets, which crowd few digits

template <int T, int SUB = 1>
__device__ uint64_t block_kth_key(const uint64_t* keys, int n, int k, uint32_t* hist, uint32_t* ctl) {
  static_assert(T / kWave <= 64, "per-wave words fit the histogram array");
  static_assert(SUB == 1 || SUB == 2 || SUB == 4, "lanes spread over 1, 2 or 4 histogram copies");
  const int tid = threadIdx.x;
  // Leading bytes that every key shares (where the AND and the OR of the
  // keys' order words agree) need no histogram pass: candidates near a
  // threshold often share their sign and exponent byte.
  uint32_t wa = 0xffffffffu, wo = 0;
  for (int i = tid; i < n; i += T) {
    const uint32_t o = key_ord(keys[i]);
    wa &= o;
    wo |= o;
  }
  wa = wave_reduce_dpp(wa, [](uint32_t x, uint32_t y) { return x & y; });
  wo = wave_reduce_dpp(wo, [](uint32_t x, uint32_t y) { return x | y; });
  if (lane_id() == 0) {
    hist[2 * (tid / kWave)] = wa;
    hist[2 * (tid / kWave) + 1] = wo;
  }
  __syncthreads();
  wa = 0xffffffffu;
  wo = 0;
#pragma unroll
  for (int w = 0; w < T / kWave; ++w) {
    wa &= hist[2 * w];
    wo |= hist[2 * w + 1];
  }
  __syncthreads();
  const uint32_t diff = wa ^ wo;
  const int common = diff == 0 ? 4 : __builtin_clz(diff) / 8;  // shared leading bytes of the order word
  uint64_t prefix = common == 0 ? 0 : ((uint64_t)(wa & (0xffffffffu << (32 - 8 * common))) << 32);
  int rem = k;
  for (int shift = 56 - 8 * common; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256 * SUB; i += T) hist[i] = 0;
    __syncthreads();
    uint32_t* hsub = hist + 256 * (lane_id() % SUB);  // keys of one digit in a wave hit SUB addresses
    const uint64_t hi_prefix = (shift == 56) ? 0 : (prefix >> (shift + 8));
    for (int i0 = 0; i0 < n; i0 += 2 * T) {
      uint64_t kk[2];  // two loads in flight
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int i = i0 + u * T + tid;
        kk[u] = i < n ? keys[i] : 0;
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const bool match = i0 + u * T + tid < n && ((shift == 56) || ((kk[u] >> (shift + 8)) == hi_prefix));
        hist_add(hsub, (uint32_t)(kk[u] >> shift) & 255u, match);
      }
    }
    __syncthreads();
    if (tid < kWave) {
      // lane l owns digits 255-4l .. 252-4l (high to low)
      uint32_t h[4];
      int s = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h[j] = hist[255 - 4 * tid - j];
#pragma unroll
        for (int c = 1; c < SUB; ++c) h[j] += hist[256 * c + 255 - 4 * tid - j];
        s += (int)h[j];
      }
      int incl = wave_incl_scan(s);  // keys in digits above this lane's low end
      int excl = incl - s;
      if (excl < rem && rem <= incl) {
        int acc = excl;
        int d = 0;
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (d == 0 && acc + (int)h[j] >= rem) {
            d = 255 - 4 * tid - j + 1;  // stored +1 so 0 means "not found yet"
            cnt = h[j];
          } else if (d == 0) {
            acc += (int)h[j];
          }
        }
        ctl[0] = (uint32_t)(d - 1);
        ctl[1] = (uint32_t)(rem - acc);
        ctl[2] = cnt;
        ctl[3] = 0;
      }
    }
    __syncthreads();
    const uint32_t digit = ctl[0];
    const int new_rem = (int)ctl[1];
    const uint32_t cnt = ctl[2];
    __syncthreads();
    prefix |= (uint64_t)digit << shift;
    rem = new_rem;
    if ((int)cnt == rem) break;  // every key with this prefix is in
    if (cnt <= (uint32_t)kWave && shift > 0) {
      // gather the keys with the prefix (two 32-bit words each)
      const uint64_t want = prefix >> shift;
      for (int i0 = 0; i0 < n; i0 += T) {
        const int i = i0 + tid;
        const uint64_t key = i < n ? keys[i] : 0;
        const bool m = i < n && (key >> shift) == want;
        const uint64_t msk = __ballot(m);
        if (msk) {
          uint32_t pos = 0;
          if (lane_id() == 0) pos = atomicAdd(&ctl[3], (uint32_t)__popcll(msk));
          pos = wave_lane0(pos);
          if (m) {
            const uint32_t slot = pos + lanes_below(msk);
            hist[2 * slot] = (uint32_t)key;
            hist[2 * slot + 1] = (uint32_t)(key >> 32);
          }
        }
      }
      __syncthreads();
      if (tid < kWave) {
        // lane l holds gathered key l; the rem-th largest has fewer than rem
        // keys above it and at least rem at or above it
        const bool own = tid < (int)cnt;
        const uint32_t lo = own ? hist[2 * tid] : 0u, hi = own ? hist[2 * tid + 1] : 0u;
        const uint64_t mine = ((uint64_t)hi << 32) | lo;
        int above = 0, same = 0;
        for (int j = 0; j < (int)cnt; ++j) {
          const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, j) << 32) |
                             (uint32_t)__builtin_amdgcn_readlane((int)lo, j);
          above += o > mine;
          same += o == mine;
        }
        if (own && above < rem && rem <= above + same) {
          ctl[0] = lo;
          ctl[1] = hi;
        }
      }
      __syncthreads();
      const uint64_t t = ((uint64_t)ctl[1] << 32) | ctl[0];
      __syncthreads();
      return t;
    }
  }
  return prefix;
}

// The k-th largest of n unique keys in LDS (1 <= k <= n), for candidate
// sets whose order words spread over a range: 512 equal-width bins over
// [min, max] of the order words (bin 0 holds the largest), one LDS atomic per
// key, a block scan of the bin counts for the bin holding the k-th key, and
// one wave ranking the keys of that bin.  When every key has the same order
// word, or that bin holds more than 64 keys, the radix select above decides
// instead.  `hist` holds 1024 words and `ctl` 8; both are overwritten.
template <int T>
__device__ __forceinline__ uint64_t block_kth_key_binned(const uint64_t* keys, int n, int k, uint32_t* hist, uint32_t* ctl) {
  constexpr int NB = 512;
  constexpr int NW = T / kWave;
  static_assert(T >= NB && NW <= 32, "one bin per thread of the first 512");
  uint32_t* mm = hist + NB;            // [NW] minima, [NW] maxima, [8] scan totals
  uint32_t* gath = hist + NB + 2 * NW + 8;  // up to 64 gathered keys (two words each)
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  uint32_t lo = 0xffffffffu, hi = 0;
  for (int i = tid; i < n; i += T) {
    const uint32_t o = key_ord(keys[i]);
    lo = min(lo, o);
    hi = max(hi, o);
  }
  lo = wave_reduce_dpp(lo, [](uint32_t x, uint32_t y) { return min(x, y); });
  hi = wave_reduce_dpp(hi, [](uint32_t x, uint32_t y) { return max(x, y); });
  if (lane == 0) {
    mm[wave] = lo;
    mm[NW + wave] = hi;
  }
  if (tid < NB) hist[tid] = 0;
  if (tid == 0) ctl[3] = 0;
  __syncthreads();
  lo = 0xffffffffu;
  hi = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    lo = min(lo, mm[w]);
    hi = max(hi, mm[NW + w]);
  }
  const uint32_t range = hi - lo;
  if (range == 0) {
    __syncthreads();
    return block_kth_key<T, kKthSub>(keys, n, k, hist, ctl);
  }
  // bin of order word o: (hi - o) scaled to [0, NB), monotone in o
  const uint64_t inv = ((uint64_t)NB << 32) / ((uint64_t)range + 1);
  for (int i = tid; i < n; i += T) {
    const uint32_t d = hi - key_ord(keys[i]);
    atomicAdd(&hist[(uint32_t)(((uint64_t)d * inv) >> 32)], 1u);
  }
  __syncthreads();
  // the bin where the running count from the top reaches k
  const int c = tid < NB ? (int)hist[tid] : 0;
  const int incl = wave_incl_scan(c);
  if (lane == kWave - 1 && tid < NB) mm[2 * NW + wave] = (uint32_t)incl;
  __syncthreads();
  if (tid < NB) {
    int before = incl - c;
#pragma unroll
    for (int w = 0; w < NB / kWave; ++w) before += w < wave ? (int)mm[2 * NW + w] : 0;
    if (before < k && k <= before + c) {
      ctl[0] = (uint32_t)tid;
      ctl[1] = (uint32_t)(k - before);
      ctl[2] = (uint32_t)c;
    }
  }
  __syncthreads();
  const uint32_t bin = ctl[0];
  const int rem = (int)ctl[1];
  const int cnt = (int)ctl[2];
  if (cnt > kWave) {
    __syncthreads();
    return block_kth_key<T, kKthSub>(keys, n, k, hist, ctl);
  }
  for (int i0 = 0; i0 < n; i0 += T) {
    const int i = i0 + tid;
    const uint64_t key = i < n ? keys[i] : 0;
    const bool m = i < n && (uint32_t)(((uint64_t)(hi - key_ord(key)) * inv) >> 32) == bin;
    const uint64_t msk = __ballot(m);
    if (msk) {
      uint32_t pos = 0;
      if (lane == 0) pos = atomicAdd(&ctl[3], (uint32_t)__popcll(msk));
      pos = wave_lane0(pos);
      if (m) {
        const uint32_t slot = pos + lanes_below(msk);
        gath[2 * slot] = (uint32_t)key;
        gath[2 * slot + 1] = (uint32_t)(key >> 32);
      }
    }
  }
  __syncthreads();
  if (tid < kWave) {
    // lane l holds gathered key l; the rem-th largest has rem - 1 above it
    const bool own = tid < cnt;
    const uint32_t klo = own ? gath[2 * tid] : 0u, khi = own ? gath[2 * tid + 1] : 0u;
    const uint64_t mine = ((uint64_t)khi << 32) | klo;
    int above = 0;
    for (int j = 0; j < cnt; ++j) {
      const uint64_t o = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)khi, j) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((int)klo, j);
      above += o > mine;
    }
    if (own && above == rem - 1) {
      ctl[4] = klo;
      ctl[5] = khi;
    }
  }
  __syncthreads();
  const uint64_t res = ((uint64_t)ctl[5] << 32) | ctl[4];
  __syncthreads();  // every thread has read ctl before a caller reuses it
  return res;
}

// Sort keys[0..n_pow2) descending in LDS (bitonic network).
template <int T>
__device__ void block_sort_desc(uint64_t* keys, int n_pow2) {
  const int tid = threadIdx.x;
  for (int size = 2; size <= n_pow2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      __syncthreads();
      for (int i = tid; i < (n_pow2 >> 1); i += T) {
        int lo = 2 * stride * (i / stride) + (i % stride);
        int hi = lo + stride;
        bool desc = (lo & size) == 0;
        uint64_t a = keys[lo], c = keys[hi];
        bool swap = desc ? (a < c) : (a > c);
        if (swap) {
          keys[lo] = c;
          keys[hi] = a;
        }
      }
    }
  }
  __syncthreads();
}

// The number of keys[0..n16) above `key`: keys in LDS, 16-byte aligned, n16 a
// multiple of 16 (the caller pads with zero keys, which are above none).
// Eight 16-byte broadcast reads are in flight per step, so the count runs at
// LDS throughput rather than one read latency per comparison.
__device__ __forceinline__ int count_above16(const uint64_t* keys, int n16, uint64_t key) {
  int c = 0;
  for (int j = 0; j < n16; j += 16) {
    ulonglong2 p[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) p[u] = *reinterpret_cast<const ulonglong2*>(keys + j + 2 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u) c += (p[u].x > key ? 1 : 0) + (p[u].y > key ? 1 : 0);
  }
  return c;
}

// Zero keys[n .. n rounded up to 16) and return that length (all threads of
// the block; the caller synchronises before the keys are read).
__device__ __forceinline__ int block_pad16(uint64_t* keys, int n) {
  const int n16 = (n + 15) & ~15;
  for (int i = n + (int)threadIdx.x; i < n16; i += (int)blockDim.x) keys[i] = 0;
  return n16;
}

// The n unique nonzero keys of keys[0..n) (LDS, capacity cap >= 2048, a
// power of two) in descending order, returned as a pointer into keys: for
// n <= 1024 each key's rank -- the number of larger keys, counted over the
// whole set -- is its place in keys[cap/2 ..]; beyond that the keys are
// sorted in place (bitonic).  Ends with a barrier.  Reductions over the
// selected keys read them in this order, so their floating-point result does
// not depend on the order in which the keys arrived.
template <int T>
__device__ uint64_t* block_order_desc(uint64_t* keys, int n, int cap) {
  if (n <= 1024) {
    uint64_t* dst = keys + cap / 2;
    const int n16 = block_pad16(keys, n);
    __syncthreads();
    for (int c = (int)threadIdx.x; c < n; c += T) {
      const uint64_t key = keys[c];
      dst[count_above16(keys, n16, key)] = key;
    }
    __syncthreads();
    return dst;
  }
  int npow = 1;
  while (npow < n) npow <<= 1;
  for (int i = n + (int)threadIdx.x; i < npow && i < cap; i += T) keys[i] = 0;
  block_sort_desc<T>(keys, npow);
  return keys;
}

// Keep the keys >= thr of keys[0..n) at the front IN THEIR ORDER and return
// their count to every thread.  Slot i = j*T + tid is read into registers
// first (n <= T * MAXPER), each wave counts its kept keys of every j into
// `scratch` (MAXPER * T/64 LDS words), and a key's place is the number of
// kept keys at smaller slots.  The result depends only on the input order,
// never on the order in which waves arrive.
template <int T, int MAXPER>
__device__ __forceinline__ int block_compact_ge_stable(uint64_t* keys, int n, uint64_t thr, uint32_t* scratch) {
  constexpr int NW = T / kWave;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int jn = (n + T - 1) / T;  // block-uniform
  uint64_t v[MAXPER];
  uint64_t msk[MAXPER];
#pragma unroll
  for (int j = 0; j < MAXPER; ++j) {
    const int i = j * T + tid;
    v[j] = (j < jn && i < n) ? keys[i] : 0;
    msk[j] = 0;
    if (j < jn) {
      msk[j] = __ballot(i < n && v[j] >= thr);
      if (lane_id() == 0) scratch[j * NW + wave] = (uint32_t)__popcll(msk[j]);
    }
  }
  __syncthreads();
  int total = 0;
  int pos[MAXPER];
#pragma unroll
  for (int j = 0; j < MAXPER; ++j) {
    pos[j] = 0;
    if (j < jn) {
      int before = 0, all = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = (int)scratch[j * NW + w];
        before += w < wave ? c : 0;
        all += c;
      }
      pos[j] = total + before;
      total += all;
    }
  }
#pragma unroll
  for (int j = 0; j < MAXPER; ++j)
    if (j < jn && ((msk[j] >> lane_id()) & 1)) keys[pos[j] + lanes_below(msk[j])] = v[j];
  __syncthreads();
  return total;
}

// Keep the keys >= thr of keys[0..n) at the front (order not kept) and
// return their count to every thread.  n <= T * MAXPER: every thread first
// reads its MAXPER slots into registers, so the in-place writes cannot
// overwrite unread keys.  `ctl` is one LDS word.
template <int T, int MAXPER>
__device__ int block_compact_ge(uint64_t* keys, int n, uint64_t thr, uint32_t* ctl) {
  const int tid = threadIdx.x;
  uint64_t v[MAXPER];
#pragma unroll
  for (int j = 0; j < MAXPER; ++j) {
    int i = j * T + tid;
    v[j] = (i < n) ? keys[i] : 0;
  }
  if (tid == 0) ctl[0] = 0;
  __syncthreads();
  // one LDS atomic per wave for every four slots' kept keys
#pragma unroll
  for (int j0 = 0; j0 < MAXPER; j0 += 4) {
    uint64_t masks[4];
    uint32_t total = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      masks[j] = j0 + j < MAXPER ? __ballot(v[j0 + j] != 0 && v[j0 + j] >= thr) : 0;
      total += (uint32_t)__popcll(masks[j]);
    }
    if (total) {
      uint32_t pos = 0;
      if (lane_id() == 0) pos = atomicAdd(&ctl[0], total);
      pos = wave_lane0(pos);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if ((masks[j] >> lane_id()) & 1) keys[pos + lanes_below(masks[j])] = v[j0 + j];
        pos += (uint32_t)__popcll(masks[j]);
      }
    }
  }
  __syncthreads();
  const int cnt = (int)ctl[0];
  __syncthreads();
  return cnt;
}

// Radix select over 32-bit order keys, 8-bit digits from the top: the
// largest v with #{keys >= v} >= k (the k-th largest key, with
// multiplicity).  `count(mask, prefix, shift)` histograms, into hist[256],
// the digit at `shift` of every key whose bits under `mask` equal `prefix`.
// Returns v; *rem_out = how many copies of v the top k take.  When every key
// shares its `common` leading bytes, `lead` (those bytes in place, the rest
// zero) skips their passes.
template <int T, typename Count>
__device__ uint32_t block_radix_kth32(int k, uint32_t* hist, uint32_t* ctl, Count&& count, int* rem_out,
                                      int common = 0, uint32_t lead = 0) {
  const int t = threadIdx.x;
  uint32_t prefix = common > 0 ? lead : 0u, mask = common > 0 ? 0xffffffffu << (32 - 8 * common) : 0u;
  int rem = k;
  for (int shift = 24 - 8 * common; shift >= 0; shift -= 8) {
    for (int i = t; i < 256; i += T) hist[i] = 0;
    __syncthreads();
    count(mask, prefix, shift);
    __syncthreads();
    if (t < kWave) {
      // lane l owns digits 255-4l .. 252-4l (high to low)
      uint32_t h[4];
      int s = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[q] = hist[255 - 4 * t - q];
        s += (int)h[q];
      }
      const int incl = wave_incl_scan(s);
      const int excl = incl - s;
      if (excl < rem && rem <= incl) {
        int acc = excl;
        int d = -1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (d < 0) {
            if (acc + (int)h[q] >= rem)
              d = 255 - 4 * t - q;
            else
              acc += (int)h[q];
          }
        }
        ctl[0] = (uint32_t)d;
        ctl[1] = (uint32_t)(rem - acc);
      }
    }
    __syncthreads();
    prefix |= ctl[0] << shift;
    mask |= 255u << shift;
    rem = (int)ctl[1];
    __syncthreads();
  }
  *rem_out = rem;
  return prefix;
}

// Exact top-k of a whole row by radix select over its order keys:
// ord_at(i) is the order key of element i (0 <= i < n).  The k-th largest
// order key v, then every element above v (fewer than k) and the
// lowest-index elements equal to v, in index order.  Leaves the k keys in
// cand[0..k) (unsorted); hist holds 256 words, ctl 3.
template <int T, typename Ord>
__device__ void block_row_topk(Ord&& ord_at, int n, int k, uint64_t* cand, uint32_t* hist, uint32_t* ctl) {
  const int t = threadIdx.x;
  int rem;
  const uint32_t v = block_radix_kth32<T>(
      k, hist, ctl,
      [&](uint32_t mask, uint32_t prefix, int shift) {
        for (int i0 = 0; i0 < n; i0 += T) {
          const int i = i0 + t;
          const uint32_t o = i < n ? ord_at(i) : 0u;
          hist_add(hist, (o >> shift) & 255u, i < n && (o & mask) == prefix);
        }
      },
      &rem);
  const int above = k - rem;  // elements with order key > v
  if (t == 0) ctl[2] = 0;
  __syncthreads();
  for (int i0 = 0; i0 < n; i0 += T) {
    const int i = i0 + t;
    const uint32_t o = i < n ? ord_at(i) : 0u;
    const bool keep = i < n && o > v;
    const uint64_t m = __ballot(keep);
    if (m) {
      uint32_t pos = 0;
      if (lane_id() == 0) pos = atomicAdd(&ctl[2], (uint32_t)__popcll(m));
      pos = wave_lane0(pos);
      if (keep) cand[pos + lanes_below(m)] = make_key(o, (uint32_t)i);
    }
  }
  // ties in index order, one tile of T consecutive elements at a time
  const int wave = t / kWave;
  int taken = 0;
  for (int base = 0; base < n && taken < rem; base += T) {
    const int i = base + t;
    const bool eq = i < n && ord_at(i) == v;
    const uint64_t m = __ballot(eq);
    if (lane_id() == 0) hist[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    int before = 0, total = 0;
    for (int w = 0; w < T / kWave; ++w) {
      const int c = (int)hist[w];
      before += w < wave ? c : 0;
      total += c;
    }
    const int pos = taken + before + (int)lanes_below(m);
    if (eq && pos < rem) cand[above + pos] = make_key(v, (uint32_t)i);
    taken += total;
    __syncthreads();
  }
  __syncthreads();
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

}  // namespace atopk
