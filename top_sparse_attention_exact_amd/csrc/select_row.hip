// One workgroup per row: single-launch exact and bucketed top-k for batches
// with enough rows to occupy the chip (one 1024-thread workgroup per CU).
//
// Bucketed ("Approximate Top-k for Increased Parallelism", Pith review page,
// "What carries the argument"): every lane keeps a sorted k_b-queue per
// element slot of its 16-byte loads.  For bf16 the key is packed into 32 bits
// -- the 16-bit order key of the value above a 16-bit complemented ordinal
// of the element inside its bucket (i = r + b*j) -- so a queue insert is one
// v_max_u32 plus one v_med3_u32 per further slot, and the value/tie order is
// decided by one unsigned compare.  Queues of lanes that share a bucket are
// merged by cross-lane shuffles, then by a tree across the 16 waves through
// LDS, and the final exact top-k of the b*k_b candidates is taken in LDS.
//
// Exact (same page, "The reading"; Figures 11-14 on radix select and its
// tie "collect" step): the row is streamed once through a threshold filter.
// The first tile seeds the threshold with a provable lower bound of the k-th
// largest value -- in each of the a waves that hold elements (16 unless the
// row is short) the ceil(k/a)-th largest of its 64 lane maxima; a*ceil(k/a)
// >= k distinct elements reach the smallest of those -- so from the start
// only a small fraction of elements is appended
// to the LDS candidate buffer, which is compacted by radix select when full.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace atopk {

namespace {

constexpr int kRowT = 1024;
constexpr int kRowWaves = kRowT / kWave;
constexpr int kRowLds = 65536;  // bytes: tree-merge exchange, then final candidates

typedef int16_t i16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Order keys of the two bf16 halves of w, packed the same way: per 16-bit
// half, a positive h maps to h ^ 0x8000 and a negative h to -h mod 2^16, so
// -0.0 and +0.0 both map to 0x8000 (packed 16-bit integer ops, 4 per word).
__device__ __forceinline__ uint32_t ord_bf16x2(uint32_t w) {
  const i16x2 s = __builtin_bit_cast(i16x2, w);
  const u16x2 m = __builtin_bit_cast(u16x2, (i16x2)(s >> (i16x2)(15)));
  const u16x2 u = __builtin_bit_cast(u16x2, w) ^ (m | (u16x2)(0x8000));
  return __builtin_bit_cast(uint32_t, (u16x2)(u - m));
}

// bf16 bits of a 16-bit order key (0x8000 -> +0.0).
__device__ __forceinline__ uint16_t bf16_from_ord16(uint32_t o) {
  return (uint16_t)((o & 0x8000u) ? (o & 0x7fffu) : ((0x10000u - o) & 0xffffu));
}

// Final exact top-k of n <= kRowT unique keys in LDS, written sorted with no
// sort: the rank of a key (how many keys beat it) is its output position.
// `per` threads share one key, each counting over a strided part of the set.
template <typename Writer>
__device__ __forceinline__ void block_rank_final(const uint64_t* cand, int n, int k, Writer&& write) {
  const int t = threadIdx.x;
  int per = 1;
  while (per < kWave && n * per * 2 <= kRowT) per *= 2;
  const int c = t / per;
  const int part = t % per;
  if (c < n) {
    const uint64_t key = cand[c];
    // parts interleave (j = part + per*m) so a wave reads `per` adjacent
    // keys per step: distinct banks, each broadcast to its group
    int cnt0 = 0, cnt1 = 0, cnt2 = 0, cnt3 = 0;
    int j = part;
    for (; j + 7 * per < n; j += 8 * per) {  // eight reads in flight
      const uint64_t a0 = cand[j], a1 = cand[j + per], a2 = cand[j + 2 * per], a3 = cand[j + 3 * per];
      const uint64_t a4 = cand[j + 4 * per], a5 = cand[j + 5 * per], a6 = cand[j + 6 * per], a7 = cand[j + 7 * per];
      cnt0 += (a0 > key ? 1 : 0) + (a4 > key ? 1 : 0);
      cnt1 += (a1 > key ? 1 : 0) + (a5 > key ? 1 : 0);
      cnt2 += (a2 > key ? 1 : 0) + (a6 > key ? 1 : 0);
      cnt3 += (a3 > key ? 1 : 0) + (a7 > key ? 1 : 0);
    }
    for (; j < n; j += per) cnt0 += cand[j] > key ? 1 : 0;
    int cnt = cnt0 + cnt1 + cnt2 + cnt3;
    for (int o = per / 2; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, kWave);
    if (part == 0 && cnt < k) write(cnt, key);
  }
}

// Exact top-k of n unique keys in LDS, sorted, written through `write`
// (every thread calls; n <= kRowLds / 8).
template <typename Writer>
__device__ void block_final(uint64_t* cand, int n, int k, uint32_t* hist, uint32_t* ctl, Writer&& write) {
  const int t = threadIdx.x;
  if (n <= 256) {
    block_rank_final(cand, n, k, write);
    return;
  }
  if (n <= kRowT) {
    block_sortmerge_final<kRowT>(cand, cand, n, k, write);
    return;
  }
  int cnt = n;
  if (cnt > k) {
    const uint64_t thr = block_kth_key<kRowT>(cand, cnt, k, hist, ctl);
    cnt = block_compact_ge<kRowT, (kRowLds / 8) / kRowT>(cand, cnt, thr, ctl);
  }
  if (cnt <= kRowT) {
    block_sortmerge_final<kRowT>(cand, cand, cnt, k, write);
    return;
  }
  int npow = 1;
  while (npow < k) npow <<= 1;
  for (int i = cnt + t; i < npow; i += kRowT) cand[i] = 0;
  block_sort_desc<kRowT>(cand, npow);
  for (int j = t; j < k; j += kRowT) write(j, cand[j]);
}

// Maximum over the wave: DPP inside each row of 16 lanes, then the 4 rows.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xb1, 0xf, 0xf, true));   // quad_perm 1,0,3,2
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4e, 0xf, 0xf, true));   // quad_perm 2,3,0,1
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xf, 0xf, true));  // row_half_mirror
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xf, 0xf, true));  // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

// c-th largest (1-based, duplicates counted) of one value per lane: c rounds
// of "take the maximum, retire one lane holding it".
__device__ __forceinline__ uint32_t wave_cth_largest(uint32_t v, int c) {
  uint32_t m = 0;
  for (int r = 0; r < c; ++r) {
    m = wave_max_u32(v);
    const uint64_t hit = __ballot(v == m);
    const int first = __builtin_ctzll(hit);
    if (lane_id() == first) v = 0;
  }
  return m;
}

// ------------------------------------------------------------- bucketed ----

template <int KB, bool FINAL>
__global__ __launch_bounds__(kRowT) void row_bucket_bf16_kernel(const uint8_t* __restrict__ x, int64_t ld_bytes,
                                                               int n, int b, int kb, int k,
                                                               uint16_t* __restrict__ out_vals,
                                                               int32_t* __restrict__ out_idx) {
  constexpr int T = kRowT;
  constexpr int V = 8;        // bf16 per 16-byte load
  constexpr int U = 4;        // loads in flight per lane
  constexpr int SW = T * V;   // elements per sweep
  __shared__ __align__(16) uint8_t smem[kRowLds];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t ctl[8];
  uint32_t* xch = reinterpret_cast<uint32_t*>(smem);
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem);

  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = t / kWave;
  const int row = blockIdx.x;
  const uint16_t* xr = reinterpret_cast<const uint16_t*>(x + (int64_t)row * ld_bytes);

  uint32_t q[V][KB];
#pragma unroll
  for (int e = 0; e < V; ++e)
#pragma unroll
    for (int j = 0; j < KB; ++j) q[e][j] = 0;

  // Element (t, e) of sweep s has index s*SW + t*V + e, bucket (t*V + e) mod b
  // and ordinal j = s*(SW/b) + (t*V)/b inside its bucket (b >= 8, b | SW).
  const uint32_t step = (uint32_t)(SW / b);
  const uint32_t pos0 = 0xffffu - (uint32_t)((t * V) / b);
  const int full_sweeps = n / SW;

  auto consume = [&](const uint4& w, uint32_t pos) {
    const uint32_t word[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const uint32_t o = ord_bf16x2(word[h]);
      queue_insert<KB>(q[2 * h], (o << 16) | pos);
      queue_insert<KB>(q[2 * h + 1], (o & 0xffff0000u) | pos);
    }
  };

  int s = 0;
  for (; s + U <= full_sweeps; s += U) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = *reinterpret_cast<const uint4*>(xr + (int64_t)(s + u) * SW + t * V);
#pragma unroll
    for (int u = 0; u < U; ++u) consume(w[u], pos0 - (uint32_t)(s + u) * step);
  }
  for (; s < full_sweeps; ++s) consume(*reinterpret_cast<const uint4*>(xr + (int64_t)s * SW + t * V), pos0 - (uint32_t)s * step);
  if ((int64_t)s * SW < n) {  // ragged last sweep, element by element
    const uint32_t pos = pos0 - (uint32_t)s * step;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int64_t i = (int64_t)s * SW + t * V + e;
      if (i < n) {
        const uint32_t o = ord_bf16x2((uint32_t)xr[i]) << 16;
        queue_insert<KB>(q[e], o | pos);
      }
    }
  }

  // Lanes l and l ^ m hold the same buckets when 8*m is a multiple of b.
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    if (m * V >= b) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        uint32_t o[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) o[j] = (uint32_t)__shfl_xor((int)q[e][j], m, kWave);
        queue_merge<KB>(q[e], o);
      }
    }
  }
  const int64_t nc = (int64_t)b * kb;
  // Bucket r's final top-k_b -> bucket-major output, or a final-stage key.
  auto emit = [&](int r, const uint32_t (&a)[KB]) {
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      if (j < kb) {
        const uint32_t key = a[j];
        const uint32_t idx = (uint32_t)r + (uint32_t)b * (0xffffu - (key & 0xffffu));
        if constexpr (FINAL) {
          cand[r * kb + j] = make_key(key & 0xffff0000u, idx);
        } else {
          const uint32_t o16 = key >> 16;
          const int64_t at = (int64_t)row * nc + (int64_t)r * kb + j;
          out_idx[at] = (int32_t)idx;
          out_vals[at] = o16 == 0x8000u ? xr[idx] : bf16_from_ord16(o16);
        }
      }
    }
  };

  if (b <= kWave * V && kRowWaves * b * KB * 4 <= kRowLds) {
    // Every wave holds all b buckets (lanes with lane*8 + e < b): one LDS
    // exchange, then thread r merges the 16 copies of bucket r.
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int r = lane * V + e;
      if (r < b) {
#pragma unroll
        for (int j = 0; j < KB; ++j) xch[(wave * b + r) * KB + j] = q[e][j];
      }
    }
    __syncthreads();
    uint32_t a[KB];
    if (t < b) {
#pragma unroll
      for (int j = 0; j < KB; ++j) a[j] = xch[t * KB + j];
      uint32_t o[kRowWaves - 1][KB];
#pragma unroll
      for (int w2 = 1; w2 < kRowWaves; ++w2)
#pragma unroll
        for (int j = 0; j < KB; ++j) o[w2 - 1][j] = xch[(w2 * b + t) * KB + j];
#pragma unroll
      for (int w2 = 1; w2 < kRowWaves; ++w2) queue_merge<KB>(a, o[w2 - 1]);
    }
    __syncthreads();
    if (t < b) emit(t, a);
  } else {
    // Tree across waves: waves w and w + st hold the same buckets when
    // 512 * st is a multiple of b.
    const int smin = b > kWave * V ? b / (kWave * V) : 1;
    for (int st = kRowWaves / 2; st >= smin; st >>= 1) {
      if (wave >= st && wave < 2 * st) {
#pragma unroll
        for (int e = 0; e < V; ++e)
#pragma unroll
          for (int j = 0; j < KB; ++j) xch[(((wave - st) * kWave + lane) * V + e) * KB + j] = q[e][j];
      }
      __syncthreads();
      if (wave < st) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          uint32_t o[KB];
#pragma unroll
          for (int j = 0; j < KB; ++j) o[j] = xch[((wave * kWave + lane) * V + e) * KB + j];
          queue_merge<KB>(q[e], o);
        }
      }
      __syncthreads();
    }
    // Waves < smin now hold every bucket once: slot p = wave*512 + lane*8 + e
    // is bucket p when b >= 512; for b < 512 the lanes with lane*8 + e < b.
    if (wave < smin) {
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const int r = wave * kWave * V + lane * V + e;
        if (r < b) emit(r, q[e]);
      }
    }
  }
  if constexpr (FINAL) {
    __syncthreads();
    block_final(cand, (int)nc, k, hist, ctl, [&](int i, uint64_t key) {
      const uint32_t idx = key_idx(key);
      const uint32_t o16 = key_ord(key) >> 16;
      out_idx[(int64_t)row * k + i] = (int32_t)idx;
      out_vals[(int64_t)row * k + i] = o16 == 0x8000u ? xr[idx] : bf16_from_ord16(o16);
    });
  }
}

// ---------------------------------------------------------------- exact ----

template <int DT>
struct RowIn {
  static constexpr int V = DT == IN_F32 ? 4 : 8;  // elements per 16-byte load
  static constexpr int U = 4;                      // loads per lane per tile
  static constexpr int ES = DT == IN_F32 ? 4 : 2;
};

// Order key (ord32) of element e of a 16-byte vector.
template <int DT>
__device__ __forceinline__ uint32_t ord_elem(const uint4& w, int e) {
  const uint32_t word[4] = {w.x, w.y, w.z, w.w};
  if constexpr (DT == IN_F32) {
    return ord_f32(word[e]);
  } else {
    const uint32_t p = ord_bf16x2(word[e >> 1]);
    return (e & 1) ? (p & 0xffff0000u) : (p << 16);
  }
}

// Load vector u of a tile: whole 16-byte loads when the tile is inside the
// row, element by element (zero-filled) in the row's last tile.
template <int DT, int T>
__device__ __forceinline__ void load_tile(const uint8_t* xr, int64_t base, int n, int t, uint4 (&w)[RowIn<DT>::U]) {
  constexpr int V = RowIn<DT>::V, U = RowIn<DT>::U, ES = RowIn<DT>::ES;
  const int64_t tile = (int64_t)T * V * U;
  if (base + tile <= n) {
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = *reinterpret_cast<const uint4*>(xr + (base + (int64_t)u * T * V + t * V) * ES);
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t word[4] = {0, 0, 0, 0};
      const int64_t i0 = base + (int64_t)u * T * V + t * V;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if (i0 + e < n) {
          if constexpr (DT == IN_F32) {
            word[e] = reinterpret_cast<const uint32_t*>(xr)[i0 + e];
          } else {
            word[e >> 1] |= (uint32_t)reinterpret_cast<const uint16_t*>(xr)[i0 + e] << ((e & 1) * 16);
          }
        }
      }
      w[u] = make_uint4(word[0], word[1], word[2], word[3]);
    }
  }
}

// Every wave keeps its own candidate region in LDS and its own threshold, so
// the streaming loop has no workgroup barrier: the wave's top-k of the
// elements it reads contains the row's top-k restricted to those elements.
// Lower bounds of the row's k-th largest value are shared through LDS
// without synchronisation (each published value is valid whenever read).
constexpr int kRowExactMaxK = 64;
constexpr int kWaveRegion = kRowLds / 8 / kRowWaves;  // keys per wave (512)

// Keep the wave's top-k of its region (cnt keys) at the front; return the
// order key of the k-th (the wave's new lower bound) -- wave-synchronous.
__device__ __noinline__ uint32_t wave_compact_region(uint64_t* mine, int cnt, int k) {
  constexpr int P = kWaveRegion / kWave;
  const int lane = lane_id();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  uint64_t key[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int i = lane * P + p;
    key[p] = i < cnt ? mine[i] : 0;
  }
  wave_sort_desc<P>(key);
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int i = lane * P + p;
    if (i < k) mine[i] = key[p];
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  uint64_t kth = 0;
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (lane * P + p == k - 1) kth = key[p];
  return (uint32_t)(shfl_u64(kth, (k - 1) / P) >> 32);
}

// Largest order key among the elements of a 16-byte vector.
template <int DT>
__device__ __forceinline__ uint32_t vec_max_ord(const uint4& w) {
  const uint32_t word[4] = {w.x, w.y, w.z, w.w};
  if constexpr (DT == IN_F32) {
    return max(max(ord_f32(word[0]), ord_f32(word[1])), max(ord_f32(word[2]), ord_f32(word[3])));
  } else {
    u16x2 m = __builtin_bit_cast(u16x2, ord_bf16x2(word[0]));
#pragma unroll
    for (int h = 1; h < 4; ++h) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, ord_bf16x2(word[h])));
    return (uint32_t)max(m.x, m.y) << 16;
  }
}

template <int DT>
__global__ __launch_bounds__(kRowT) void row_exact_kernel(const uint8_t* __restrict__ x, int64_t ld_bytes, int n, int k,
                                                         uint8_t* __restrict__ out_vals,
                                                         int32_t* __restrict__ out_idx) {
  constexpr int T = kRowT;
  constexpr int V = RowIn<DT>::V;
  constexpr int U = RowIn<DT>::U;
  constexpr int ES = RowIn<DT>::ES;
  constexpr int TILE = T * U * V;
  __shared__ uint64_t buf[kRowLds / 8];
  // Bounds published by the waves, read fresh every tile and written without
  // barriers: relaxed workgroup-scope atomics (a volatile access would also
  // wait for the next tile's loads in flight).
  __shared__ uint32_t pub[kRowWaves];
  __shared__ uint32_t packed;  // keys in the final run
  auto pub_store = [&](int w2, uint32_t v) {
    __hip_atomic_store(&pub[w2], v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  };
  auto pub_load = [&](int w2) { return __hip_atomic_load(&pub[w2], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP); };

  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = t / kWave;
  const int row = blockIdx.x;
  const uint8_t* xr = x + (int64_t)row * ld_bytes;
  uint64_t* mine = buf + wave * kWaveRegion;
  // Waves that hold elements: on a row shorter than one pass of the block
  // the last waves hold none, and a bound pooled over them would be 0.
  // Each of the `act` waves vouches for ceil(k / act) <= 64 lane maxima; the
  // others publish no bound.
  const int64_t waves_n = ((int64_t)n + kWave * V - 1) / (kWave * V);
  const int act = waves_n < kRowWaves ? (int)waves_n : kRowWaves;
  const int cpw = (k + act - 1) / act;  // lane maxima each wave vouches for

  uint32_t lmax = 0;  // largest order key this lane has seen
  uint32_t thr = 1;   // filter: order key >= thr (real keys are >= 0x00800000)
  int cnt = 0;        // keys in this wave's region (wave-uniform)
  bool first = true;

  // One tile: lane t holds elements base + u*T*V + t*V + e.  `full` tiles are
  // whole 16-byte vectors; the last, partial tile is zero-filled and checked.
  auto tile = [&](const uint4 (&w)[U], int64_t base, auto full_c) {
    constexpr bool full = decltype(full_c)::value;
    uint32_t vm[U];  // largest order key of each vector (in-row elements only)
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (full) {
        vm[u] = vec_max_ord<DT>(w[u]);
      } else {
        vm[u] = 0;
#pragma unroll
        for (int e = 0; e < V; ++e)
          if (base + (int64_t)u * T * V + t * V + e < n) vm[u] = max(vm[u], ord_elem<DT>(w[u], e));
      }
      lmax = max(lmax, vm[u]);
    }
    // The c-th largest lane maximum of each active wave, c = ceil(k / act):
    // act * c >= k distinct elements reach the smallest of the published
    // values.  The first tile waits once for every wave to publish: the
    // pooled bound is far tighter than any one wave's.
    const uint32_t tc = wave < act ? wave_cth_largest(lmax, cpw) : 0xffffffffu;
    if (lane == 0) pub_store(wave, tc);
    if (first) {
      lds_barrier();
      first = false;
    }
    uint32_t tm = 0xffffffffu;
#pragma unroll
    for (int w2 = 0; w2 < kRowWaves; ++w2) tm = min(tm, pub_load(w2));
    thr = max(thr, tm);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // after the first tile almost no vector holds an element that passes
      if (__ballot(vm[u] >= thr) == 0) continue;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const uint32_t idx0 = (uint32_t)(base + u * T * V + t * V + e);
        const uint32_t oe = ord_elem<DT>(w[u], e);
        bool pass = oe >= thr && (full || (int64_t)idx0 < n);
        uint64_t mask = __ballot(pass);
        if (mask) {
          if (cnt + kWave > kWaveRegion) {  // region full: keep the wave's top-k
            thr = max(thr, wave_compact_region(mine, cnt, k));
            cnt = k;
            pass = pass && oe >= thr;
            mask = __ballot(pass);
          }
          const uint32_t idx = (uint32_t)(base + u * T * V + t * V + e);
          if (pass) mine[cnt + lanes_below(mask)] = make_key(oe, idx);
          cnt += __popcll(mask);
        }
      }
    }
  };

  // Full tiles through two register sets: the next tile's loads are always
  // in flight while a tile is filtered.  Inside the loop the prefetch is
  // unconditional (the loop stops while tile it + 2 still exists), so the
  // code stays straight and the wait before a tile covers only that tile's
  // own loads; the last one or two tiles are handled after the loop.
  const int nfull = n / TILE;
  uint4 wa[U], wb[U];
  auto load_full = [&](uint4 (&w)[U], int it) {
    const int64_t base = (int64_t)it * TILE;
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = *reinterpret_cast<const uint4*>(xr + (base + (int64_t)u * T * V + t * V) * ES);
  };
  if (nfull > 0) {
    int it = 0;
    load_full(wa, 0);
    for (; it + 2 < nfull; it += 2) {
      load_full(wb, it + 1);
      tile(wa, (int64_t)it * TILE, std::true_type{});
      load_full(wa, it + 2);
      tile(wb, (int64_t)(it + 1) * TILE, std::true_type{});
    }
    if (it + 1 < nfull) {
      load_full(wb, it + 1);
      tile(wa, (int64_t)it * TILE, std::true_type{});
      tile(wb, (int64_t)(it + 1) * TILE, std::true_type{});
    } else {
      tile(wa, (int64_t)it * TILE, std::true_type{});
    }
  }
  if ((int64_t)nfull * TILE < n) {
    load_tile<DT, T>(xr, (int64_t)nfull * TILE, n, t, wa);
    tile(wa, (int64_t)nfull * TILE, std::false_type{});
  }

  // Each wave reduces its region to at most k keys (its top-k when it holds
  // more than a wave's worth).  Once every wave has streamed, the published
  // bounds are final and their minimum bounds the row's k-th largest from
  // below (as in the first tile), far tighter than the bounds the keys were
  // admitted with: the keys that reach it are packed into one run at the
  // front of `buf`, and each key's rank in that run -- its output position
  // -- is counted directly.
  if (cnt > kWave) {
    wave_compact_region(mine, cnt, k);
    cnt = k;
  }
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront", "local");
  const uint64_t key = lane < cnt ? mine[lane] : 0;
  if (t == 0) packed = 0;
  __syncthreads();
  uint32_t bound = 0xffffffffu;
#pragma unroll
  for (int w2 = 0; w2 < kRowWaves; ++w2) bound = min(bound, pub_load(w2));
  const bool keep = key != 0 && key_ord(key) >= bound;
  const uint64_t kmask = __ballot(keep);
  if (kmask) {
    uint32_t pos = 0;
    if (lane == 0) pos = atomicAdd(&packed, (uint32_t)__popcll(kmask));
    pos = wave_lane0(pos);
    if (keep) buf[pos + lanes_below(kmask)] = key;
  }
  __syncthreads();
  const int total = (int)packed;
  block_rank_final(buf, total, k, [&](int i, uint64_t kk) {
    // the order key gives the value back, except the sign of a zero
    const uint32_t idx = key_idx(kk);
    const uint32_t o = key_ord(kk);
    const int64_t at = (int64_t)row * k + i;
    out_idx[at] = (int32_t)idx;
    if constexpr (DT == IN_F32) {
      reinterpret_cast<uint32_t*>(out_vals)[at] =
          o == 0x80000000u ? reinterpret_cast<const uint32_t*>(xr)[idx] : bits_from_ord(o);
    } else {
      const uint32_t o16 = o >> 16;
      reinterpret_cast<uint16_t*>(out_vals)[at] =
          o16 == 0x8000u ? reinterpret_cast<const uint16_t*>(xr)[idx] : bf16_from_ord16(o16);
    }
  });
}

// ------------------------------------------------------------ contiguous ----

// Contiguous assignment (same page, Figures 6 and 8 compare it with the
// interleaved one): bucket r holds the positions i with floor(i * b / n) ==
// r, a run of consecutive elements.  Each wave owns whole buckets (r = wave,
// wave + 16, ...): its lanes stream the run with coalesced loads into a
// k_b-queue of (order key, index) keys each, a butterfly of shuffles merges
// the 64 queues into the bucket's top-k_b, and the final exact top-k of the
// b * k_b candidates is taken in LDS.  vec: every run starts and ends on a
// 16-byte boundary (the runs are then read as 16-byte vectors).
template <int DT, int KB, bool FINAL, bool PACK>
__global__ __launch_bounds__(kRowT) void row_contig_kernel(const uint8_t* __restrict__ x, int64_t ld_bytes, int n,
                                                          int b, int kb, int k, int vec,
                                                          uint8_t* __restrict__ out_vals,
                                                          int32_t* __restrict__ out_idx) {
  // PACK (bf16, runs of at most 65536): 32-bit keys, the 16-bit order key
  // above the complemented position inside the run; otherwise 64-bit keys.
  using Key = std::conditional_t<PACK, uint32_t, uint64_t>;
  constexpr int V = RowIn<DT>::V;
  constexpr int ES = RowIn<DT>::ES;
  constexpr int U = 4;
  __shared__ uint64_t cand[kRowLds / 8];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t ctl[8];
  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = t / kWave;
  const int row = blockIdx.x;
  const uint8_t* xr = x + (int64_t)row * ld_bytes;

  auto write = [&](int64_t at, uint64_t key) {
    // the order key gives the value back, except the sign of a zero
    const uint32_t idx = key_idx(key);
    const uint32_t o = key_ord(key);
    out_idx[at] = (int32_t)idx;
    if constexpr (DT == IN_F32) {
      reinterpret_cast<uint32_t*>(out_vals)[at] =
          o == 0x80000000u ? reinterpret_cast<const uint32_t*>(xr)[idx] : bits_from_ord(o);
    } else {
      const uint32_t o16 = o >> 16;
      reinterpret_cast<uint16_t*>(out_vals)[at] =
          o16 == 0x8000u ? reinterpret_cast<const uint16_t*>(xr)[idx] : bf16_from_ord16(o16);
    }
  };

  for (int r = wave; r < b; r += kRowWaves) {
    const int s0 = (int)(((int64_t)r * n + b - 1) / b);
    const int s1 = (int)(((int64_t)(r + 1) * n + b - 1) / b);
    // key of the element with order key o (ord32 layout) at position i
    auto mk = [&](uint32_t o, int i) -> Key {
      if constexpr (PACK)
        return (o & 0xffff0000u) | (0xffffu - (uint32_t)(i - s0));
      else
        return make_key(o, (uint32_t)i);
    };
    Key q[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) q[j] = 0;
    if (vec) {
      const int nv = (s1 - s0) / V;
      for (int v0 = lane; v0 < nv; v0 += kWave * U) {
        uint4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int v = v0 + u * kWave;
          w[u] = v < nv ? *reinterpret_cast<const uint4*>(xr + ((int64_t)s0 + (int64_t)v * V) * ES)
                        : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int v = v0 + u * kWave;
          if (v < nv) {
#pragma unroll
            for (int e = 0; e < V; ++e) queue_insert<KB>(q, mk(ord_elem<DT>(w[u], e), s0 + v * V + e));
          }
        }
      }
    } else {
      for (int i0 = s0 + lane; i0 < s1; i0 += kWave * U) {
        uint32_t bits[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * kWave;
          if constexpr (DT == IN_F32)
            bits[u] = i < s1 ? reinterpret_cast<const uint32_t*>(xr)[i] : 0u;
          else
            bits[u] = i < s1 ? (uint32_t)reinterpret_cast<const uint16_t*>(xr)[i] : 0u;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int i = i0 + u * kWave;
          if (i < s1) {
            const uint32_t o = DT == IN_F32 ? ord_f32(bits[u]) : (ord_bf16x2(bits[u]) << 16);
            queue_insert<KB>(q, mk(o, i));
          }
        }
      }
    }
    // every lane ends with the bucket's top-KB
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      Key c[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        if constexpr (PACK)
          c[j] = (Key)__shfl_xor((int)q[j], o, kWave);
        else
          c[j] = shfl_xor_u64(q[j], o);
      }
      queue_merge<KB>(q, c);
    }
    Key mine = 0;
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if (j == lane) mine = q[j];
    uint64_t key;
    if constexpr (PACK)
      key = make_key(mine & 0xffff0000u, (uint32_t)s0 + (0xffffu - (mine & 0xffffu)));
    else
      key = mine;
    if (lane < kb) {
      if constexpr (FINAL)
        cand[r * kb + lane] = key;
      else
        write(((int64_t)row * b + r) * kb + lane, key);
    }
  }
  if constexpr (FINAL) {
    __syncthreads();
    block_final(cand, b * kb, k, hist, ctl, [&](int i, uint64_t key) { write((int64_t)row * k + i, key); });
  }
}

// Exact top-k of a row that fits LDS whole (n <= kRowLds / 8 elements, any
// alignment, any k <= n): every element becomes an (order key, index) key
// and the block's radix select and exact final rank them: one read of the
// row and no threshold filter.  Short rows with k above the filtering kernel's limit
// otherwise pay several launches for a few KiB.
constexpr int kRowSmallMaxN = kRowLds / 8;

template <int DT>
__global__ __launch_bounds__(kRowT) void row_small_exact_kernel(const uint8_t* __restrict__ x, int64_t ld_bytes,
                                                               int n, int k, uint8_t* __restrict__ out_vals,
                                                               int32_t* __restrict__ out_idx) {
  __shared__ uint64_t cand[kRowSmallMaxN];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t ctl[8];
  const int row = blockIdx.x;
  const uint8_t* xr = x + (int64_t)row * ld_bytes;
  for (int i = threadIdx.x; i < n; i += kRowT) {
    uint32_t o;
    if constexpr (DT == IN_F32)
      o = ord_f32(reinterpret_cast<const uint32_t*>(xr)[i]);
    else
      o = ord_bf16x2((uint32_t)reinterpret_cast<const uint16_t*>(xr)[i]) << 16;
    cand[i] = make_key(o, (uint32_t)i);
  }
  __syncthreads();
  // Above 256 keys, select the k-th key and keep the k keys that reach it
  // first: the final then ranks or sorts k keys instead of the whole row.
  int cnt = n;
  if (n > 256 && k < n) {
    const uint64_t thr = block_kth_key<kRowT>(cand, n, k, hist, ctl);
    cnt = block_compact_ge<kRowT, kRowSmallMaxN / kRowT>(cand, n, thr, ctl);
  }
  block_final(cand, cnt, k, hist, ctl, [&](int i, uint64_t kk) {
    // the order key gives the value back, except the sign of a zero
    const uint32_t idx = key_idx(kk);
    const uint32_t o = key_ord(kk);
    const int64_t at = (int64_t)row * k + i;
    out_idx[at] = (int32_t)idx;
    if constexpr (DT == IN_F32) {
      reinterpret_cast<uint32_t*>(out_vals)[at] =
          o == 0x80000000u ? reinterpret_cast<const uint32_t*>(xr)[idx] : bits_from_ord(o);
    } else {
      const uint32_t o16 = o >> 16;
      reinterpret_cast<uint16_t*>(out_vals)[at] =
          o16 == 0x8000u ? reinterpret_cast<const uint16_t*>(xr)[idx] : bf16_from_ord16(o16);
    }
  });
}

}  // namespace

bool row_bucket_ok(int dtype, int64_t m, int64_t n, int64_t b, int64_t kb, bool aligned) {
  if (dtype != IN_BF16 || !aligned) return false;
  if (b < 8 || b > 8192 || (b & (b - 1)) != 0) return false;
  if (n / b > 65535 + 1) return false;  // ordinal fits 16 bits
  if ((n + b - 1) / b > 65536) return false;
  if (kb > 4) return false;
  if (b * kb > kRowLds / 8) return false;
  if ((int64_t)(kRowWaves / 2) * kWave * 8 * (kb <= 1 ? 1 : kb <= 2 ? 2 : 4) * 4 > kRowLds) return false;
  return m >= 128 || n <= 65536;
}

bool row_exact_ok(int dtype, int64_t m, int64_t n, int64_t k, bool aligned) {
  if (!aligned || k > kRowExactMaxK) return false;
  return m >= 128 || n <= 65536;
}

bool row_small_exact_ok(int dtype, int64_t m, int64_t n, int64_t k) {
  (void)m;
  (void)k;
  return (dtype == IN_F32 || dtype == IN_BF16) && n <= kRowSmallMaxN;
}

hipError_t launch_row_bucket(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b,
                             int64_t kb, int final_exact, void* out_vals, int32_t* out_idx, hipStream_t s) {
  (void)dtype;
  const int64_t ld_bytes = ldx * 2;
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  uint16_t* ov = static_cast<uint16_t*>(out_vals);
  dim3 grid((unsigned)m);
  const int kbs = kb <= 1 ? 1 : kb <= 2 ? 2 : 4;
#define ATOPK_RB(KBV, FIN)                                                                                  \
  ATOPK_LAUNCH((row_bucket_bf16_kernel<KBV, FIN>), grid, dim3(kRowT), 0, s, xb, ld_bytes, (int)n, \
                     (int)b, (int)kb, (int)k, ov, out_idx)
  if (final_exact) {
    if (kbs == 1) ATOPK_RB(1, true);
    else if (kbs == 2) ATOPK_RB(2, true);
    else ATOPK_RB(4, true);
  } else {
    if (kbs == 1) ATOPK_RB(1, false);
    else if (kbs == 2) ATOPK_RB(2, false);
    else ATOPK_RB(4, false);
  }
#undef ATOPK_RB
  return hipGetLastError();
}

bool row_contig_ok(int64_t n, int64_t b, int64_t kb, int final_exact) {
  return kb >= 1 && kb <= 16 && n / b >= kb && n <= INT32_MAX && (!final_exact || b * kb <= kRowLds / 8);
}

template <int DT, int KB, bool FIN>
void launch_contig_t(dim3 grid, hipStream_t s, const uint8_t* xb, int64_t ld_bytes, int64_t n, int64_t b, int64_t kb,
                     int64_t k, int vec, bool pack, uint8_t* ov, int32_t* out_idx) {
  if constexpr (DT == IN_BF16) {
    if (pack) {
      ATOPK_LAUNCH((row_contig_kernel<DT, KB, FIN, true>), grid, dim3(kRowT), 0, s, xb, ld_bytes, (int)n, (int)b,
                         (int)kb, (int)k, vec, ov, out_idx);
      return;
    }
  }
  ATOPK_LAUNCH((row_contig_kernel<DT, KB, FIN, false>), grid, dim3(kRowT), 0, s, xb, ld_bytes, (int)n, (int)b,
                     (int)kb, (int)k, vec, ov, out_idx);
}

template <int DT, bool FIN>
void launch_contig_kb(int kbs, dim3 grid, hipStream_t s, const uint8_t* xb, int64_t ld_bytes, int64_t n, int64_t b,
                      int64_t kb, int64_t k, int vec, bool pack, uint8_t* ov, int32_t* out_idx) {
  if (kbs == 1) launch_contig_t<DT, 1, FIN>(grid, s, xb, ld_bytes, n, b, kb, k, vec, pack, ov, out_idx);
  else if (kbs == 2) launch_contig_t<DT, 2, FIN>(grid, s, xb, ld_bytes, n, b, kb, k, vec, pack, ov, out_idx);
  else if (kbs == 4) launch_contig_t<DT, 4, FIN>(grid, s, xb, ld_bytes, n, b, kb, k, vec, pack, ov, out_idx);
  else if (kbs == 8) launch_contig_t<DT, 8, FIN>(grid, s, xb, ld_bytes, n, b, kb, k, vec, pack, ov, out_idx);
  else launch_contig_t<DT, 16, FIN>(grid, s, xb, ld_bytes, n, b, kb, k, vec, pack, ov, out_idx);
}

hipError_t launch_row_contig(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, int64_t b,
                             int64_t kb, int final_exact, bool aligned, void* out_vals, int32_t* out_idx,
                             hipStream_t s) {
  const int64_t es = dtype == IN_F32 ? 4 : 2;
  const int64_t vlen = 16 / es;
  const int vec = aligned && n % b == 0 && (n / b) % vlen == 0 ? 1 : 0;
  const bool pack = (n + b - 1) / b <= 65536;  // positions inside a run fit 16 bits
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  uint8_t* ov = static_cast<uint8_t*>(out_vals);
  const dim3 grid((unsigned)m);
  const int kbs = kb <= 1 ? 1 : kb <= 2 ? 2 : kb <= 4 ? 4 : kb <= 8 ? 8 : 16;
  if (dtype == IN_F32) {
    if (final_exact) launch_contig_kb<IN_F32, true>(kbs, grid, s, xb, ldx * es, n, b, kb, k, vec, pack, ov, out_idx);
    else launch_contig_kb<IN_F32, false>(kbs, grid, s, xb, ldx * es, n, b, kb, k, vec, pack, ov, out_idx);
  } else {
    if (final_exact) launch_contig_kb<IN_BF16, true>(kbs, grid, s, xb, ldx * es, n, b, kb, k, vec, pack, ov, out_idx);
    else launch_contig_kb<IN_BF16, false>(kbs, grid, s, xb, ldx * es, n, b, kb, k, vec, pack, ov, out_idx);
  }
  return hipGetLastError();
}

hipError_t launch_row_small_exact(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k,
                                  void* out_vals, int32_t* out_idx, hipStream_t s) {
  if (n > kRowSmallMaxN || k > n) return hipErrorInvalidValue;
  dim3 grid((unsigned)m);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  uint8_t* ov = static_cast<uint8_t*>(out_vals);
  if (dtype == IN_F32) {
    ATOPK_LAUNCH((row_small_exact_kernel<IN_F32>), grid, dim3(kRowT), 0, s, xb, ldx * 4, (int)n, (int)k, ov, out_idx);
  } else {
    ATOPK_LAUNCH((row_small_exact_kernel<IN_BF16>), grid, dim3(kRowT), 0, s, xb, ldx * 2, (int)n, (int)k, ov,
                 out_idx);
  }
  return hipGetLastError();
}

hipError_t launch_row_exact(const void* x, int dtype, int64_t m, int64_t n, int64_t ldx, int64_t k, void* out_vals,
                            int32_t* out_idx, hipStream_t s) {
  dim3 grid((unsigned)m);
  const uint8_t* xb = static_cast<const uint8_t*>(x);
  uint8_t* ov = static_cast<uint8_t*>(out_vals);
  if (dtype == IN_F32) {
    ATOPK_LAUNCH((row_exact_kernel<IN_F32>), grid, dim3(kRowT), 0, s, xb, ldx * 4, (int)n, (int)k, ov, out_idx);
  } else {
    ATOPK_LAUNCH((row_exact_kernel<IN_BF16>), grid, dim3(kRowT), 0, s, xb, ldx * 2, (int)n, (int)k, ov, out_idx);
  }
  return hipGetLastError();
}

}  // namespace atopk
