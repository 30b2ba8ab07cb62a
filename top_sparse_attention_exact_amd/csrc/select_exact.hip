// Exact top-k of long rows: a one-pass threshold filter with an LDS
// candidate buffer, compacted by radix select.
//
// "Approximate Top-k for Increased Parallelism" (Pith review page), Figures
// 11-14 describe serial and parallel radix select (a bitwise search for the
// k-th value from the most significant bit, then a "collect" step because the
// k-th value may be tied).  Here the row is streamed once: an element enters
// the LDS buffer only if its 64-bit key (value, then lower index) beats the
// current threshold, the k-th best key seen so far.  When the buffer is
// nearly full, a radix select over the buffered keys (8-bit digits, LDS
// histogram) finds the k-th key, the buffer is compacted to the k keys at or
// above it, and that key becomes the new threshold.  Because the index is
// part of the key, every key is unique and the "collect" of tied values is
// the same compaction.  After warm-up almost every element costs one
// comparison, so the pass runs at streaming speed.
#include "common.h"
#include "launch.h"

namespace atopk {

namespace {

constexpr int kExactThreads = 256;
constexpr int kExactStep = 2048;  // elements appended per iteration (upper bound)

template <int IN>
struct ExactIn {
  static constexpr int V = IN == IN_F32 ? 4 : (IN == IN_BF16 ? 8 : 2);   // per 16-byte load
  static constexpr int ES = IN == IN_F32 ? 4 : (IN == IN_BF16 ? 2 : 8);  // bytes per element
  static constexpr int U = kExactStep / (kExactThreads * V);             // loads per lane per step
};

template <int IN>
__device__ __forceinline__ uint64_t key_from_vec(const uint4& w, int e, uint32_t idx) {
  if constexpr (IN == IN_KEY64) {
    return e == 0 ? (((uint64_t)w.y << 32) | w.x) : (((uint64_t)w.w << 32) | w.z);
  } else if constexpr (IN == IN_F32) {
    const uint32_t word[4] = {w.x, w.y, w.z, w.w};
    return make_key(ord_f32(word[e]), idx);
  } else {
    const uint32_t word[4] = {w.x, w.y, w.z, w.w};
    const uint32_t v = word[e >> 1];
    return make_key(ord_f32((e & 1) ? (v & 0xffff0000u) : (v << 16)), idx);
  }
}

template <int IN>
__device__ __forceinline__ uint64_t key_at(const uint8_t* row, int64_t i) {
  if constexpr (IN == IN_KEY64) {
    return reinterpret_cast<const uint64_t*>(row)[i];
  } else if constexpr (IN == IN_F32) {
    return make_key(ord_f32(reinterpret_cast<const uint32_t*>(row)[i]), (uint32_t)i);
  } else {
    return make_key(ord_f32((uint32_t)reinterpret_cast<const uint16_t*>(row)[i] << 16), (uint32_t)i);
  }
}

template <int IN, int CAP>
__global__ __launch_bounds__(kExactThreads) void exact_filter_kernel(
    const uint8_t* __restrict__ x, int64_t ld_bytes, int n, int k, int64_t chunk, int splits, int aligned,
    uint64_t* __restrict__ part, const uint8_t* __restrict__ src, int64_t src_ld_bytes, int src_dt,
    uint8_t* __restrict__ out_vals, int32_t* __restrict__ out_idx) {
  constexpr int T = kExactThreads;
  constexpr int V = ExactIn<IN>::V;
  constexpr int ES = ExactIn<IN>::ES;
  constexpr int U = ExactIn<IN>::U;
  constexpr int NS = U * V;
  constexpr int MAXPER = CAP / T;
  __shared__ uint64_t buf[CAP];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t ctl[8];  // [0..2] radix select / compaction scratch, [4..6] append counters

  const int t = threadIdx.x;
  const int lane = lane_id();
  const int row = blockIdx.y;
  const int split = blockIdx.x;
  const int64_t c0 = (int64_t)split * chunk;
  const int64_t c1 = min((int64_t)n, c0 + chunk);
  const uint8_t* xr = x + (int64_t)row * ld_bytes;

  // Buffer fill: `count` is kept identical in every thread.  Appends of one
  // iteration count up a per-iteration counter (three in rotation, so the one
  // being cleared is never being read or incremented).
  if (t < 3) ctl[4 + t] = 0;
  uint64_t thr = 0;  // keys must be strictly greater to enter
  int count = 0;
  int it = 0;
  __syncthreads();

  for (int64_t base = c0; base < c1; base += kExactStep, ++it) {
    uint64_t key[NS];
    if (aligned && base + kExactStep <= c1) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i0 = base + (int64_t)u * T * V + (int64_t)t * V;
        const uint4 w = *reinterpret_cast<const uint4*>(xr + i0 * ES);
#pragma unroll
        for (int e = 0; e < V; ++e) key[u * V + e] = key_from_vec<IN>(w, e, (uint32_t)(i0 + e));
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t i0 = base + (int64_t)u * T * V + (int64_t)t * V;
#pragma unroll
        for (int e = 0; e < V; ++e) key[u * V + e] = (i0 + e < c1) ? key_at<IN>(xr, i0 + e) : 0;
      }
    }
    if (count + kExactStep > CAP) {  // same decision in every thread
      thr = block_kth_key<T>(buf, count, k, hist, ctl);
      count = block_compact_ge<T, MAXPER>(buf, count, thr, ctl);
    }
    uint32_t* ctr = &ctl[4 + it % 3];
    if (t == 0) ctl[4 + (it + 1) % 3] = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bool pass = key[s] > thr;
      const uint64_t mask = __ballot(pass);
      if (mask) {
        uint32_t pos = 0;
        if (lane == 0) pos = atomicAdd(ctr, (uint32_t)__popcll(mask));
        pos = wave_lane0(pos);
        if (pass) buf[count + pos + lanes_below(mask)] = key[s];
      }
    }
    __syncthreads();
    count += (int)*ctr;
  }

  __syncthreads();
  if (count > k) {
    thr = block_kth_key<T>(buf, count, k, hist, ctl);
    count = block_compact_ge<T, MAXPER>(buf, count, thr, ctl);
  }
  if (part != nullptr) {
    uint64_t* dst = part + ((int64_t)row * splits + split) * k;
    for (int j = t; j < k; j += T) dst[j] = (j < count) ? buf[j] : 0;
    return;
  }
  int npow = 1;
  while (npow < k) npow <<= 1;
  for (int i = count + t; i < npow; i += T) buf[i] = 0;
  block_sort_desc<T>(buf, npow);
  const uint8_t* sr = src + (int64_t)row * src_ld_bytes;
  for (int j = t; j < k; j += T) {
    const uint64_t key = buf[j];
    const uint32_t idx = key_idx(key);
    const int64_t o = (int64_t)row * k + j;
    out_idx[o] = (int32_t)idx;
    if (src_dt == IN_F32) {
      reinterpret_cast<uint32_t*>(out_vals)[o] = reinterpret_cast<const uint32_t*>(sr)[idx];
    } else {
      reinterpret_cast<uint16_t*>(out_vals)[o] = reinterpret_cast<const uint16_t*>(sr)[idx];
    }
  }
}

template <int IN>
hipError_t launch_exact_in(const ExactPlan& p, const void* x, int64_t m, int64_t n, int64_t ld, int64_t k,
                           uint64_t* part, const void* src, int src_dtype, int64_t src_ld, void* out_vals,
                           int32_t* out_idx, hipStream_t s) {
  const int64_t ld_bytes = ld * ExactIn<IN>::ES;
  const int64_t src_ld_bytes = src_ld * (src_dtype == IN_F32 ? 4 : 2);
  dim3 grid((unsigned)p.splits, (unsigned)m);
  const int aligned = ((reinterpret_cast<uintptr_t>(x) | (uintptr_t)ld_bytes) & 15) == 0;
  if (p.cap == 4096) {
    ATOPK_LAUNCH((exact_filter_kernel<IN, 4096>), grid, dim3(kExactThreads), 0, s,
                       static_cast<const uint8_t*>(x), ld_bytes, (int)n, (int)k, p.chunk, p.splits, aligned, part,
                       static_cast<const uint8_t*>(src), src_ld_bytes, src_dtype,
                       static_cast<uint8_t*>(out_vals), out_idx);
  } else {
    ATOPK_LAUNCH((exact_filter_kernel<IN, 10240>), grid, dim3(kExactThreads), 0, s,
                       static_cast<const uint8_t*>(x), ld_bytes, (int)n, (int)k, p.chunk, p.splits, aligned, part,
                       static_cast<const uint8_t*>(src), src_ld_bytes, src_dtype,
                       static_cast<uint8_t*>(out_vals), out_idx);
  }
  return hipGetLastError();
}

}  // namespace

ExactPlan plan_exact(int in_kind, int64_t m, int64_t n, int64_t k) {
  ExactPlan p{};
  p.cap = k <= 2048 ? 4096 : 10240;
  int64_t splits = 1;
  if (in_kind != IN_KEY64) {
    splits = (512 + m - 1) / (m > 0 ? m : 1);
    splits = std::min<int64_t>(splits, std::max<int64_t>(1, n / std::max<int64_t>(4 * k, 16384)));
    splits = std::max<int64_t>(splits, 1);
  }
  int64_t chunk = (n + splits - 1) / splits;
  chunk = (chunk + kExactStep - 1) / kExactStep * kExactStep;
  p.chunk = chunk;
  p.splits = (int)((n + chunk - 1) / chunk);
  return p;
}

hipError_t launch_exact(const ExactPlan& p, const void* x, int in_kind, int64_t m, int64_t n, int64_t ld, int64_t k,
                        uint64_t* part, const void* src, int src_dtype, int64_t src_ld, void* out_vals,
                        int32_t* out_idx, hipStream_t s) {
  switch (in_kind) {
    case IN_F32:
      return launch_exact_in<IN_F32>(p, x, m, n, ld, k, part, src, src_dtype, src_ld, out_vals, out_idx, s);
    case IN_BF16:
      return launch_exact_in<IN_BF16>(p, x, m, n, ld, k, part, src, src_dtype, src_ld, out_vals, out_idx, s);
    default:
      return launch_exact_in<IN_KEY64>(p, x, m, n, ld, k, part, src, src_dtype, src_ld, out_vals, out_idx, s);
  }
}

}  // namespace atopk
