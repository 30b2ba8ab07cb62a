// Candidate-set rerank decode.
//
// "Recall Before You Rank: Similarity-Guided Top-K Reuse ..." (fugumt page),
// Abstract: instead of scoring the query against the whole KV cache, the
// supports of the most similar cached queries are united with a recent
// window, and only that compact candidate set is reranked with exact
// current-query scores; the Top-K of it feeds softmax and value aggregation.
// This is that inner step (the cache of query / support pairs and the
// fallback policy stay with the caller).
//
// Two kernels:
//  1. (query head, split) workgroups: the candidates in the split's position
//     range -- the head's given indices inside [0, ctx) and the last `window`
//     positions -- made unique with an LDS bitmap over the range; their
//     scores: 16 lanes read one 256-byte key row with 16-byte loads and form
//     its dot product with the query (packed bf16 dot products, fp32
//     accumulation, DPP row sums), scaled in fp32; keys to the workspace
//     (and, when asked, each score to its position in a [heads, ctx] dump).
//     Splitting by position keeps every workgroup's bitmap small and puts
//     the whole chip on the gather when there are few heads.
//  2. one workgroup per query head: exact Top-K of its keys by (score desc,
//     index asc) -- radix select in LDS -- or the whole set when it holds
//     fewer than K keys; softmax over the selected scores (maximum
//     subtracted) and the weighted sum of their V rows, rounded to bf16.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace atopk {

namespace {

constexpr int kD = 128;
constexpr int kRT = 512;
constexpr int kGroups = kRT / 16;
constexpr int64_t kRerankTargetBlocks = 512;  // scoring workgroups to aim for

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b) {
  float acc = 0.0f;
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  return acc;
}

__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, true));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4e, 0xf, 0xf, true));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, true));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xf, 0xf, true));  // row_mirror
  return v;
}

// Kernel 1: workgroup (head, split) takes the candidates whose positions fall
// in the split's range [lo, hi) (so every position has one owner and the
// bitmap only covers the range), makes them unique, scores them and writes
// their keys to keys_out[(head * S + split) * cap ...], count to cnt_out.
__global__ __launch_bounds__(kRT) void rerank_score_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ K, int hq, int hkv, int ctx,
                                                          int64_t ctx_stride, float scale,
                                                          const int32_t* __restrict__ cand, int ncand,
                                                          int64_t cand_stride, int window, int range,
                                                          uint64_t* __restrict__ keys_out,
                                                          int* __restrict__ cnt_out, float* __restrict__ scores) {
  constexpr int T = kRT;
  __shared__ uint32_t list[kRerankMaxCand];
  __shared__ uint32_t bits[kRerankMaxCtx / 32];
  __shared__ int wsum[T / kWave];

  const int t = threadIdx.x;
  const int r_out = blockIdx.x;  // = bi * hq + h
  const int sp = blockIdx.y;
  const int S = gridDim.y;
  const int bi = r_out / hq;
  const int h = r_out - bi * hq;
  const int kvh = h / (hq / hkv);
  const int64_t bh = (int64_t)bi * hkv + kvh;
  const int lo = sp * range;
  const int hi = min(ctx, lo + range);

  // 1. the split's candidates, made unique: a bitmap over the range, then
  // its set bits listed in position order (thread t owns a run of words; a
  // block scan of the runs' counts gives each run its place)
  const int words = (max(hi - lo, 0) + 31) / 32;
  for (int i = t; i < words; i += T) bits[i] = 0;
  __syncthreads();
  const int32_t* cr = cand + (int64_t)r_out * cand_stride;
  const int total = ncand + window;
  for (int i = t; i < total; i += T) {
    const int j = i < ncand ? cr[i] : ctx - window + (i - ncand);
    if (j >= lo && j < hi) {
      const int jl = j - lo;
      atomicOr(&bits[jl >> 5], 1u << (jl & 31));
    }
  }
  __syncthreads();
  const int per = (words + T - 1) / T;
  const int w0 = min(words, t * per), w1 = min(words, w0 + per);
  int mine = 0;
  for (int w = w0; w < w1; ++w) mine += __popc(bits[w]);
  const int incl = wave_incl_scan(mine);
  if (lane_id() == kWave - 1) wsum[t / kWave] = incl;
  __syncthreads();
  int pos = incl - mine, nc = 0;
#pragma unroll
  for (int w = 0; w < T / kWave; ++w) {
    pos += w < t / kWave ? wsum[w] : 0;
    nc += wsum[w];  // <= ncand + window
  }
  for (int w = w0; w < w1; ++w) {
    uint32_t m = bits[w];
    while (m) {
      list[pos++] = (uint32_t)(lo + 32 * w + __builtin_ctz(m));
      m &= m - 1;
    }
  }
  __syncthreads();

  // 2. scores
  const int group = t >> 4;
  const int sub = t & 15;
  const uint4 qv = *reinterpret_cast<const uint4*>(q + (int64_t)r_out * kD + sub * 8);
  const uint16_t* kh = K + bh * ctx_stride * kD + sub * 8;
  uint64_t* dst = keys_out + ((int64_t)r_out * S + sp) * total;
  constexpr int U = 8;
  for (int i0 = 0; i0 < nc; i0 += kGroups * U) {
    uint32_t jj[U];
    uint4 kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + group + kGroups * u;
      jj[u] = i < nc ? list[i] : 0u;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + group + kGroups * u;
      kv[u] = i < nc ? *reinterpret_cast<const uint4*>(kh + (int64_t)jj[u] * kD) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + group + kGroups * u;
      const float sc = row16_sum(dot8_bf16(kv[u], qv)) * scale;
      if (i < nc && sub == 0) {
        dst[i] = make_key(ord_f32(__float_as_uint(sc)), jj[u]);
        if (scores != nullptr) scores[(int64_t)r_out * ctx + jj[u]] = sc;
      }
    }
  }
  if (t == 0) cnt_out[(int64_t)r_out * S + sp] = nc;
}

// Kernel 2, one workgroup per query head: the keys of its S splits, the
// exact Top-K of them (all of them when fewer), softmax and the weighted sum
// of the selected V rows.
constexpr int kST = 1024;              // select kernel threads
constexpr int kRerankStableMax = 1024;  // selections up to this size are summed in position order
constexpr int kSGroups = kST / 16;

__global__ __launch_bounds__(kST) void rerank_select_kernel(const uint64_t* __restrict__ keys_in,
                                                           const int* __restrict__ cnt_in, int S, int total,
                                                           int hq, int hkv, int64_t ctx_stride,
                                                           const uint16_t* __restrict__ V, int k_sel,
                                                           uint16_t* __restrict__ out, int32_t* __restrict__ sel_idx) {
  constexpr int T = kST;
  __shared__ alignas(16) uint64_t keys[kRerankMaxCand];
  __shared__ uint32_t hist[256 * kKthSub];
  __shared__ uint32_t ctl[8];
  __shared__ float w_lds[kSGroups];
  __shared__ float red[T / kWave];

  const int t = threadIdx.x;
  const int r_out = blockIdx.x;
  const int bi = r_out / hq;
  const int h = r_out - bi * hq;
  const int kvh = h / (hq / hkv);
  const int64_t bh = (int64_t)bi * hkv + kvh;

  int n = 0;
  for (int sp = 0; sp < S; ++sp) {
    const int c = cnt_in[(int64_t)r_out * S + sp];
    const uint64_t* src = keys_in + ((int64_t)r_out * S + sp) * total;
    for (int i = t; i < c; i += T) keys[n + i] = src[i];
    n += c;  // <= total <= kRerankMaxCand (positions are unique across splits)
  }
  __syncthreads();

  // 3. exact Top-K of the set (the whole set when it is smaller), kept in
  // position order: the keys arrive in position order (splits in order, each
  // split's list ascending) and the compaction keeps it, so the softmax-V
  // sums below run in one order whether or not the selection is written;
  // past kRerankStableMax keys the selection is sorted instead
  if (n > k_sel) {
    const uint64_t thr = block_kth_key_binned<T>(keys, n, k_sel, hist, ctl);
    n = block_compact_ge_stable<T, kRerankMaxCand / T>(keys, n, thr, hist);
  }
  const bool sorted = n > kRerankStableMax;
  const uint64_t* sel = sorted ? block_order_desc<T>(keys, n, kRerankMaxCand) : keys;
  if (sel_idx != nullptr) {
    int32_t* dst = sel_idx + (int64_t)r_out * k_sel;
    for (int i = n + t; i < k_sel; i += T) dst[i] = -1;
    if (sorted) {
      for (int i = t; i < n; i += T) dst[i] = (int32_t)key_idx(sel[i]);
    } else {
      // a key's place: the number of larger keys (the padding past n is read
      // by the count only)
      const int n16 = block_pad16(keys, n);
      __syncthreads();
      for (int c = t; c < n; c += T) dst[count_above16(keys, n16, keys[c])] = (int32_t)key_idx(keys[c]);
    }
  }

  // 4. softmax over the selected scores, weighted sum of their V rows
  float mx = -INFINITY;
  for (int i = t; i < n; i += T) mx = fmaxf(mx, key_value_f32(sel[i]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  if (lane_id() == 0) red[t / kWave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < T / kWave; ++w) mx = fmaxf(mx, red[w]);

  constexpr int U = 8;
  const int group = t >> 4;
  const int sub = t & 15;
  const uint16_t* vh = V + bh * ctx_stride * kD + sub * 8;
  float acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = 0.0f;
  float wsum = 0.0f;
  for (int i = group; i < n; i += kSGroups * U) {
    uint4 v[U];
    float w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ii = i + kSGroups * u;
      if (ii < n) {
        const uint64_t key = sel[ii];
        v[u] = *reinterpret_cast<const uint4*>(vh + (int64_t)key_idx(key) * kD);
        w[u] = expf(key_value_f32(key) - mx);
      } else {
        v[u] = make_uint4(0, 0, 0, 0);
        w[u] = 0.0f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t word[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        acc[2 * d] += w[u] * __uint_as_float(word[d] << 16);
        acc[2 * d + 1] += w[u] * __uint_as_float(word[d] & 0xffff0000u);
      }
      wsum += w[u];
    }
  }
  // the selected keys are no longer read: their LDS takes the partial sums
  __syncthreads();
  float (*acc_lds)[kD] = reinterpret_cast<float (*)[kD]>(keys);
  static_assert(sizeof(keys) >= sizeof(float) * kSGroups * kD, "the partial sums fit in the key array");
#pragma unroll
  for (int d = 0; d < 8; ++d) acc_lds[group][sub * 8 + d] = acc[d];
  if (sub == 0) w_lds[group] = wsum;
  __syncthreads();
  if (t < kD) {
    float s = 0.0f, wt = 0.0f;
#pragma unroll
    for (int gg = 0; gg < kSGroups; ++gg) {
      s += acc_lds[gg][t];
      wt += w_lds[gg];
    }
    out[(int64_t)r_out * kD + t] = f32_to_bf16_rne(s / wt);
  }
}

}  // namespace

int rerank_splits(int64_t batch, int64_t hq, int64_t ncand, int64_t window) {
  const int64_t heads = std::max<int64_t>(1, batch * hq);
  int64_t S = (kRerankTargetBlocks + heads - 1) / heads;
  S = std::min<int64_t>(S, std::max<int64_t>(1, (ncand + window) / 256));
  return (int)std::max<int64_t>(1, std::min<int64_t>(S, 8));
}

size_t rerank_ws_bytes(int64_t batch, int64_t hq, int64_t ncand, int64_t window) {
  const int64_t rows = batch * hq * rerank_splits(batch, hq, ncand, window);
  const size_t keys = ((size_t)rows * (ncand + window) * 8 + 255) / 256 * 256;
  return keys + (size_t)rows * 4;
}

hipError_t launch_rerank(const uint16_t* q, const uint16_t* K, const uint16_t* V, int64_t batch, int64_t hq,
                         int64_t hkv, int64_t ctx, int64_t ctx_stride, float scale, const int32_t* cand, int64_t ncand,
                         int64_t cand_stride, int64_t window, int64_t k_sel, uint16_t* out, int32_t* sel_idx,
                         float* scores, void* ws, hipStream_t s) {
  const int S = rerank_splits(batch, hq, ncand, window);
  const int64_t rows = batch * hq * S;
  const int64_t total = ncand + window;
  uint64_t* keys = static_cast<uint64_t*>(ws);
  int* cnt = reinterpret_cast<int*>(static_cast<uint8_t*>(ws) + ((size_t)rows * total * 8 + 255) / 256 * 256);
  int range = (int)((ctx + S - 1) / S);
  range = (range + 31) / 32 * 32;
  ATOPK_LAUNCH(rerank_score_kernel, dim3((unsigned)(batch * hq), (unsigned)S), dim3(kRT), 0, s, q, K, (int)hq,
                     (int)hkv, (int)ctx, ctx_stride, scale, cand, (int)ncand, cand_stride, (int)window, range, keys, cnt, scores);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  ATOPK_LAUNCH(rerank_select_kernel, dim3((unsigned)(batch * hq)), dim3(kST), 0, s, keys, cnt, S, (int)total,
                     (int)hq, (int)hkv, ctx_stride, V, (int)k_sel, out, sel_idx);
  return hipGetLastError();
}

}  // namespace atopk
