// Fused top-K sparse-attention decode: scoring + bucketed stage 1 in one
// pass over K, then per query head the merge, the final exact Top-K and the
// softmax / value aggregation over the selected keys.
//
// "Recall Before You Rank ..." (fugumt page), Abstract: every cached key is
// scored against the new query, the K best keys are kept, and the attention
// softmax and the weighted value sum run over those K keys only.
// "Approximate Top-k for Increased Parallelism" (Pith review page), "What
// carries the argument": the two-stage bucketed selection stands in for the
// single global Top-K.
//
// Kernel 1 (grid: context chunks or bucket ranges x (batch, KV head)): 16
// lanes read one 256-byte key row with 16-byte loads and form its dot
// products with the g query heads that share the KV head (packed bf16 dot
// products, fp32 accumulation, DPP row sums; query-head groups on the matrix
// cores).  Scores of 512 keys at a time are staged in LDS (double buffered,
// one LDS-only barrier per step, so K loads stay in flight); then every
// thread folds the staged scores of the (head, bucket) pairs it owns into
// sorted k_b-queues of 64-bit keys (order key of the score, then ~key index).
// In bucket-range mode a workgroup owns whole buckets over the whole context,
// so its lists are final.  A workgroup visits its steps in a rotated order,
// so that the workgroups in flight read different offsets of their ranges.
// Scores never go to HBM unless a debug dump is asked for.  Each workgroup
// writes its per-pair lists to the workspace -- except when one workgroup
// holds every candidate of its query head and the b*k_b candidates are the
// selection (b*k_b = K, one context chunk, one query head per KV head): then
// it runs kernel 2's softmax and value sum itself, right after its own
// scoring, while other workgroups still stream (no second launch; the same
// order of every floating-point sum, so the same output bits).
//
// With b = 0 kernel 1 only writes every score (the exact Top-K route selects
// on the written scores).
//
// Kernel 2 (grid: batch x query heads): merge the chunk lists of every
// bucket (bucket-range lists need none), take the exact Top-K of the b*k_b
// candidates in LDS (binned select, order-preserving compaction), then the
// softmax over the selected scores (maximum subtracted, fp32) and the
// weighted sum of the gathered V rows in rank order, rounded to bf16.
#include "common.h"
#include "launch.h"

namespace atopk {

namespace {

constexpr int kD = 128;
constexpr int kT1 = 256;
constexpr int kSub = 512;          // keys staged per step
constexpr int kSubPad = kSub + 1;  // LDS row pitch (heads on different banks)
constexpr int kMaxG = 8;
constexpr int kStableMax = 1024;  // selections up to this size are summed in compaction order
constexpr int kVGroups = 32;      // 16-lane groups of the finish's softmax-V sums (kernel 2's 512 threads / 16)
constexpr int kVU = 16;           // V rows in flight per lane group

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

// Staged scores of one step (G head rows of nk keys from key s0) to
// scores[row0 + g][s0 + li]: 16-byte stores when the rows allow them.
template <int T>
__device__ __forceinline__ void dump_scores(float* __restrict__ scores, int64_t row0, int ctx, int s0, int G, int nk,
                                            const float (*scb)[kSubPad]) {
  const int t = threadIdx.x;
  if (nk == kSub && (ctx & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0) {
    constexpr int Q = kSub / 4;
    for (int i = t; i < G * Q; i += T) {
      const int g = i / Q, li = (i - g * Q) * 4;
      const float4 v = make_float4(scb[g][li], scb[g][li + 1], scb[g][li + 2], scb[g][li + 3]);
      *reinterpret_cast<float4*>(scores + (row0 + g) * ctx + s0 + li) = v;
    }
  } else {
    for (int i = t; i < G * nk; i += T) {
      const int g = i / nk, li = i - g * nk;
      scores[(row0 + g) * ctx + s0 + li] = scb[g][li];
    }
  }
}

// Bucket-range mode: a workgroup owns the R buckets [r0, r0 + R) (R a power
// of two dividing kSub) of one (batch, KV head) over the whole context; step
// s stages the keys of sweeps m = s*M .. s*M + M - 1 (M = kSub / R): slot li
// is key m*b + r0 + (li mod R) of sweep m = s*M + li / R, live when it is
// below ctx.  A thread folds the slots of its (head, bucket) pair.
__device__ __forceinline__ int brange_key(int s, int li, int lgR, int b, int r0) {
  const int M = kSub >> lgR;
  return (s * M + (li >> lgR)) * b + r0 + (li & ((1 << lgR) - 1));
}

template <int T>
__device__ __forceinline__ void dump_scores_brange(float* __restrict__ scores, int64_t row0, int ctx, int s, int lgR,
                                                   int b, int r0, int G, const float (*scb)[kSubPad]) {
  for (int i = threadIdx.x; i < G * kSub; i += T) {
    const int g = i / kSub, li = i - g * kSub;
    const int j = brange_key(s, li, lgR, b, r0);
    if (j < ctx) scores[(row0 + g) * ctx + j] = scb[g][li];
  }
}

// Fold of one step in bucket-range mode: the thread's pair (g, rl) takes the
// slots li = mm*R + rl, mm = part, part + tpp, ... < M.
template <int KB>
__device__ __forceinline__ void fold_brange(uint64_t (&qq)[KB], const float (*scb)[kSubPad], int g, int rl, int part,
                                            int tpp, int s, int lgR, int b, int r0, int ctx) {
  const int M = kSub >> lgR;
  for (int mm = part; mm < M; mm += tpp) {
    const int li = (mm << lgR) + rl;
    const int j = brange_key(s, li, lgR, b, r0);
    if (j < ctx) queue_insert<KB>(qq, make_key(ord_f32(__float_as_uint(scb[g][li])), (uint32_t)j));
  }
}

// The tpp partial queues of a pair (consecutive lanes) merged into lane
// part 0's.
template <int KB>
__device__ __forceinline__ void merge_parts(uint64_t (&qq)[KB], int tpp) {
  for (int o = 1; o < tpp; o <<= 1) {
    uint64_t other[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) other[j] = shfl_xor_u64(qq[j], o);
    queue_merge<KB>(qq, other);
  }
}

// Kernel 2's work for a head whose candidates one workgroup of T threads holds
// (queue i of thread t: bucket t + T i) and whose b*k_b candidates are the
// selection: candidates to LDS in kernel 2's layout (slot r k_b + j), sel_idx
// by rank counting, the maximum score, then the weighted V sums in kernel 2's
// 32 lane groups (lane group g of this workgroup takes groups g, g + T/16, ...,
// each with kernel 2's row order and in-flight batch) and the same final sum
// over the groups.  `lds` holds at least 2 (kStableMax + 16) + 32 (kD + 1) + 16
// floats, 16-byte aligned; the caller's last reads of it are done.
template <int T, int PPT, int KB>
__device__ __forceinline__ void finish_in_place(const uint64_t (&qq)[PPT][KB], int b, int kb, float* lds,
                                                const uint16_t* __restrict__ vh, uint16_t* __restrict__ outp,
                                                int32_t* __restrict__ selp) {
  uint64_t* cand = reinterpret_cast<uint64_t*>(lds);
  float (*acc_lds)[kD] = reinterpret_cast<float (*)[kD]>(lds + 2 * (kStableMax + 16));
  float* w_lds = lds + 2 * (kStableMax + 16) + kVGroups * kD;
  float* red = w_lds + kVGroups;
  const int t = threadIdx.x;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int r = t + T * i;
    if (r < b) {
#pragma unroll
      for (int j = 0; j < KB; ++j)
        if (j < kb) cand[r * kb + j] = qq[i][j];
    }
  }
  __syncthreads();
  const int n = b * kb;
  if (selp != nullptr) {
    const int n16 = block_pad16(cand, n);
    __syncthreads();
    for (int c = t; c < n; c += T) selp[count_above16(cand, n16, cand[c])] = (int32_t)key_idx(cand[c]);
  }
  float mx = -INFINITY;
  for (int i = t; i < n; i += T) mx = fmaxf(mx, key_value_f32(cand[i]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  if (lane_id() == 0) red[t / kWave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < T / kWave; ++w) mx = fmaxf(mx, red[w]);
  const int sub = t & 15;
  const uint16_t* vrow = vh + sub * 8;
  for (int group = t >> 4; group < kVGroups; group += T / 16) {
    float acc[8];
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[d] = 0.0f;
    float wsum = 0.0f;
    for (int i = group; i < n; i += kVGroups * kVU) {
      uint4 v[kVU];
      float w[kVU];
#pragma unroll
      for (int u = 0; u < kVU; ++u) {
        const int ii = i + kVGroups * u;
        const uint64_t key = ii < n ? cand[ii] : 0;
        v[u] = key != 0 ? *reinterpret_cast<const uint4*>(vrow + (int64_t)key_idx(key) * kD) : make_uint4(0, 0, 0, 0);
        w[u] = key != 0 ? expf(key_value_f32(key) - mx) : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kVU; ++u) {
        const uint32_t word[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          acc[2 * d] += w[u] * __uint_as_float(word[d] << 16);
          acc[2 * d + 1] += w[u] * __uint_as_float(word[d] & 0xffff0000u);
        }
        wsum += w[u];
      }
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) acc_lds[group][sub * 8 + d] = acc[d];
    if (sub == 0) w_lds[group] = wsum;
  }
  __syncthreads();
  if (t < kD) {
    float sum = 0.0f, wt = 0.0f;
#pragma unroll
    for (int gg = 0; gg < kVGroups; ++gg) {
      sum += acc_lds[gg][t];
      wt += w_lds[gg];
    }
    outp[t] = f32_to_bf16_rne(sum / wt);
  }
}

// PPT (head, bucket) pairs per thread, KB queue slots per pair.  Context
// chunks (lgR < 0) or bucket ranges (lgR >= 0, tpp threads per pair), as in
// decode_select_mfma_kernel below.  finish != 0: the head's softmax-V in
// place (finish_in_place; one chunk, G = 1, b*kb = K <= kStableMax).
template <int PPT, int KB>
__global__ __launch_bounds__(kT1) void decode_select_kernel(const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ K, int hq, int hkv,
                                                           int ctx, int64_t ctx_stride, float scale, int b,
                                                           int64_t chunk, int nchunks, int lgR, int tpp,
                                                           uint64_t* __restrict__ partial,
                                                           float* __restrict__ scores, int finish, int kb,
                                                           const uint16_t* __restrict__ V,
                                                           uint16_t* __restrict__ out,
                                                           int32_t* __restrict__ sel_idx, int k_sel) {
  constexpr int U = 8;                 // keys in flight per 16-lane group
  constexpr int PASSES = kSub / (16 * U);
  __shared__ alignas(16) float sc[2][kMaxG][kSubPad];
  static_assert(sizeof(sc) >= sizeof(float) * (2 * (kStableMax + 16) + kVGroups * (kD + 1) + 16),
                "the in-place finish fits in the staged-score tile");

  const int t = threadIdx.x;
  const int sub = t & 15;   // 16-byte slice of a key row
  const int slot = t >> 4;  // key slot (16 per workgroup step)
  const int bh = blockIdx.y;
  const int bi = bh / hkv;
  const int h = bh - bi * hkv;
  const int G = hq / hkv;
  const int c = blockIdx.x;
  const bool brange = lgR >= 0;
  const int j0 = brange ? 0 : (int)(c * chunk);
  const int j1 = brange ? ctx : (int)min((int64_t)ctx, (int64_t)j0 + chunk);
  const int r0 = brange ? (c << lgR) : 0;
  const int nsteps = brange ? ((ctx + b - 1) / b + (kSub >> lgR) - 1) / (kSub >> lgR) : (j1 - j0 + kSub - 1) / kSub;

  uint4 qv[kMaxG];
#pragma unroll
  for (int g = 0; g < kMaxG; ++g)
    qv[g] = g < G ? *reinterpret_cast<const uint4*>(q + ((int64_t)(bi * hq + h * G + g) * kD + sub * 8))
                  : make_uint4(0, 0, 0, 0);
  const uint16_t* kh = K + (int64_t)bh * ctx_stride * kD + sub * 8;

  uint64_t qq[PPT][KB];
#pragma unroll
  for (int i = 0; i < PPT; ++i)
#pragma unroll
    for (int j = 0; j < KB; ++j) qq[i][j] = 0;
  const int npairs = G * (brange ? (1 << lgR) : b);
  const int bpr = brange ? t / tpp : 0;
  const int bpart = brange ? t - bpr * tpp : 0;

  // steps in rotated order: workgroups in flight together read different
  // offsets of their key ranges instead of one offset of every range (which
  // crowds a few HBM channels); the selection does not depend on the order
  const int rot = nsteps > 0 ? (int)((blockIdx.x + blockIdx.y) % (unsigned)nsteps) : 0;
  int buf = 0;
  for (int st0 = 0; st0 < nsteps; ++st0) {
    const int st = st0 + rot < nsteps ? st0 + rot : st0 + rot - nsteps;
    const int s0 = j0 + st * kSub;
    const int s1 = min(j1, s0 + kSub);
    // score the staged slots li = slot + 16 * (u + U * p)
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      uint4 kv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int li = slot + 16 * (u + U * p);
        const int jj = brange ? brange_key(st, li, lgR, b, r0) : s0 + li;
        kv[u] = jj < (brange ? ctx : s1) ? *reinterpret_cast<const uint4*>(kh + (int64_t)jj * kD)
                                         : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int li = slot + 16 * (u + U * p);
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) {
          if (g < G) {
            const float s = row16_sum(dot8_bf16(kv[u], qv[g])) * scale;
            if (sub == g) sc[buf][g][li] = s;
          }
        }
      }
    }
    lds_barrier();
    if (brange) {
      if (scores != nullptr) dump_scores_brange<kT1>(scores, (int64_t)(bi * hq + h * G), ctx, st, lgR, b, r0, G, sc[buf]);
      if (bpr < npairs) fold_brange<KB>(qq[0], sc[buf], bpr >> lgR, bpr & ((1 << lgR) - 1), bpart, tpp, st, lgR, b, r0, ctx);
    } else {
      const int nk = s1 - s0;
      if (scores != nullptr) dump_scores<kT1>(scores, (int64_t)(bi * hq + h * G), ctx, s0, G, nk, sc[buf]);
      // fold the staged scores of the owned (head, bucket) pairs: bucket r
      // holds keys j with j mod b == r
      const int rs = b > 0 ? s0 % b : 0;  // b == 0: scores only
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int pr = t + kT1 * i;
        if (pr < npairs) {
          const int g = pr / b;
          const int r = pr - g * b;
          for (int li = r - rs + (r < rs ? b : 0); li < nk; li += b) {
            const uint32_t bits = __float_as_uint(sc[buf][g][li]);
            queue_insert<KB>(qq[i], make_key(ord_f32(bits), (uint32_t)(s0 + li)));
          }
        }
      }
    }
    buf ^= 1;
  }
  if (brange) {
    merge_parts<KB>(qq[0], tpp);
    if (bpr < npairs && bpart == 0) {
      const int g = bpr >> lgR;
      const int r = r0 + (bpr & ((1 << lgR) - 1));
      uint64_t* dst = partial + (((int64_t)bh * G + g) * b + r) * KB;
#pragma unroll
      for (int j = 0; j < KB; ++j) dst[j] = qq[0][j];
    }
    return;
  }
  if (finish) {
    finish_in_place<kT1, PPT, KB>(qq, b, kb, &sc[0][0][0], V + (int64_t)bh * ctx_stride * kD,
                                  out + (int64_t)bh * kD, sel_idx != nullptr ? sel_idx + (int64_t)bh * k_sel : nullptr);
    return;
  }
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int pr = t + kT1 * i;
    if (pr < npairs) {
      const int g = pr / b;
      const int r = pr - g * b;
      uint64_t* dst = partial + ((((int64_t)bh * nchunks + c) * G + g) * b + r) * KB;
#pragma unroll
      for (int j = 0; j < KB; ++j) dst[j] = qq[i][j];
    }
  }
}

// Kernel 1 for query-head groups (G >= 2): the g dot products of a key are a
// dense contraction, Q [G x 128] times K^T [128 x keys], so they go to the
// matrix cores: v_mfma_f32_16x16x32_bf16 with the G query rows as A (rows G..15
// zero) and 16 keys as B; lane l holds A row l % 16 / B column l % 16 over
// k = 8 (l / 16) .. + 8 of each 32-wide k step, and gets C rows 4 (l / 16) + i,
// column l % 16.  A key row is read as 4 x 64 contiguous bytes per k step.
// 512 threads, so each thread owns half as many (head, bucket) queues.
constexpr int kT1M = 512;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int PPT, int KB>
__global__ __launch_bounds__(kT1M, 2) void decode_select_mfma_kernel(const uint16_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ K, int hq, int hkv,
                                                                 int ctx, int64_t ctx_stride, float scale, int b,
                                                                 int64_t chunk, int nchunks, int lgR, int tpp,
                                                                 uint64_t* __restrict__ partial,
                                                                 float* __restrict__ scores) {
  constexpr int NW = kT1M / kWave;  // 8 waves
  constexpr int GR = kSub / (NW * 16);  // 16-key groups per wave per step
  constexpr int KS = kD / 32;           // k steps of one MFMA each
  __shared__ float sc[2][kMaxG][kSubPad];

  const int t = threadIdx.x;
  const int lane = lane_id();
  const int wave = t / kWave;
  const int bh = blockIdx.y;
  const int bi = bh / hkv;
  const int h = bh - bi * hkv;
  const int G = hq / hkv;
  const int c = blockIdx.x;
  // context-chunk mode (lgR < 0): keys [j0, j1); bucket-range mode: buckets
  // [r0, r0 + 2^lgR) over the whole context, nsteps steps
  const bool brange = lgR >= 0;
  const int j0 = brange ? 0 : (int)(c * chunk);
  const int j1 = brange ? ctx : (int)min((int64_t)ctx, (int64_t)j0 + chunk);
  const int r0 = brange ? (c << lgR) : 0;
  const int nsteps = brange ? ((ctx + b - 1) / b + (kSub >> lgR) - 1) / (kSub >> lgR) : (j1 - j0 + kSub - 1) / kSub;

  const int col = lane & 15;         // A row (query head) / B column (key)
  const int kq = 8 * (lane >> 4);    // k offset inside a k step
  bf16x8_t qa[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 v = col < G ? *reinterpret_cast<const uint4*>(q + ((int64_t)(bi * hq + h * G + col) * kD + 32 * ks + kq))
                            : make_uint4(0, 0, 0, 0);
    qa[ks] = __builtin_bit_cast(bf16x8_t, v);
  }
  const uint16_t* kh = K + (int64_t)bh * ctx_stride * kD + kq;

  uint64_t qq[PPT][KB];
#pragma unroll
  for (int i = 0; i < PPT; ++i)
#pragma unroll
    for (int j = 0; j < KB; ++j) qq[i][j] = 0;
  const int npairs = G * (brange ? (1 << lgR) : b);

  // key of staged slot li in step st (ctx or beyond when it is not live)
  auto key_of = [&](int st, int li) {
    if (brange) return brange_key(st, li, lgR, b, r0);
    const int jj = j0 + st * kSub + li;
    return jj < j1 ? jj : ctx;
  };
  // 16-key groups through two register sets: a group's loads are in flight
  // while the previous group is on the matrix cores, and the next step's
  // first group loads during this step's fold (after the score stores, which
  // share the load counter).  Loads of keys that are not live are masked off.
  static_assert(GR == 4, "the group schedule below is written for 4 groups per wave and step");
  uint4 kv0[KS], kv1[KS];
  // steps in rotated order: workgroups in flight together read different
  // offsets of their key ranges instead of one offset of every range (which
  // crowds a few HBM channels); the selection does not depend on the order.
  // phys(nsteps) = nsteps: the prefetch past the last step loads nothing.
  const int rot = nsteps > 0 ? (int)((blockIdx.x + blockIdx.y) % (unsigned)nsteps) : 0;
  auto phys = [&](int st) { return st >= nsteps ? nsteps : (st + rot < nsteps ? st + rot : st + rot - nsteps); };
  auto load_grp = [&](uint4 (&kv)[KS], int st, int gi) {
    const int ps = phys(st);
    const int jj = ps < nsteps ? key_of(ps, (wave * GR + gi) * 16 + col) : ctx;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kv[ks] = jj < ctx ? *reinterpret_cast<const uint4*>(kh + (int64_t)jj * kD + 32 * ks) : make_uint4(0, 0, 0, 0);
  };
  int buf = 0;
  auto mma_grp = [&](const uint4 (&kv)[KS], int gi) {
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], __builtin_bit_cast(bf16x8_t, kv[ks]), acc, 0, 0, 0);
    const int li = (wave * GR + gi) * 16 + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * (lane >> 4) + i;
      if (g < G) sc[buf][g][li] = acc[i] * scale;
    }
  };
  // fold ownership: chunk mode, PPT pairs per thread; bucket-range mode,
  // tpp threads per pair (PPT == 1), each taking every tpp-th sweep
  const int bpr = brange ? t / tpp : 0;
  const int bpart = brange ? t - bpr * tpp : 0;
  load_grp(kv0, 0, 0);
  for (int st = 0; st < nsteps; ++st) {
    load_grp(kv1, st, 1);
    mma_grp(kv0, 0);
    load_grp(kv0, st, 2);
    mma_grp(kv1, 1);
    load_grp(kv1, st, 3);
    mma_grp(kv0, 2);
    mma_grp(kv1, 3);
    lds_barrier();
    const int ps = phys(st);
    if (brange) {
      if (scores != nullptr) dump_scores_brange<kT1M>(scores, (int64_t)(bi * hq + h * G), ctx, ps, lgR, b, r0, G, sc[buf]);
      load_grp(kv0, st + 1, 0);
      if (bpr < npairs) fold_brange<KB>(qq[0], sc[buf], bpr >> lgR, bpr & ((1 << lgR) - 1), bpart, tpp, ps, lgR, b, r0, ctx);
    } else {
      const int s0 = j0 + ps * kSub;
      const int nk = min(j1, s0 + kSub) - s0;
      if (scores != nullptr) dump_scores<kT1M>(scores, (int64_t)(bi * hq + h * G), ctx, s0, G, nk, sc[buf]);
      load_grp(kv0, st + 1, 0);
      // fold the staged scores of the owned (head, bucket) pairs: bucket r
      // holds keys j with j mod b == r
      const int rs = b > 0 ? s0 % b : 0;  // b == 0: scores only
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int pr = t + kT1M * i;
        if (pr < npairs) {
          const int g = pr / b;
          const int r = pr - g * b;
          for (int li = r - rs + (r < rs ? b : 0); li < nk; li += b) {
            const uint32_t bits = __float_as_uint(sc[buf][g][li]);
            queue_insert<KB>(qq[i], make_key(ord_f32(bits), (uint32_t)(s0 + li)));
          }
        }
      }
    }
    buf ^= 1;
  }
  if (brange) {
    merge_parts<KB>(qq[0], tpp);
    if (bpr < npairs && bpart == 0) {
      const int g = bpr >> lgR;
      const int r = r0 + (bpr & ((1 << lgR) - 1));
      uint64_t* dst = partial + (((int64_t)bh * G + g) * b + r) * KB;
#pragma unroll
      for (int j = 0; j < KB; ++j) dst[j] = qq[0][j];
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < PPT; ++i) {
    const int pr = t + kT1M * i;
    if (pr < npairs) {
      const int g = pr / b;
      const int r = pr - g * b;
      uint64_t* dst = partial + ((((int64_t)bh * nchunks + c) * G + g) * b + r) * KB;
#pragma unroll
      for (int j = 0; j < KB; ++j) dst[j] = qq[i][j];
    }
  }
}

constexpr int kT2 = 512;
constexpr int kMaxCand = 8192;
static_assert(kVGroups == kT2 / 16, "kernel 2 sums in one group per 16 of its threads");

constexpr int kFlagMax = 256;  // flagged buckets rescanned in LDS; more take the full-row fallback

__device__ __noinline__ void decode_row_fallback(const float* srow, int ctx, int k, uint64_t* cand, uint32_t* hist,
                                                 uint32_t* ctl) {
  block_row_topk<kT2>([&](int i) { return ord_f32(__float_as_uint(srow[i])); }, ctx, k, cand, hist, ctl);
}

// For a rescan that overflows (one query head per KV head): the workgroup
// recomputes every score of its head exactly as the scoring kernel does
// (16-lane groups) into its own row `srow` of the workspace, then selects
// from that row.
__device__ __noinline__ void decode_fill_scores(const uint16_t* qrow, const uint16_t* krow, float scale, int ctx,
                                                float* srow) {
  const int t = threadIdx.x;
  const int grp = t >> 4, sub = t & 15;
  const uint4 qv = *reinterpret_cast<const uint4*>(qrow + sub * 8);
  for (int j0 = 0; j0 < ctx; j0 += kVGroups) {
    const int j = j0 + grp;
    const uint4 kv = j < ctx ? *reinterpret_cast<const uint4*>(krow + (int64_t)j * kD + sub * 8) : make_uint4(0, 0, 0, 0);
    const float sc = row16_sum(dot8_bf16(kv, qv)) * scale;
    if (sub == 0 && j < ctx) srow[j] = sc;
  }
  __threadfence_block();
  __syncthreads();
}

// Matrix-core counterpart of decode_fill_scores for query-head groups: the
// scoring kernel's own v_mfma_f32_16x16x32_bf16 chain (the G query rows of
// the KV head as A rows 0..G-1, 16 keys as B, the k steps in order from a zero
// accumulator, then the scaling), row g of the result to `srow`.
__device__ __noinline__ void decode_fill_scores_mfma(const uint16_t* qg, int G, int g, const uint16_t* kh, float scale,
                                                     int ctx, float* srow) {
  constexpr int KS = kD / 32;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int col = lane & 15, kq = 8 * (lane >> 4);
  bf16x8_t qa[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qa[ks] = __builtin_bit_cast(bf16x8_t, col < G ? *reinterpret_cast<const uint4*>(qg + (int64_t)col * kD + 32 * ks + kq)
                                                  : make_uint4(0, 0, 0, 0));
  const bool mine = (lane >> 4) == (g >> 2);  // the lanes that hold C row g
  for (int j0 = 0; j0 < ctx; j0 += kT2 / kWave * 16) {
    const int j = j0 + wave * 16 + col;
    uint4 kv[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kv[ks] = j < ctx ? *reinterpret_cast<const uint4*>(kh + (int64_t)j * kD + 32 * ks + kq) : make_uint4(0, 0, 0, 0);
    f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], __builtin_bit_cast(bf16x8_t, kv[ks]), acc, 0, 0, 0);
    if (mine && j < ctx) srow[j] = acc[g & 3] * scale;
  }
  __threadfence_block();
  __syncthreads();
}

// Keys that a rescan keeps go after the k_sel selected ones (ctl[6] counts
// them; slots past the LDS array are dropped and the count reports the
// overflow).  Called by every lane of the wave.
__device__ __forceinline__ void append_kept(bool keep, uint64_t key, int k_sel, uint64_t* cand, uint32_t* ctl) {
  const uint64_t msk = __ballot(keep);
  if (msk) {
    uint32_t pos = 0;
    if (lane_id() == 0) pos = atomicAdd(&ctl[6], (uint32_t)__popcll(msk));
    pos = wave_lane0(pos);
    const uint32_t slot = (uint32_t)k_sel + pos + lanes_below(msk);
    if (keep && slot < (uint32_t)kMaxCand) cand[slot] = key;
  }
}

// Slot sl of the flagged buckets' keys: bucket f = sl / S, key
// r_f + (sl % S) * b with S = ceil(ctx / b); ctx for a slot past the list or
// past the context.
__device__ __forceinline__ int flagged_key(int sl, int total, int S, int b, const uint32_t* flg_r, int* f) {
  *f = sl < total ? sl / S : 0;
  return sl < total ? (int)flg_r[*f] + (sl - *f * S) * b : INT32_MAX;
}

// Rescan of the flagged buckets with one query head per KV head: 16-lane
// groups recompute the scores with the scoring kernel's arithmetic (packed
// bf16 dot products, the same row sum, the same scaling), U keys per group
// and step so that their loads are in flight together.
__device__ __forceinline__ void decode_rescan_dot(const uint16_t* qrow, const uint16_t* kh, float scale, int ctx, int b,
                                                  int nflag, const uint32_t* flg_r, const uint64_t* flg_c,
                                                  uint64_t thr, int k_sel, uint64_t* cand, uint32_t* ctl) {
  constexpr int U = 4;
  const int t = threadIdx.x;
  const int grp = t >> 4, sub = t & 15;
  const uint4 qv = *reinterpret_cast<const uint4*>(qrow + sub * 8);
  const int S = (ctx + b - 1) / b;
  const int total = nflag * S;
  for (int s0 = 0; s0 < total; s0 += kVGroups * U) {
    int jj[U], ff[U];
    uint4 kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      jj[u] = flagged_key(s0 + u * kVGroups + grp, total, S, b, flg_r, &ff[u]);
      kv[u] = jj[u] < ctx ? *reinterpret_cast<const uint4*>(kh + (int64_t)jj[u] * kD + sub * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = jj[u];
      const float sc = row16_sum(dot8_bf16(kv[u], qv)) * scale;
      const uint64_t key = j < ctx ? make_key(ord_f32(__float_as_uint(sc)), (uint32_t)j) : 0;
      append_kept(sub == 0 && j < ctx && key > thr && key < flg_c[ff[u]], key, k_sel, cand, ctl);
    }
  }
}

// Rescan of the flagged buckets for query-head groups: every wave recomputes
// 16 keys per MFMA chain, two chains per step, with the scoring kernel's
// operands in the same places (the G query rows as A rows 0..G-1, the k
// steps in order from a zero accumulator, then the scaling).  A result
// element of v_mfma depends only on its own A row, B column and accumulator
// element, so the recomputed scores are the ones that were ranked, wherever
// a key sits among the 16 columns.
__device__ __forceinline__ void decode_rescan_mfma(const uint16_t* qg, int G, int g, const uint16_t* kh, float scale,
                                                int ctx, int b, int nflag, const uint32_t* flg_r,
                                                const uint64_t* flg_c, uint64_t thr, int k_sel, uint64_t* cand,
                                                uint32_t* ctl) {
  constexpr int KS = kD / 32;
  constexpr int GR = 2;
  constexpr int STEP = kT2 / kWave * 16 * GR;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int col = lane & 15, kq = 8 * (lane >> 4);
  bf16x8_t qa[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qa[ks] = __builtin_bit_cast(bf16x8_t, col < G ? *reinterpret_cast<const uint4*>(qg + (int64_t)col * kD + 32 * ks + kq)
                                                  : make_uint4(0, 0, 0, 0));
  const bool mine = (lane >> 4) == (g >> 2);
  const int S = (ctx + b - 1) / b;
  const int total = nflag * S;
  for (int s0 = 0; s0 < total; s0 += STEP) {
    uint4 kv[GR][KS];
    int jj[GR], ff[GR];
#pragma unroll
    for (int gi = 0; gi < GR; ++gi) {
      jj[gi] = flagged_key(s0 + (wave * GR + gi) * 16 + col, total, S, b, flg_r, &ff[gi]);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kv[gi][ks] = jj[gi] < ctx ? *reinterpret_cast<const uint4*>(kh + (int64_t)jj[gi] * kD + 32 * ks + kq)
                                  : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int gi = 0; gi < GR; ++gi) {
      f32x4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[ks], __builtin_bit_cast(bf16x8_t, kv[gi][ks]), acc, 0, 0, 0);
      const int j = jj[gi];
      const float sc = acc[g & 3] * scale;
      const uint64_t key = j < ctx ? make_key(ord_f32(__float_as_uint(sc)), (uint32_t)j) : 0;
      append_kept(mine && j < ctx && key > thr && key < flg_c[ff[gi]], key, k_sel, cand, ctl);
    }
  }
}

// certify != 0 makes the Top-K exact over every score of the head: with T
// the k_sel-th candidate key, a bucket that kept k_b keys all >= T may hide
// more of the Top-K (any missing key beats T); those buckets are rescanned
// for keys between T and their k_b-th kept key, and the Top-K of the
// enlarged pool is the exact one.  The rescan recomputes the flagged
// buckets' scores from q and K with the scoring kernel's own arithmetic, so
// they are bit-identical to the ones that were ranked: certify == 1 (query-
// head groups) on the matrix cores, certify == 2 (one query head per KV head)
// with the 16-lane dot products.  Past kFlagMax flagged buckets, or past the
// LDS candidate array, the workgroup recomputes every score of its head into
// its row of `scores` ([B*Hq, ctx] workspace) and selects from that row.
// MP: register slots per thread of the compaction of the b*kb <= kT2 * MP
// candidates; the certification's second compaction (after a rescan) keeps
// kMaxCand / kT2.
template <int KB, int MP>
__global__ __launch_bounds__(kT2) __attribute__((amdgpu_waves_per_eu(4))) void decode_finish_kernel(const uint64_t* __restrict__ partial, int nchunks, int hq,
                                                           int hkv, int b, int kb, int k_sel,
                                                           const uint16_t* __restrict__ V, int64_t ctx_stride,
                                                           uint16_t* __restrict__ out, int32_t* __restrict__ sel_idx,
                                                           int certify, float* __restrict__ scores, int ctx,
                                                           const uint16_t* __restrict__ q,
                                                           const uint16_t* __restrict__ K, float scale) {
  constexpr int T = kT2;
  __shared__ alignas(16) uint64_t cand[kMaxCand];
  __shared__ uint32_t hist[256 * kKthSub];
  __shared__ uint32_t ctl[8];
  __shared__ uint32_t flg_r[kFlagMax];
  __shared__ uint64_t flg_c[kFlagMax];
  __shared__ float w_lds[kVGroups];
  __shared__ float red[T / kWave];

  const int t = threadIdx.x;
  const int G = hq / hkv;
  // r_out = bi * hq + hh.  Workgroups are dealt to the 8 XCDs round-robin by
  // id: the G query heads of one KV head go to one XCD, where the V rows
  // they share meet in one L2.
  int r_out = blockIdx.x;
  if (G > 1 && gridDim.x % (8 * G) == 0) {
    const int x = blockIdx.x & 7, kk = blockIdx.x >> 3;
    r_out = ((kk / G) * 8 + x) * G + kk % G;
  }
  const int bi = r_out / hq;
  const int hh = r_out - bi * hq;
  const int kvh = hh / G;
  const int g = hh - kvh * G;
  const int bh = bi * hkv + kvh;

  // merge the chunk lists of every bucket, every list of a batch in flight
  // at once (lists past the last chunk read as empty and change nothing)
  constexpr int kLB = KB >= 16 ? 2 : 32 / KB;  // lists per batch: 32 keys in registers
  for (int r = t; r < b; r += T) {
    const uint64_t* src = partial + ((((int64_t)bh * nchunks) * G + g) * b + r) * KB;
    const int64_t cstride = (int64_t)G * b * KB;
    uint64_t a[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) a[j] = 0;
    for (int c0 = 0; c0 < nchunks; c0 += kLB) {
      uint64_t o[kLB][KB];
#pragma unroll
      for (int u = 0; u < kLB; ++u) {
        const bool live = c0 + u < nchunks;
        const uint64_t* p = src + (int64_t)(c0 + u) * cstride;
        if constexpr (KB >= 2) {
#pragma unroll
          for (int j = 0; j < KB; j += 2) {
            const uint4 w = live ? *reinterpret_cast<const uint4*>(p + j) : make_uint4(0, 0, 0, 0);
            o[u][j] = ((uint64_t)w.y << 32) | w.x;
            o[u][j + 1] = ((uint64_t)w.w << 32) | w.z;
          }
        } else {
          o[u][0] = live ? p[0] : 0;
        }
      }
#pragma unroll
      for (int u = 0; u < kLB; ++u) queue_merge<KB>(a, o[u]);
    }
#pragma unroll
    for (int j = 0; j < KB; ++j)
      if (j < kb) cand[r * kb + j] = a[j];
  }
  __syncthreads();
  int n = b * kb;
  // Order of the selection for the softmax-V sums (and its ranks for
  // sel_idx): the stable compaction's order -- a function of the candidates
  // alone, a rescan's keys put in descending order behind them -- or, after a
  // fallback (which collects keys in arrival order), a rescan of more than T
  // keys, and for selections above kStableMax keys, descending order.
  bool sorted = false;
  if (certify) {
    const uint64_t thr = block_kth_key_binned<T>(cand, n, k_sel, hist, ctl);
    if (t == 0) {
      ctl[5] = 0;
      ctl[6] = 0;
    }
    __syncthreads();
    for (int r = t; r < b; r += T) {
      const uint64_t c = cand[r * kb + kb - 1];
      if ((ctx - r + b - 1) / b > kb && c >= thr) {
        const uint32_t f = atomicAdd(&ctl[5], 1u);
        if (f < (uint32_t)kFlagMax) {
          flg_r[f] = (uint32_t)r;
          flg_c[f] = c;
        }
      }
    }
    n = block_compact_ge_stable<T, MP>(cand, n, thr, hist);  // k_sel keys
    const int nflag = (int)ctl[5];
    if (nflag > 0) {
      bool overflow = nflag > kFlagMax;
      const uint16_t* kh = K + (int64_t)bh * ctx_stride * kD;
      const uint16_t* qg = q + (int64_t)(r_out - g) * kD;  // the G query rows of the KV head
      if (!overflow) {
        if (certify == 1)
          decode_rescan_mfma(qg, G, g, kh, scale, ctx, b, nflag, flg_r, flg_c, thr, k_sel, cand, ctl);
        else
          decode_rescan_dot(q + (int64_t)r_out * kD, kh, scale, ctx, b, nflag, flg_r, flg_c, thr, k_sel, cand, ctl);
        __syncthreads();
        const int extra = (int)ctl[6];
        __syncthreads();
        overflow = k_sel + extra > kMaxCand;
        if (!overflow && extra > 0) {
          n = k_sel + extra;
          // The rescan appended its keys in the order its waves' atomics ran;
          // put them in descending order so that the list -- the selected
          // keys in their stable order, then these -- is one function of the
          // scores and the compaction below keeps a canonical order.  More
          // than T of them: the selection is sorted instead.
          if (extra <= T) {
            uint64_t key = 0;
            int rank = 0;
            if (t < extra) {
              key = cand[k_sel + t];
              for (int j = 0; j < extra; ++j) rank += cand[k_sel + j] > key ? 1 : 0;
            }
            __syncthreads();
            if (t < extra) cand[k_sel + rank] = key;
            __syncthreads();
          } else {
            sorted = true;
          }
          const uint64_t thr2 = block_kth_key<T, kKthSub>(cand, n, k_sel, hist, ctl);
          n = block_compact_ge_stable<T, kMaxCand / T>(cand, n, thr2, hist);
        }
      }
      if (overflow) {
        sorted = true;
        float* row = scores + (int64_t)r_out * ctx;
        if (certify == 1)
          decode_fill_scores_mfma(qg, G, g, kh, scale, ctx, row);
        else
          decode_fill_scores(q + (int64_t)r_out * kD, kh, scale, ctx, row);
        decode_row_fallback(row, ctx, k_sel, cand, hist, ctl);
        n = k_sel;
      }
    }
  } else if (n > k_sel) {
    const uint64_t thr = block_kth_key_binned<T>(cand, n, k_sel, hist, ctl);
    n = block_compact_ge_stable<T, MP>(cand, n, thr, hist);
  }
  sorted = sorted || n > kStableMax;
  const uint64_t* sel = sorted ? block_order_desc<T>(cand, n, kMaxCand) : cand;
  if (sel_idx != nullptr) {
    int32_t* dst = sel_idx + (int64_t)r_out * k_sel;
    if (sorted) {
      for (int i = t; i < n; i += T) dst[i] = (int32_t)key_idx(sel[i]);
    } else {
      // a key's place in descending order: the number of larger keys (the
      // padding past n is read by the count only)
      const int n16 = block_pad16(cand, n);
      __syncthreads();
      for (int c = t; c < n; c += T) dst[count_above16(cand, n16, cand[c])] = (int32_t)key_idx(cand[c]);
    }
  }

  // softmax over the selected scores, weighted sum of their V rows
  float mx = -INFINITY;
  for (int i = t; i < n; i += T) mx = fmaxf(mx, key_value_f32(sel[i]));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  if (lane_id() == 0) red[t / kWave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < T / kWave; ++w) mx = fmaxf(mx, red[w]);

  // lane group `group` takes rows group, group + kVGroups, ...; all U rows of
  // a batch are loaded before any is summed
  constexpr int U = 16;
  const int group = t >> 4;
  const int sub = t & 15;
  const uint16_t* vh = V + (int64_t)bh * ctx_stride * kD + sub * 8;
  float acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = 0.0f;
  float wsum = 0.0f;
  for (int i = group; i < n; i += kVGroups * U) {
    uint4 v[U];
    float w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ii = i + kVGroups * u;
      const uint64_t key = ii < n ? sel[ii] : 0;
      v[u] = key != 0 ? *reinterpret_cast<const uint4*>(vh + (int64_t)key_idx(key) * kD) : make_uint4(0, 0, 0, 0);
      w[u] = key != 0 ? expf(key_value_f32(key) - mx) : 0.0f;
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
  float (*acc_lds)[kD] = reinterpret_cast<float (*)[kD]>(cand);
  static_assert(sizeof(cand) >= sizeof(float) * kVGroups * kD, "the partial sums fit in the key array");
#pragma unroll
  for (int d = 0; d < 8; ++d) acc_lds[group][sub * 8 + d] = acc[d];
  if (sub == 0) w_lds[group] = wsum;
  __syncthreads();
  if (t < kD) {
    float s = 0.0f, wt = 0.0f;
#pragma unroll
    for (int gg = 0; gg < kVGroups; ++gg) {
      s += acc_lds[gg][t];
      wt += w_lds[gg];
    }
    out[(int64_t)r_out * kD + t] = f32_to_bf16_rne(s / wt);
  }
}

int kb_pow2(int64_t kb) {
  int v = 1;
  while (v < kb) v <<= 1;
  return v;
}

}  // namespace

DecodePlan plan_decode(int64_t batch, int64_t hq, int64_t hkv, int64_t ctx, int64_t k_sel, int64_t b, int64_t kb) {
  DecodePlan p{};
  const int64_t g = hq / hkv;
  const int kbs = kb_pow2(kb);
  p.mfma = g >= 2;  // the G dot products of a key on the matrix cores
  const int threads = p.mfma ? kT1M : kT1;
  int ppt = 1;
  while ((int64_t)ppt * threads < g * b) ppt *= 2;
  p.ppt = ppt;
  p.fused = !(b == 1 && kb == k_sel) && ppt <= 8 && (int64_t)ppt * kbs <= 64 && b * kb <= kMaxCand && kbs <= 16;
  // chunks: enough workgroups to fill the chip, long enough that the lists
  // written per chunk stay small next to the K bytes read.  The matrix-core
  // kernel streams as fast with one 512-thread workgroup per CU as with two,
  // and half the chunks halve the lists the finish merges (gqa-128k: 215 ->
  // 211 us per call).
  const int64_t heads = batch * hkv;
  const int64_t target = p.mfma ? 256 : 512;  // workgroups
  int64_t nchunks = std::max<int64_t>(1, (target + heads - 1) / std::max<int64_t>(heads, 1));
  nchunks = std::min<int64_t>(nchunks, std::max<int64_t>(1, ctx / 4096));
  int64_t chunk = (ctx + nchunks - 1) / nchunks;
  chunk = (chunk + kSub - 1) / kSub * kSub;
  p.chunk = chunk;
  p.nchunks = (int)((ctx + chunk - 1) / chunk);
  p.nsplit = p.nchunks;
  p.lgR = -1;
  p.tpp = 1;
  // Bucket-range mode: with b a power of two, split the buckets instead of
  // the context -- workgroup c owns buckets [c*R, c*R + R) over every sweep
  // of the keys -- so each workgroup's lists are final and the finish merges
  // nothing.  Needs runs of R >= 16 consecutive keys (whole 16-key groups)
  // and at most one (head, bucket) pair per thread.
  // Its lists do not grow with the number of workgroups, so it takes up to
  // two scoring workgroups per CU (512) for more loads in flight, as long as
  // the ranges keep 32 buckets (16-key runs measured slower).
  if (p.fused && p.nchunks >= 2 && b >= 16 && (b & (b - 1)) == 0) {
    const int64_t want = (512 + heads - 1) / heads;
    int64_t ns = 1;
    while (ns < p.nchunks) ns <<= 1;
    while (ns < want && b / (2 * ns) >= 32) ns <<= 1;
    while (ns <= b / 16 && g * (b / ns) > threads) ns <<= 1;
    if (ns <= b / 16 && b / ns <= kSub) {
      const int64_t R = b / ns;
      int lg = 0;
      while ((1LL << lg) < R) ++lg;
      int tpp = 1;
      while (g * R * tpp * 2 <= threads && tpp * 2 <= kSub / R && tpp * 2 <= kWave) tpp *= 2;
      p.lgR = lg;
      p.tpp = tpp;
      p.ppt = 1;
      p.nsplit = (int)ns;
      p.nchunks = 1;
    }
  }
  p.partial_bytes = (size_t)heads * p.nchunks * g * b * kbs * 8;
  return p;
}

hipError_t launch_decode_scores(const uint16_t* q, const uint16_t* K, int64_t batch, int64_t hq, int64_t hkv,
                                int64_t ctx, int64_t ctx_stride, float scale, float* scores, hipStream_t s) {
  // the scoring kernels with no bucket (b = 0): every score to `scores`
  const DecodePlan p = plan_decode(batch, hq, hkv, ctx, 1, 1, 1);  // context chunks (b = 1)
  dim3 g1((unsigned)p.nchunks, (unsigned)(batch * hkv));
  if (p.mfma)
    ATOPK_LAUNCH((decode_select_mfma_kernel<1, 1>), g1, dim3(kT1M), 0, s, q, K, (int)hq, (int)hkv, (int)ctx,
                       ctx_stride, scale, 0, p.chunk, p.nchunks, -1, 1, nullptr, scores);
  else
    ATOPK_LAUNCH((decode_select_kernel<1, 1>), g1, dim3(kT1), 0, s, q, K, (int)hq, (int)hkv, (int)ctx,
                       ctx_stride, scale, 0, p.chunk, p.nchunks, -1, 1, nullptr, scores, 0, 1, nullptr, nullptr,
                       nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_decode_fused(const DecodePlan& p, const uint16_t* q, const uint16_t* K, const uint16_t* V,
                               int64_t batch, int64_t hq, int64_t hkv, int64_t ctx, int64_t ctx_stride, float scale,
                               int64_t k_sel, int64_t b, int64_t kb, uint64_t* partial, uint16_t* out,
                               int32_t* sel_idx, float* scores, int certify, float* cert_buf, hipStream_t s) {
  if (certify && cert_buf == nullptr) return hipErrorInvalidValue;
  if (certify && certify != (p.mfma ? 1 : 2)) return hipErrorInvalidValue;  // the rescan repeats kernel 1's arithmetic
  const int kbs = kb_pow2(kb);
  dim3 g1((unsigned)p.nsplit, (unsigned)(batch * hkv));
  // one workgroup holds every candidate of its head and they are the
  // selection: the scoring kernel finishes the head itself
  const int in_place = !p.mfma && p.lgR < 0 && p.nchunks == 1 && hq == hkv && b * kb == k_sel && certify == 0 &&
                       k_sel <= kStableMax;
#define ATOPK_D1(P, KBV)                                                                                            \
  if (p.ppt == P && kbs == KBV) {                                                                                   \
    if (p.mfma)                                                                                                     \
      ATOPK_LAUNCH((decode_select_mfma_kernel<P, KBV>), g1, dim3(kT1M), 0, s, q, K, (int)hq, (int)hkv,         \
                         (int)ctx, ctx_stride, scale, (int)b, p.chunk, p.nchunks, p.lgR, p.tpp, partial, scores);    \
    else                                                                                                            \
      ATOPK_LAUNCH((decode_select_kernel<P, KBV>), g1, dim3(kT1), 0, s, q, K, (int)hq, (int)hkv, (int)ctx,     \
                         ctx_stride, scale, (int)b, p.chunk, p.nchunks, p.lgR, p.tpp, partial, scores, in_place,     \
                         (int)kb, V, out, sel_idx, (int)k_sel);                                                     \
  } else
  ATOPK_D1(1, 1) ATOPK_D1(1, 2) ATOPK_D1(1, 4) ATOPK_D1(1, 8) ATOPK_D1(1, 16)
  ATOPK_D1(2, 1) ATOPK_D1(2, 2) ATOPK_D1(2, 4) ATOPK_D1(2, 8) ATOPK_D1(2, 16)
  ATOPK_D1(4, 1) ATOPK_D1(4, 2) ATOPK_D1(4, 4) ATOPK_D1(4, 8) ATOPK_D1(4, 16)
  ATOPK_D1(8, 1) ATOPK_D1(8, 2) ATOPK_D1(8, 4) ATOPK_D1(8, 8)
  { return hipErrorInvalidValue; }
#undef ATOPK_D1
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || in_place) return e;
  dim3 g2((unsigned)(batch * hq));
#define ATOPK_D2(KBV)                                                                                              \
  case KBV:                                                                                                        \
    if (b * kb <= (int64_t)kT2 * 4)                                                                                \
      ATOPK_LAUNCH((decode_finish_kernel<KBV, 4>), g2, dim3(kT2), 0, s, partial, p.nchunks, (int)hq, (int)hkv,    \
                   (int)b, (int)kb, (int)k_sel, V, ctx_stride, out, sel_idx, certify, cert_buf, (int)ctx, q, K,     \
                   scale);                                                                                         \
    else                                                                                                           \
      ATOPK_LAUNCH((decode_finish_kernel<KBV, kMaxCand / kT2>), g2, dim3(kT2), 0, s, partial, p.nchunks, (int)hq,  \
                   (int)hkv, (int)b, (int)kb, (int)k_sel, V, ctx_stride, out, sel_idx, certify, cert_buf, (int)ctx, \
                   q, K, scale);                                                                                   \
    break;
  switch (kbs) {
    ATOPK_D2(1) ATOPK_D2(2) ATOPK_D2(4) ATOPK_D2(8) ATOPK_D2(16)
    default: return hipErrorInvalidValue;
  }
#undef ATOPK_D2
  return hipGetLastError();
}

}  // namespace atopk
