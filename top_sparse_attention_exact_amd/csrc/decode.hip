// Top-K sparse-attention decode: scoring against the whole KV cache and the
// softmax / value aggregation over the selected keys.
//
// "Recall Before You Rank ..." (fugumt page), Abstract: the current query is
// scored against the full KV cache, a global Top-K is taken, and softmax and
// value aggregation run over only that subset.  STARC (Pith review page),
// Figure 3 caption: q in R^{1 x d_h}, K, V in R^{L x d_h} per head.
//
// Scoring is a matrix-vector product per KV head: each 256-byte key row is
// read once with 16-byte loads by 16 lanes (8 bf16 each), multiplied against
// the g = hq/hkv query heads that share it with packed bf16 dot products
// accumulated in fp32, and summed across the 16 lanes with DPP row
// operations.  It is bound by HBM bandwidth, not by the ALUs or the matrix
// cores, so no MFMA is used.
#include "common.h"
#include "launch.h"

namespace atopk {

namespace {

constexpr int kD = 128;
constexpr int kDecThreads = 256;
constexpr int kKeysPerBlock = 2048;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  return acc;
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xb1, 0xf, 0xf, true));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4e, 0xf, 0xf, true));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, true));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x140, 0xf, 0xf, true));  // row_mirror
  return v;
}

template <int G>
__global__ __launch_bounds__(kDecThreads) void decode_scores_kernel(const uint16_t* __restrict__ q,
                                                                   const uint16_t* __restrict__ K, int hq, int hkv,
                                                                   int ctx, int64_t ctx_stride, float scale,
                                                                   float* __restrict__ scores) {
  constexpr int U = 8;
  const int t = threadIdx.x;
  const int sub = t & 15;   // 16-byte slice of the key row
  const int slot = t >> 4;  // 16 keys in flight per block step
  const int bh = blockIdx.y;
  const int bi = bh / hkv;
  const int h = bh - bi * hkv;
  const int j0 = blockIdx.x * kKeysPerBlock;
  const int j1 = min(ctx, j0 + kKeysPerBlock);

  uint4 qv[G];
#pragma unroll
  for (int g = 0; g < G; ++g)
    qv[g] = *reinterpret_cast<const uint4*>(q + ((int64_t)(bi * hq + h * G + g) * kD + sub * 8));
  const uint16_t* kh = K + (int64_t)bh * ctx_stride * kD + sub * 8;
  float* srow = scores + (int64_t)(bi * hq + h * G) * ctx;

  for (int j = j0 + slot; j < j1; j += 16 * U) {
    uint4 kv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j + 16 * u;
      kv[u] = (jj < j1) ? *reinterpret_cast<const uint4*>(kh + (int64_t)jj * kD) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j + 16 * u;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float s = row16_sum(dot8_bf16(kv[u], qv[g], 0.0f)) * scale;
        if (sub == g && jj < j1) srow[(int64_t)g * ctx + jj] = s;
      }
    }
  }
}

__global__ __launch_bounds__(kDecThreads) void sparse_softmax_v_kernel(const float* __restrict__ sel_vals,
                                                                      const int32_t* __restrict__ sel_idx,
                                                                      const uint16_t* __restrict__ V, int hq,
                                                                      int hkv, int64_t ctx_stride, int ks,
                                                                      uint16_t* __restrict__ out) {
  constexpr int U = 4;
  __shared__ float acc_lds[16][kD];
  __shared__ float w_lds[16];
  __shared__ float red[kDecThreads / kWave];
  const int t = threadIdx.x;
  const int r = blockIdx.x;
  const int bi = r / hq;
  const int h = r - bi * hq;
  const int kvh = h / (hq / hkv);
  const float* sv = sel_vals + (int64_t)r * ks;
  const int32_t* si = sel_idx + (int64_t)r * ks;

  float mx = -INFINITY;
  for (int j = t; j < ks; j += kDecThreads) mx = fmaxf(mx, sv[j]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  if (lane_id() == 0) red[t / kWave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < kDecThreads / kWave; ++w) mx = fmaxf(mx, red[w]);

  const int group = t >> 4;
  const int sub = t & 15;
  const uint16_t* vh = V + ((int64_t)bi * hkv + kvh) * ctx_stride * kD + sub * 8;
  float acc[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) acc[d] = 0.0f;
  float wsum = 0.0f;
  for (int j = group; j < ks; j += 16 * U) {
    uint4 v[U];
    float w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j + 16 * u;
      if (jj < ks) {
        v[u] = *reinterpret_cast<const uint4*>(vh + (int64_t)si[jj] * kD);
        w[u] = expf(sv[jj] - mx);
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
#pragma unroll
  for (int d = 0; d < 8; ++d) acc_lds[group][sub * 8 + d] = acc[d];
  if (sub == 0) w_lds[group] = wsum;
  __syncthreads();
  if (t < kD) {
    float s = 0.0f, wt = 0.0f;
#pragma unroll
    for (int g = 0; g < 16; ++g) {
      s += acc_lds[g][t];
      wt += w_lds[g];
    }
    out[(int64_t)r * kD + t] = f32_to_bf16_rne(s / wt);
  }
}

}  // namespace

hipError_t launch_decode_scores(const uint16_t* q, const uint16_t* K, int64_t batch, int64_t hq, int64_t hkv,
                                int64_t ctx, int64_t ctx_stride, float scale, float* scores, hipStream_t s) {
  dim3 grid((unsigned)((ctx + kKeysPerBlock - 1) / kKeysPerBlock), (unsigned)(batch * hkv));
  const int g = (int)(hq / hkv);
#define ATOPK_DS(GV)                                                                                              \
  case GV:                                                                                                        \
    hipLaunchKernelGGL((decode_scores_kernel<GV>), grid, dim3(kDecThreads), 0, s, q, K, (int)hq, (int)hkv, (int)ctx, \
                       ctx_stride, scale, scores);                                                                \
    break;
  switch (g) {
    ATOPK_DS(1) ATOPK_DS(2) ATOPK_DS(3) ATOPK_DS(4) ATOPK_DS(5) ATOPK_DS(6) ATOPK_DS(7) ATOPK_DS(8)
    default: return hipErrorInvalidValue;
  }
#undef ATOPK_DS
  return hipGetLastError();
}

hipError_t launch_sparse_softmax_v(const float* sel_vals, const int32_t* sel_idx, const uint16_t* V, int64_t batch,
                                   int64_t hq, int64_t hkv, int64_t ctx_stride, int64_t k_sel, uint16_t* out,
                                   hipStream_t s) {
  dim3 grid((unsigned)(batch * hq));
  hipLaunchKernelGGL(sparse_softmax_v_kernel, grid, dim3(kDecThreads), 0, s, sel_vals, sel_idx, V, (int)hq, (int)hkv,
                     ctx_stride, (int)k_sel, out);
  return hipGetLastError();
}

}  // namespace atopk
