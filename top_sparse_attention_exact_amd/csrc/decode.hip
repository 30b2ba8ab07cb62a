// Softmax / value aggregation over the selected keys of the exact Top-K
// decode (its scores come from the scoring kernels in scores-only mode).
//
// "Recall Before You Rank ..." (fugumt page), Abstract: the current query is
// scored against the full KV cache, a global Top-K is taken, and softmax and
// value aggregation run over only that subset.  STARC (Pith review page),
// Figure 3 caption: q in R^{1 x d_h}, K, V in R^{L x d_h} per head.
#include "common.h"
#include "launch.h"

namespace atopk {

namespace {

constexpr int kD = 128;
constexpr int kDecThreads = 512;
constexpr int kGroups = kDecThreads / 16;  // 16-lane groups gathering V rows

__global__ __launch_bounds__(kDecThreads) void sparse_softmax_v_kernel(const float* __restrict__ sel_vals,
                                                                      const int32_t* __restrict__ sel_idx,
                                                                      const uint16_t* __restrict__ V, int hq,
                                                                      int hkv, int64_t ctx_stride, int ks,
                                                                      uint16_t* __restrict__ out) {
  constexpr int U = 8;
  __shared__ float acc_lds[kGroups][kD];
  __shared__ float w_lds[kGroups];
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
  for (int j = group; j < ks; j += kGroups * U) {
    uint4 v[U];
    float w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int jj = j + kGroups * u;
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
    for (int g = 0; g < kGroups; ++g) {
      s += acc_lds[g][t];
      wt += w_lds[g];
    }
    out[(int64_t)r * kD + t] = f32_to_bf16_rne(s / wt);
  }
}

}  // namespace

hipError_t launch_sparse_softmax_v(const float* sel_vals, const int32_t* sel_idx, const uint16_t* V, int64_t batch,
                                   int64_t hq, int64_t hkv, int64_t ctx_stride, int64_t k_sel, uint16_t* out,
                                   hipStream_t s) {
  dim3 grid((unsigned)(batch * hq));
  ATOPK_LAUNCH(sparse_softmax_v_kernel, grid, dim3(kDecThreads), 0, s, sel_vals, sel_idx, V, (int)hq, (int)hkv,
                     ctx_stride, (int)k_sel, out);
  return hipGetLastError();
}

}  // namespace atopk
