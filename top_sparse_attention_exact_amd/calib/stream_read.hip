// Measurement yardstick, not part of the selection library: a plain
// streaming read of a device buffer, the best a kernel that only reads its
// input can do on this GPU at a given size.  Every thread reads 16-byte
// vectors (8 in flight) in a grid-stride loop and folds them into one word;
// each workgroup writes its word so the reads cannot be dropped.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ x, int64_t nvec,
                                                             uint32_t* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < nvec; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = x[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < nvec; i += stride) {
    const uint4 v = x[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  __shared__ uint32_t red[kThreads / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace

// Read `bytes` (a multiple of 16, 16-byte aligned) at x with `blocks`
// workgroups on `stream`; out holds `blocks` words.  Returns a hipError_t.
extern "C" int atopk_calib_stream_read(const void* x, int64_t bytes, int blocks, uint32_t* out, void* stream) {
  if (x == nullptr || out == nullptr || bytes < 16 || (bytes & 15) != 0 || blocks < 1 ||
      (reinterpret_cast<uintptr_t>(x) & 15) != 0)
    return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(x), bytes / 16, out);
  return (int)hipGetLastError();
}
