// Deterministic reductions shared by the edge convolution and the ladder.
#include "fc_reduce.h"

#include "fc_common.h"

namespace fc {

// out[i] = sum_b part[b][i] in a fixed order: a block of four waves covers
// 64 consecutive i, wave w sums the w-th quarter of the b range in b order,
// and the four quarter sums are added in wave order.
__global__ __launch_bounds__(256) void block_sum_kernel(int nblk, int n, const float* __restrict__ part,
                                                        float* __restrict__ out) {
  __shared__ float red[3][kWave];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int i = blockIdx.x * kWave + lane;
  const int per = (nblk + 3) / 4;
  const int b0 = min(nblk, wave * per), b1 = min(nblk, b0 + per);
  float t = 0.f;
  if (i < n) {
    const float* src = part + i;
    int b = b0;
    for (; b + 8 <= b1; b += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = src[(size_t)(b + j) * n];
#pragma unroll
      for (int j = 0; j < 8; ++j) t += v[j];
    }
    for (; b < b1; ++b) t += src[(size_t)b * n];
  }
  if (wave > 0) red[wave - 1][lane] = t;
  __syncthreads();
  if (wave == 0 && i < n) out[i] = ((t + red[0][lane]) + red[1][lane]) + red[2][lane];
}

void launch_block_sum(int nblk, int n, const float* part, float* out, hipStream_t st) {
  if (n <= 0) return;
  hipLaunchKernelGGL(block_sum_kernel, dim3((n + kWave - 1) / kWave), dim3(4 * kWave), 0, st, nblk, n, part, out);
}

__global__ __launch_bounds__(256) void add_kernel(size_t n, const float* __restrict__ src, float* __restrict__ dst) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] += src[i];
}

__global__ __launch_bounds__(256) void zero_kernel(size_t n, float* __restrict__ dst) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    dst[i] = 0.f;
}

static dim3 elementwise_grid(size_t n) {
  const size_t b = (n + 255) / 256;
  return dim3((unsigned)(b < 8192 ? b : 8192));
}

void launch_add(size_t n, const float* src, float* dst, hipStream_t st) {
  if (n == 0) return;
  hipLaunchKernelGGL(add_kernel, elementwise_grid(n), dim3(256), 0, st, n, src, dst);
}

void launch_zero(size_t n, float* dst, hipStream_t st) {
  if (n == 0) return;
  hipLaunchKernelGGL(zero_kernel, elementwise_grid(n), dim3(256), 0, st, n, dst);
}

}  // namespace fc
