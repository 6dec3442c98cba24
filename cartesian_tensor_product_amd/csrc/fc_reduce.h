// Deterministic reductions shared by the edge convolution and the ladder.
#pragma once

#include <hip/hip_runtime.h>

namespace fc {

// out[i] = sum_{b < nblk} part[b * n + i] for i < n, in a fixed order that
// depends only on nblk (bitwise reproducible).
void launch_block_sum(int nblk, int n, const float* part, float* out, hipStream_t st);

// dst[i] += src[i] for i < n.
void launch_add(size_t n, const float* src, float* dst, hipStream_t st);

// dst[i] = 0 for i < n (a kernel, so that it may sit in a captured graph).
void launch_zero(size_t n, float* dst, hipStream_t st);

}  // namespace fc
