// Deterministic reductions shared by the edge convolution and the ladder.
#pragma once

#include <hip/hip_runtime.h>

namespace fc {

// out[i] = sum_{b < nblk} part[b * n + i] for i < n, in a fixed order that
// depends only on nblk (bitwise reproducible).
void launch_block_sum(int nblk, int n, const float* part, float* out, hipStream_t st);

}  // namespace fc
