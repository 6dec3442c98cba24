// Equivariant RMS normalisation of node features (launch interface).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace fc {

inline constexpr int kNormMaxChannels = 512;
inline constexpr int kNormMaxRank = 5;

// Blocks of the VJP (each sums the weight gradient of its nodes).
int rms_norm_vjp_blocks(int N);

void launch_rms_norm_fwd(int l_max, int N, int C, float eps, const float* x, const float* gamma, float* y,
                         float* inv_s, hipStream_t st);
// part: [rms_norm_vjp_blocks(N)][l_max + 1][C] when gamma_grad is wanted
void launch_rms_norm_vjp(int l_max, int N, int C, const float* x, const float* gamma, const float* inv_s,
                         const float* g, float* x_grad, float* part, float* gamma_grad, hipStream_t st);

}  // namespace fc
