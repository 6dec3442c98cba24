// Helpers of the energy/force composition (see fc_block.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>

namespace fc {

// pos_w = a W, neg_w = -a W (neg_w nullable), n floats each
void block_scaled_weights(const float* W, size_t n, float a, float* pos_w, float* neg_w, hipStream_t st);
void block_unit_cotangent(float* g, int N, int rows, int C, hipStream_t st);
int block_energy_parts(int N);
void block_energy(const float* z, int N, int rows, int C, float* e_atom, double* part, double* energy,
                  hipStream_t st);

}  // namespace fc
