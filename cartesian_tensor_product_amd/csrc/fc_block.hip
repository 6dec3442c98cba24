// One message-passing block evaluated for energy and forces (FlashCart
// paper, App. E "Model architecture": an equivariant convolution with scalar
// sender features, the 1/sqrt(N_bar) neighbour normalisation of Eq. E1, then
// the product ladder whose final block returns scalars; E = sum of the
// rank-0 outputs; §2: F_u = -dE/dr_u).  Residual updates, normalisation,
// gates and the readout carry trained weights and are not part of it.
//
// Small kernels used by the composition: scaling (in place, and of the
// radial weights into a scaled and a negated copy), a deterministic fp64
// energy reduction and the unit cotangent of the energy.
#include <hip/hip_runtime.h>

#include "fc_block.h"

namespace fc {

namespace {

// pos_w = a W and neg_w = -a W (nullable): the radial weights with the
// convolution scale folded in, for the forward and (negated, so that the
// VJP to the positions is the force) for the backward pass.
__global__ __launch_bounds__(256) void scaled_pair_kernel(size_t n, float a, const float* __restrict__ W,
                                                          float* __restrict__ pos_w, float* __restrict__ neg_w) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = a * W[i];
  pos_w[i] = v;
  if (neg_w) neg_w[i] = -v;
}

// dE/dz: 1 on the rank-0 rows, 0 elsewhere.
__global__ __launch_bounds__(256) void unit_cotangent_kernel(size_t n, int rows, int C, float* __restrict__ g) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) g[i] = ((i / C) % rows) == 0 ? 1.f : 0.f;
}

// Per-atom energies e_u = sum_k z[u, 0, k] (one wave per atom, fixed order),
// written as fp64 partials of 256 atoms per block.
__global__ __launch_bounds__(256) void atom_energy_kernel(int N, int rows, int C, const float* __restrict__ z,
                                                          float* __restrict__ e_atom, double* __restrict__ part) {
  __shared__ double s[4];
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  double acc = 0.0;
  for (int u = blockIdx.x * 4 + w; u < N; u += gridDim.x * 4) {
    double t = 0.0;
    for (int k = lane; k < C; k += 64) t += (double)z[((size_t)u * rows) * C + k];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
    if (lane == 0 && e_atom) e_atom[u] = (float)t;
    acc += t;
  }
  if (lane == 0) s[w] = acc;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = (s[0] + s[1]) + (s[2] + s[3]);
}

// One wave: lane l sums part[l], part[l + 64], ... in order, then a butterfly
// (fixed order, the same bits in every lane).
__global__ __launch_bounds__(64) void energy_sum_kernel(int n, const double* __restrict__ part,
                                                        double* __restrict__ energy) {
  const int lane = threadIdx.x;
  double t = 0.0;
  for (int i = lane; i < n; i += 64) t += part[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
  if (lane == 0) *energy = t;
}

}  // namespace

void block_scaled_weights(const float* W, size_t n, float a, float* pos_w, float* neg_w, hipStream_t st) {
  if (n)
    hipLaunchKernelGGL(scaled_pair_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, n, a, W, pos_w,
                       neg_w);
}

void block_unit_cotangent(float* g, int N, int rows, int C, hipStream_t st) {
  const size_t n = (size_t)N * rows * C;
  hipLaunchKernelGGL(unit_cotangent_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, n, rows, C, g);
}

int block_energy_parts(int N) { return std::min(1024, (N + 3) / 4); }

void block_energy(const float* z, int N, int rows, int C, float* e_atom, double* part, double* energy,
                  hipStream_t st) {
  const int nb = block_energy_parts(N);
  hipLaunchKernelGGL(atom_energy_kernel, dim3(nb), dim3(256), 0, st, N, rows, C, z, e_atom, part);
  hipLaunchKernelGGL(energy_sum_kernel, dim3(1), dim3(64), 0, st, nb, (const double*)part, energy);
}

}  // namespace fc
