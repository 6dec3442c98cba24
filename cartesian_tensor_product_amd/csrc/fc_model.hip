// Pieces of a full message-passing block for gfx950 (FlashCart paper, App. E
// "Model architecture": after normalisation, nonlinear functions of the
// scalar features gate the equivariant channels; scalar channels pass
// through a readout MLP to the atomic energy; App. F: scalar SiLU gates,
// readout MLP with two hidden layers of width 64).  Gates: one thread per
// (node, channel).  Readout: one wave per node, lanes = hidden units, the
// hidden activations exchanged by lane shuffles.
#include "fc_model.h"

#include "fc_common.h"

namespace fc {
namespace {

__device__ __forceinline__ float silu(float a) { return a / (1.f + expf(-a)); }
__device__ __forceinline__ float silu_grad(float a) {
  const float s = 1.f / (1.f + expf(-a));
  return s * (1.f + a * (1.f - s));
}

__global__ __launch_bounds__(256) void gate_fwd_kernel(int N, int C, int R, const float* __restrict__ n,
                                                       float* __restrict__ y, float* __restrict__ A) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)N * C) return;
  const size_t u = i / C, k = i % C;
  const float* nu = n + u * R * C + k;
  float* yu = y + u * R * C + k;
  float* Au = A + u * R * C + k;
  const float s = nu[0], sg = silu(s);
  yu[0] = sg;
  Au[0] = s;
  for (int r = 1; r < R; ++r) {
    const float v = nu[(size_t)r * C];
    yu[(size_t)r * C] = sg * v;
    Au[(size_t)r * C] = v;
  }
}

__global__ __launch_bounds__(256) void gate_vjp_kernel(int N, int C, int R, const float* __restrict__ n,
                                                       const float* __restrict__ Ab, const float* __restrict__ yb,
                                                       float* __restrict__ nb) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)N * C) return;
  const size_t u = i / C, k = i % C, base = u * R * C + k;
  const float s = n[base];
  const float sg = silu(s);
  float t = yb[base];
  for (int r = 1; r < R; ++r) {
    const size_t o = base + (size_t)r * C;
    t = fmaf(yb[o], n[o], t);
    nb[o] = fmaf(sg, yb[o], Ab[o]);
  }
  nb[base] = fmaf(silu_grad(s), t, Ab[base]);
}

constexpr int kReadWaves = 4;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// lane j: a1_j = f . Wr1[:, j], h1_j = SiLU(a1_j), a2_j = h1 . Wr2[:, j]
__device__ __forceinline__ void readout_hidden(int C, const float* __restrict__ fu, const float* __restrict__ Wr1,
                                               const float* __restrict__ Wr2, int j, float& a1, float& h1,
                                               float& a2) {
  a1 = 0.f;
  for (int k = 0; k < C; ++k) a1 = fmaf(fu[k], Wr1[(size_t)k * kReadoutHidden + j], a1);
  h1 = silu(a1);
  a2 = 0.f;
#pragma unroll 8
  for (int i = 0; i < kReadoutHidden; ++i) a2 = fmaf(__shfl(h1, i), Wr2[i * kReadoutHidden + j], a2);
}

__global__ __launch_bounds__(kReadWaves * kWave) void readout_fwd_kernel(int N, int C, const float* __restrict__ f,
                                                                         const float* __restrict__ Wr1,
                                                                         const float* __restrict__ Wr2,
                                                                         const float* __restrict__ wr3,
                                                                         float* __restrict__ e) {
  const int u = blockIdx.x * kReadWaves + threadIdx.x / kWave, j = threadIdx.x % kWave;
  if (u >= N) return;   // whole waves; no barrier
  float a1, h1, a2;
  readout_hidden(C, f + (size_t)u * C, Wr1, Wr2, j, a1, h1, a2);
  const float t = wave_sum(silu(a2) * wr3[j]);
  if (j == 0) e[u] = t;
}

__global__ __launch_bounds__(kReadWaves * kWave) void readout_vjp_kernel(int N, int C, const float* __restrict__ f,
                                                                         const float* __restrict__ Wr1,
                                                                         const float* __restrict__ Wr2,
                                                                         const float* __restrict__ wr3,
                                                                         float* __restrict__ fb) {
  const int u = blockIdx.x * kReadWaves + threadIdx.x / kWave, j = threadIdx.x % kWave;
  if (u >= N) return;
  float a1, h1, a2;
  readout_hidden(C, f + (size_t)u * C, Wr1, Wr2, j, a1, h1, a2);
  const float ab2 = wr3[j] * silu_grad(a2);
  // lane i: h1_bar_i = sum_j a2_bar_j Wr2[i, j]
  float hb1 = 0.f;
#pragma unroll 8
  for (int jj = 0; jj < kReadoutHidden; ++jj) hb1 = fmaf(__shfl(ab2, jj), Wr2[j * kReadoutHidden + jj], hb1);
  const float ab1 = hb1 * silu_grad(a1);
  // every lane runs every chunk, so that the shuffles read active lanes
  for (int k0 = 0; k0 < C; k0 += kWave) {
    const int k = k0 + j;
    const bool in = k < C;
    const float* wrow = Wr1 + (size_t)(in ? k : 0) * kReadoutHidden;
    float t = 0.f;
#pragma unroll 8
    for (int i = 0; i < kReadoutHidden; ++i) t = fmaf(__shfl(ab1, i), wrow[i], t);
    if (in) fb[(size_t)u * C + k] = t;
  }
}

dim3 elem_grid(size_t n) { return dim3((unsigned)((n + 255) / 256)); }

}  // namespace

void launch_gate_fwd(int N, int C, int l_max, const float* n, float* y, float* A, hipStream_t st) {
  hipLaunchKernelGGL(gate_fwd_kernel, elem_grid((size_t)N * C), dim3(256), 0, st, N, C, nrank(l_max), n, y, A);
}

void launch_gate_vjp(int N, int C, int l_max, const float* n, const float* Abar, const float* ybar, float* nbar,
                     hipStream_t st) {
  hipLaunchKernelGGL(gate_vjp_kernel, elem_grid((size_t)N * C), dim3(256), 0, st, N, C, nrank(l_max), n, Abar, ybar,
                     nbar);
}

void launch_readout_fwd(int N, int C, const float* f, const float* Wr1, const float* Wr2, const float* wr3, float* e,
                        hipStream_t st) {
  hipLaunchKernelGGL(readout_fwd_kernel, dim3((N + kReadWaves - 1) / kReadWaves), dim3(kReadWaves * kWave), 0, st, N,
                     C, f, Wr1, Wr2, wr3, e);
}

void launch_readout_vjp(int N, int C, const float* f, const float* Wr1, const float* Wr2, const float* wr3,
                        float* fbar, hipStream_t st) {
  hipLaunchKernelGGL(readout_vjp_kernel, dim3((N + kReadWaves - 1) / kReadWaves), dim3(kReadWaves * kWave), 0, st, N,
                     C, f, Wr1, Wr2, wr3, fbar);
}

}  // namespace fc
