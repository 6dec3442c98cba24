// Edge-convolution dispatch: every (l_in, l_edge, l_out) of the build lives
// in its own generated translation unit (generated/conv_inst_*.hip) so that
// the heavily unrolled kernels compile in parallel.
#include "fc_conv.h"

namespace fc {

// Receiver pass: pos_bar[u] -= sum of r_bar over the incoming edges of u
// (one wave per node, fixed per-lane order and a fixed butterfly, so the
// result is deterministic).
__global__ __launch_bounds__(256) void conv_vjp_receiver_kernel(int N, const int* __restrict__ rowptr,
                                                                const float* __restrict__ rbar,
                                                                float* __restrict__ pos_bar) {
  const int u = blockIdx.x * 4 + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (u >= N) return;
  const int e0 = rowptr[u], e1 = rowptr[u + 1];
  float sx = 0.f, sy = 0.f, sz = 0.f;
  for (int e = e0 + lane; e < e1; e += kWave) {
    sx += rbar[3 * (size_t)e];
    sy += rbar[3 * (size_t)e + 1];
    sz += rbar[3 * (size_t)e + 2];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    sx += __shfl_xor(sx, o);
    sy += __shfl_xor(sy, o);
    sz += __shfl_xor(sz, o);
  }
  if (lane == 0) {
    pos_bar[3 * u] -= sx;
    pos_bar[3 * u + 1] -= sy;
    pos_bar[3 * u + 2] -= sz;
  }
}

void launch_vjp_receiver(const ConvArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(conv_vjp_receiver_kernel, dim3((a.N + 3) / 4), dim3(256), 0, st, a.N, a.rowptr, a.rbar,
                     a.pos_bar);
}

#define FC_CONV_DECL(A, B, Cc) bool conv_run_##A##B##Cc(int op, const ConvArgs& args, hipStream_t stream);
FC_CONV_CONFIGS(FC_CONV_DECL)

#define FC_CONV_CASE(A, B, Cc) \
  case (A) * 25 + (B) * 5 + (Cc): return conv_run_##A##B##Cc(op, args, stream);

#define FC_CONV_SUPPORTED(A, B, Cc) \
  case (A) * 25 + (B) * 5 + (Cc): return true;

bool conv_supported(int l_in, int l_edge, int l_out) {
  switch (l_in * 25 + l_edge * 5 + l_out) {
    FC_CONV_CONFIGS(FC_CONV_SUPPORTED)
    default: return false;
  }
}

bool conv_dispatch(int op, int l_in, int l_edge, int l_out, const ConvArgs& args, hipStream_t stream) {
  switch (l_in * 25 + l_edge * 5 + l_out) {
    FC_CONV_CONFIGS(FC_CONV_CASE)
    default: return false;
  }
}

}  // namespace fc
