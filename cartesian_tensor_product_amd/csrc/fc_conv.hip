// Edge-convolution dispatch: every (l_in, l_edge, l_out) of the build lives
// in its own generated translation unit (generated/conv_inst_*.hip) so that
// the heavily unrolled kernels compile in parallel.
#include "fc_conv.h"
#include "generated/fc_conv_configs.h"

namespace fc {

// Combine pass, one block per node v, fixed summation order (deterministic):
//   x_bar[v]   = sum_s x_part[v, s]                         (when S > 1)
//   pos_bar[v] = sum_s p_part[v, s] - sum_{e: u_e = v} r_bar_e
// With S == 1 the sender kernel wrote x_bar and the sender part of pos_bar
// directly and only the receiver sum is applied.
__global__ __launch_bounds__(256) void conv_vjp_combine_kernel(int S, int row, const int* __restrict__ rowptr,
                                                               const float* __restrict__ rbar,
                                                               const float* __restrict__ p_part,
                                                               const float* __restrict__ x_part,
                                                               float* __restrict__ x_bar, float* __restrict__ pos_bar) {
  const int v = blockIdx.x;
  const int tid = threadIdx.x;
  if (x_part && S > 1) {
    for (int i = tid; i < row; i += blockDim.x) {
      float t = 0.f;
      for (int s = 0; s < S; ++s) t += x_part[((size_t)v * S + s) * row + i];
      x_bar[(size_t)v * row + i] = t;
    }
  }
  if (pos_bar && tid < kWave) {
    const int e0 = rowptr[v], e1 = rowptr[v + 1];
    float sx = 0.f, sy = 0.f, sz = 0.f;
    for (int e = e0 + tid; e < e1; e += kWave) {
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
    if (tid == 0) {
      const float* pp = S > 1 ? p_part + (size_t)3 * v * S : pos_bar + 3 * (size_t)v;
      float px = 0.f, py = 0.f, pz = 0.f;
      for (int s = 0; s < (S > 1 ? S : 1); ++s) {
        px += pp[3 * s];
        py += pp[3 * s + 1];
        pz += pp[3 * s + 2];
      }
      pos_bar[3 * (size_t)v] = px - sx;
      pos_bar[3 * (size_t)v + 1] = py - sy;
      pos_bar[3 * (size_t)v + 2] = pz - sz;
    }
  }
}

// pos_bar[v] = sum_{e out of v} r_bar_e - sum_{e into v} r_bar_e, one wave
// per node, fixed order (after the receiver-side VJP, which stores r_bar per
// edge only).
__global__ __launch_bounds__(kWave) void conv_pos_from_edges_kernel(int N, const int* __restrict__ rowptr,
                                                                    const int* __restrict__ t_rowptr,
                                                                    const int* __restrict__ t_edge,
                                                                    const float* __restrict__ rbar,
                                                                    float* __restrict__ pos_bar) {
  const int v = blockIdx.x, lane = threadIdx.x;
  float s[3] = {0.f, 0.f, 0.f};
  for (int i = t_rowptr[v] + lane; i < t_rowptr[v + 1]; i += kWave) {
    const size_t e = (size_t)t_edge[i];
    s[0] += rbar[3 * e];
    s[1] += rbar[3 * e + 1];
    s[2] += rbar[3 * e + 2];
  }
  for (int e = rowptr[v] + lane; e < rowptr[v + 1]; e += kWave) {
    s[0] -= rbar[3 * (size_t)e];
    s[1] -= rbar[3 * (size_t)e + 1];
    s[2] -= rbar[3 * (size_t)e + 2];
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s[i] += __shfl_xor(s[i], o);
  }
  if (lane == 0) {
    pos_bar[3 * (size_t)v] = s[0];
    pos_bar[3 * (size_t)v + 1] = s[1];
    pos_bar[3 * (size_t)v + 2] = s[2];
  }
}

void launch_pos_from_edges(const ConvArgs& a, const float* rbar, hipStream_t st) {
  hipLaunchKernelGGL(conv_pos_from_edges_kernel, dim3(a.N), dim3(kWave), 0, st, a.N, a.rowptr, a.t_rowptr, a.t_edge,
                     rbar, a.pos_bar);
}

void launch_vjp_combine(const ConvArgs& a, const VjpWorkspace& w, int nin, hipStream_t st) {
  if (w.S == 1 && !a.pos_bar) return;
  hipLaunchKernelGGL(conv_vjp_combine_kernel, dim3(a.N), dim3(256), 0, st, w.S, nin * a.C, a.rowptr, w.rbar,
                     w.p_part, a.x_bar ? w.x_part : nullptr, a.x_bar, a.pos_bar);
}

#define FC_CONV_DECL(A, B, Cc) bool conv_run_##A##B##Cc(int op, const ConvArgs& args, hipStream_t stream);
FC_CONV_CONFIGS(FC_CONV_DECL)

#define FC_CONV_CASE(A, B, Cc) \
  case (A) * 1024 + (B) * 32 + (Cc): return conv_run_##A##B##Cc(op, args, stream);

#define FC_CONV_SUPPORTED(A, B, Cc) \
  case (A) * 1024 + (B) * 32 + (Cc): return true;

bool conv_supported(int l_in, int l_edge, int l_out) {
  switch (l_in * 1024 + l_edge * 32 + l_out) {
    FC_CONV_CONFIGS(FC_CONV_SUPPORTED)
    default: return false;
  }
}

bool conv_vv_supported(int l_in, int l_edge, int l_out) {
  switch (l_in * 1024 + l_edge * 32 + l_out) {
    FC_CONV_VV_CONFIGS(FC_CONV_SUPPORTED)
    default: return false;
  }
}

bool conv_dispatch(int op, int l_in, int l_edge, int l_out, const ConvArgs& args, hipStream_t stream) {
  switch (l_in * 1024 + l_edge * 32 + l_out) {
    FC_CONV_CONFIGS(FC_CONV_CASE)
    default: return false;
  }
}

void run_vjp_vjp(const VVParts& parts, int nin, int P, const ConvArgs& a, hipStream_t st) {
  if (a.g_hat) parts.recv(a, st);
  if (a.W_bar) parts.wgrad(a, st);
  if (!a.x_bar && !a.pos_bar) return;
  if (a.v_x) parts.sender_vx(a, st);
  else parts.sender(a, st);
  const VjpWorkspace wsl(a.N, a.E, a.C, nin, P, true, a.rbar);
  launch_vjp_combine(a, wsl, nin, st);
}

bool conv_vv_w_supported(int l_in, int l_edge, int l_out) {
  switch (l_in * 1024 + l_edge * 32 + l_out) {
    FC_CONV_VV_W_CONFIGS(FC_CONV_SUPPORTED)
    default: return false;
  }
}

#define FC_CONV_W_DECL(A, B, Cc) void conv_run_w_##A##B##Cc(const ConvArgs& args, hipStream_t stream);
FC_CONV_VV_W_CONFIGS(FC_CONV_W_DECL)

#define FC_CONV_W_CASE(A, B, Cc)            \
  case (A) * 1024 + (B) * 32 + (Cc):         \
    conv_run_w_##A##B##Cc(args, stream);     \
    return true;

bool conv_vv_w_dispatch(int l_in, int l_edge, int l_out, const ConvArgs& args, hipStream_t stream) {
  switch (l_in * 1024 + l_edge * 32 + l_out) {
    FC_CONV_VV_W_CONFIGS(FC_CONV_W_CASE)
    default: return false;
  }
}

#define FC_CONV_MLP_DECL(A, B, Cc) void conv_run_mlp_##A##B##Cc(int op, const ConvArgs& args, hipStream_t stream);
FC_CONV_MLP_CONFIGS(FC_CONV_MLP_DECL)

#define FC_CONV_MLP_CASE(A, B, Cc)            \
  case (A) * 1024 + (B) * 32 + (Cc):           \
    conv_run_mlp_##A##B##Cc(op, args, stream); \
    return true;

bool conv_mlp_dispatch(int op, int l_in, int l_edge, int l_out, const ConvArgs& args, hipStream_t stream) {
  switch (l_in * 1024 + l_edge * 32 + l_out) {
    FC_CONV_MLP_CONFIGS(FC_CONV_MLP_CASE)
    default: return false;
  }
}

bool conv_mlp_supported(int l_in, int l_edge, int l_out) {
  switch (l_in * 1024 + l_edge * 32 + l_out) {
    FC_CONV_MLP_CONFIGS(FC_CONV_SUPPORTED)
    default: return false;
  }
}

bool conv_mlp_fwd_fused(int l_in, int l_edge, int l_out) {
  switch (l_in * 1024 + l_edge * 32 + l_out) {
    FC_CONV_MLP_FWD_FUSED_CONFIGS(FC_CONV_SUPPORTED)
    default: return false;
  }
}

}  // namespace fc
