// The pages' radial network for gfx950 (FlashCart paper, App. E "Model
// architecture", the radial weights of Eq. E1, and App. F "Model
// architecture and training"): eight Chebyshev functions of the
// cosine-transformed distance, T_n(cos(pi r / r_max)), times a p = 6
// polynomial envelope u(d) = 1 - 28 d^6 + 48 d^7 - 21 d^8 (value and first
// two derivatives zero at d = r / r_max = 1), fed to a bias-free MLP with two
// SiLU hidden layers of width 64 and one output per path and channel.
//
// The two hidden layers are per-edge work (one lane per edge, weights in
// LDS); the output layer w [E][P C] = h2 [E][64] W3 [64][P C] is a dense
// contraction and runs as an MFMA GEMM, as do the backward products
// h2_bar = w_bar W3^T and the weight gradients (split-K over edges, fixed
// summation order).  Per-edge position terms q_e = (dL/dr_e) r_hat_e are
// summed per node in a fixed order (out-edges minus in-edges).
#include "fc_radial.h"

#include "fc_common.h"
#include "fc_gemm.h"
#include "fc_reduce.h"

namespace fc {
namespace {

constexpr int kRadBlock = 256;
constexpr int kW1 = kRadFeat * kRadHidden, kW2 = kRadHidden * kRadHidden;

__device__ __forceinline__ float silu(float a) { return a / (1.f + expf(-a)); }
__device__ __forceinline__ float silu_grad(float a) {
  const float s = 1.f / (1.f + expf(-a));
  return s * (1.f + a * (1.f - s));
}

// Edge vector r = pos[sender] - pos[receiver] + shift.
__device__ __forceinline__ void edge_vec(int e, const int* __restrict__ receiver, const int* __restrict__ sender,
                                         const float* __restrict__ pos, const float* __restrict__ shift, float* rv) {
  const int u = receiver[e], v = sender[e];
  rv[0] = pos[3 * v] - pos[3 * u];
  rv[1] = pos[3 * v + 1] - pos[3 * u + 1];
  rv[2] = pos[3 * v + 2] - pos[3 * u + 2];
  if (shift) {
    rv[0] += shift[3 * e];
    rv[1] += shift[3 * e + 1];
    rv[2] += shift[3 * e + 2];
  }
}

// phi_n = T_n(cos t) u(d) with t = pi d, d = r / r_max (Chebyshev recurrence
// T_{n+1} = 2x T_n - T_{n-1} on x = cos t, which gives cos(n t); sin(n t)
// follows the same recurrence); dphi = d phi / d r.  Zero for d >= 1 and for
// r = 0 (an edge without a direction takes no part).
__device__ __forceinline__ void features(float r, float rmax, float* phi, float* dphi) {
  const float d = r / rmax;
  if (!(d < 1.f) || !(r > 0.f)) {
#pragma unroll
    for (int n = 0; n < kRadFeat; ++n) phi[n] = dphi[n] = 0.f;
    return;
  }
  float s1, c1;
  sincosf(kPi * d, &s1, &c1);
  const float d2 = d * d, d5 = d2 * d2 * d, d6 = d5 * d, om = 1.f - d;
  const float u = 1.f + d6 * (-28.f + d * (48.f - 21.f * d));
  const float du = -168.f * d5 * om * om / rmax;
  const float k = kPi / rmax;
  float cp = 1.f, c = c1, sp = 0.f, s = s1;   // cos/sin of (n-1) t and n t
  phi[0] = u;
  dphi[0] = du;
#pragma unroll
  for (int n = 1; n < kRadFeat; ++n) {
    phi[n] = c * u;
    dphi[n] = fmaf(-float(n) * k * s, u, c * du);
    const float cn = 2.f * c1 * c - cp, sn = 2.f * c1 * s - sp;
    cp = c;
    c = cn;
    sp = s;
    s = sn;
  }
}

// acc[i] = sum_j h[j] w2[j][j0 + i] for i < NJ (j ascending, as a dot product
// per output would add them): the loop over j is outside, so that every
// 128-bit LDS read of a W2 row segment feeds four accumulators instead of one
// scalar read per FMA.
template <int NJ>
__device__ __forceinline__ void layer2(const float* h, const float* w2, int j0, float* acc) {
#pragma unroll
  for (int i = 0; i < NJ; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < kRadHidden; ++j) {
    const float4* row = reinterpret_cast<const float4*>(w2 + j * kRadHidden + j0);
#pragma unroll
    for (int q = 0; q < NJ / 4; ++q) {
      const float4 w = row[q];
      acc[4 * q] = fmaf(h[j], w.x, acc[4 * q]);
      acc[4 * q + 1] = fmaf(h[j], w.y, acc[4 * q + 1]);
      acc[4 * q + 2] = fmaf(h[j], w.z, acc[4 * q + 2]);
      acc[4 * q + 3] = fmaf(h[j], w.w, acc[4 * q + 3]);
    }
  }
}

// h1 = SiLU(phi W1) (and its r-derivative with dphi), W1 rows read as float4.
template <bool D>
__device__ __forceinline__ void layer1(const float* phi, const float* dphi, const float* w1, float* h1, float* dh1) {
  float a[kRadHidden], da[D ? kRadHidden : 1];
#pragma unroll
  for (int j = 0; j < kRadHidden; ++j) {
    a[j] = 0.f;
    if constexpr (D) da[j] = 0.f;
  }
#pragma unroll
  for (int n = 0; n < kRadFeat; ++n) {
    const float4* row = reinterpret_cast<const float4*>(w1 + n * kRadHidden);
#pragma unroll
    for (int q = 0; q < kRadHidden / 4; ++q) {
      const float4 w = row[q];
      const float wq[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        a[4 * q + t] = fmaf(phi[n], wq[t], a[4 * q + t]);
        if constexpr (D) da[4 * q + t] = fmaf(dphi[n], wq[t], da[4 * q + t]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kRadHidden; ++j) {
    h1[j] = silu(a[j]);
    if constexpr (D) dh1[j] = silu_grad(a[j]) * da[j];
  }
}

__device__ __forceinline__ void load_hidden_weights(const float* __restrict__ W, float* w1, float* w2) {
  for (int i = threadIdx.x; i < kW1; i += blockDim.x) w1[i] = W[i];
  for (int i = threadIdx.x; i < kW2; i += blockDim.x) w2[i] = W[kW1 + i];
  __syncthreads();
}

__global__ __launch_bounds__(kRadBlock) void radial_hidden_kernel(int E, float rmax, const int* __restrict__ receiver,
                                                                  const int* __restrict__ sender,
                                                                  const float* __restrict__ pos,
                                                                  const float* __restrict__ shift,
                                                                  const float* __restrict__ W, float* __restrict__ h2t,
                                                                  int ld) {
  __shared__ float w1[kW1], w2[kW2];
  load_hidden_weights(W, w1, w2);
  const int e = blockIdx.x * kRadBlock + threadIdx.x;
  if (e >= E) return;   // no barrier below
  float rv[3], phi[kRadFeat], dphi[kRadFeat];
  edge_vec(e, receiver, sender, pos, shift, rv);
  features(sqrtf(rv[0] * rv[0] + rv[1] * rv[1] + rv[2] * rv[2]), rmax, phi, dphi);
  float h1[kRadHidden];
  layer1<false>(phi, dphi, w1, h1, nullptr);
  float a2[kRadHidden];
  layer2<kRadHidden>(h1, w2, 0, a2);
#pragma unroll
  for (int j2 = 0; j2 < kRadHidden; ++j2) h2t[(size_t)j2 * ld + e] = silu(a2[j2]);
}

// Row e of hh: h2 (64 floats), then dh2/dr (64 floats), by forward-mode
// differentiation of the two hidden layers along the edge length.
__global__ __launch_bounds__(kRadBlock) void radial_hidden_rows_kernel(int E, float rmax,
                                                                       const int* __restrict__ receiver,
                                                                       const int* __restrict__ sender,
                                                                       const float* __restrict__ pos,
                                                                       const float* __restrict__ shift,
                                                                       const float* __restrict__ W,
                                                                       float* __restrict__ hh) {
  __shared__ float w1[kW1], w2[kW2];
  load_hidden_weights(W, w1, w2);
  const int e = blockIdx.x * kRadBlock + threadIdx.x;
  if (e >= E) return;   // no barrier below
  float rv[3], phi[kRadFeat], dphi[kRadFeat];
  edge_vec(e, receiver, sender, pos, shift, rv);
  features(sqrtf(rv[0] * rv[0] + rv[1] * rv[1] + rv[2] * rv[2]), rmax, phi, dphi);
  float h1[kRadHidden], dh1[kRadHidden];
  layer1<true>(phi, dphi, w1, h1, dh1);
  float4* row = reinterpret_cast<float4*>(hh + (size_t)e * kRadRow);
  // the second layer and its derivative in quarters of 16 outputs (registers)
#pragma unroll 1
  for (int part = 0; part < 4; ++part) {
    float a[16], da[16];
    layer2<16>(h1, w2, 16 * part, a);
    layer2<16>(dh1, w2, 16 * part, da);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float h[4], dh[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        h[t] = silu(a[4 * q + t]);
        dh[t] = silu_grad(a[4 * q + t]) * da[4 * q + t];
      }
      row[4 * part + q] = make_float4(h[0], h[1], h[2], h[3]);
      row[(kRadHidden + 16 * part) / 4 + q] = make_float4(dh[0], dh[1], dh[2], dh[3]);
    }
  }
}

// Backward of the hidden layers for one edge from h2_bar = hbar[e][:]:
// q_e = (sum_n phi_bar_n dphi_n / dr) r_hat and, with a2bt, the operands of
// the W2 / W1 gradients (a2_bar, h1, a1_bar edge-minor; phi edge-minor).
__global__ __launch_bounds__(kRadBlock) void radial_back_kernel(
    int E, float rmax, const int* __restrict__ receiver, const int* __restrict__ sender, const float* __restrict__ pos,
    const float* __restrict__ shift, const float* __restrict__ W, const float* __restrict__ hbar,
    float* __restrict__ q, float* __restrict__ a2bt, float* __restrict__ h1t, float* __restrict__ a1bt,
    float* __restrict__ phit) {
  __shared__ float w1[kW1], w2[kW2];
  load_hidden_weights(W, w1, w2);
  const int e = blockIdx.x * kRadBlock + threadIdx.x;
  if (e >= E) return;
  float rv[3], phi[kRadFeat], dphi[kRadFeat];
  edge_vec(e, receiver, sender, pos, shift, rv);
  const float r = sqrtf(rv[0] * rv[0] + rv[1] * rv[1] + rv[2] * rv[2]);
  features(r, rmax, phi, dphi);
  // pass 1: a2 = h1 W2 and a2_bar = h2_bar * SiLU'(a2), h1 then dropped
  float ab2[kRadHidden];
  {
    float h1[kRadHidden];
    layer1<false>(phi, dphi, w1, h1, nullptr);
    if (a1bt) {
#pragma unroll
      for (int j = 0; j < kRadHidden; ++j) h1t[(size_t)j * E + e] = h1[j];
    }
    layer2<kRadHidden>(h1, w2, 0, ab2);
    const float4* hb = reinterpret_cast<const float4*>(hbar + (size_t)e * kRadHidden);
#pragma unroll
    for (int q = 0; q < kRadHidden / 4; ++q) {
      const float4 h = hb[q];
      const float hq[4] = {h.x, h.y, h.z, h.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) ab2[4 * q + t] = hq[t] * silu_grad(ab2[4 * q + t]);
    }
    if (a2bt) {
#pragma unroll
      for (int j2 = 0; j2 < kRadHidden; ++j2) a2bt[(size_t)j2 * E + e] = ab2[j2];
    }
  }
  // pass 2, one hidden unit j at a time: h1_bar_j = a2_bar . W2[j, :],
  // a1_bar_j = h1_bar_j SiLU'(a1_j), phi_bar += a1_bar_j W1[:, j]
  float phib[kRadFeat];
#pragma unroll
  for (int n = 0; n < kRadFeat; ++n) phib[n] = 0.f;
  for (int j = 0; j < kRadHidden; ++j) {
    float hb1 = 0.f;
#pragma unroll
    for (int j2 = 0; j2 < kRadHidden; ++j2) hb1 = fmaf(ab2[j2], w2[j * kRadHidden + j2], hb1);
    float a = 0.f;
#pragma unroll
    for (int n = 0; n < kRadFeat; ++n) a = fmaf(phi[n], w1[n * kRadHidden + j], a);
    const float ab = hb1 * silu_grad(a);
    if (a1bt) a1bt[(size_t)j * E + e] = ab;
#pragma unroll
    for (int n = 0; n < kRadFeat; ++n) phib[n] = fmaf(ab, w1[n * kRadHidden + j], phib[n]);
  }
  float rb = 0.f;
#pragma unroll
  for (int n = 0; n < kRadFeat; ++n) {
    rb = fmaf(phib[n], dphi[n], rb);
    if (phit) phit[(size_t)n * E + e] = phi[n];
  }
  const float s = r > 0.f ? rb / r : 0.f;
  q[3 * (size_t)e] = s * rv[0];
  q[3 * (size_t)e + 1] = s * rv[1];
  q[3 * (size_t)e + 2] = s * rv[2];
}

// pos_grad[v] += sum_{e out of v} q_e - sum_{e into v} q_e (one wave per
// node, fixed order).
__global__ __launch_bounds__(kWave) void radial_pos_kernel(int N, const int* __restrict__ rowptr,
                                                           const int* __restrict__ t_rowptr,
                                                           const int* __restrict__ t_edge,
                                                           const float* __restrict__ q, float* __restrict__ pos_grad) {
  const int v = blockIdx.x, lane = threadIdx.x;
  float s[3] = {0.f, 0.f, 0.f};
  for (int i = t_rowptr[v] + lane; i < t_rowptr[v + 1]; i += kWave) {
    const int e = t_edge[i];
    s[0] += q[3 * (size_t)e];
    s[1] += q[3 * (size_t)e + 1];
    s[2] += q[3 * (size_t)e + 2];
  }
  for (int e = rowptr[v] + lane; e < rowptr[v + 1]; e += kWave) {
    s[0] -= q[3 * (size_t)e];
    s[1] -= q[3 * (size_t)e + 1];
    s[2] -= q[3 * (size_t)e + 2];
  }
#pragma unroll
  for (int i = 0; i < 3; ++i) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s[i] += __shfl_xor(s[i], o);
  }
  if (lane == 0) {
    pos_grad[3 * (size_t)v] += s[0];
    pos_grad[3 * (size_t)v + 1] += s[1];
    pos_grad[3 * (size_t)v + 2] += s[2];
  }
}

constexpr int kRadSplitTarget = 256;   // blocks per split-K weight-gradient GEMM

GemmProblem problem(int M, int N, int K, GView A, GView Bt, GOut C) {
  GemmProblem p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.alpha = 1.f;
  p.A = A;
  p.Bt = Bt;
  p.C = C;
  p.C2 = no_out();
  p.ksplit = 1;
  return p;
}

}  // namespace

void launch_radial_hidden(const RadialArgs& a, float* h2t, hipStream_t st) {
  if (a.E == 0) return;
  hipLaunchKernelGGL(radial_hidden_kernel, dim3((a.E + kRadBlock - 1) / kRadBlock), dim3(kRadBlock), 0, st, a.E,
                     a.r_max, a.receiver, a.sender, a.pos, a.shift, a.weights, h2t, radial_ld(a.E));
}

void launch_radial_out(const RadialArgs& a, const float* h2t, float* w, hipStream_t st) {
  if (a.E == 0) return;
  const long long PC = (long long)a.P * a.C;
  const float* W3 = a.weights + kW1 + kW2;
  GemmGroup g{};
  // the first E4 = 4 floor(E / 4) edges with 128-bit operand loads, the rest
  // (at most three) with scalar ones
  const int ld = radial_ld(a.E), E4 = a.E / 4 * 4;
  if (E4 > 0)
    g.prob[g.count++] = problem(E4, (int)PC, kRadHidden, plain_view_t(h2t, ld), plain_view_t(W3, PC),
                                plain_out(w, PC, 0));
  if (a.E > E4)
    g.prob[g.count++] = problem(a.E - E4, (int)PC, kRadHidden, plain_view_t(h2t + E4, ld), plain_view_t(W3, PC),
                                plain_out(w + (size_t)E4 * PC, PC, 0));
  gemm_group(g, st);
}

void launch_radial_hidden_rows(const RadialArgs& a, float* hh, hipStream_t st) {
  if (a.E == 0) return;
  hipLaunchKernelGGL(radial_hidden_rows_kernel, dim3((a.E + kRadBlock - 1) / kRadBlock), dim3(kRadBlock), 0, st,
                     a.E, a.r_max, a.receiver, a.sender, a.pos, a.shift, a.weights, hh);
}

size_t radial_vjp_scratch_floats(int E, int P, int C) {
  const size_t PC = (size_t)P * C;
  size_t part = (size_t)gemm_ksplit(kRadHidden, (int)PC, E, kRadSplitTarget) * kRadHidden * PC;
  const size_t p2 = (size_t)gemm_ksplit(kRadHidden, kRadHidden, E, kRadSplitTarget) * kW2 +
                    (size_t)gemm_ksplit(kRadFeat, kRadHidden, E, kRadSplitTarget) * kW1;
  if (p2 > part) part = p2;
  return (size_t)E * kRadHidden * 4 + (size_t)E * kRadFeat + part;
}

void launch_radial_vjp(const RadialArgs& a, const float* h2t, const float* w_bar, float* q, float* pos_grad,
                       float* w_grad, float* scratch, hipStream_t st) {
  if (a.E == 0) {
    if (w_grad) launch_zero(radial_weight_floats(a.P, a.C), w_grad, st);
    return;
  }
  const int E = a.E;
  const long long PC = (long long)a.P * a.C;
  const float* W3 = a.weights + kW1 + kW2;
  float* hbar = scratch;
  float* a2bt = hbar + (size_t)E * kRadHidden;
  float* h1t = a2bt + (size_t)E * kRadHidden;
  float* a1bt = h1t + (size_t)E * kRadHidden;
  float* phit = a1bt + (size_t)E * kRadHidden;
  float* part = phit + (size_t)E * kRadFeat;
  {  // hbar = w_bar W3^T; W3_bar = h2^T w_bar
    GemmGroup g{};
    g.prob[g.count++] = problem(E, kRadHidden, (int)PC, plain_view(w_bar, PC), plain_view(W3, PC),
                                plain_out(hbar, kRadHidden, 0));
    if (w_grad) {
      GemmProblem d = problem(kRadHidden, (int)PC, E, plain_view(h2t, radial_ld(E)), plain_view_t(w_bar, PC),
                              plain_out(w_grad + kW1 + kW2, PC, 0));
      d.ksplit = gemm_ksplit(d.M, d.N, d.K, kRadSplitTarget);
      d.part = part;
      g.prob[g.count++] = d;
    }
    gemm_group(g, st);
  }
  hipLaunchKernelGGL(radial_back_kernel, dim3((E + kRadBlock - 1) / kRadBlock), dim3(kRadBlock), 0, st, E, a.r_max,
                     a.receiver, a.sender, a.pos, a.shift, a.weights, (const float*)hbar, q,
                     w_grad ? a2bt : nullptr, h1t, w_grad ? a1bt : nullptr, w_grad ? phit : nullptr);
  if (w_grad) {  // W2_bar = h1^T a2_bar; W1_bar = phi^T a1_bar
    GemmGroup g{};
    GemmProblem d2 = problem(kRadHidden, kRadHidden, E, plain_view(h1t, E), plain_view(a2bt, E),
                             plain_out(w_grad + kW1, kRadHidden, 0));
    d2.ksplit = gemm_ksplit(d2.M, d2.N, d2.K, kRadSplitTarget);
    d2.part = part;
    GemmProblem d1 = problem(kRadFeat, kRadHidden, E, plain_view(phit, E), plain_view(a1bt, E),
                             plain_out(w_grad, kRadHidden, 0));
    d1.ksplit = gemm_ksplit(d1.M, d1.N, d1.K, kRadSplitTarget);
    d1.part = part + (size_t)d2.ksplit * kW2;
    g.prob[g.count++] = d2;
    g.prob[g.count++] = d1;
    gemm_group(g, st);
  }
  if (pos_grad)
    hipLaunchKernelGGL(radial_pos_kernel, dim3(a.N), dim3(kWave), 0, st, a.N, a.rowptr, a.t_rowptr, a.t_edge,
                       (const float*)q, pos_grad);
}

}  // namespace fc
