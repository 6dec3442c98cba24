// Equivariant RMS normalisation of node features for gfx950 (FlashCart
// paper, App. E "Model architecture": scalar invariants from the generated
// (l, l) -> 0 couplings, combined over ranks and channels into one scale per
// atom, without batch statistics).  With q[u, l, k] = f_(l,l)->0(x_l, x_l):
//   s[u] = sqrt(sum_{l,k} q[u, l, k] / ((l_max + 1) C) + eps),
//   y[u, l, k] = gamma[l, k] x[u, l, k] / s[u],
// and for L = <g, y>, with B[u] = sum <g, gamma x> and (K x) the symmetric
// (l, l) -> 0 form applied to x:
//   x_bar = gamma g / s - B (K x) / (s^3 (l_max + 1) C),
//   gamma_bar[l, k] = sum_u <g, x>[u, l, k] / s[u].
// One wave per node, channels across lanes; the node's rows are read twice
// (the second time from cache).  Wave sums use a butterfly, which leaves
// the same bits in every lane.
#include "fc_norm.h"

#include "fc_common.h"
#include "fc_reduce.h"

namespace fc {
namespace {

inline constexpr int kNormWaves = 4;

// sum over ranks l <= LMAX of the (l, l) -> 0 invariant of one channel
template <int LMAX>
__device__ __forceinline__ float invariant_sum(const float* xv) {
  float q = 0.f;
  static_for<LMAX + 1>([&](auto li) {
    constexpr int l = li, o = rank_off(l), t = path_type(l, l, 0);
    constexpr int tb = tab::kTermBegin[t], te = tab::kTermBegin[t + 1];
    static_for<te - tb>([&](auto ti) {
      constexpr tab::Term T = tab::kTerms[tb + ti];
      q = fmaf(T.c * xv[o + T.b1], xv[o + T.b2], q);
    });
  });
  return q;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int LMAX>
__global__ __launch_bounds__(kNormWaves * kWave) void rms_norm_fwd_kernel(int N, int C, float eps,
                                                                          const float* __restrict__ x,
                                                                          const float* __restrict__ gamma,
                                                                          float* __restrict__ y,
                                                                          float* __restrict__ inv_s) {
  constexpr int R = nrank(LMAX);
  const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int u = blockIdx.x * kNormWaves + wv;
  if (u >= N) return;   // whole waves; the kernel has no barrier
  const float* xu = x + (size_t)u * R * C;
  float q = 0.f;
  for (int k = lane; k < C; k += kWave) {
    float xv[R];
    static_for<R>([&](auto r) { xv[r] = xu[(size_t)r * C + k]; });
    q += invariant_sum<LMAX>(xv);
  }
  q = wave_sum(q);
  const float is = 1.f / sqrtf(q / float((LMAX + 1) * C) + eps);
  if (inv_s && lane == 0) inv_s[u] = is;
  float* yu = y + (size_t)u * R * C;
  for (int k = lane; k < C; k += kWave) {
    static_for<LMAX + 1>([&](auto li) {
      constexpr int l = li;
      const float sc = (gamma ? gamma[(size_t)l * C + k] : 1.f) * is;
      static_for<ncomp(l)>([&](auto c) {
        constexpr int r = rank_off(l) + c;
        yu[(size_t)r * C + k] = xu[(size_t)r * C + k] * sc;
      });
    });
  }
}

template <int LMAX>
__global__ __launch_bounds__(kNormWaves * kWave) void rms_norm_vjp_kernel(
    int N, int C, const float* __restrict__ x, const float* __restrict__ gamma, const float* __restrict__ inv_s,
    const float* __restrict__ g, float* __restrict__ xb, float* __restrict__ part) {
  constexpr int R = nrank(LMAX), NL = LMAX + 1;
  extern __shared__ float lds[];   // [kNormWaves][NL][C] when part is set
  const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  float* gp = lds + (size_t)wv * NL * C;
  if (part)   // each lane clears the entries it accumulates
    for (int l = 0; l < NL; ++l)
      for (int k = lane; k < C; k += kWave) gp[l * C + k] = 0.f;
  const float inv_den = 1.f / float(NL * C);
  for (int u = blockIdx.x * kNormWaves + wv; u < N; u += gridDim.x * kNormWaves) {
    const float is = inv_s[u];
    const float* xu = x + (size_t)u * R * C;
    const float* gu = g + (size_t)u * R * C;
    float B = 0.f;
    for (int k = lane; xb && k < C; k += kWave) {
      static_for<NL>([&](auto li) {
        constexpr int l = li;
        float t = 0.f;
        static_for<ncomp(l)>([&](auto c) {
          constexpr int r = rank_off(l) + c;
          t = fmaf(gu[(size_t)r * C + k], xu[(size_t)r * C + k], t);
        });
        B = fmaf(gamma ? gamma[(size_t)l * C + k] : 1.f, t, B);
      });
    }
    B = wave_sum(B);
    const float coef = B * is * is * is * inv_den;
    float* xo = xb ? xb + (size_t)u * R * C : nullptr;
    for (int k = lane; k < C; k += kWave) {
      float xv[R], gv[R];
      static_for<R>([&](auto r) {
        xv[r] = xu[(size_t)r * C + k];
        gv[r] = gu[(size_t)r * C + k];
      });
      static_for<NL>([&](auto li) {
        constexpr int l = li, o = rank_off(l), t = path_type(l, l, 0);
        constexpr int tb = tab::kTermBegin[t], te = tab::kTermBegin[t + 1];
        float kx[ncomp(l)];
        static_for<ncomp(l)>([&](auto c) { kx[c] = 0.f; });
        static_for<te - tb>([&](auto ti) {
          constexpr tab::Term T = tab::kTerms[tb + ti];
          kx[T.b1] = fmaf(0.5f * T.c, xv[o + T.b2], kx[T.b1]);
          kx[T.b2] = fmaf(0.5f * T.c, xv[o + T.b1], kx[T.b2]);
        });
        const float gs = (gamma ? gamma[(size_t)l * C + k] : 1.f) * is;
        float gx = 0.f;
        static_for<ncomp(l)>([&](auto c) {
          if (xb) xo[(size_t)(o + c) * C + k] = fmaf(gs, gv[o + c], -coef * kx[c]);
          gx = fmaf(gv[o + c], xv[o + c], gx);
        });
        if (part) gp[l * C + k] = fmaf(gx, is, gp[l * C + k]);
      });
    }
  }
  if (!part) return;
  __syncthreads();
  const float* w0 = lds;
  float* dst = part + (size_t)blockIdx.x * NL * C;
  for (int i = threadIdx.x; i < NL * C; i += kNormWaves * kWave) {
    float t = w0[i];
#pragma unroll
    for (int w = 1; w < kNormWaves; ++w) t += w0[(size_t)w * NL * C + i];
    dst[i] = t;
  }
}

template <int LMAX>
void fwd_l(int N, int C, float eps, const float* x, const float* gamma, float* y, float* inv_s, hipStream_t st) {
  hipLaunchKernelGGL(rms_norm_fwd_kernel<LMAX>, dim3((N + kNormWaves - 1) / kNormWaves), dim3(kNormWaves * kWave), 0,
                     st, N, C, eps, x, gamma, y, inv_s);
}

template <int LMAX>
void vjp_l(int N, int C, const float* x, const float* gamma, const float* inv_s, const float* g, float* xb,
           float* part, float* gamma_grad, hipStream_t st) {
  const int nblk = rms_norm_vjp_blocks(N);
  const size_t lds = part ? sizeof(float) * kNormWaves * (LMAX + 1) * C : 0;
  hipLaunchKernelGGL(rms_norm_vjp_kernel<LMAX>, dim3(nblk), dim3(kNormWaves * kWave), lds, st, N, C, x, gamma, inv_s,
                     g, xb, part);
  if (part) launch_block_sum(nblk, (LMAX + 1) * C, part, gamma_grad, st);
}

}  // namespace

int rms_norm_vjp_blocks(int N) {
  const int b = (N + kNormWaves - 1) / kNormWaves;
  return b < 1024 ? b : 1024;
}

void launch_rms_norm_fwd(int l_max, int N, int C, float eps, const float* x, const float* gamma, float* y,
                         float* inv_s, hipStream_t st) {
  switch (l_max) {
    case 0: fwd_l<0>(N, C, eps, x, gamma, y, inv_s, st); break;
    case 1: fwd_l<1>(N, C, eps, x, gamma, y, inv_s, st); break;
    case 2: fwd_l<2>(N, C, eps, x, gamma, y, inv_s, st); break;
    case 3: fwd_l<3>(N, C, eps, x, gamma, y, inv_s, st); break;
    case 4: fwd_l<4>(N, C, eps, x, gamma, y, inv_s, st); break;
    default: fwd_l<5>(N, C, eps, x, gamma, y, inv_s, st); break;
  }
}

void launch_rms_norm_vjp(int l_max, int N, int C, const float* x, const float* gamma, const float* inv_s,
                         const float* g, float* x_grad, float* part, float* gamma_grad, hipStream_t st) {
  switch (l_max) {
    case 0: vjp_l<0>(N, C, x, gamma, inv_s, g, x_grad, part, gamma_grad, st); break;
    case 1: vjp_l<1>(N, C, x, gamma, inv_s, g, x_grad, part, gamma_grad, st); break;
    case 2: vjp_l<2>(N, C, x, gamma, inv_s, g, x_grad, part, gamma_grad, st); break;
    case 3: vjp_l<3>(N, C, x, gamma, inv_s, g, x_grad, part, gamma_grad, st); break;
    case 4: vjp_l<4>(N, C, x, gamma, inv_s, g, x_grad, part, gamma_grad, st); break;
    default: vjp_l<5>(N, C, x, gamma, inv_s, g, x_grad, part, gamma_grad, st); break;
  }
}

}  // namespace fc
