// Edge convolution kernels for gfx950: forward (receiver-sorted, FlashCart
// paper §4 Eq. 1) and VJP (App. C Eq. C1 with the chain rule to positions),
// the VJP run sender-sorted so that every output is written exactly once.
//
// Mapping: one wavefront per (node, 64-channel tile); channel k lives in lane
// k % 64, so every gather of a neighbour row is one coalesced 256-byte
// transaction per stored component.  Per-edge geometry (direction tensor
// components, Bessel radial values, neighbour id) is computed once per edge
// by a lane of its own (lane j <-> edge j of a 64-edge chunk), parked in LDS
// and read back by all 64 lanes as a broadcast, so it is shared by all
// channels.  The coupling polynomials come from the generated tables and are
// fully unrolled; all accumulators stay in VGPRs.
#pragma once

#include "fc_conv.h"

namespace fc {

// Largest number of output rows one launch accumulates per lane (the pages
// group output ranks to about 100 stored components per channel).
inline constexpr int kGroupRows = 100;
// Channels of one VJP block: up to 4 waves (C <= 256).
inline constexpr int kMaxVjpWaves = 4;

template <class Cfg, int LOUT>
constexpr int group_end(int lo) {
  int rows = 0, hi = lo;
  for (int L = lo; L <= LOUT; ++L) {
    const int r = ncomp(L) * Cfg::count_L(L);
    if (L > lo && rows + r > kGroupRows) break;
    rows += r;
    hi = L;
  }
  return hi;
}

// ============================================================== forward ====
template <int LIN, int LEDGE, int LOUT, int LLO, int LHI>
__global__ __launch_bounds__(kWave) void conv_fwd_kernel(
    int C, const int* __restrict__ rowptr, const int* __restrict__ sender,
    const float* __restrict__ pos, const float* __restrict__ shift,
    const float* __restrict__ x, const float* __restrict__ W, float* __restrict__ z, float rc) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using G = Group<Cfg, LLO, LHI>;
  constexpr int NIN = Cfg::NIN, NE = Cfg::NE, P = Cfg::P, NOUT = Cfg::NOUT;
  constexpr int REC = NE + kNB + 1;
  constexpr bool WREG = kNB * G::NP <= 128;
  __shared__ float geo[kWave * REC];

  const int u = blockIdx.x;
  const int lane = threadIdx.x;
  const int k = blockIdx.y * kWave + lane;
  const bool act = k < C;
  const int kk = act ? k : 0;

  float Wr[WREG ? kNB * G::NP : 1];
  if constexpr (WREG) {
    static_for<kNB * G::NP>([&](auto i) {
      constexpr int b = i / G::NP, p = i % G::NP;
      Wr[i] = W[(size_t)(b * P + G::p0 + p) * C + kk];
    });
  }
  float acc[G::NR];
  static_for<G::NR>([&](auto i) { acc[i] = 0.f; });

  const int e0 = rowptr[u], e1 = rowptr[u + 1];
  const float pux = pos[3 * u], puy = pos[3 * u + 1], puz = pos[3 * u + 2];
  for (int base = e0; base < e1; base += kWave) {
    const int cnt = min(kWave, e1 - base);
    if (lane < cnt) {
      const int e = base + lane;
      const int s = sender[e];
      float rx = pos[3 * s] - pux, ry = pos[3 * s + 1] - puy, rz = pos[3 * s + 2] - puz;
      if (shift) {
        rx += shift[3 * e];
        ry += shift[3 * e + 1];
        rz += shift[3 * e + 2];
      }
      const float r = sqrtf(rx * rx + ry * ry + rz * rz);
      const float inv = r > 0.f ? 1.f / r : 0.f;
      float y[NE], R[kNB];
      direction_tensors<LEDGE>(rx * inv, ry * inv, rz * inv, y);
      radial<false>(r, rc, R, nullptr);
      float* rec = geo + lane * REC;
      static_for<NE>([&](auto c) { rec[c] = y[c]; });
      static_for<kNB>([&](auto b) { rec[NE + b] = R[b]; });
      rec[NE + kNB] = __int_as_float(s);
    }
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const float* rec = geo + j * REC;
      const int s = uniform_int(__float_as_int(rec[NE + kNB]));
      const float* xs = x + (size_t)s * NIN * C + kk;
      float xv[NIN], y[NE], R[kNB];
      static_for<NIN>([&](auto c) { xv[c] = xs[(size_t)c * C]; });
      static_for<NE>([&](auto c) { y[c] = rec[c]; });
      static_for<kNB>([&](auto b) { R[b] = rec[NE + b]; });
      static_for<G::NP>([&](auto pi) {
        constexpr int p = G::p0 + pi;
        constexpr PathInfo PI = Cfg::paths[p];
        float w = 0.f;
        static_for<kNB>([&](auto b) {
          float wb;
          if constexpr (WREG) wb = Wr[b * G::NP + pi];
          else wb = W[(size_t)(b * P + p) * C + kk];
          w = fmaf(R[b], wb, w);
        });
        constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
        float t[ncomp(PI.L)];
        static_for<ncomp(PI.L)>([&](auto a) { t[a] = 0.f; });
        static_for<te - tb>([&](auto ti) {
          constexpr tab::Term T = tab::kTerms[tb + ti];
          t[T.a] = fmaf(T.c * y[rank_off(PI.l2) + T.b2], xv[rank_off(PI.l1) + T.b1], t[T.a]);
        });
        static_for<ncomp(PI.L)>([&](auto a) {
          constexpr int row = Cfg::row(p, a) - G::r0;
          acc[row] = fmaf(w, t[a], acc[row]);
        });
      });
    }
    __syncthreads();
  }
  if (act) {
    float* zo = z + (size_t)u * NOUT * C + k;
    static_for<G::NR>([&](auto i) { zo[(size_t)(G::r0 + i) * C] = acc[i]; });
  }
}

template <int LIN, int LEDGE, int LOUT, int LLO>
void launch_fwd_groups(const ConvArgs& a, hipStream_t st) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  constexpr int LHI = group_end<Cfg, LOUT>(LLO);
  dim3 grid(a.N, (a.C + kWave - 1) / kWave);
  hipLaunchKernelGGL((conv_fwd_kernel<LIN, LEDGE, LOUT, LLO, LHI>), grid, dim3(kWave), 0, st,
                     a.C, a.rowptr, a.sender, a.pos, a.shift, a.x, a.W, a.z, a.rc);
  if constexpr (LHI < LOUT) launch_fwd_groups<LIN, LEDGE, LOUT, LHI + 1>(a, st);
}

// ================================================================== VJP ====
// Sender-sorted pass: block = NW = ceil(C/64) waves covering all C channels
// of sender v (C <= 256).
// For every outgoing edge e = (v -> u): gather g[u], then
//   x_bar[v]  += sum_p w_p VJP1_p(g_p, y)                  (per lane)
//   y_bar_e   = sum_{p,k} w_p VJP2_p(g_p, x_v)             (across lanes)
//   rho_e[b]  = sum_{p,k} <g_p, f_p(x_v, y)> W[b,p,k]      (across lanes)
// and the edge's position cotangent
//   r_bar_e = (sum_b dR_b/dr rho_b) r_hat + (I - r_hat r_hat^T)/r (sum_c y_bar_c grad_n y_c),
// which is added to the sender here and stored per edge for the receiver pass.
template <int LIN, int LEDGE, int LOUT, bool NEED_X, bool NEED_POS>
__global__ __launch_bounds__(kMaxVjpWaves * kWave) void conv_vjp_sender_kernel(
    int C, const int* __restrict__ t_rowptr, const int* __restrict__ t_edge,
    const int* __restrict__ receiver, const float* __restrict__ pos,
    const float* __restrict__ shift, const float* __restrict__ x,
    const float* __restrict__ W, const float* __restrict__ g, float* __restrict__ x_bar,
    float* __restrict__ pos_bar, float* __restrict__ rbar, float rc) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  constexpr int NIN = Cfg::NIN, NE = Cfg::NE, P = Cfg::P, NOUT = Cfg::NOUT;
  constexpr int REC = NE + kNB + 1;
  constexpr int NRED = NE + kNB;
  constexpr bool WREG = kNB * P <= 128;
  __shared__ float geo[kWave * REC];
  __shared__ float red[NEED_POS ? kMaxVjpWaves * kWave * NRED : 1];
  const int NW = blockDim.x / kWave;

  const int v = blockIdx.x;
  const int tid = threadIdx.x;
  const int wv = tid / kWave, lane = tid % kWave;
  const int k = tid;
  const bool act = k < C;
  const int kk = act ? k : 0;

  float Wr[WREG ? kNB * P : 1];
  if constexpr (WREG) {
    static_for<kNB * P>([&](auto i) { Wr[i] = act ? W[(size_t)i * C + kk] : 0.f; });
  }
  float xv[NIN];
  {
    const float* xs = x + (size_t)v * NIN * C + kk;
    static_for<NIN>([&](auto c) { xv[c] = act ? xs[(size_t)c * C] : 0.f; });
  }
  float xb[NIN];
  static_for<NIN>([&](auto c) { xb[c] = 0.f; });
  float psum[3] = {0.f, 0.f, 0.f};

  const int e0 = t_rowptr[v], e1 = t_rowptr[v + 1];
  const float pvx = pos[3 * v], pvy = pos[3 * v + 1], pvz = pos[3 * v + 2];
  for (int base = e0; base < e1; base += kWave) {
    const int cnt = min(kWave, e1 - base);
    if (wv == 0 && lane < cnt) {
      const int e = t_edge[base + lane];
      const int u = receiver[e];
      float rx = pvx - pos[3 * u], ry = pvy - pos[3 * u + 1], rz = pvz - pos[3 * u + 2];
      if (shift) {
        rx += shift[3 * e];
        ry += shift[3 * e + 1];
        rz += shift[3 * e + 2];
      }
      const float r = sqrtf(rx * rx + ry * ry + rz * rz);
      const float inv = r > 0.f ? 1.f / r : 0.f;
      float y[NE], R[kNB];
      direction_tensors<LEDGE>(rx * inv, ry * inv, rz * inv, y);
      radial<false>(r, rc, R, nullptr);
      float* rec = geo + lane * REC;
      static_for<NE>([&](auto c) { rec[c] = y[c]; });
      static_for<kNB>([&](auto b) { rec[NE + b] = R[b]; });
      rec[NE + kNB] = __int_as_float(u);
    }
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const float* rec = geo + j * REC;
      const int u = uniform_int(__float_as_int(rec[NE + kNB]));
      const float* gs = g + (size_t)u * NOUT * C + kk;
      float y[NE], R[kNB];
      static_for<NE>([&](auto c) { y[c] = rec[c]; });
      static_for<kNB>([&](auto b) { R[b] = rec[NE + b]; });
      float yb[NE], rho[kNB];
      static_for<NE>([&](auto c) { yb[c] = 0.f; });
      static_for<kNB>([&](auto b) { rho[b] = 0.f; });
      static_for<P>([&](auto pc) {
        constexpr int p = pc;
        constexpr PathInfo PI = Cfg::paths[p];
        constexpr int na = ncomp(PI.L), n1 = ncomp(PI.l1), n2 = ncomp(PI.l2);
        constexpr int o1 = rank_off(PI.l1), o2 = rank_off(PI.l2);
        float gp[na];
        static_for<na>([&](auto a) { gp[a] = act ? gs[(size_t)Cfg::row(p, a) * C] : 0.f; });
        float w = 0.f;
        static_for<kNB>([&](auto b) {
          float wb;
          if constexpr (WREG) wb = Wr[b * P + p];
          else wb = act ? W[(size_t)(b * P + p) * C + kk] : 0.f;
          w = fmaf(R[b], wb, w);
        });
        constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
        if constexpr (NEED_X) {
          float v1[n1];
          static_for<n1>([&](auto c) { v1[c] = 0.f; });
          static_for<te - tb>([&](auto ti) {
            constexpr tab::Term T = tab::kTerms[tb + ti];
            v1[T.b1] = fmaf(T.c * y[o2 + T.b2], gp[T.a], v1[T.b1]);
          });
          static_for<n1>([&](auto c) { xb[o1 + c] = fmaf(w, v1[c], xb[o1 + c]); });
        }
        if constexpr (NEED_POS) {
          float v2[n2];
          static_for<n2>([&](auto c) { v2[c] = 0.f; });
          static_for<te - tb>([&](auto ti) {
            constexpr tab::Term T = tab::kTerms[tb + ti];
            v2[T.b2] = fmaf(T.c * gp[T.a], xv[o1 + T.b1], v2[T.b2]);
          });
          float wbar = 0.f;
          static_for<n2>([&](auto c) {
            yb[o2 + c] = fmaf(w, v2[c], yb[o2 + c]);
            wbar = fmaf(v2[c], y[o2 + c], wbar);
          });
          static_for<kNB>([&](auto b) {
            float wb;
            if constexpr (WREG) wb = Wr[b * P + p];
            else wb = act ? W[(size_t)(b * P + p) * C + kk] : 0.f;
            rho[b] = fmaf(wbar, wb, rho[b]);
          });
        }
      });
      if constexpr (NEED_POS) {
        // wave reduction of the per-lane partials, then park them in LDS
        float* dst = red + ((size_t)wv * kWave + j) * NRED;
        static_for<NE>([&](auto c) {
          float t = yb[c];
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
          if (lane == 0) dst[c] = t;
        });
        static_for<kNB>([&](auto b) {
          float t = rho[b];
#pragma unroll
          for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
          if (lane == 0) dst[NE + b] = t;
        });
      }
    }
    __syncthreads();
    if constexpr (NEED_POS) {
      if (wv == 0 && lane < cnt) {
        const int e = t_edge[base + lane];
        const int u = receiver[e];
        float tot[NRED];
        static_for<NRED>([&](auto i) { tot[i] = 0.f; });
        for (int w2 = 0; w2 < NW; ++w2) {
          const float* src = red + ((size_t)w2 * kWave + lane) * NRED;
          static_for<NRED>([&](auto i) { tot[i] += src[i]; });
        }
        float rx = pvx - pos[3 * u], ry = pvy - pos[3 * u + 1], rz = pvz - pos[3 * u + 2];
        if (shift) {
          rx += shift[3 * e];
          ry += shift[3 * e + 1];
          rz += shift[3 * e + 2];
        }
        const float r = sqrtf(rx * rx + ry * ry + rz * rz);
        float ox = 0.f, oy = 0.f, oz = 0.f;
        if (r > 0.f) {
          const float inv = 1.f / r;
          const float nx = rx * inv, ny = ry * inv, nz = rz * inv;
          float R[kNB], dR[kNB];
          radial<true>(r, rc, R, dR);
          float srad = 0.f;
          static_for<kNB>([&](auto b) { srad = fmaf(dR[b], tot[NE + b], srad); });
          float dy[3 * NE];
          direction_tensor_grads<LEDGE>(nx, ny, nz, dy);
          float gx = 0.f, gy = 0.f, gz = 0.f;
          static_for<NE>([&](auto c) {
            gx = fmaf(tot[c], dy[3 * c], gx);
            gy = fmaf(tot[c], dy[3 * c + 1], gy);
            gz = fmaf(tot[c], dy[3 * c + 2], gz);
          });
          const float gn = gx * nx + gy * ny + gz * nz;
          ox = srad * nx + (gx - gn * nx) * inv;
          oy = srad * ny + (gy - gn * ny) * inv;
          oz = srad * nz + (gz - gn * nz) * inv;
        }
        rbar[3 * (size_t)e] = ox;
        rbar[3 * (size_t)e + 1] = oy;
        rbar[3 * (size_t)e + 2] = oz;
        psum[0] += ox;
        psum[1] += oy;
        psum[2] += oz;
      }
      __syncthreads();
    }
  }
  if (NEED_X && x_bar && act) {
    float* xo = x_bar + (size_t)v * NIN * C + k;
    static_for<NIN>([&](auto c) { xo[(size_t)c * C] = xb[c]; });
  }
  if constexpr (NEED_POS) {
    if (wv == 0) {
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        float t = psum[i];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) t += __shfl_xor(t, o);
        psum[i] = t;
      }
      if (lane == 0) {
        pos_bar[3 * v] = psum[0];
        pos_bar[3 * v + 1] = psum[1];
        pos_bar[3 * v + 2] = psum[2];
      }
    }
  }
}

template <int LIN, int LEDGE, int LOUT>
void launch_vjp(const ConvArgs& a, hipStream_t st) {
  const bool nx = a.x_bar != nullptr, np = a.pos_bar != nullptr;
  const int nw = (a.C + kWave - 1) / kWave;
  dim3 grid(a.N), block(nw * kWave);
  if (nx && np)
    hipLaunchKernelGGL((conv_vjp_sender_kernel<LIN, LEDGE, LOUT, true, true>), grid, block, 0, st, a.C,
                       a.t_rowptr, a.t_edge, a.receiver, a.pos, a.shift, a.x, a.W, a.g, a.x_bar, a.pos_bar,
                       a.rbar, a.rc);
  else if (nx)
    hipLaunchKernelGGL((conv_vjp_sender_kernel<LIN, LEDGE, LOUT, true, false>), grid, block, 0, st, a.C,
                       a.t_rowptr, a.t_edge, a.receiver, a.pos, a.shift, a.x, a.W, a.g, a.x_bar, a.pos_bar,
                       a.rbar, a.rc);
  else
    hipLaunchKernelGGL((conv_vjp_sender_kernel<LIN, LEDGE, LOUT, false, true>), grid, block, 0, st, a.C,
                       a.t_rowptr, a.t_edge, a.receiver, a.pos, a.shift, a.x, a.W, a.g, a.x_bar, a.pos_bar,
                       a.rbar, a.rc);
  if (np) launch_vjp_receiver(a, st);
}

}  // namespace fc
