// VJP-of-VJP of the edge convolution for gfx950 (FlashCart paper, App. C
// Eq. C2, carried through the direction tensors and radial weights).
//
// For s = <v_x, x_bar> + <v_pos, pos_bar>, with per edge e = (u <- v)
//   dv_e = v_pos[v] - v_pos[u],   ydot = J_y dv_e,   wdot = w'(r) (r_hat . dv_e),
// the outputs are
//   g_hat[u]  = sum_{e into u} w (f(v_x, y) + f(x, ydot)) + wdot f(x, y)
//   x_hat[v]  = sum_{e out of v} VJP1(g_u, w ydot + wdot y)
//   pos_hat  += q_e at v, -= q_e at u, with q_e = d psi_e / d r_e,
//   q_e = S1 r_hat + J_y^T (Ya + nd Yd) + H_y[Yb] dv + S2 nd r_hat + S3 (dv - nd r_hat) / r,
// nd = r_hat . dv, and per-edge channel sums (beta = VJP2(g, x),
// alpha = VJP2(g, v_x)):
//   Ya = sum w alpha, Yb = sum w beta, Yd = sum w' beta,
//   S1 = sum w' (<alpha, y> + <beta, ydot>), S2 = sum w'' <beta, y>,
//   S3 = sum w' <beta, y>.
// g_hat runs receiver-sorted like the forward; x_hat and q_e run
// sender-sorted like the VJP and share its slice/combine passes.
#pragma once

#include "fc_conv_kernels.h"

namespace fc {

// Geometry of one edge: unit direction, length, dv and its derived terms.
struct VVGeo {
  float nx, ny, nz, r, inv, dvx, dvy, dvz, nd, ndx, ndy, ndz;   // ndot = (dv - nd n) / r
};

__device__ __forceinline__ VVGeo vv_geo(float rx, float ry, float rz, float dvx, float dvy, float dvz) {
  VVGeo G;
  G.r = sqrtf(rx * rx + ry * ry + rz * rz);
  G.inv = G.r > 0.f ? 1.f / G.r : 0.f;
  G.nx = rx * G.inv;
  G.ny = ry * G.inv;
  G.nz = rz * G.inv;
  G.dvx = dvx;
  G.dvy = dvy;
  G.dvz = dvz;
  G.nd = G.nx * dvx + G.ny * dvy + G.nz * dvz;
  G.ndx = (dvx - G.nd * G.nx) * G.inv;
  G.ndy = (dvy - G.nd * G.ny) * G.inv;
  G.ndz = (dvz - G.nd * G.nz) * G.inv;
  return G;
}

// y and ydot = J_y dv (= grad_n y . ndot) for all ranks <= LE.
template <int LE>
__device__ __forceinline__ void vv_tensors(const VVGeo& G, float* y, float* yd) {
  constexpr int NE = nrank(LE);
  direction_tensors<LE>(G.nx, G.ny, G.nz, y);
  float dy[3 * NE];
  direction_tensor_grads<LE>(G.nx, G.ny, G.nz, dy);
  static_for<NE>([&](auto c) { yd[c] = dy[3 * c] * G.ndx + dy[3 * c + 1] * G.ndy + dy[3 * c + 2] * G.ndz; });
}

// ------------------------------------------------------------ g_hat pass --
__host__ __device__ constexpr int vv_recv_budget(int nin) { return 200 - 3 * nin; }

// XW: per-edge weights W = w [E][P][C] with the weight cotangent vw (same
// layout, nullable) in place of the radial weights (Alg. 3's interface):
// w_dot = vw instead of w'(r) nd, and an edge of zero length takes no part.
template <int LIN, int LEDGE, int LOUT, int P0, int P1, bool HAS_VX, bool XW = false>
__global__ __launch_bounds__(kWave) void conv_vv_recv_kernel(
    int N, int C, const int* __restrict__ rowptr, const int* __restrict__ sender, const float* __restrict__ pos,
    const float* __restrict__ shift, const float* __restrict__ x, const float* __restrict__ W,
    const float* __restrict__ v_x, const float* __restrict__ v_pos, float* __restrict__ g_hat, float rc,
    const float* __restrict__ vw = nullptr) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using G = PathGroup<Cfg, P0, P1>;
  constexpr int NIN = Cfg::NIN, NE = Cfg::NE, P = Cfg::P, NOUT = Cfg::NOUT;
  constexpr int REC = 2 * NE + 2 * kNB + 2;   // y, ydot, R, R', nd, sender
  __shared__ float geo[kWave * REC];

  const int u = xcd_node(blockIdx.x, N);
  const int lane = threadIdx.x;
  const int k = blockIdx.y * kWave + lane;
  const bool act = k < C;
  const int kk = act ? k : 0;
  const int voff = kk * 4;

  float Wr[XW ? 1 : kNB * G::NP];
  if constexpr (!XW) {
    static_for<kNB * G::NP>([&](auto i) {
      constexpr int b = i / G::NP, p = i % G::NP;
      Wr[i] = W[(size_t)(b * P + P0 + p) * C + kk];
    });
  }
  float acc[G::NR];
  static_for<G::NR>([&](auto i) { acc[i] = 0.f; });

  const int e0 = rowptr[u], e1 = rowptr[u + 1];
  const float pux = pos[3 * u], puy = pos[3 * u + 1], puz = pos[3 * u + 2];
  const float vux = v_pos ? v_pos[3 * u] : 0.f, vuy = v_pos ? v_pos[3 * u + 1] : 0.f,
              vuz = v_pos ? v_pos[3 * u + 2] : 0.f;
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
      float dvx = 0.f, dvy = 0.f, dvz = 0.f;
      if (v_pos) {
        dvx = v_pos[3 * s] - vux;
        dvy = v_pos[3 * s + 1] - vuy;
        dvz = v_pos[3 * s + 2] - vuz;
      }
      const VVGeo Gm = vv_geo(rx, ry, rz, dvx, dvy, dvz);
      float y[NE], yd[NE];
      vv_tensors<LEDGE>(Gm, y, yd);
      float* rec = geo + lane * REC;
      static_for<NE>([&](auto c) {
        rec[c] = y[c];
        rec[NE + c] = yd[c];
      });
      if constexpr (XW) {
        rec[2 * NE] = Gm.r > 0.f ? 1.f : 0.f;
      } else {
        float R[kNB], dR[kNB];
        radial<true>(Gm.r, rc, R, dR);
        static_for<kNB>([&](auto b) {
          rec[2 * NE + b] = R[b];
          rec[2 * NE + kNB + b] = dR[b];
        });
      }
      rec[2 * NE + 2 * kNB] = Gm.nd;
      rec[2 * NE + 2 * kNB + 1] = __int_as_float(s);
    }
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const float* rec = geo + j * REC;
      const int s = uniform_int(__float_as_int(rec[2 * NE + 2 * kNB + 1]));
      const float nd = rec[2 * NE + 2 * kNB];
      const auto xs = node_rsrc(x, s, NIN * C);
      const auto vs = node_rsrc(HAS_VX ? v_x : x, s, NIN * C);
      float xv[NIN], vx[HAS_VX ? NIN : 1];
      static_for<NIN>([&](auto c) { xv[c] = buf_load(xs, voff, c * C * 4); });
      if constexpr (HAS_VX) static_for<NIN>([&](auto c) { vx[c] = buf_load(vs, voff, c * C * 4); });
      float we[XW ? G::NP : 1], wve[XW ? G::NP : 1];
      if constexpr (XW) {
        const float valid = rec[2 * NE];
        const size_t erow = (size_t)(base + j) * P * C + kk;
        static_for<G::NP>([&](auto pi) {
          we[pi] = valid * W[erow + (size_t)(P0 + pi) * C];
          wve[pi] = vw ? valid * vw[erow + (size_t)(P0 + pi) * C] : 0.f;
        });
      }
      static_for<G::NP>([&](auto pi) {
        constexpr int p = P0 + pi;
        constexpr PathInfo PI = Cfg::paths[p];
        constexpr int n1 = ncomp(PI.l1), o1 = rank_off(PI.l1), o2 = rank_off(PI.l2);
        constexpr int lo = G::loff(p);
        float w = 0.f, w1 = 0.f;
        if constexpr (XW) {
          w = we[pi];
        } else {
          static_for<kNB>([&](auto b) {
            constexpr int bb = b;
            const float wb = Wr[bb * G::NP + pi];
            w = fmaf(rec[2 * NE + bb], wb, w);
            w1 = fmaf(rec[2 * NE + kNB + bb], wb, w1);
          });
        }
        const float wd = XW ? wve[pi] : w1 * nd;
        float xw[n1], xd[n1], vxw[HAS_VX ? n1 : 1];
        static_for<n1>([&](auto c) {
          xw[c] = w * xv[o1 + c];
          xd[c] = wd * xv[o1 + c];
          if constexpr (HAS_VX) vxw[c] = w * vx[o1 + c];
        });
        constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
        static_for<te - tb>([&](auto ti) {
          constexpr tab::Term T = tab::kTerms[tb + ti];
          const float cy = T.c * rec[o2 + T.b2];
          const float cyd = T.c * rec[NE + o2 + T.b2];
          float a = fmaf(cy, xd[T.b1], acc[lo + T.a]);
          a = fmaf(cyd, xw[T.b1], a);
          if constexpr (HAS_VX) a = fmaf(cy, vxw[T.b1], a);
          acc[lo + T.a] = a;
        });
      });
    }
    __syncthreads();
  }
  if (act) {
    float* zo = g_hat + (size_t)u * NOUT * C + k;
    static_for<G::NP>([&](auto pi) {
      constexpr int p = P0 + pi;
      if constexpr (!G::owner(p)) return;
      static_for<ncomp(Cfg::paths[p].L)>([&](auto c) {
        constexpr int row = Cfg::row(p, c), li = G::loff(p) + c;
        if constexpr (G::carry(p)) zo[(size_t)row * C] += acc[li];
        else zo[(size_t)row * C] = acc[li];
      });
    });
  }
}

template <int LIN, int LEDGE, int LOUT, bool XW = false>
void launch_vv_recv(const ConvArgs& a, hipStream_t st) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using GS = PathGroups<Cfg, vv_recv_budget(Cfg::NIN)>;
  dim3 grid(a.N, (a.C + kWave - 1) / kWave);
  const float* Wt = XW ? a.w_edge : a.W;
  static_for<GS::n>([&](auto gi) {
    constexpr int p0 = GS::start[gi], p1 = GS::start[gi + 1];
    if (a.v_x)
      hipLaunchKernelGGL((conv_vv_recv_kernel<LIN, LEDGE, LOUT, p0, p1, true, XW>), grid, dim3(kWave), 0, st, a.N,
                         a.C, a.rowptr, a.sender, a.pos, a.shift, a.x, Wt, a.v_x, a.v_pos, a.g_hat, a.rc,
                         a.v_w_edge);
    else
      hipLaunchKernelGGL((conv_vv_recv_kernel<LIN, LEDGE, LOUT, p0, p1, false, XW>), grid, dim3(kWave), 0, st, a.N,
                         a.C, a.rowptr, a.sender, a.pos, a.shift, a.x, Wt, a.v_x, a.v_pos, a.g_hat, a.rc,
                         a.v_w_edge);
  });
}

// --------------------------------------------------------- W_hat pass --
// W_hat[b, p, k] = d W_bar[b, p, k] / d eps along (v_x, v_pos):
//   sum_e R'_b nd <g_u, f_p(x_v, y)> + R_b <g_u, f_p(x_v, ydot) + f_p(v_x[v], y)>,
// nd = r_hat . dv_e, ydot = J_y dv_e.  Same block shape and fixed-order
// reduction as the W_bar pass; edges are staged 32 per chunk so that the
// four waves' records (y, ydot, R, R' nd, sender) fit in LDS at rank 4.
inline constexpr int kWhChunk = 32;
// path-group budget: g (2L+1) and kNB accumulators per path, below the g_hat
// pass's budget by the per-path f and f-dot temporaries
__host__ __device__ constexpr int wgrad_vv_budget(int nin) { return 176 - 3 * nin; }

template <int LIN, int LEDGE, int LOUT, int P0, int P1, bool HAS_VX>
__global__ __launch_bounds__(kWgWaves * kWave) void conv_wgrad_vv_kernel(
    int N, int C, const int* __restrict__ rowptr, const int* __restrict__ sender, const float* __restrict__ pos,
    const float* __restrict__ shift, const float* __restrict__ x, const float* __restrict__ g,
    const float* __restrict__ v_x, const float* __restrict__ v_pos, float* __restrict__ wpart, float rc) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using G = PathGroup<Cfg, P0, P1>;
  constexpr int NIN = Cfg::NIN, NE = Cfg::NE, P = Cfg::P, NOUT = Cfg::NOUT;
  constexpr int REC = 2 * NE + 2 * kNB + 1;   // y, ydot, R, R' nd, sender
  constexpr int NACC = kNB * G::NP;
  constexpr int LDS = (kWgWaves * kWhChunk * REC > kWave * NACC) ? kWgWaves * kWhChunk * REC : kWave * NACC;
  __shared__ float lds[LDS];

  const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int u0 = blockIdx.x * kWgWaves, u = u0 + wv;
  const bool has_u = u < N;
  const int k = blockIdx.y * kWave + lane;
  const bool act = k < C;
  const int kk = act ? k : 0;
  const int voff = kk * 4;
  float* geo = lds + wv * kWhChunk * REC;

  float gv[G::NR];
  static_for<G::NP>([&](auto pi) {
    constexpr int p = P0 + pi;
    if constexpr (!G::owner(p)) return;
    static_for<ncomp(Cfg::paths[p].L)>([&](auto c) {
      constexpr int row = Cfg::row(p, c), li = G::loff(p) + c;
      gv[li] = (act && has_u) ? g[((size_t)u * NOUT + row) * C + k] : 0.f;
    });
  });
  float acc[NACC];
  static_for<NACC>([&](auto i) { acc[i] = 0.f; });

  int nch = 0;
  for (int i = 0; i < kWgWaves; ++i)
    if (u0 + i < N) nch = max(nch, (rowptr[u0 + i + 1] - rowptr[u0 + i] + kWhChunk - 1) / kWhChunk);
  const int e0 = has_u ? rowptr[u] : 0, e1 = has_u ? rowptr[u + 1] : 0;
  const float pux = has_u ? pos[3 * u] : 0.f, puy = has_u ? pos[3 * u + 1] : 0.f, puz = has_u ? pos[3 * u + 2] : 0.f;
  const bool vp = v_pos != nullptr && has_u;
  const float vux = vp ? v_pos[3 * u] : 0.f, vuy = vp ? v_pos[3 * u + 1] : 0.f, vuz = vp ? v_pos[3 * u + 2] : 0.f;
  for (int ch = 0; ch < nch; ++ch) {
    const int base = e0 + ch * kWhChunk;
    const int cnt = max(0, min(kWhChunk, e1 - base));
    if (lane < cnt) {
      const int e = base + lane;
      const int s = sender[e];
      float rx = pos[3 * s] - pux, ry = pos[3 * s + 1] - puy, rz = pos[3 * s + 2] - puz;
      if (shift) {
        rx += shift[3 * e];
        ry += shift[3 * e + 1];
        rz += shift[3 * e + 2];
      }
      float dvx = 0.f, dvy = 0.f, dvz = 0.f;
      if (vp) {
        dvx = v_pos[3 * s] - vux;
        dvy = v_pos[3 * s + 1] - vuy;
        dvz = v_pos[3 * s + 2] - vuz;
      }
      const VVGeo Gm = vv_geo(rx, ry, rz, dvx, dvy, dvz);
      float y[NE], yd[NE], R[kNB], dR[kNB];
      vv_tensors<LEDGE>(Gm, y, yd);
      radial<true>(Gm.r, rc, R, dR);
      float* rec = geo + lane * REC;
      static_for<NE>([&](auto c) {
        rec[c] = y[c];
        rec[NE + c] = yd[c];
      });
      static_for<kNB>([&](auto b) {
        rec[2 * NE + b] = R[b];
        rec[2 * NE + kNB + b] = dR[b] * Gm.nd;
      });
      rec[2 * NE + 2 * kNB] = __int_as_float(s);
    }
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const float* rec = geo + j * REC;
      const int s = uniform_int(__float_as_int(rec[2 * NE + 2 * kNB]));
      const auto xs = node_rsrc(x, s, NIN * C);
      const auto vs = node_rsrc(HAS_VX ? v_x : x, s, NIN * C);
      float xv[NIN], vx[HAS_VX ? NIN : 1];
      static_for<NIN>([&](auto c) { xv[c] = buf_load(xs, voff, c * C * 4); });
      if constexpr (HAS_VX) static_for<NIN>([&](auto c) { vx[c] = buf_load(vs, voff, c * C * 4); });
      static_for<G::NP>([&](auto pi) {
        constexpr int p = P0 + pi;
        constexpr PathInfo PI = Cfg::paths[p];
        constexpr int na = ncomp(PI.L), o1 = rank_off(PI.l1), o2 = rank_off(PI.l2);
        constexpr int lo = G::loff(p);
        constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
        float f[na], fd[na];
        static_for<te - tb>([&](auto ti) {
          constexpr tab::Term T = tab::kTerms[tb + ti];
          const float cy = T.c * rec[o2 + T.b2];
          const float cyd = T.c * rec[NE + o2 + T.b2];
          float d = cyd * xv[o1 + T.b1];
          if constexpr (HAS_VX) d = fmaf(cy, vx[o1 + T.b1], d);
          if constexpr (T.fa) {
            f[T.a] = cy * xv[o1 + T.b1];
            fd[T.a] = d;
          } else {
            f[T.a] = fmaf(cy, xv[o1 + T.b1], f[T.a]);
            fd[T.a] += d;
          }
        });
        float wb = 0.f, wbd = 0.f;
        static_for<na>([&](auto a) {
          wb = fmaf(gv[lo + a], f[a], wb);
          wbd = fmaf(gv[lo + a], fd[a], wbd);
        });
        static_for<kNB>([&](auto b) {
          constexpr int bb = b;
          float t = fmaf(rec[2 * NE + kNB + bb], wb, acc[bb * G::NP + pi]);
          acc[bb * G::NP + pi] = fmaf(rec[2 * NE + bb], wbd, t);
        });
      });
    }
    __syncthreads();
  }
  wgrad_block_store<G::NP, P0, P>(acc, lds, wv, lane, k, act, C, wpart);
}

template <int LIN, int LEDGE, int LOUT>
void launch_wgrad_vv(const ConvArgs& a, float* wpart, hipStream_t st) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using GS = PathGroups<Cfg, wgrad_vv_budget(Cfg::NIN)>;
  const int nblk = wgrad_blocks(a.N);
  dim3 grid(nblk, (a.C + kWave - 1) / kWave);
  static_for<GS::n>([&](auto gi) {
    constexpr int p0 = GS::start[gi], p1 = GS::start[gi + 1];
    if (a.v_x)
      hipLaunchKernelGGL((conv_wgrad_vv_kernel<LIN, LEDGE, LOUT, p0, p1, true>), grid, dim3(kWgWaves * kWave), 0, st,
                         a.N, a.C, a.rowptr, a.sender, a.pos, a.shift, a.x, a.g, a.v_x, a.v_pos, wpart, a.rc);
    else
      hipLaunchKernelGGL((conv_wgrad_vv_kernel<LIN, LEDGE, LOUT, p0, p1, false>), grid, dim3(kWgWaves * kWave), 0,
                         st, a.N, a.C, a.rowptr, a.sender, a.pos, a.shift, a.x, a.g, a.v_x, a.v_pos, wpart, a.rc);
  });
  launch_block_sum(nblk, kNB * Cfg::P * a.C, wpart, a.W_bar, st);
}

// ------------------------------------------------- x_hat / pos_hat pass --
template <int LIN, int LEDGE, int LOUT, bool HAS_VX>
struct VVShape {
  static constexpr int NIN = nrank(LIN);
  static constexpr int NE = nrank(LEDGE);
  // reductions: Yb, Yd, [Ya], S1, S2, S3
  static constexpr int NRED = (HAS_VX ? 3 : 2) * NE + 3;
  static constexpr int REC = 2 * NE + 3 * kNB + 2;   // y, ydot, R, R', R'', nd, receiver
  // register budget of one path group; with natural-parity, path-separated
  // rank-3 senders capped at 100 (3.68 -> 3.44 ms for the micro workload's
  // VJP-of-VJP; smaller groups were slower at rank 4, where each sweep
  // repeats 2 NE + 3 sums per edge, and with every parity)
  static constexpr int base_budget = 200 - (HAS_VX ? 3 : 2) * (NIN + NE);
  static constexpr int budget = LOUT < kAllParities && NIN == 16 && base_budget > 100 ? 100 : base_budget;
  // edge records of a chunk of ch edges plus the per-wave row sums
  static constexpr size_t lds_bytes(int nw, int ch) {
    return sizeof(float) * ((size_t)ch * REC + (size_t)nw * ch * NRED * 4);
  }
  // edges per chunk: the largest of 64, 32, 16 whose LDS fits the 160 KB a
  // workgroup may hold with the most channel waves (C = 256) and lets two
  // blocks of two waves (C = 128) share a CU (LDS otherwise caps occupancy)
  static constexpr bool fits(int ch) {
    return lds_bytes(kMaxVjpWaves, ch) <= kLdsBytes && lds_bytes(2, ch) <= kLdsBytes / 2;
  }
  static constexpr int CH = fits(64) ? 64 : fits(32) ? 32 : 16;
  static_assert(lds_bytes(kMaxVjpWaves, CH) <= kLdsBytes, "VJP-of-VJP chunk does not fit in LDS");
};

// CH: edges per chunk (64, or 32 when the per-wave row sums of 64 edges would
// not fit in LDS: many channel waves at rank 4).
// XW: per-edge weights W = w [E][P][C] with the weight cotangent vw (nullable)
// as in conv_vv_recv_kernel; w_dot = vw enters J_y^T with coefficient 1 (no
// radial terms), and wh_out (nullable) receives the per-edge
// w_hat = <g, f(v_x, y) + f(x, ydot)> = <alpha, y> + <beta, ydot> (Eq. C2).
template <int LIN, int LEDGE, int LOUT, bool HAS_VX, bool NEED_X, bool NEED_POS, int CH, bool XW = false>
__global__ __launch_bounds__(kMaxVjpWaves * kWave) void conv_vv_sender_kernel(
    int N, int C, const int* __restrict__ t_rowptr, const int* __restrict__ t_edge,
    const int* __restrict__ receiver, const float* __restrict__ pos, const float* __restrict__ shift,
    const float* __restrict__ x, const float* __restrict__ W, const float* __restrict__ g,
    const float* __restrict__ v_x, const float* __restrict__ v_pos, float* __restrict__ x_out,
    float* __restrict__ p_out, float* __restrict__ qbar, float rc, const float* __restrict__ vw = nullptr,
    float* __restrict__ wh_out = nullptr) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using Sh = VVShape<LIN, LEDGE, LOUT, HAS_VX>;
  using GS = PathGroups<Cfg, Sh::budget>;
  constexpr int NIN = Cfg::NIN, NE = Cfg::NE, P = Cfg::P, NOUT = Cfg::NOUT;
  constexpr int REC = Sh::REC, NRED = Sh::NRED;
  constexpr int IYB = 0, IYD = NE, IYA = 2 * NE, IS = (HAS_VX ? 3 : 2) * NE;
  extern __shared__ float lds[];
  float* geo = lds;
  float* part = lds + CH * REC;
  const int NW = blockDim.x / kWave;

  const int v = xcd_node(blockIdx.x, N);
  const int S = gridDim.y, sl = blockIdx.y;
  const int tid = threadIdx.x;
  const int wv = tid / kWave, lane = tid % kWave;
  const int k = tid;
  const bool act = k < C;
  const int kk = act ? k : 0;
  const int voff = kk * 4;

  float xv[NIN], vx[HAS_VX ? NIN : 1];
  {
    const float* xs = x + (size_t)v * NIN * C + kk;
    static_for<NIN>([&](auto c) { xv[c] = xs[(size_t)c * C]; });
    if constexpr (HAS_VX) {
      const float* vs = v_x + (size_t)v * NIN * C + kk;
      static_for<NIN>([&](auto c) { vx[c] = vs[(size_t)c * C]; });
    }
  }
  float xh[NIN];
  static_for<NIN>([&](auto c) { xh[c] = 0.f; });
  float psum[3] = {0.f, 0.f, 0.f};

  const int v0 = t_rowptr[v], deg = t_rowptr[v + 1] - v0;
  const int e0 = v0 + (int)(((long long)sl * deg) / S), e1 = v0 + (int)(((long long)(sl + 1) * deg) / S);
  const float pvx = pos[3 * v], pvy = pos[3 * v + 1], pvz = pos[3 * v + 2];
  const float vvx = v_pos ? v_pos[3 * v] : 0.f, vvy = v_pos ? v_pos[3 * v + 1] : 0.f,
              vvz = v_pos ? v_pos[3 * v + 2] : 0.f;
  auto edge_geo = [&](int e, int u) -> VVGeo {
    float rx = pvx - pos[3 * u], ry = pvy - pos[3 * u + 1], rz = pvz - pos[3 * u + 2];
    if (shift) {
      rx += shift[3 * e];
      ry += shift[3 * e + 1];
      rz += shift[3 * e + 2];
    }
    float dvx = 0.f, dvy = 0.f, dvz = 0.f;
    if (v_pos) {
      dvx = vvx - v_pos[3 * u];
      dvy = vvy - v_pos[3 * u + 1];
      dvz = vvz - v_pos[3 * u + 2];
    }
    return vv_geo(rx, ry, rz, dvx, dvy, dvz);
  };
  // One sweep over the slice per path group, as in the VJP: x_hat stays in
  // registers, q_e (linear in the per-edge sums) is summed over the sweeps.
  static_for<GS::n>([&](auto gi) {
    using G = typename GS::template group<gi>;
    constexpr bool FIRST = gi == 0;
    constexpr uint64_t MASK = G::comp_mask();
    float Wr[XW ? 1 : kNB * G::NP];
    if constexpr (!XW) {
      static_for<kNB * G::NP>([&](auto i) {
        constexpr int b = i / G::NP, pi = i % G::NP;
        Wr[i] = act ? W[(size_t)(b * P + G::p0 + pi) * C + kk] : 0.f;
      });
    }
    for (int base = e0; base < e1; base += CH) {
      const int cnt = min(CH, e1 - base);
      if (wv == 0 && lane < cnt) {
        const int e = t_edge[base + lane];
        const int u = receiver[e];
        const VVGeo Gm = edge_geo(e, u);
        float y[NE], yd[NE];
        vv_tensors<LEDGE>(Gm, y, yd);
        float* rec = geo + lane * REC;
        static_for<NE>([&](auto c) {
          rec[c] = y[c];
          rec[NE + c] = yd[c];
        });
        if constexpr (XW) {
          rec[2 * NE] = __int_as_float(e);
          rec[2 * NE + 1] = Gm.r > 0.f ? 1.f : 0.f;
        } else {
          float R[kNB], dR[kNB], d2R[kNB];
          radial2(Gm.r, rc, R, dR, d2R);
          static_for<kNB>([&](auto b) {
            rec[2 * NE + b] = R[b];
            rec[2 * NE + kNB + b] = dR[b];
            rec[2 * NE + 2 * kNB + b] = d2R[b];
          });
        }
        rec[2 * NE + 3 * kNB] = Gm.nd;
        rec[2 * NE + 3 * kNB + 1] = __int_as_float(u);
      }
      __syncthreads();
      for (int j = 0; j < cnt; ++j) {
        const float* rec = geo + j * REC;
        const int u = uniform_int(__float_as_int(rec[2 * NE + 3 * kNB + 1]));
        const float nd = rec[2 * NE + 3 * kNB];
        const auto gu = node_rsrc(g, u, NOUT * C);
        float gv[G::NR];
        static_for<G::NP>([&](auto pi) {
          constexpr int p = G::p0 + pi;
          if constexpr (!G::owner(p)) return;
          static_for<ncomp(Cfg::paths[p].L)>([&](auto c) {
            constexpr int row = Cfg::row(p, c), li = G::loff(p) + c;
            gv[li] = buf_load(gu, voff, row * C * 4);
          });
        });
        float red[NRED];
        static_for<NRED>([&](auto i) { red[i] = 0.f; });
        float we[XW ? G::NP : 1], wve[XW ? G::NP : 1];
        [[maybe_unused]] size_t erow = 0;
        [[maybe_unused]] float valid = 1.f;
        if constexpr (XW) {
          // lanes past the last channel read channel 0 and must add nothing
          // to the per-edge row sums
          valid = act ? rec[2 * NE + 1] : 0.f;
          erow = (size_t)uniform_int(__float_as_int(rec[2 * NE])) * P * C + kk;
          static_for<G::NP>([&](auto pi) {
            we[pi] = valid * W[erow + (size_t)(G::p0 + pi) * C];
            wve[pi] = vw ? valid * vw[erow + (size_t)(G::p0 + pi) * C] : 0.f;
          });
        }
        static_for<G::NP>([&](auto pi) {
          constexpr int p = G::p0 + pi;
          constexpr PathInfo PI = Cfg::paths[p];
          constexpr int na = ncomp(PI.L), n2 = ncomp(PI.l2);
          constexpr int o1 = rank_off(PI.l1), o2 = rank_off(PI.l2);
          constexpr int lo = G::loff(p);
          constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
          float w = 0.f, w1 = 0.f, w2 = 0.f;
          if constexpr (XW) {
            w = we[pi];
            w1 = wve[pi];   // enters J_y^T with coefficient 1 (no nd factor)
          } else {
            static_for<kNB>([&](auto b) {
              constexpr int bb = b;
              const float wb = Wr[bb * G::NP + pi];
              w = fmaf(rec[2 * NE + bb], wb, w);
              w1 = fmaf(rec[2 * NE + kNB + bb], wb, w1);
              if constexpr (NEED_POS) w2 = fmaf(rec[2 * NE + 2 * kNB + bb], wb, w2);
            });
          }
          const float wd = XW ? w1 : w1 * nd;
          if constexpr (NEED_X) {
            // x_hat[b1] += sum c g[a] (w ydot[b2] + wdot y[b2])
            float gw[na], gd[na];
            static_for<na>([&](auto a) {
              gw[a] = w * gv[lo + a];
              gd[a] = wd * gv[lo + a];
            });
            static_for<te - tb>([&](auto ti) {
              constexpr tab::Term T = tab::kTerms[tb + ti];
              float t = fmaf(T.c * rec[NE + o2 + T.b2], gw[T.a], xh[o1 + T.b1]);
              xh[o1 + T.b1] = fmaf(T.c * rec[o2 + T.b2], gd[T.a], t);
            });
          }
          if (NEED_POS || (XW && wh_out)) {
            float be[n2], al[HAS_VX ? n2 : 1];
            static_for<n2>([&](auto c) {
              be[c] = 0.f;
              if constexpr (HAS_VX) al[c] = 0.f;
            });
            static_for<te - tb>([&](auto ti) {
              constexpr tab::Term T = tab::kTerms[tb + ti];
              const float cg = T.c * gv[lo + T.a];
              be[T.b2] = fmaf(cg, xv[o1 + T.b1], be[T.b2]);
              if constexpr (HAS_VX) al[T.b2] = fmaf(cg, vx[o1 + T.b1], al[T.b2]);
            });
            float by = 0.f, bd = 0.f, ay = 0.f;
            static_for<n2>([&](auto c) {
              by = fmaf(be[c], rec[o2 + c], by);
              bd = fmaf(be[c], rec[NE + o2 + c], bd);
              red[IYB + o2 + c] = fmaf(w, be[c], red[IYB + o2 + c]);
              red[IYD + o2 + c] = fmaf(w1, be[c], red[IYD + o2 + c]);
              if constexpr (HAS_VX) {
                ay = fmaf(al[c], rec[o2 + c], ay);
                red[IYA + o2 + c] = fmaf(w, al[c], red[IYA + o2 + c]);
              }
            });
            if constexpr (XW) {
              if (wh_out && act) wh_out[erow + (size_t)p * C] = valid * (ay + bd);
            } else {
              red[IS] = fmaf(w1, ay + bd, red[IS]);
              red[IS + 1] = fmaf(w2, by, red[IS + 1]);
              red[IS + 2] = fmaf(w1, by, red[IS + 2]);
            }
          }
        });
        if constexpr (NEED_POS) {
          float* dst = part + ((size_t)(wv * CH + j) * NRED) * 4 + (lane >> 4);
          static_for<NRED>([&](auto i) {
            if constexpr (i >= IS || ((MASK >> (i % NE)) & 1)) {
              const float t = row_sum16(red[i]);
              if ((lane & 15) == 0) dst[i * 4] = t;
            }
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
            const float4* src = reinterpret_cast<const float4*>(part + ((size_t)(w2 * CH + lane) * NRED) * 4);
            static_for<NRED>([&](auto i) {
              if constexpr (i >= IS || ((MASK >> (i % NE)) & 1)) {
                const float4 q = src[i];
                tot[i] += (q.x + q.y) + (q.z + q.w);
              }
            });
          }
          const VVGeo Gm = edge_geo(e, u);
          float ox = 0.f, oy = 0.f, oz = 0.f;
          if (Gm.r > 0.f) {
            // J_y^T (Ya + nd Yd) = (gA - n (n.gA)) / r, gA = grad_n of (Ya + nd Yd) . y
            float cA[NE];
            static_for<NE>([&](auto c) {
              cA[c] = XW ? tot[IYD + c] : Gm.nd * tot[IYD + c];
              if constexpr (HAS_VX) cA[c] += tot[IYA + c];
            });
            float gA[3], HA[6], gB[3], HB[6];
            direction_contract_d2<LEDGE, MASK>(cA, Gm.nx, Gm.ny, Gm.nz, gA, HA);
            direction_contract_d2<LEDGE, MASK>(tot + IYB, Gm.nx, Gm.ny, Gm.nz, gB, HB);
            const float ngA = Gm.nx * gA[0] + Gm.ny * gA[1] + Gm.nz * gA[2];
            ox = (gA[0] - Gm.nx * ngA) * Gm.inv;
            oy = (gA[1] - Gm.ny * ngA) * Gm.inv;
            oz = (gA[2] - Gm.nz * ngA) * Gm.inv;
            // H_y[Yb] dv = [gdot - ndot (n.g) - n (ndot.g + n.gdot)] / r - nd (g - n (n.g)) / r^2
            const float gdx = HB[0] * Gm.ndx + HB[3] * Gm.ndy + HB[4] * Gm.ndz;
            const float gdy = HB[3] * Gm.ndx + HB[1] * Gm.ndy + HB[5] * Gm.ndz;
            const float gdz = HB[4] * Gm.ndx + HB[5] * Gm.ndy + HB[2] * Gm.ndz;
            const float ng = Gm.nx * gB[0] + Gm.ny * gB[1] + Gm.nz * gB[2];
            const float ndg = Gm.ndx * gB[0] + Gm.ndy * gB[1] + Gm.ndz * gB[2];
            const float ngd = Gm.nx * gdx + Gm.ny * gdy + Gm.nz * gdz;
            const float t1 = ndg + ngd;
            ox += (gdx - Gm.ndx * ng - Gm.nx * t1) * Gm.inv - Gm.nd * (gB[0] - Gm.nx * ng) * Gm.inv * Gm.inv;
            oy += (gdy - Gm.ndy * ng - Gm.ny * t1) * Gm.inv - Gm.nd * (gB[1] - Gm.ny * ng) * Gm.inv * Gm.inv;
            oz += (gdz - Gm.ndz * ng - Gm.nz * t1) * Gm.inv - Gm.nd * (gB[2] - Gm.nz * ng) * Gm.inv * Gm.inv;
            // radial terms
            const float sn = tot[IS] + tot[IS + 1] * Gm.nd;
            ox += sn * Gm.nx + tot[IS + 2] * Gm.ndx;
            oy += sn * Gm.ny + tot[IS + 2] * Gm.ndy;
            oz += sn * Gm.nz + tot[IS + 2] * Gm.ndz;
          }
          float* qe = qbar + 3 * (size_t)e;
          if constexpr (FIRST) {
            qe[0] = ox;
            qe[1] = oy;
            qe[2] = oz;
          } else {
            qe[0] += ox;
            qe[1] += oy;
            qe[2] += oz;
          }
          psum[0] += ox;
          psum[1] += oy;
          psum[2] += oz;
        }
        __syncthreads();
      }
    }
  });
  const size_t slot = (size_t)v * S + sl;
  if (NEED_X && act) {
    float* xo = x_out + slot * NIN * C + k;
    static_for<NIN>([&](auto c) { xo[(size_t)c * C] = xh[c]; });
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
        p_out[3 * slot] = psum[0];
        p_out[3 * slot + 1] = psum[1];
        p_out[3 * slot + 2] = psum[2];
      }
    }
  }
}

template <int LIN, int LEDGE, int LOUT, bool HAS_VX, bool XW = false>
void launch_vv_sender_vx(const ConvArgs& a, const VjpWorkspace& wsl, hipStream_t st) {
  const bool nx = a.x_bar != nullptr, np = a.pos_bar != nullptr;
  const int nw = (a.C + kWave - 1) / kWave;
  float* xo = wsl.S == 1 ? a.x_bar : wsl.x_part;
  float* po = wsl.S == 1 ? a.pos_bar : wsl.p_part;
  dim3 grid(a.N, wsl.S), block(nw * kWave);
  using Sh = VVShape<LIN, LEDGE, LOUT, HAS_VX>;
  const size_t lds = Sh::lds_bytes(np ? nw : 0, Sh::CH);
#define FC_VV(NX, NP)                                                                                    \
  hipLaunchKernelGGL((conv_vv_sender_kernel<LIN, LEDGE, LOUT, HAS_VX, NX, NP, Sh::CH, XW>), grid, block, lds, st, \
                     a.N, a.C, a.t_rowptr, a.t_edge, a.receiver, a.pos, a.shift, a.x, XW ? a.w_edge : a.W, a.g,  \
                     a.v_x, a.v_pos, xo, po, wsl.rbar, a.rc, a.v_w_edge, XW ? a.w_edge_bar : nullptr)
  if (nx && np) FC_VV(true, true);
  else if (nx) FC_VV(true, false);
  else if (np || !XW) FC_VV(false, true);
  else if constexpr (XW) FC_VV(false, false);   // w_hat alone
#undef FC_VV
}

// The passes of the VJP-of-VJP, each a separate launch sequence (the
// g_hat pass, the W_hat pass, the sender pass for x_hat and the per-edge
// position terms without and with a feature cotangent); at the highest
// ranks each is instantiated in a unit of its own and composed by
// run_vjp_vjp.
template <int LIN, int LEDGE, int LOUT>
void vv_part_recv(const ConvArgs& a, hipStream_t st) {
  launch_vv_recv<LIN, LEDGE, LOUT>(a, st);
}
template <int LIN, int LEDGE, int LOUT>
void vv_part_wgrad(const ConvArgs& a, hipStream_t st) {
  const VjpWorkspace wsl(a.N, a.E, a.C, nrank(LIN), ConvCfg<LIN, LEDGE, LOUT>::P, true, a.rbar);
  launch_wgrad_vv<LIN, LEDGE, LOUT>(a, wsl.w_part, st);
}
template <int LIN, int LEDGE, int LOUT, bool HAS_VX>
void vv_part_sender(const ConvArgs& a, hipStream_t st) {
  const VjpWorkspace wsl(a.N, a.E, a.C, nrank(LIN), ConvCfg<LIN, LEDGE, LOUT>::P, true, a.rbar);
  launch_vv_sender_vx<LIN, LEDGE, LOUT, HAS_VX>(a, wsl, st);
}

// g_hat, W_hat (W_bar of the arguments), then x_hat / pos_hat, each when
// requested.
template <int LIN, int LEDGE, int LOUT>
void launch_vjp_vjp(const ConvArgs& a, hipStream_t st) {
  run_vjp_vjp(VVParts{vv_part_recv<LIN, LEDGE, LOUT>, vv_part_wgrad<LIN, LEDGE, LOUT>,
                      vv_part_sender<LIN, LEDGE, LOUT, false>, vv_part_sender<LIN, LEDGE, LOUT, true>},
              nrank(LIN), ConvCfg<LIN, LEDGE, LOUT>::P, a, st);
}

// Explicit per-edge weights w = a.w_edge [E][P][C] (receiver-sorted edge
// order) with cotangent a.v_w_edge (nullable): g_hat, then x_hat / pos_hat
// and w_hat (a.w_edge_bar), each when requested.  The workspace is the VJP's.
template <int LIN, int LEDGE, int LOUT>
void launch_vjp_vjp_w(const ConvArgs& a, hipStream_t st) {
  if (a.g_hat) launch_vv_recv<LIN, LEDGE, LOUT, true>(a, st);
  if (!a.x_bar && !a.pos_bar && !a.w_edge_bar) return;
  const VjpWorkspace wsl(a.N, a.E, a.C, nrank(LIN), ConvCfg<LIN, LEDGE, LOUT>::P, true, a.rbar);
  if (a.v_x) launch_vv_sender_vx<LIN, LEDGE, LOUT, true, true>(a, wsl, st);
  else launch_vv_sender_vx<LIN, LEDGE, LOUT, false, true>(a, wsl, st);
  launch_vjp_combine(a, wsl, nrank(LIN), st);
}

}  // namespace fc
