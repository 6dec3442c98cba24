// Edge convolution kernels for gfx950: forward (receiver-sorted, FlashCart
// paper §4 Eq. 1) and VJP (App. C Eq. C1 with the chain rule to positions),
// the VJP run sender-sorted so that every output is written exactly once.
//
// Mapping: one wavefront per (node, 64-channel tile); channel k lives in lane
// k % 64, so every gather of a neighbour row is one coalesced 256-byte
// buffer load per stored component.  Per-edge geometry (direction tensor
// components or their coefficient products, Bessel radial values, neighbour
// id) is computed once per edge by a lane of its own (lane j <-> edge j of a
// 64-edge chunk), parked in LDS and read back by all 64 lanes as a broadcast,
// so it is shared by all channels.  The coupling polynomials come from the
// generated tables and are fully unrolled; all accumulators stay in VGPRs.
#pragma once

#include "fc_conv.h"
#include "fc_radial.h"

namespace fc {

// Register budgets of the path groups (see PathGroups): what is left of
// about 200 VGPRs per lane once the per-lane arrays that do not depend on the
// group (gathered features, their weighted copies, accumulated cotangents)
// are counted.
__host__ __device__ constexpr int fwd_budget(int nin) { return 200 - 2 * nin; }

// Whether output component a (resp. input component b1) occurs among the
// terms [tb, te) of a path type.
__host__ __device__ constexpr bool term_has_a(int tb, int te, int a) {
  for (int t = tb; t < te; ++t)
    if (tab::kTerms[t].a == a) return true;
  return false;
}
__host__ __device__ constexpr bool term_has_b1(int tb, int te, int b) {
  for (int t = tb; t < te; ++t)
    if (tab::kTerms[t].b1 == b) return true;
  return false;
}
// Register budget of one VJP path group (2L+1 cotangent rows plus the radial
// weights of each path).  With natural-parity, path-separated outputs and
// senders of rank 3 or 4 it is sized so that the sender kernel stays within
// the 256 registers of two waves per SIMD: one wave per SIMD had cost
// 1.67 / 5.44 ms where two take 1.15 / 4.22 ms at the micro workload (ranks
// 3 / 4), despite more sweeps per sender (the formula is fitted there).  The
// same budgets made the every-parity and summed-path kernels slower (more
// paths per rank, more repeated sums per sweep); they and the other ranks
// keep the wider groups.
__host__ __device__ constexpr int vjp_budget(int nin, int ne, bool natural_separate) {
  return natural_separate && nin >= 16 && nin <= 25 && ne <= 25 ? 190 - 3 * nin - 2 * ne : 200 - 2 * nin - ne;
}
// With one wave per sender (C <= 64) each extra sweep's records and
// per-edge sums serve half as many channels: at rank 4 the wider groups
// are faster there (1.62 / 2.64 ms against 2.02 / 3.49 ms at 64 / 128
// neighbours); at rank 3 the narrower ones still win (0.51 / 0.71 ms
// against 0.50 / 0.81 ms).
__host__ __device__ constexpr bool vjp_wide_when_narrow(int nin, int ne, bool natural_separate) {
  return natural_separate && nin == 25 && ne == 25;
}
// Channels of one VJP block: up to 4 waves (C <= 256).
inline constexpr int kMaxVjpWaves = 4;
// LDS one workgroup may hold on gfx950.
inline constexpr size_t kLdsBytes = 160 * 1024;

// Node of the block with x index b in a grid whose x extent is N.  The
// dispatcher deals consecutive workgroups to the chip's eight XCDs in turn,
// so block b runs on XCD b % 8; this numbering gives each XCD one contiguous
// range of nodes, so that when the nodes are numbered in space (a lattice, a
// sorted cell list) the neighbour rows an XCD gathers meet in its own L2.
// A bijection of [0, N) for any N.
__device__ __forceinline__ int xcd_node(int b, int N) {
  const int q = N >> 3, r = N & 7, k = b & 7;
  return k * q + (k < r ? k : r) + (b >> 3);
}
// Per-edge products |c| y[g] are broadcast from LDS when a configuration uses
// at most this many; larger tables multiply inline from y.
inline constexpr int kCYMax = 48;
// Per-sender products |c| x[g] stay in registers up to this many.
inline constexpr int kCXMax = 20;

// Per-edge coefficient products of one configuration.
template <int LIN, int LEDGE, int LOUT>
struct EdgeProducts {
  using CYt = tab::CY<LIN, LEDGE, LOUT % kSumPaths>;
  using CXt = tab::CX<LIN, LEDGE, LOUT % kSumPaths>;
  static constexpr int NE = nrank(LEDGE);
  static constexpr bool kLDS = CYt::n <= kCYMax;
  static constexpr bool kCXReg = CXt::n <= kCXMax;
  static constexpr int NY = kLDS ? CYt::n : NE;   // record floats holding y (first NE) and products

  // record entries from y (lane-per-edge stage)
  __device__ __forceinline__ static void fill(const float* y, float* rec) {
    if constexpr (kLDS) {
      static_for<CYt::n>([&](auto i) {
        constexpr int ii = i;
        constexpr float c = CYt::c[ii];
        if constexpr (c == 1.f) rec[ii] = y[CYt::g[ii]];
        else rec[ii] = c * y[CYt::g[ii]];
      });
    } else {
      static_for<NE>([&](auto i) { rec[i] = y[i]; });
    }
  }
  // signed c * y[g2] of global term TERM (g2 = l2^2 + b2)
  template <int TERM, int G2>
  __device__ __forceinline__ static float cy(const float* rec) {
    constexpr tab::Term T = tab::kTerms[TERM];
    constexpr float ac = T.c < 0.f ? -T.c : T.c;
    float v;
    if constexpr (kLDS) v = rec[CYt::term[TERM]];
    else if constexpr (ac == 1.f) v = rec[G2];
    else v = ac * rec[G2];
    return T.c < 0.f ? -v : v;
  }
};

// ------------------------------------------------ fused radial network ----
// With the radial network's output layer fused into the convolution (MLP),
// w[e, p, k] = sum_h h2[e, h] W3[h, p, k] (and, for the VJP, dw/dr from the
// r-derivatives of h2) is formed per lane (channel k) for a batch of B
// consecutive edges of a chunk: the edges' 64 activations are staged in LDS
// (rows of kMlpRow floats, or kMlpRow2 with the derivatives) and read as
// broadcasts, the W3 entries of the lane's channel are read from the cache
// once per batch, and w never leaves the registers.
inline constexpr int kMlpRow = kRadHidden + 4;        // padded: the lanes' row stores spread over the banks
inline constexpr int kMlpRow2 = 2 * kRadHidden + 4;   // h2, then dh2/dr
// Edges per batch for a path group of np paths: each W3 entry read serves
// one FMA per edge of the batch (two in the VJP: w and dw/dr), so the batch
// is as large as the registers allow: the forward holds 16 np weights (np
// <= 6) or 8 np; the VJP holds 2 np per edge within 66 registers (3 edges
// at the 11 paths of ranks <= 2, whose four would take the kernel past the
// 256 registers of two waves per SIMD; 8 for four paths).
#ifndef FC_MLP_VJP_CAP
#define FC_MLP_VJP_CAP 8
#endif
#ifndef FC_MLP_FWD_REGS
#define FC_MLP_FWD_REGS 96
#endif
__host__ __device__ constexpr int mlp_batch_fwd(int np) {
  int b = 16;
  while (b > 1 && b * np > FC_MLP_FWD_REGS) b /= 2;
  return b;
}
__host__ __device__ constexpr int mlp_batch_vjp(int np) {
  return np >= 33 ? 1 : (33 / np > FC_MLP_VJP_CAP ? FC_MLP_VJP_CAP : 33 / np);
}
inline constexpr int kMlpBatchVjpMax = 8;
static_assert(FC_MLP_VJP_CAP <= kMlpBatchVjpMax, "LDS rows past the chunk");
// edges per chunk of the fused forward: 32 keep its LDS (records and
// activation rows) low enough for two one-wave blocks per SIMD
inline constexpr int kMlpChunkFwd = 32;
static_assert(kMlpChunkFwd % 16 == 0, "forward batches tile the chunk");

// w[b NP + i] = sum_h hs[b HR + h] w3[h ldw + i C] for b < B (and, with D,
// dw from the derivative rows at hs + b HR + kRadHidden).  HS hidden units
// (2 or 4) per step; the W3 entries of step h + HS are requested before the
// products of step h, so that their latency overlaps the FMAs (the last
// step requests its own entries again, unused).
template <int B, int NP, bool D, int HR, int HS>
__device__ __forceinline__ void mlp_batch_weights(const float* hs, const float* __restrict__ w3, size_t ldw, int C,
                                                  float* w, float* dw) {
  static_assert(HS == 2 || HS == 4, "2 or 4 hidden units per step");
  using V = typename std::conditional<HS == 4, float4, float2>::type;
  static_for<B * NP>([&](auto i) {
    w[i] = 0.f;
    if constexpr (D) dw[i] = 0.f;
  });
  auto fetch = [&](float* dst, int h) {
    static_for<HS * NP>([&](auto i) {
      constexpr int q = i / NP, pi = i % NP;
      dst[i] = w3[(size_t)(h + q) * ldw + (size_t)pi * C];
    });
  };
  float wv[HS * NP];
  fetch(wv, 0);
#pragma unroll 2
  for (int h = 0; h < kRadHidden; h += HS) {
    float wn[HS * NP];
    fetch(wn, min(h + HS, kRadHidden - HS));
    auto madd = [&](const V& v, float* acc, auto pi, int o) {
      acc[o] = fmaf(v.x, wv[pi], acc[o]);
      acc[o] = fmaf(v.y, wv[NP + pi], acc[o]);
      if constexpr (HS == 4) {
        acc[o] = fmaf(v.z, wv[2 * NP + pi], acc[o]);
        acc[o] = fmaf(v.w, wv[3 * NP + pi], acc[o]);
      }
    };
    static_for<B>([&](auto b) {
      constexpr int bb = b;
      const V hv = *reinterpret_cast<const V*>(hs + bb * HR + h);
      static_for<NP>([&](auto pi) { madd(hv, w, pi, bb * NP + pi); });
      if constexpr (D) {
        const V dv = *reinterpret_cast<const V*>(hs + bb * HR + kRadHidden + h);
        static_for<NP>([&](auto pi) { madd(dv, dw, pi, bb * NP + pi); });
      }
    });
    static_for<HS * NP>([&](auto i) { wv[i] = wn[i]; });
  }
}

// Copies n floats (a multiple of 4) from global src to LDS dst.
template <int NF>
__device__ __forceinline__ void copy_row(const float* __restrict__ src, float* dst) {
  static_for<NF / 4>([&](auto q) {
    reinterpret_cast<float4*>(dst)[q] = reinterpret_cast<const float4*>(src)[q];
  });
}

// Receiver-sorted edge record: direction-tensor entries (or their coefficient
// products), the eight radial values and the sender id of edge e into u.
// With explicit per-edge weights (XW) the first radial slot holds 1 for an
// edge of nonzero length and 0 otherwise (such an edge has no direction and
// takes no part), and the radial basis is not evaluated.
template <int LIN, int LEDGE, int LOUT, bool XW = false>
__device__ __forceinline__ void recv_edge_record(int e, const int* __restrict__ sender, const float* __restrict__ pos,
                                                 const float* __restrict__ shift, float pux, float puy, float puz,
                                                 float rc, float* rec) {
  using EP = EdgeProducts<LIN, LEDGE, LOUT>;
  constexpr int NE = nrank(LEDGE);
  const int s = sender[e];
  float rx = pos[3 * s] - pux, ry = pos[3 * s + 1] - puy, rz = pos[3 * s + 2] - puz;
  if (shift) {
    rx += shift[3 * e];
    ry += shift[3 * e + 1];
    rz += shift[3 * e + 2];
  }
  const float r = sqrtf(rx * rx + ry * ry + rz * rz);
  const float inv = r > 0.f ? 1.f / r : 0.f;
  float y[NE];
  direction_tensors<LEDGE>(rx * inv, ry * inv, rz * inv, y);
  EP::fill(y, rec);
  if constexpr (XW) {
    rec[EP::NY] = r > 0.f ? 1.f : 0.f;
  } else {
    float R[kNB];
    radial<false>(r, rc, R, nullptr);
    static_for<kNB>([&](auto b) { rec[EP::NY + b] = R[b]; });
  }
  rec[EP::NY + kNB] = __int_as_float(s);
}

// ============================================================== forward ====
// One launch per path group G: z rows of G's paths for node u and 64 channels.
// XW: the weights are given per edge, W = w [E][P][C] (receiver-sorted edge
// order), instead of being formed from the radial basis and W [8][P][C].
// MLP: W = W3 [64][P][C] and hh [E][2][64] the second hidden layer of the
// radial network per edge (and its r-derivative, unused here); w = h2 W3 is
// formed in the lanes.
template <int LIN, int LEDGE, int LOUT, int P0, int P1, bool XW, bool MLP = false>
__global__ __launch_bounds__(kWave) void conv_fwd_kernel(
    int N, int C, const int* __restrict__ rowptr, const int* __restrict__ sender,
    const float* __restrict__ pos, const float* __restrict__ shift,
    const float* __restrict__ x, const float* __restrict__ W, float* __restrict__ z, float rc,
    const float* __restrict__ hh) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using G = PathGroup<Cfg, P0, P1>;
  using EP = EdgeProducts<LIN, LEDGE, LOUT>;
  constexpr int NIN = Cfg::NIN, NE = Cfg::NE, P = Cfg::P, NOUT = Cfg::NOUT;
  constexpr int REC = EP::NY + kNB + 1;
  constexpr int MB = mlp_batch_fwd(G::NP), CHF = MLP ? kMlpChunkFwd : kWave;
  __shared__ float geo[CHF * REC];
  __shared__ __align__(16) float hsh[MLP ? CHF * kMlpRow : 4];

  const int u = xcd_node(blockIdx.x, N);
  const int lane = threadIdx.x;
  const int k = blockIdx.y * kWave + lane;
  const bool act = k < C;
  const int kk = act ? k : 0;
  const int voff = kk * 4;

  float Wr[XW || MLP ? 1 : kNB * G::NP];
  if constexpr (!XW && !MLP) {
    static_for<kNB * G::NP>([&](auto i) {
      constexpr int b = i / G::NP, p = i % G::NP;
      Wr[i] = W[(size_t)(b * P + P0 + p) * C + kk];
    });
  }
  float acc[G::NR];
  static_for<G::NR>([&](auto i) { acc[i] = 0.f; });

  const int e0 = rowptr[u], e1 = rowptr[u + 1];
  const float pux = pos[3 * u], puy = pos[3 * u + 1], puz = pos[3 * u + 2];
  for (int base = e0; base < e1; base += CHF) {
    const int cnt = min(CHF, e1 - base);
    if (lane < cnt) {
      recv_edge_record<LIN, LEDGE, LOUT, XW || MLP>(base + lane, sender, pos, shift, pux, puy, puz, rc,
                                                     geo + lane * REC);
      if constexpr (MLP) copy_row<kRadHidden>(hh + (size_t)(base + lane) * kRadRow, hsh + lane * kMlpRow);
    }
    __syncthreads();
    // XW: the weights of edge j + 1 are requested after the gather of edge
    // j, so that waiting for the gather leaves the prefetch in flight
    float wn[XW ? G::NP : 1];
    if constexpr (XW) {
      if (cnt > 0) {
        const float* wrow = W + (size_t)base * P * C + kk;
        static_for<G::NP>([&](auto pi) { wn[pi] = wrow[(size_t)(P0 + pi) * C]; });
      }
    }
    // one edge; wm(pi) gives the fused network's weight of path P0 + pi
    auto edge = [&](int j, auto wm) {
      const float* rec = geo + j * REC;
      const int s = uniform_int(__float_as_int(rec[EP::NY + kNB]));
      const auto xs = node_rsrc(x, s, NIN * C);
      float xv[NIN];
      static_for<NIN>([&](auto c) { xv[c] = buf_load(xs, voff, c * C * 4); });
      float we[XW ? G::NP : 1];
      if constexpr (XW) {
        static_for<G::NP>([&](auto pi) { we[pi] = rec[EP::NY] * wn[pi]; });
        if (j + 1 < cnt) {
          const float* wrow = W + (size_t)(base + j + 1) * P * C + kk;
          static_for<G::NP>([&](auto pi) { wn[pi] = wrow[(size_t)(P0 + pi) * C]; });
        }
      }
      static_for<G::NP>([&](auto pi) {
        constexpr int p = P0 + pi;
        constexpr PathInfo PI = Cfg::paths[p];
        constexpr int n1 = ncomp(PI.l1), o1 = rank_off(PI.l1), o2 = rank_off(PI.l2);
        constexpr int lo = G::loff(p);
        float w = 0.f;
        if constexpr (XW) {
          w = we[pi];
        } else if constexpr (MLP) {
          w = wm(pi);
        } else {
          static_for<kNB>([&](auto b) {
            constexpr int bb = b;
            w = fmaf(rec[EP::NY + bb], Wr[bb * G::NP + pi], w);
          });
        }
        constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
        constexpr int na = ncomp(PI.L);
        if constexpr (na < n1) {
          // fewer outputs than inputs: weight the 2L+1 products, not the 2l1+1 inputs
          float t[na];
          static_for<te - tb>([&](auto ti) {
            constexpr int tt = tb + ti;
            constexpr tab::Term T = tab::kTerms[tt];
            const float cy = EP::template cy<tt, o2 + T.b2>(rec);
            if constexpr (T.fa) t[T.a] = cy * xv[o1 + T.b1];
            else t[T.a] = fmaf(cy, xv[o1 + T.b1], t[T.a]);
          });
          static_for<na>([&](auto a) {
            if constexpr (term_has_a(tb, te, a)) acc[lo + a] = fmaf(w, t[a], acc[lo + a]);
          });
        } else {
          float xw[n1];
          static_for<n1>([&](auto c) { xw[c] = w * xv[o1 + c]; });
          static_for<te - tb>([&](auto ti) {
            constexpr int tt = tb + ti;
            constexpr tab::Term T = tab::kTerms[tt];
            acc[lo + T.a] = fmaf(EP::template cy<tt, o2 + T.b2>(rec), xw[T.b1], acc[lo + T.a]);
          });
        }
      });
    };
    if constexpr (MLP) {
      for (int jb = 0; jb < cnt; jb += MB) {
        float wb[MB * G::NP];
        mlp_batch_weights<MB, G::NP, false, kMlpRow, 2>(hsh + jb * kMlpRow, W + (size_t)P0 * C + kk, (size_t)P * C, C,
                                                    wb, nullptr);
        static_for<MB>([&](auto bi) {
          constexpr int b = bi;
          if (jb + b < cnt) edge(jb + b, [&](auto pi) { return wb[b * G::NP + pi]; });
        });
      }
    } else {
      for (int j = 0; j < cnt; ++j) edge(j, [](auto) { return 0.f; });
    }
    __syncthreads();
  }
  if (act) {
    float* zo = z + (size_t)u * NOUT * C + k;
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

template <int LIN, int LEDGE, int LOUT>
void launch_fwd(const ConvArgs& a, hipStream_t st) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using GS = PathGroups<Cfg, fwd_budget(Cfg::NIN)>;
  dim3 grid(a.N, (a.C + kWave - 1) / kWave);
  static_for<GS::n>([&](auto gi) {
    constexpr int p0 = GS::start[gi], p1 = GS::start[gi + 1];
    if (a.w_edge)
      hipLaunchKernelGGL((conv_fwd_kernel<LIN, LEDGE, LOUT, p0, p1, true>), grid, dim3(kWave), 0, st, a.N, a.C,
                         a.rowptr, a.sender, a.pos, a.shift, a.x, a.w_edge, a.z, a.rc, nullptr);
    else
      hipLaunchKernelGGL((conv_fwd_kernel<LIN, LEDGE, LOUT, p0, p1, false>), grid, dim3(kWave), 0, st, a.N, a.C,
                         a.rowptr, a.sender, a.pos, a.shift, a.x, a.W, a.z, a.rc, nullptr);
  });
}

// Forward with the radial network fused (a.W = W3, a.mlp_h = h2 [E][64]).
template <int LIN, int LEDGE, int LOUT>
void launch_fwd_mlp(const ConvArgs& a, hipStream_t st) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using GS = PathGroups<Cfg, fwd_budget(Cfg::NIN)>;
  dim3 grid(a.N, (a.C + kWave - 1) / kWave);
  static_for<GS::n>([&](auto gi) {
    constexpr int p0 = GS::start[gi], p1 = GS::start[gi + 1];
    hipLaunchKernelGGL((conv_fwd_kernel<LIN, LEDGE, LOUT, p0, p1, false, true>), grid, dim3(kWave), 0, st, a.N, a.C,
                       a.rowptr, a.sender, a.pos, a.shift, a.x, a.W, a.z, a.rc, a.mlp_h);
  });
}

// ============================================ radial-weight gradient ====
// W_bar[b, p, k] = sum_e R_b(r_e) <g[u_e, p, k], f_p(x[v_e, k], y_e)>, the
// weight-gradient line of Eq. C1 carried through w = R W.  Receiver-sorted
// like the forward: a block of kWgWaves waves covers kWgWaves consecutive
// receivers (one each) and 64 channels; wave w keeps g[u_w] of the group's
// paths in registers, evaluates f_p(x_v, y_e) for every incoming edge from
// the broadcast edge record, and accumulates R_b w_bar_p in kNB x NP
// registers.  The waves' sums are added in wave order through LDS and the
// block writes one partial [kNB][P][C] slab; launch_block_sum adds the slabs
// in block order.  One launch per path group.
// Adds the kWgWaves waves' accumulators acc[b * NP + pi] in wave order
// (through `red`, kWave * kNB * NP floats that every wave may overwrite)
// and stores the block's slab rows b, P0 + pi of wpart [blocks][kNB][P][C].
template <int NP, int P0, int P>
__device__ __forceinline__ void wgrad_block_store(float* acc, float* red, int wv, int lane, int k, bool act, int C,
                                                  float* __restrict__ wpart) {
  constexpr int NACC = kNB * NP;
  for (int w = 1; w < kWgWaves; ++w) {
    __syncthreads();
    if (wv == w) static_for<NACC>([&](auto i) { red[i * kWave + lane] = acc[i]; });
    __syncthreads();
    if (wv == 0) static_for<NACC>([&](auto i) { acc[i] += red[i * kWave + lane]; });
  }
  if (wv == 0 && act) {
    float* dst = wpart + (size_t)blockIdx.x * kNB * P * C + k;
    static_for<NACC>([&](auto i) {
      constexpr int b = i / NP, pi = i % NP;
      dst[((size_t)b * P + P0 + pi) * C] = acc[i];
    });
  }
}

template <int LIN, int LEDGE, int LOUT, int P0, int P1>
__global__ __launch_bounds__(kWgWaves * kWave) void conv_wgrad_kernel(
    int N, int C, const int* __restrict__ rowptr, const int* __restrict__ sender,
    const float* __restrict__ pos, const float* __restrict__ shift, const float* __restrict__ x,
    const float* __restrict__ g, float* __restrict__ wpart, float rc) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using G = PathGroup<Cfg, P0, P1>;
  using EP = EdgeProducts<LIN, LEDGE, LOUT>;
  constexpr int NIN = Cfg::NIN, P = Cfg::P, NOUT = Cfg::NOUT;
  constexpr int REC = EP::NY + kNB + 1;
  constexpr int NACC = kNB * G::NP;
  // edge records of every wave; reused afterwards for the cross-wave sums
  constexpr int LDS = (kWgWaves * kWave * REC > kWave * NACC) ? kWgWaves * kWave * REC : kWave * NACC;
  __shared__ float lds[LDS];

  const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int u0 = blockIdx.x * kWgWaves, u = u0 + wv;
  const bool has_u = u < N;
  const int k = blockIdx.y * kWave + lane;
  const bool act = k < C;
  const int kk = act ? k : 0;
  const int voff = kk * 4;
  float* geo = lds + wv * kWave * REC;

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

  // chunk count shared by the block's waves (they meet at every barrier)
  int nch = 0;
  for (int i = 0; i < kWgWaves; ++i)
    if (u0 + i < N) nch = max(nch, (rowptr[u0 + i + 1] - rowptr[u0 + i] + kWave - 1) / kWave);
  const int e0 = has_u ? rowptr[u] : 0, e1 = has_u ? rowptr[u + 1] : 0;
  const float pux = has_u ? pos[3 * u] : 0.f, puy = has_u ? pos[3 * u + 1] : 0.f, puz = has_u ? pos[3 * u + 2] : 0.f;
  for (int ch = 0; ch < nch; ++ch) {
    const int base = e0 + ch * kWave;
    const int cnt = max(0, min(kWave, e1 - base));
    if (lane < cnt)
      recv_edge_record<LIN, LEDGE, LOUT>(base + lane, sender, pos, shift, pux, puy, puz, rc, geo + lane * REC);
    __syncthreads();
    for (int j = 0; j < cnt; ++j) {
      const float* rec = geo + j * REC;
      const int s = uniform_int(__float_as_int(rec[EP::NY + kNB]));
      const auto xs = node_rsrc(x, s, NIN * C);
      float xv[NIN];
      static_for<NIN>([&](auto c) { xv[c] = buf_load(xs, voff, c * C * 4); });
      static_for<G::NP>([&](auto pi) {
        constexpr int p = P0 + pi;
        constexpr PathInfo PI = Cfg::paths[p];
        constexpr int na = ncomp(PI.L), o1 = rank_off(PI.l1), o2 = rank_off(PI.l2);
        constexpr int lo = G::loff(p);
        constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
        float f[na];
        static_for<te - tb>([&](auto ti) {
          constexpr int tt = tb + ti;
          constexpr tab::Term T = tab::kTerms[tt];
          const float cy = EP::template cy<tt, o2 + T.b2>(rec);
          if constexpr (T.fa) f[T.a] = cy * xv[o1 + T.b1];
          else f[T.a] = fmaf(cy, xv[o1 + T.b1], f[T.a]);
        });
        float wb = 0.f;
        static_for<na>([&](auto a) { wb = fmaf(gv[lo + a], f[a], wb); });
        static_for<kNB>([&](auto b) {
          constexpr int bb = b;
          acc[bb * G::NP + pi] = fmaf(rec[EP::NY + bb], wb, acc[bb * G::NP + pi]);
        });
      });
    }
    __syncthreads();
  }
  wgrad_block_store<G::NP, P0, P>(acc, lds, wv, lane, k, act, C, wpart);
}

template <int LIN, int LEDGE, int LOUT>
void launch_wgrad(const ConvArgs& a, float* wpart, hipStream_t st) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using GS = PathGroups<Cfg, fwd_budget(Cfg::NIN)>;
  const int nblk = wgrad_blocks(a.N);
  dim3 grid(nblk, (a.C + kWave - 1) / kWave);
  static_for<GS::n>([&](auto gi) {
    constexpr int p0 = GS::start[gi], p1 = GS::start[gi + 1];
    hipLaunchKernelGGL((conv_wgrad_kernel<LIN, LEDGE, LOUT, p0, p1>), grid, dim3(kWgWaves * kWave), 0, st, a.N, a.C,
                       a.rowptr, a.sender, a.pos, a.shift, a.x, a.g, wpart, a.rc);
  });
  launch_block_sum(nblk, kNB * Cfg::P * a.C, wpart, a.W_bar, st);
}

// ================================================================== VJP ====
// Sender-sorted pass: a block of NW = ceil(C/64) waves holds all C channels
// of sender v (C <= 256) and one of S contiguous slices of v's outgoing
// edges (slices balance the unequal out-degrees; their partial x_bar and
// position sums are combined in a fixed order by conv_vjp_combine_kernel).
// For every outgoing edge e = (v -> u), gather g[u] and accumulate
//   x_bar[v]  += sum_p w_p VJP1_p(g_p, y)                       (per lane)
//   y_bar_e    = sum_{p,k} w_p VJP2_p(g_p, x_v)                 (over lanes)
//   s_e        = sum_{p,k} <g_p, f_p(x_v, y)> dw_p/dr            (over lanes)
// with w_p = sum_b R_b W[b,p] and dw_p/dr = sum_b R'_b W[b,p].  The edge's
// position cotangent is
//   r_bar_e = s_e r_hat + (I - r_hat r_hat^T)/r (sum_c y_bar_c grad_n y_c);
// it is added to the sender and stored per edge for the combine pass.
// The NE+1 per-edge sums over lanes use DPP row rotations (16 lanes) and the
// four row totals of every wave are combined from LDS once per chunk of
// edges (64, or 32 where LDS would not hold 64 at rank 5).
template <int LIN, int LEDGE, int LOUT>
struct VjpShape {
  using EP = EdgeProducts<LIN, LEDGE, LOUT>;
  static constexpr int NE = nrank(LEDGE);
  static constexpr int NRED = NE + 1;                      // y_bar components, s
  static constexpr int REC = EP::NY + 2 * kNB + 2;         // y / products, R, R', receiver, edge id
  static constexpr int budget = vjp_budget(nrank(LIN), NE, LOUT < kAllParities) - (EP::kCXReg ? EP::CXt::n : 0);
  static constexpr int wide_budget = vjp_budget(nrank(LIN), NE, false) - (EP::kCXReg ? EP::CXt::n : 0);
  static constexpr bool wide_when_narrow = vjp_wide_when_narrow(nrank(LIN), NE, LOUT < kAllParities);
  // edge records of a chunk of ch edges plus the per-wave row sums
  static constexpr size_t lds_bytes(int nw, int ch) {
    return sizeof(float) * ((size_t)ch * REC + (size_t)nw * ch * NRED * 4);
  }
  // edges per chunk: 64, or 32 where 64 would not fit the 160 KB of a
  // workgroup at 256 channels or would keep two blocks of two waves (128
  // channels) from sharing a CU
  static constexpr bool fits(int ch) {
    return lds_bytes(kMaxVjpWaves, ch) <= kLdsBytes && lds_bytes(2, ch) <= kLdsBytes / 2;
  }
  static constexpr int CH = fits(64) ? 64 : 32;
  static_assert(lds_bytes(kMaxVjpWaves, CH) <= kLdsBytes, "VJP chunk does not fit in LDS");
};

__device__ __forceinline__ float row_sum16(float v) {
  // every lane of a 16-lane row ends with the row total
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xF, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xF, 0xF, false));
  return v;
}

// XW: explicit per-edge weights, W = w [E][P][C]; the radial term of the
// position cotangent is absent (w is held fixed), the first radial slot of
// the edge record flags an edge of nonzero length, and (wb_out non-null)
// w_bar[e, p, k] = <g_p, f_p(x, y)> is stored per edge.
// CH: edges staged per chunk (the shape's default, or 32 for short slices,
// which halves the block's LDS).
// MLP: W = W3 [64][P][C] and hh [E][2][64] the second hidden layer of the
// radial network and its r-derivative per edge; w and dw/dr are formed in
// the lanes for batches of mlp_batch_vjp(paths of the group) edges.
// WIDE: the wider path groups of vjp_budget(.., false) (one-wave blocks at rank 4).
template <int LIN, int LEDGE, int LOUT, bool NEED_X, bool NEED_POS, bool XW, int CH = VjpShape<LIN, LEDGE, LOUT>::CH,
          bool MLP = false, bool WIDE = false>
__global__ __launch_bounds__(kMaxVjpWaves * kWave) void conv_vjp_sender_kernel(
    int N, int C, const int* __restrict__ t_rowptr, const int* __restrict__ t_edge,
    const int* __restrict__ receiver, const float* __restrict__ pos,
    const float* __restrict__ shift, const float* __restrict__ x,
    const float* __restrict__ W, const float* __restrict__ g, float* __restrict__ x_out,
    float* __restrict__ p_out, float* __restrict__ rbar, float* __restrict__ wb_out, float rc,
    const float* __restrict__ hh) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using Sh = VjpShape<LIN, LEDGE, LOUT>;
  using EP = typename Sh::EP;
  using CXt = typename EP::CXt;
  constexpr int NIN = Cfg::NIN, NE = Cfg::NE, P = Cfg::P, NOUT = Cfg::NOUT;
  constexpr int REC = Sh::REC, NRED = Sh::NRED, NY = EP::NY;
  using GS = PathGroups<Cfg, WIDE ? Sh::wide_budget : Sh::budget>;
  extern __shared__ float lds[];
  float* geo = lds;                      // [CH][REC]
  float* part = lds + CH * REC;          // [NW][CH edges][NRED][4 rows]
  const int NW = blockDim.x / kWave;
  // MLP: [CH + kMlpBatchVjpMax][HR] activations (and their derivatives) of
  // the chunk's edges (a last batch may read rows past the chunk; unused)
  constexpr int HR = NEED_POS ? kMlpRow2 : kMlpRow;
  float* hsh = part + (NEED_POS ? NW : 0) * CH * NRED * 4;

  const int v = xcd_node(blockIdx.x, N);
  const int S = gridDim.y, sl = blockIdx.y;   // slice sl of S of v's outgoing edges
  const int tid = threadIdx.x;
  const int wv = tid / kWave, lane = tid % kWave;
  const int k = tid;
  const bool act = k < C;
  const int kk = act ? k : 0;
  const int voff = kk * 4;

  float xv[NIN];
  {
    const float* xs = x + (size_t)v * NIN * C + kk;
    static_for<NIN>([&](auto c) { xv[c] = xs[(size_t)c * C]; });
  }
  float cxr[EP::kCXReg && CXt::n > 0 ? CXt::n : 1];
  if constexpr (EP::kCXReg) {
    static_for<CXt::n>([&](auto i) {
      constexpr int ii = i;
      cxr[ii] = CXt::c[ii] * xv[CXt::g[ii]];
    });
  }
  float xb[NIN];
  static_for<NIN>([&](auto c) { xb[c] = 0.f; });
  float psum[3] = {0.f, 0.f, 0.f};

  const int v0 = t_rowptr[v], deg = t_rowptr[v + 1] - v0;
  const int e0 = v0 + (int)(((long long)sl * deg) / S), e1 = v0 + (int)(((long long)(sl + 1) * deg) / S);
  const float pvx = pos[3 * v], pvy = pos[3 * v + 1], pvz = pos[3 * v + 2];

  // One sweep over the slice per path group; x_bar accumulates in registers
  // across the sweeps, and each edge's position cotangent (linear in the
  // per-edge sums) is the sum of the sweeps' parts, added in group order.
  static_for<GS::n>([&](auto gi) {
    using G = typename GS::template group<gi>;
    constexpr bool FIRST = gi == 0;
    // radial weights of this lane's channel for the group's paths (zero for
    // idle lanes, so their contributions to the sums over lanes vanish)
    float Wr[XW || MLP ? 1 : kNB * G::NP];
    if constexpr (!XW && !MLP) {
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
        float rx = pvx - pos[3 * u], ry = pvy - pos[3 * u + 1], rz = pvz - pos[3 * u + 2];
        if (shift) {
          rx += shift[3 * e];
          ry += shift[3 * e + 1];
          rz += shift[3 * e + 2];
        }
        const float r = sqrtf(rx * rx + ry * ry + rz * rz);
        const float inv = r > 0.f ? 1.f / r : 0.f;
        float y[NE];
        direction_tensors<LEDGE>(rx * inv, ry * inv, rz * inv, y);
        float* rec = geo + lane * REC;
        EP::fill(y, rec);
        if constexpr (XW) {
          rec[NY] = r > 0.f ? 1.f : 0.f;
        } else if constexpr (MLP) {
          copy_row<NEED_POS ? kRadRow : kRadHidden>(hh + (size_t)e * kRadRow, hsh + lane * HR);
        } else {
          float R[kNB], dR[kNB];
          radial<true>(r, rc, R, dR);
          static_for<kNB>([&](auto b) {
            rec[NY + b] = R[b];
            rec[NY + kNB + b] = dR[b];
          });
        }
        rec[NY + 2 * kNB] = __int_as_float(u);
        rec[NY + 2 * kNB + 1] = __int_as_float(e);
      }
      __syncthreads();
      // XW: the weights of edge j + 1 are requested after the gather of
      // edge j, so that waiting for the gather leaves the prefetch in flight
      float wn[XW ? G::NP : 1];
      auto w_row = [&](int jj) -> size_t {
        return (size_t)uniform_int(__float_as_int(geo[jj * REC + NY + 2 * kNB + 1])) * P * C + kk;
      };
      if constexpr (XW) {
        if (cnt > 0) {
          const size_t r0 = w_row(0);
          static_for<G::NP>([&](auto pi) { wn[pi] = W[r0 + (size_t)(G::p0 + pi) * C]; });
        }
      }
      // one edge; wm(pi) / dwm(pi) give the fused network's weight of path
      // p0 + pi and its r-derivative
      auto edge = [&](int j, auto wm, auto dwm) {
        const float* rec = geo + j * REC;
        const int u = uniform_int(__float_as_int(rec[NY + 2 * kNB]));
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
        float we[XW ? G::NP : 1];
        [[maybe_unused]] size_t erow = 0;
        if constexpr (XW) {
          erow = w_row(j);
          static_for<G::NP>([&](auto pi) { we[pi] = act ? rec[NY] * wn[pi] : 0.f; });
          if (j + 1 < cnt) {
            const size_t rn = w_row(j + 1);
            static_for<G::NP>([&](auto pi) { wn[pi] = W[rn + (size_t)(G::p0 + pi) * C]; });
          }
        }
        float yb[NE];
        static_for<NE>([&](auto c) { yb[c] = 0.f; });
        float sacc = 0.f;
        static_for<G::NP>([&](auto pi) {
          constexpr int p = G::p0 + pi;
          constexpr PathInfo PI = Cfg::paths[p];
          constexpr int na = ncomp(PI.L), n2 = ncomp(PI.l2);
          constexpr int o1 = rank_off(PI.l1), o2 = rank_off(PI.l2);
          constexpr int lo = G::loff(p);
          constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
          float w = 0.f;
          if constexpr (XW) {
            w = we[pi];
          } else if constexpr (MLP) {
            w = wm(pi);
          } else {
            static_for<kNB>([&](auto b) {
              constexpr int bb = b;
              w = fmaf(rec[NY + bb], Wr[bb * G::NP + pi], w);
            });
          }
          if constexpr (NEED_X) {
            // x_bar[b1] += sum_terms c y[b2] (w g[a]); with fewer inputs than
            // outputs the 2l1+1 sums are weighted instead of the 2L+1 g rows
            constexpr int n1 = ncomp(PI.l1);
            if constexpr (n1 < na) {
              float u[n1];
              static_for<te - tb>([&](auto ti) {
                constexpr int tt = tb + ti;
                constexpr tab::Term T = tab::kTerms[tt];
                const float cy = EP::template cy<tt, o2 + T.b2>(rec);
                if constexpr (T.f1) u[T.b1] = cy * gv[lo + T.a];
                else u[T.b1] = fmaf(cy, gv[lo + T.a], u[T.b1]);
              });
              static_for<n1>([&](auto c) {
                if constexpr (term_has_b1(tb, te, c)) xb[o1 + c] = fmaf(w, u[c], xb[o1 + c]);
              });
            } else {
              float gw[na];
              static_for<na>([&](auto a) { gw[a] = w * gv[lo + a]; });
              static_for<te - tb>([&](auto ti) {
                constexpr int tt = tb + ti;
                constexpr tab::Term T = tab::kTerms[tt];
                xb[o1 + T.b1] = fmaf(EP::template cy<tt, o2 + T.b2>(rec), gw[T.a], xb[o1 + T.b1]);
              });
            }
          }
          if (NEED_POS || (XW && wb_out)) {
            // v2[b2] = sum_terms c g[a] x[b1]  (VJP_2(g, x), unweighted)
            float v2[n2];
            static_for<te - tb>([&](auto ti) {
              constexpr int tt = tb + ti;
              constexpr tab::Term T = tab::kTerms[tt];
              constexpr float ac = T.c < 0.f ? -T.c : T.c;
              float cx;
              if constexpr (ac == 1.f) cx = xv[o1 + T.b1];
              else if constexpr (EP::kCXReg) cx = cxr[CXt::term[tt]];
              else cx = ac * xv[o1 + T.b1];
              if constexpr (T.c < 0.f) cx = -cx;
              if constexpr (T.f2) v2[T.b2] = gv[lo + T.a] * cx;
              else v2[T.b2] = fmaf(gv[lo + T.a], cx, v2[T.b2]);
            });
            float wbar = 0.f;
            static_for<n2>([&](auto c) {
              yb[o2 + c] = fmaf(w, v2[c], yb[o2 + c]);
              wbar = fmaf(v2[c], rec[o2 + c], wbar);
            });
            if constexpr (XW) {
              if (wb_out && act) wb_out[erow + (size_t)p * C] = rec[NY] * wbar;
            } else {
              float dw = 0.f;
              if constexpr (MLP) {
                dw = dwm(pi);
              } else {
                static_for<kNB>([&](auto b) {
                  constexpr int bb = b;
                  dw = fmaf(rec[NY + kNB + bb], Wr[bb * G::NP + pi], dw);
                });
              }
              sacc = fmaf(wbar, dw, sacc);
            }
          }
        });
        if constexpr (NEED_POS) {
          float* dst = part + ((size_t)(wv * CH + j) * NRED) * 4 + (lane >> 4);
          static_for<NE>([&](auto c) {
            if constexpr (G::uses_comp(c)) {
              const float t = row_sum16(yb[c]);
              if ((lane & 15) == 0) dst[c * 4] = t;
            }
          });
          const float t = row_sum16(sacc);
          if ((lane & 15) == 0) dst[NE * 4] = t;
        }
      };
      if constexpr (MLP) {
        constexpr int MB = mlp_batch_vjp(G::NP);
        for (int jb = 0; jb < cnt; jb += MB) {
          float wb[MB * G::NP], dwb[MB * G::NP];
          mlp_batch_weights<MB, G::NP, NEED_POS, HR, 2>(hsh + jb * HR, W + (size_t)G::p0 * C + kk, (size_t)P * C, C, wb,
                                                     dwb);
          // idle lanes carry weight 0 (their products must not reach the sums over lanes)
          if (!act) {
            static_for<MB * G::NP>([&](auto i) {
              wb[i] = 0.f;
              dwb[i] = 0.f;
            });
          }
          static_for<MB>([&](auto bi) {
            constexpr int b = bi;
            if (jb + b < cnt)
              edge(jb + b, [&](auto pi) { return wb[b * G::NP + pi]; }, [&](auto pi) { return dwb[b * G::NP + pi]; });
          });
        }
      } else {
        for (int j = 0; j < cnt; ++j) edge(j, [](auto) { return 0.f; }, [](auto) { return 0.f; });
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
              if constexpr (i == NE || G::uses_comp(i)) {
                const float4 q = src[i];
                tot[i] += (q.x + q.y) + (q.z + q.w);
              }
            });
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
            const float srad = tot[NE];
            float dy[3 * NE];
            direction_tensor_grads<LEDGE>(nx, ny, nz, dy);
            float gx = 0.f, gy = 0.f, gz = 0.f;
            static_for<NE>([&](auto c) {
              if constexpr (G::uses_comp(c)) {
                gx = fmaf(tot[c], dy[3 * c], gx);
                gy = fmaf(tot[c], dy[3 * c + 1], gy);
                gz = fmaf(tot[c], dy[3 * c + 2], gz);
              }
            });
            const float gn = gx * nx + gy * ny + gz * nz;
            ox = srad * nx + (gx - gn * nx) * inv;
            oy = srad * ny + (gy - gn * ny) * inv;
            oz = srad * nz + (gz - gn * nz) * inv;
          }
          float* re = rbar + 3 * (size_t)e;
          if constexpr (FIRST) {
            re[0] = ox;
            re[1] = oy;
            re[2] = oz;
          } else {
            re[0] += ox;
            re[1] += oy;
            re[2] += oz;
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
        p_out[3 * slot] = psum[0];
        p_out[3 * slot + 1] = psum[1];
        p_out[3 * slot + 2] = psum[2];
      }
    }
  }
}

// ==================================================== receiver-side VJP ====
// Without x_bar (the message blocks ask for the forces and w_bar only) the
// VJP needs no sender order: a block of NW = ceil(C/64) waves holds all
// channels of receiver u with its cotangent rows g[u] in registers and
// walks u's incoming edges like the forward, gathering the senders' x.  Per
// edge and path it forms v2 = VJP2_p(g, x) per lane and
//   y_bar_e        = sum_{p,k} w_p v2_p        (over lanes, DPP rows + LDS)
//   w_bar[e, p, k] = <v2_p, y>                 (stored when wb_out)
// and the edge lane turns y_bar_e into r_bar_e = (I - r_hat r_hat^T)/r
// grad_n(y_bar . y), stored per edge; launch_pos_from_edges then sums the
// out-edges minus the in-edges of every node in a fixed order.  Each row of
// g is read once per receiver instead of once per incoming edge in sender
// order, where the rows of the receivers in flight on an XCD outgrow its L2.
// Explicit per-edge weights only (the weights w [E][P][C] are read in edge
// order, w_bar written in edge order).
template <int LIN, int LEDGE, int LOUT, bool NEED_POS, int CH>
__global__ __launch_bounds__(kMaxVjpWaves * kWave) void conv_vjp_recv_kernel(
    int N, int C, const int* __restrict__ rowptr, const int* __restrict__ sender,
    const float* __restrict__ pos, const float* __restrict__ shift, const float* __restrict__ x,
    const float* __restrict__ W, const float* __restrict__ g, float* __restrict__ rbar,
    float* __restrict__ wb_out) {
  using Cfg = ConvCfg<LIN, LEDGE, LOUT>;
  using Sh = VjpShape<LIN, LEDGE, LOUT>;
  using EP = typename Sh::EP;
  constexpr int NIN = Cfg::NIN, NE = Cfg::NE, P = Cfg::P, NOUT = Cfg::NOUT;
  constexpr int REC = Sh::REC, NRED = Sh::NRED, NY = EP::NY;
  using GS = PathGroups<Cfg, Sh::budget>;
  extern __shared__ float lds[];
  float* geo = lds;                      // [CH][REC]
  float* part = lds + CH * REC;          // [NW][CH edges][NRED][4 rows]

  const int NW = blockDim.x / kWave;
  const int u = xcd_node(blockIdx.x, N);
  const int tid = threadIdx.x;
  const int wv = tid / kWave, lane = tid % kWave;
  const int k = tid;
  const bool act = k < C;
  const int kk = act ? k : 0;
  const int voff = kk * 4;
  const int e0 = rowptr[u], e1 = rowptr[u + 1];
  const float pux = pos[3 * u], puy = pos[3 * u + 1], puz = pos[3 * u + 2];

  // one sweep over u's edges per path group; the groups' parts of each
  // edge's position term are added in group order
  static_for<GS::n>([&](auto gi) {
    using G = typename GS::template group<gi>;
    constexpr bool FIRST = gi == 0;
    float gv[G::NR];
    {
      const float* gu = g + (size_t)u * NOUT * C + kk;
      static_for<G::NP>([&](auto pi) {
        constexpr int p = G::p0 + pi;
        if constexpr (!G::owner(p)) return;
        static_for<ncomp(Cfg::paths[p].L)>([&](auto c) {
          constexpr int row = Cfg::row(p, c), li = G::loff(p) + c;
          gv[li] = gu[(size_t)row * C];
        });
      });
    }
    for (int base = e0; base < e1; base += CH) {
      const int cnt = min(CH, e1 - base);
      if (wv == 0 && lane < cnt) {
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
        float y[NE];
        direction_tensors<LEDGE>(rx * inv, ry * inv, rz * inv, y);
        float* rec = geo + lane * REC;
        EP::fill(y, rec);
        rec[NY] = r > 0.f ? 1.f : 0.f;   // an edge without a direction takes no part
        rec[NY + 2 * kNB] = __int_as_float(s);
      }
      __syncthreads();
      // the weights of edge j + 1 are requested after the gather of edge j
      float wn[G::NP];
      if (cnt > 0) {
        const float* wrow = W + (size_t)base * P * C + kk;
        static_for<G::NP>([&](auto pi) { wn[pi] = wrow[(size_t)(G::p0 + pi) * C]; });
      }
      for (int j = 0; j < cnt; ++j) {
        const float* rec = geo + j * REC;
        const int s = uniform_int(__float_as_int(rec[NY + 2 * kNB]));
        const auto xs = node_rsrc(x, s, NIN * C);
        float xv[NIN];
        static_for<NIN>([&](auto c) { xv[c] = buf_load(xs, voff, c * C * 4); });
        float we[G::NP];
        static_for<G::NP>([&](auto pi) { we[pi] = act ? rec[NY] * wn[pi] : 0.f; });
        if (j + 1 < cnt) {
          const float* wrow = W + (size_t)(base + j + 1) * P * C + kk;
          static_for<G::NP>([&](auto pi) { wn[pi] = wrow[(size_t)(G::p0 + pi) * C]; });
        }
        float yb[NE];
        static_for<NE>([&](auto c) { yb[c] = 0.f; });
        static_for<G::NP>([&](auto pi) {
          constexpr int p = G::p0 + pi;
          constexpr PathInfo PI = Cfg::paths[p];
          constexpr int n2 = ncomp(PI.l2), o1 = rank_off(PI.l1), o2 = rank_off(PI.l2);
          constexpr int lo = G::loff(p);
          constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
          // v2[b2] = sum_terms c g[a] x[b1]  (VJP_2(g, x))
          float v2[n2];
          static_for<te - tb>([&](auto ti) {
            constexpr int tt = tb + ti;
            constexpr tab::Term T = tab::kTerms[tt];
            constexpr float ac = T.c < 0.f ? -T.c : T.c;
            float cx = ac == 1.f ? xv[o1 + T.b1] : ac * xv[o1 + T.b1];
            if constexpr (T.c < 0.f) cx = -cx;
            if constexpr (T.f2) v2[T.b2] = gv[lo + T.a] * cx;
            else v2[T.b2] = fmaf(gv[lo + T.a], cx, v2[T.b2]);
          });
          float wbar = 0.f;
          static_for<n2>([&](auto c) {
            if constexpr (NEED_POS) yb[o2 + c] = fmaf(we[pi], v2[c], yb[o2 + c]);
            wbar = fmaf(v2[c], rec[o2 + c], wbar);
          });
          if (wb_out && act) wb_out[(size_t)(base + j) * P * C + (size_t)p * C + k] = rec[NY] * wbar;
        });
        if constexpr (NEED_POS) {
          float* dst = part + ((size_t)(wv * CH + j) * NRED) * 4 + (lane >> 4);
          static_for<NE>([&](auto c) {
            if constexpr (G::uses_comp(c)) {
              const float t = row_sum16(yb[c]);
              if ((lane & 15) == 0) dst[c * 4] = t;
            }
          });
        }
      }
      __syncthreads();
      if constexpr (NEED_POS) {
        if (wv == 0 && lane < cnt) {
          const int e = base + lane;
          const int s = sender[e];
          float tot[NE];
          static_for<NE>([&](auto i) { tot[i] = 0.f; });
          for (int w2 = 0; w2 < NW; ++w2) {
            const float4* src = reinterpret_cast<const float4*>(part + ((size_t)(w2 * CH + lane) * NRED) * 4);
            static_for<NE>([&](auto i) {
              if constexpr (G::uses_comp(i)) {
                const float4 q = src[i];
                tot[i] += (q.x + q.y) + (q.z + q.w);
              }
            });
          }
          float rx = pos[3 * s] - pux, ry = pos[3 * s + 1] - puy, rz = pos[3 * s + 2] - puz;
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
            float dy[3 * NE];
            direction_tensor_grads<LEDGE>(nx, ny, nz, dy);
            float gx = 0.f, gy = 0.f, gz = 0.f;
            static_for<NE>([&](auto c) {
              if constexpr (G::uses_comp(c)) {
                gx = fmaf(tot[c], dy[3 * c], gx);
                gy = fmaf(tot[c], dy[3 * c + 1], gy);
                gz = fmaf(tot[c], dy[3 * c + 2], gz);
              }
            });
            const float gn = gx * nx + gy * ny + gz * nz;
            ox = (gx - gn * nx) * inv;
            oy = (gy - gn * ny) * inv;
            oz = (gz - gn * nz) * inv;
          }
          float* re = rbar + 3 * (size_t)e;
          if constexpr (FIRST) {
            re[0] = ox;
            re[1] = oy;
            re[2] = oz;
          } else {
            re[0] += ox;
            re[1] += oy;
            re[2] += oz;
          }
        }
        __syncthreads();
      }
    }
  });
}

template <int LIN, int LEDGE, int LOUT>
void launch_vjp(const ConvArgs& a, hipStream_t st) {
  const bool nx = a.x_bar != nullptr, np = a.pos_bar != nullptr;
  const int nw = (a.C + kWave - 1) / kWave;
  const VjpWorkspace wsl(a.N, a.E, a.C, nrank(LIN), ConvCfg<LIN, LEDGE, LOUT>::P, true, a.rbar);
  if (a.W_bar && !a.w_edge) launch_wgrad<LIN, LEDGE, LOUT>(a, wsl.w_part, st);
  if (!nx && !np && !(a.w_edge && a.w_edge_bar)) return;
  using Sh = VjpShape<LIN, LEDGE, LOUT>;
  if (a.w_edge && !nx) {
    // explicit weights without x_bar: receiver order (each g row read once)
    const int ch = Sh::CH > 32 && Sh::lds_bytes(np ? nw : 0, Sh::CH) > kLdsBytes / 4 ? 32 : Sh::CH;
#define FC_VJP_RECV(NP, CHV)                                                                                         \
  hipLaunchKernelGGL((conv_vjp_recv_kernel<LIN, LEDGE, LOUT, NP, CHV>), dim3(a.N), dim3(nw * kWave),                   \
                     Sh::lds_bytes(NP ? nw : 0, CHV), st, a.N, a.C, a.rowptr, a.sender, a.pos, a.shift, a.x, a.w_edge,  \
                     a.g, wsl.rbar, a.w_edge_bar)
    if (ch == 32) {
      if (np) FC_VJP_RECV(true, 32);
      else FC_VJP_RECV(false, 32);
    } else if constexpr (Sh::CH > 32) {
      if (np) FC_VJP_RECV(true, Sh::CH);
      else FC_VJP_RECV(false, Sh::CH);
    }
#undef FC_VJP_RECV
    if (np) launch_pos_from_edges(a, wsl.rbar, st);
    return;
  }
  float* xo = wsl.S == 1 ? a.x_bar : wsl.x_part;
  float* po = wsl.S == 1 ? a.pos_bar : wsl.p_part;
  dim3 grid(a.N, wsl.S), block(nw * kWave);
  // slices of at most 32 edges on average (e.g. 128 or fewer neighbours in
  // four slices) stage 32 edges per chunk when the block's LDS at 64 would
  // keep four blocks from sharing a CU (it then holds half as much; at ranks
  // <= 2 the registers, not the LDS, limit the blocks per CU)
  const bool short_slices = (long long)a.E <= 32LL * a.N * wsl.S &&
                            Sh::lds_bytes(np ? nw : 0, Sh::CH) > kLdsBytes / 4;
#define FC_VJP_CH(NX, NP, XW, CHV)                                                                                   \
  hipLaunchKernelGGL((conv_vjp_sender_kernel<LIN, LEDGE, LOUT, NX, NP, XW, CHV>), grid, block,                      \
                     Sh::lds_bytes(np ? nw : 0, CHV), st, a.N, a.C, a.t_rowptr, a.t_edge, a.receiver, a.pos,         \
                     a.shift, a.x, XW ? a.w_edge : a.W, a.g, xo, po, wsl.rbar, a.w_edge_bar, a.rc, nullptr)
#define FC_VJP(NX, NP, XW)                          \
  do {                                              \
    if constexpr (Sh::CH > 32) {                    \
      if (short_slices) {                           \
        FC_VJP_CH(NX, NP, XW, 32);                  \
        break;                                      \
      }                                             \
    }                                               \
    FC_VJP_CH(NX, NP, XW, Sh::CH);                  \
  } while (0)
  if (a.w_edge) {
    if (nx && np) FC_VJP(true, true, true);
    else if (nx) FC_VJP(true, false, true);
    else if (np) FC_VJP(false, true, true);
    else FC_VJP(false, false, true);
  } else if constexpr (Sh::wide_when_narrow) {
    // (32-edge chunks, as the wide groups were measured with)
#define FC_VJP_WIDE(NX, NP)                                                                                         \
  hipLaunchKernelGGL((conv_vjp_sender_kernel<LIN, LEDGE, LOUT, NX, NP, false, 32, false, true>), grid, block,        \
                     Sh::lds_bytes(np ? nw : 0, 32), st, a.N, a.C, a.t_rowptr, a.t_edge, a.receiver, a.pos, a.shift,   \
                     a.x, a.W, a.g, xo, po, wsl.rbar, nullptr, a.rc, nullptr)
    if (nw == 1) {
      if (nx && np) FC_VJP_WIDE(true, true);
      else if (nx) FC_VJP_WIDE(true, false);
      else FC_VJP_WIDE(false, true);
    } else {
      if (nx && np) FC_VJP(true, true, false);
      else if (nx) FC_VJP(true, false, false);
      else FC_VJP(false, true, false);
    }
#undef FC_VJP_WIDE
  } else {
    if (nx && np) FC_VJP(true, true, false);
    else if (nx) FC_VJP(true, false, false);
    else FC_VJP(false, true, false);
  }
#undef FC_VJP
#undef FC_VJP_CH
  launch_vjp_combine(a, wsl, nrank(LIN), st);
}

// VJP with the radial network fused (a.W = W3, a.mlp_h = [E][2][64] h2 and
// dh2/dr): x_bar and/or pos_bar, the latter with the radial term through
// w(r); 32 edges per chunk keep the activation rows within a quarter of
// the LDS at 128 channels.
template <int LIN, int LEDGE, int LOUT>
void launch_vjp_mlp(const ConvArgs& a, hipStream_t st) {
  const bool nx = a.x_bar != nullptr, np = a.pos_bar != nullptr;
  if (!nx && !np) return;
  const int nw = (a.C + kWave - 1) / kWave;
  const VjpWorkspace wsl(a.N, a.E, a.C, nrank(LIN), ConvCfg<LIN, LEDGE, LOUT>::P, false, a.rbar);
  float* xo = wsl.S == 1 ? a.x_bar : wsl.x_part;
  float* po = wsl.S == 1 ? a.pos_bar : wsl.p_part;
  dim3 grid(a.N, wsl.S), block(nw * kWave);
  using Sh = VjpShape<LIN, LEDGE, LOUT>;
  constexpr int CHM = 32;
  // activation rows of the chunk's edges, plus the rows a last partial batch reads past its end
  const size_t lds = Sh::lds_bytes(np ? nw : 0, CHM) + sizeof(float) * (CHM + kMlpBatchVjpMax) * (np ? kMlpRow2 : kMlpRow);
#define FC_VJP_MLP(NX, NP)                                                                                          \
  hipLaunchKernelGGL((conv_vjp_sender_kernel<LIN, LEDGE, LOUT, NX, NP, false, CHM, true>), grid, block, lds, st, a.N, \
                     a.C, a.t_rowptr, a.t_edge, a.receiver, a.pos, a.shift, a.x, a.W, a.g, xo, po, wsl.rbar, nullptr,  \
                     a.rc, a.mlp_h)
  if (nx && np) FC_VJP_MLP(true, true);
  else if (nx) FC_VJP_MLP(true, false);
  else FC_VJP_MLP(false, true);
#undef FC_VJP_MLP
  launch_vjp_combine(a, wsl, nrank(LIN), st);
}

}  // namespace fc
