// Node-local correlation ladder for gfx950 (FlashCart paper §5 Eq. 2 and
// App. E "Path-reduced products").
//
// Full ladder, per step q >= 2: the channel-diagonal products
// B_eta = (phi^{q-1}_{l1} (x) A_{l2})_L of every path eta and the
// path/channel mixing phi^q_L = B_L W^q_L^T run in one kernel
// (ladder_step_kernel): product waves form each K tile of B in LDS while
// MFMA waves multiply the previous one, so B never reaches memory, and the
// epilogue adds phi^q into the output sum z.  Shapes that kernel does not
// cover (C other than 64 or 128, l_prod = 4) write B to a GEMM-ready buffer
// with a VALU kernel (one row (u, component) per output rank, columns (eta,
// channel)) and run the mixing as a grouped FP32 MFMA GEMM.  The reverse
// passes always recompute B into a buffer.
// Path-reduced products: every step runs in registers per (node, channel)
// with the per-path weights a^q, and one grouped GEMM applies the final
// rank-wise maps W_L.
//
// Supported shapes: l_a = l_prod in 1..4, 0 <= l_out <= l_prod, 1 <= order
// <= 8, C a multiple of 32 in [32, 512].
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "fc_common.h"
#include "fc_gemm.h"
#include "fc_ladder.h"
#include "fc_reduce.h"

namespace fc {

constexpr int kRedWaves = 4;   // waves per block of the path-reduced reverse kernel

// ------------------------------------------------------- product kernels --

// One step of the full ladder: B rows for all paths of ConvCfg<LP, LA, LQ>.
// phi [N][phi_rows][C], A [N][a_rows][C]; B block of rank L starts at
// N * off(L) * C floats, row (u (2L+1) + a), column (eta_L C + k).  With
// acc the products are added to B.  TWO: B gets prod(phi, A) +
// prod(phi2, A2) in one pass (a tangent B' = prod(phi', A) + prod(phi, A')
// without writing and re-reading B' in between).
template <int LP, int LA, int LQ, bool TWO>
__global__ __launch_bounds__(kWave) void ladder_prod_kernel(int N, int C, const float* __restrict__ phi,
                                                            int phi_rows, const float* __restrict__ A,
                                                            int a_rows, float* __restrict__ B, int acc,
                                                            const float* __restrict__ phi2,
                                                            const float* __restrict__ A2) {
  using Cfg = ConvCfg<LP, LA, LQ>;
  const int u = blockIdx.x;
  const int k = blockIdx.y * kWave + threadIdx.x;
  if (k >= C) return;
  float x[nrank(LP)], y[nrank(LA)], x2[TWO ? nrank(LP) : 1], y2[TWO ? nrank(LA) : 1];
  static_for<nrank(LP)>([&](auto c) { x[c] = phi[((size_t)u * phi_rows + c) * C + k]; });
  static_for<nrank(LA)>([&](auto c) { y[c] = A[((size_t)u * a_rows + c) * C + k]; });
  if constexpr (TWO) {
    static_for<nrank(LP)>([&](auto c) { x2[c] = phi2[((size_t)u * phi_rows + c) * C + k]; });
    static_for<nrank(LA)>([&](auto c) { y2[c] = A2[((size_t)u * a_rows + c) * C + k]; });
  }
  static_for<Cfg::P>([&](auto pc) {
    constexpr int p = pc;
    constexpr PathInfo PI = Cfg::paths[p];
    constexpr int na = ncomp(PI.L), o1 = rank_off(PI.l1), o2 = rank_off(PI.l2);
    constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
    float t[na];
    static_for<te - tb>([&](auto ti) {
      constexpr tab::Term T = tab::kTerms[tb + ti];
      float xy = x[o1 + T.b1] * y[o2 + T.b2];
      if constexpr (TWO) xy = fmaf(x2[o1 + T.b1], y2[o2 + T.b2], xy);
      if constexpr (T.fa) t[T.a] = T.c * xy;
      else t[T.a] = fmaf(T.c, xy, t[T.a]);
    });
    float* dst = B + (size_t)N * PI.off * C + (size_t)PI.eta * C + k;
    const size_t ld = (size_t)PI.PL * C;
    static_for<na>([&](auto a) {
      float* d = dst + ((size_t)u * na + a) * ld;
      *d = acc ? *d + t[a] : t[a];
    });
  });
}

// ------------------------------------------- fused product + mixing step --
//
// One step q >= 2 of the full ladder without the product buffer: the
// channel-diagonal products are formed in LDS as the matrix-core A operand.
// A block takes 32 nodes and one output rank L; its rows are ordered (c,
// node), so each 32-row MFMA block belongs to one component c.  The K tiles
// (32 channels of one path) run channel block outer, path inner, so that the
// 2 l_prod + 1 ... rows of phi and A of a channel block are loaded once and
// serve every path of the rank.  The block's eight waves split the work:
// waves 4-7 hold those rows for one node and four channels each and form the
// products of the next K tile, while waves 0-3 run the MFMAs of the current
// one, wave w owning output columns [32 w, 32 w + 32) for every component,
// its W^q_L operand loaded straight from global memory (L2) into registers,
// as no other wave reads it.  One barrier per K tile hands the
// double-buffered product tile over.
constexpr int kStepNodes = 32;    // nodes per block: one MFMA row block per component
constexpr int kStepKPad = 36;     // LDS row length of the product tile (floats)
constexpr int kStepMaxItems = 6;

struct StepItem {
  int L;                     // output rank
  long long woff;            // offset of W^q_L [C][P_L C] in the flat weights
};
struct StepPlan {
  int count, tiles;          // items (blocks per node tile), node tiles
  StepItem item[kStepMaxItems];
};

// Whether the phi rows of path e's l1 block (A rows of its l2 block, with
// SECOND) are used by no later path of rank L: then they can be reloaded for
// the next channel block right after path e.
template <class Cfg, int FIRST, int P>
__host__ __device__ constexpr bool step_last_use(int e, bool second) {
  const int l = second ? Cfg::paths[FIRST + e].l2 : Cfg::paths[FIRST + e].l1;
  for (int f = e + 1; f < P; ++f)
    if ((second ? Cfg::paths[FIRST + f].l2 : Cfg::paths[FIRST + f].l1) == l) return false;
  return true;
}

template <int LP, int LQ, int L>
__device__ __forceinline__ void step_body(int N, int C, const float* __restrict__ phi, const float* __restrict__ A,
                                          const float* __restrict__ wl, float* __restrict__ out,
                                          float* __restrict__ z, int z_rows, int lz, int u0, float* Ps) {
  using Cfg = ConvCfg<LP, LP, LQ>;
  typedef float f4 __attribute__((ext_vector_type(4)));
  typedef float f16 __attribute__((ext_vector_type(16)));
  constexpr int R = nrank(LP);   // rows of phi, A and out per node
  constexpr int NC = ncomp(L);
  constexpr int P = Cfg::count_L(L), FIRST = Cfg::first_path_of(L);
  constexpr int TILE = ncomp(LP) * kStepNodes * kStepKPad;
  const int nkb = C / 32;   // even
  // Step t (0 .. ntiles - 1, then a final MFMA pass): the product waves form
  // K tile t (channel block t / P, path t % P) into buffer t % 2 while the
  // MFMA waves consume tile t - 1; one barrier per step.  The channel blocks
  // go in pairs, so every step of a pair is straight-line code with
  // compile-time path and buffer, and the waits on loads are exact.

  f16 acc[NC];   // MFMA waves only
  if (threadIdx.x < 256) {
    static_for<NC>([&](auto i) { static_for<16>([&](auto r) { acc[i][(int)r] = 0.f; }); });
    // ---- MFMA waves: wave wv owns columns [32 wv, 32 wv + 32)
    const int wv = threadIdx.x / 64, lane = threadIdx.x % 64, h = lane / 32;
    const bool nok = wv < nkb;
    const long long ldw = (long long)P * C;
    const float* wrow = wl + (long long)((nok ? wv : 0) * 32 + lane % 32) * ldw + 16 * h;
    // W columns of K tile (channel block kb, path e): e C + 32 kb
    auto load_w = [&](int kb, int e, f4 (&dst)[4]) {
      const float* src = wrow + (long long)e * C + kb * 32;
      static_for<4>([&](auto q) { dst[q] = *reinterpret_cast<const f4*>(src + 4 * q); });
    };
    auto mma = [&](const float* Sc, const f4 (&bw)[4]) {
      static_for<NC>([&](auto i) {
        const f4* src = reinterpret_cast<const f4*>(Sc + (i * kStepNodes + lane % 32) * kStepKPad + 16 * h);
        f4 a4[4];
        static_for<4>([&](auto q) { a4[q] = src[q]; });
        static_for<16>([&](auto s) {
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(a4[s / 4][(int)s % 4], bw[s / 4][(int)s % 4], acc[i], 0, 0,
                                                        0);
        });
      });
    };
    // W operands in two register sets by tile parity (a pair of channel
    // blocks starts at an even tile, so the parity is fixed per step): the
    // operand of tile t is requested at step t, one step before its MFMAs
    f4 wb[2][4];
    for (int kb = 0; kb < nkb; kb += 2) {
      static_for<2 * P>([&](auto sc) {
        constexpr int s = sc, par = s % 2;
        load_w(kb + s / P, s % P, wb[par]);
        if (kb > 0 || s > 0) {
          __builtin_amdgcn_sched_barrier(0);
          mma(Ps + (par ^ 1) * TILE, wb[par ^ 1]);   // tile t - 1
        }
        __syncthreads();
      });
    }
    mma(Ps + TILE, wb[1]);   // the last tile (odd: the tile count is even)
  } else {
    // ---- product waves: node pu, channels pk .. pk + 3 of a channel block
    const int pt = threadIdx.x - 256;
    const int pu = pt / 8, pk = 4 * (pt % 8);
    const size_t nbase = (size_t)(u0 + pu < N ? u0 + pu : 0) * R * C + pk;   // rows past N: node 0, never stored
    f4 x[R], y[R];
    // channel block 0 of every row block some path of rank L reads
    static_for<P>([&](auto e) {
      constexpr PathInfo PI = Cfg::paths[FIRST + e];
      if constexpr (step_last_use<Cfg, FIRST, P>(e, false)) {
        static_for<ncomp(PI.l1)>([&](auto a) {
          x[rank_off(PI.l1) + a] = *reinterpret_cast<const f4*>(phi + nbase + (size_t)(rank_off(PI.l1) + a) * C);
        });
      }
      if constexpr (step_last_use<Cfg, FIRST, P>(e, true)) {
        static_for<ncomp(PI.l2)>([&](auto a) {
          y[rank_off(PI.l2) + a] = *reinterpret_cast<const f4*>(A + nbase + (size_t)(rank_off(PI.l2) + a) * C);
        });
      }
    });
    // products of path e (the term order of the product-buffer kernel); then
    // the rows whose last use this was are reloaded for channel block kbn
    auto path_step = [&](auto ec, float* S, int kbn) {
      constexpr int e = ec;
      constexpr PathInfo PI = Cfg::paths[FIRST + e];
      constexpr int o1 = rank_off(PI.l1), o2 = rank_off(PI.l2);
      constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
      f4 t[NC];
      static_for<te - tb>([&](auto ti) {
        constexpr tab::Term T = tab::kTerms[tb + ti];
        const f4 xy = x[o1 + T.b1] * y[o2 + T.b2];
        if constexpr (T.fa) t[T.a] = T.c * xy;
        else {
#pragma unroll
          for (int k = 0; k < 4; ++k) t[T.a][k] = fmaf(T.c, xy[k], t[T.a][k]);
        }
      });
      static_for<NC>([&](auto c) { *reinterpret_cast<f4*>(S + (c * kStepNodes + pu) * kStepKPad + pk) = t[c]; });
      // keep the reloads after the products: issued earlier, they would need
      // registers of their own
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (step_last_use<Cfg, FIRST, P>(e, false)) {
        static_for<ncomp(PI.l1)>([&](auto a) {
          x[o1 + a] = *reinterpret_cast<const f4*>(phi + nbase + (size_t)(o1 + a) * C + kbn * 32);
        });
      }
      if constexpr (step_last_use<Cfg, FIRST, P>(e, true)) {
        static_for<ncomp(PI.l2)>([&](auto a) {
          y[o2 + a] = *reinterpret_cast<const f4*>(A + nbase + (size_t)(o2 + a) * C + kbn * 32);
        });
      }
    };
    for (int kb = 0; kb < nkb; kb += 2) {
      static_for<2 * P>([&](auto sc) {
        constexpr int s = sc, e = s % P, d = s / P;
        // tile kb P + s: path e of channel block kb + d (buffer s % 2, as
        // kb P is even); reloads are for the following channel block
        path_step(std::integral_constant<int, e>{}, Ps + (s % 2) * TILE, min(kb + d + 1, nkb - 1));
        __syncthreads();
      });
    }
  }

  // Epilogue through LDS (the product buffers are free after one more
  // barrier): the MFMA waves place CH components of their accumulators as
  // rows [component][node][C] (accumulator register r of lane l holds node
  // 8 (r / 4) + 4 h + r % 4 and column l % 32 of the wave's block), then all
  // 512 threads write phi^q and add into z as whole 128-bit row pieces, the
  // z values of a thread's pieces requested together.
  constexpr int TP = 128 + 4;                                        // row stride (C <= 128)
  constexpr int CH = (2 * TILE) / (kStepNodes * TP);                 // components per pass
  constexpr int IT = (CH * kStepNodes * 128 / 4 + 511) / 512;         // pieces per thread at C = 128
  const int c4 = C / 4;
  const bool addz = L <= lz;
  static_for<(NC + CH - 1) / CH>([&](auto cc) {
    constexpr int cb = cc * CH, chn = (cb + CH <= NC) ? CH : NC - cb;
    __syncthreads();
    if (threadIdx.x < 256) {
      const int wv = threadIdx.x / 64, lane = threadIdx.x % 64, h = lane / 32;
      if (wv < C / 32) {
        static_for<chn>([&](auto j) {
          static_for<16>([&](auto r) {
            constexpr int row = 8 * (r / 4) + r % 4;
            Ps[(j * kStepNodes + row + 4 * h) * TP + wv * 32 + lane % 32] = acc[cb + j][(int)r];
          });
        });
      }
    }
    __syncthreads();
    const int total = chn * kStepNodes * c4;
    typedef float f4 __attribute__((ext_vector_type(4)));
    f4 zv[IT];
    static_for<IT>([&](auto k) {
      const int idx = threadIdx.x + 512 * k;
      zv[k] = f4{0.f, 0.f, 0.f, 0.f};
      if (addz && idx < total) {
        const int j = idx / (kStepNodes * c4), row = (idx / c4) % kStepNodes, q = idx % c4;
        const int u = u0 + row;
        if (u < N) zv[k] = *reinterpret_cast<const f4*>(z + ((size_t)u * z_rows + L * L + cb + j) * C + 4 * q);
      }
    });
    static_for<IT>([&](auto k) {
      const int idx = threadIdx.x + 512 * k;
      if (idx < total) {
        const int j = idx / (kStepNodes * c4), row = (idx / c4) % kStepNodes, q = idx % c4;
        const int u = u0 + row;
        if (u < N) {
          const f4 v = *reinterpret_cast<const f4*>(Ps + (j * kStepNodes + row) * TP + 4 * q);
          if (out) *reinterpret_cast<f4*>(out + ((size_t)u * R + L * L + cb + j) * C + 4 * q) = v;
          if (addz) *reinterpret_cast<f4*>(z + ((size_t)u * z_rows + L * L + cb + j) * C + 4 * q) = zv[k] + v;
        }
      }
    });
  });
}

template <int LP, int LQ>
__global__ __launch_bounds__(512) void ladder_step_kernel(int N, int C, const float* __restrict__ phi,
                                                         const float* __restrict__ A, const float* __restrict__ w,
                                                         float* __restrict__ out, float* __restrict__ z, int z_rows,
                                                         int lz, StepPlan plan) {
  __shared__ __attribute__((aligned(16))) float Ps[2 * ncomp(LP) * kStepNodes * kStepKPad];
  const int item = blockIdx.x / plan.tiles, tile = blockIdx.x - item * plan.tiles;
  const int L = plan.item[item].L;
  const float* wl = w + plan.item[item].woff;
  static_for<LQ + 1>([&](auto Lc) {
    if (Lc != L) return;
    if constexpr (ConvCfg<LP, LP, LQ>::count_L(Lc) > 0)
      step_body<LP, LQ, Lc>(N, C, phi, A, wl, out, z, z_rows, lz, tile * kStepNodes, Ps);
  });
}

// One step of the path-reduced products in registers:
// new_L = P_L^{-1/2} sum_{eta -> L} a[eta][k] (x_{l1} (x) y_{l2})_L.
template <int LP, int LA, int LQ>
__device__ __forceinline__ void reduced_step(const float* x, const float* y, const float* __restrict__ aw, int C,
                                             int k, float* nw) {
  using Cfg = ConvCfg<LP, LA, LQ>;
  static_for<nrank(LQ)>([&](auto c) { nw[c] = 0.f; });
  static_for<Cfg::P>([&](auto pc) {
    constexpr int p = pc;
    constexpr PathInfo PI = Cfg::paths[p];
    constexpr int na = ncomp(PI.L), o1 = rank_off(PI.l1), o2 = rank_off(PI.l2), oL = rank_off(PI.L);
    constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
    const float a = aw[(size_t)p * C + k];
    float t[na];
    static_for<te - tb>([&](auto ti) {
      constexpr tab::Term T = tab::kTerms[tb + ti];
      float xy = x[o1 + T.b1] * y[o2 + T.b2];
      if constexpr (T.fa) t[T.a] = T.c * xy;
      else t[T.a] = fmaf(T.c, xy, t[T.a]);
    });
    static_for<na>([&](auto c) { nw[oL + c] = fmaf(a, t[c], nw[oL + c]); });
  });
  static_for<LQ + 1>([&](auto Lc) {
    constexpr int L = Lc;
    if constexpr (Cfg::count_L(L) > 1) {
      const float s = 1.0f / sqrtf(float(Cfg::count_L(L)));
      static_for<ncomp(L)>([&](auto c) { nw[rank_off(L) + c] *= s; });
    }
  });
}

// All steps of the path-reduced ladder for one (node, channel); writes the
// step sum S = sum_q Pi_{<= LO} phi^q and (saved != nullptr) phi^q for
// q = 1 .. order-1.
template <int LP, int LO>
__global__ __launch_bounds__(kWave) void ladder_reduced_kernel(int N, int C, int order, const float* __restrict__ A,
                                                               const float* __restrict__ a1,
                                                               const float* __restrict__ amid, int pmid,
                                                               const float* __restrict__ alast,
                                                               float* __restrict__ S, float* __restrict__ saved) {
  constexpr int NP = nrank(LP), NO = nrank(LO);
  const int u = blockIdx.x;
  const int k = blockIdx.y * kWave + threadIdx.x;
  if (k >= C) return;
  float y[NP], x[NP], s[NO];
  static_for<NP>([&](auto c) { y[c] = A[((size_t)u * NP + c) * C + k]; });
  // phi^1 = a1[l] * A_l for l <= l_1 (l_1 = LO when order == 1)
  const int l1max = order == 1 ? LO : LP;
  static_for<LP + 1>([&](auto lc) {
    constexpr int l = lc;
    const float a = l <= l1max ? a1[(size_t)l * C + k] : 0.f;
    static_for<ncomp(l)>([&](auto c) { x[rank_off(l) + c] = a * y[rank_off(l) + c]; });
  });
  static_for<NO>([&](auto c) { s[c] = x[c]; });
  if (saved && order > 1) static_for<NP>([&](auto c) { saved[((size_t)u * NP + c) * C + k] = x[c]; });
  for (int q = 2; q < order; ++q) {
    float nw[NP];
    reduced_step<LP, LP, LP>(x, y, amid + (size_t)(q - 2) * pmid * C, C, k, nw);
    static_for<NO>([&](auto c) { s[c] += nw[c]; });
    static_for<NP>([&](auto c) { x[c] = nw[c]; });
    if (saved)
      static_for<NP>([&](auto c) { saved[(((size_t)(q - 1) * N + u) * NP + c) * C + k] = x[c]; });
  }
  if (order > 1) {
    float nw[NO];
    reduced_step<LP, LP, LO>(x, y, alast, C, k, nw);
    static_for<NO>([&](auto c) { s[c] += nw[c]; });
  }
  static_for<NO>([&](auto c) { S[((size_t)u * NO + c) * C + k] = s[c]; });
}


// ------------------------------------------------------------ VJP kernels --

// Full ladder, reverse of one product step: given Bbar (layout of B),
// phi^{q-1} and A, write G^{q-1} = g_z (ranks <= l_out) + sum_eta VJP1 and
// add sum_eta VJP2 into A_bar.  acc_g adds to G^{q-1} instead (g_z unused);
// A == nullptr drops the VJP1 term, Abar == nullptr the VJP2 term.
template <int LP, int LA, int LQ>
__global__ __launch_bounds__(kWave) void ladder_prod_vjp_kernel(int N, int C, const float* __restrict__ Bbar,
                                                                const float* __restrict__ phi,
                                                                const float* __restrict__ A,
                                                                const float* __restrict__ gz, int gz_rows,
                                                                float* __restrict__ Gprev, int acc_g,
                                                                float* __restrict__ Abar) {
  using Cfg = ConvCfg<LP, LA, LQ>;
  constexpr int NP = nrank(LP), NA = nrank(LA);
  const int u = blockIdx.x;
  const int k = blockIdx.y * kWave + threadIdx.x;
  if (k >= C) return;
  float x[NP], y[NA], gp[NP], ab[NA];
  static_for<NP>([&](auto c) {
    x[c] = phi[((size_t)u * NP + c) * C + k];
    gp[c] = acc_g ? Gprev[((size_t)u * NP + c) * C + k]
                  : (c < gz_rows ? gz[((size_t)u * gz_rows + c) * C + k] : 0.f);
  });
  static_for<NA>([&](auto c) {
    y[c] = A ? A[((size_t)u * NA + c) * C + k] : 0.f;
    ab[c] = 0.f;
  });
  static_for<Cfg::P>([&](auto pc) {
    constexpr int p = pc;
    constexpr PathInfo PI = Cfg::paths[p];
    constexpr int na = ncomp(PI.L), o1 = rank_off(PI.l1), o2 = rank_off(PI.l2);
    constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
    const float* src = Bbar + (size_t)N * PI.off * C + (size_t)PI.eta * C + k;
    const size_t ld = (size_t)PI.PL * C;
    float bb[na];
    static_for<na>([&](auto a) { bb[a] = src[((size_t)u * na + a) * ld]; });
    static_for<te - tb>([&](auto ti) {
      constexpr tab::Term T = tab::kTerms[tb + ti];
      const float cb = T.c * bb[T.a];
      gp[o1 + T.b1] = fmaf(cb, y[o2 + T.b2], gp[o1 + T.b1]);
      ab[o2 + T.b2] = fmaf(cb, x[o1 + T.b1], ab[o2 + T.b2]);
    });
  });
  static_for<NP>([&](auto c) { Gprev[((size_t)u * NP + c) * C + k] = gp[c]; });
  if (Abar) static_for<NA>([&](auto c) { Abar[((size_t)u * NA + c) * C + k] += ab[c]; });
}

// Path-reduced ladder, reverse of step q for a tile of nodes: G = dL/dphi^q
// (ranks <= LQ), phi^{q-1}, A and Sbar = dL/dS.  Writes
//   G^{q-1} = Sbar (ranks <= l_out) + sum_eta s_eta a_eta VJP1(G_L, A_l2)
// (or, for q == 2, applies phi^1 = a1 A directly: A_bar += a1 G^1 and the
// a1 gradient), adds sum_eta s_eta a_eta VJP2(G_L, phi_l1) into A_bar and
// writes per-block partial gradients of a^q (and a1) summed over the tile.
// A block holds kRedWaves waves over the same 64 channels; wave w takes the
// nodes u0 + w, u0 + w + kRedWaves, ... of the tile, and the waves' partial
// weight gradients are added in wave order through LDS.
template <int LP, int LA, int LQ, bool FIRST>
__global__ __launch_bounds__(kRedWaves * kWave) void ladder_reduced_vjp_kernel(
    int N, int C, int ntile, const float* __restrict__ G, int g_rows, const float* __restrict__ phi,
    const float* __restrict__ A, const float* __restrict__ Sbar, int s_rows, const float* __restrict__ aw,
    const float* __restrict__ a1, float* __restrict__ Gprev, float* __restrict__ Abar,
    float* __restrict__ apart, float* __restrict__ a1part, int acc_abar) {
  using Cfg = ConvCfg<LP, LA, LQ>;
  constexpr int NP = nrank(LP), NA = nrank(LA), NQ = nrank(LQ);
  constexpr int NR = Cfg::P + (FIRST ? LP + 1 : 0);   // partial sums per lane
  __shared__ float red[kRedWaves - 1][NR][kWave];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int k = blockIdx.y * kWave + lane;
  const bool active = k < C;
  float aacc[Cfg::P], a1acc[LP + 1];
  static_for<Cfg::P>([&](auto i) { aacc[i] = 0.f; });
  static_for<LP + 1>([&](auto i) { a1acc[i] = 0.f; });
  float aq[Cfg::P];
  static_for<Cfg::P>([&](auto i) { aq[i] = active ? aw[(size_t)i * C + k] : 0.f; });
  const int u0 = blockIdx.x * ntile, u1 = min(N, u0 + ntile);
  for (int u = u0 + wave; active && u < u1; u += kRedWaves) {
    float g[NQ], x[NP], y[NA], gp[NP], ab[NA];
    static_for<NQ>([&](auto c) { g[c] = c < g_rows ? G[((size_t)u * g_rows + c) * C + k] : 0.f; });
    static_for<NP>([&](auto c) {
      x[c] = phi[((size_t)u * NP + c) * C + k];
      gp[c] = c < s_rows ? Sbar[((size_t)u * s_rows + c) * C + k] : 0.f;
    });
    static_for<NA>([&](auto c) {
      y[c] = A[((size_t)u * NA + c) * C + k];
      ab[c] = 0.f;
    });
    static_for<Cfg::P>([&](auto pc) {
      constexpr int p = pc;
      constexpr PathInfo PI = Cfg::paths[p];
      constexpr int na = ncomp(PI.L), o1 = rank_off(PI.l1), o2 = rank_off(PI.l2), oL = rank_off(PI.L);
      constexpr int tb = tab::kTermBegin[PI.type], te = tab::kTermBegin[PI.type + 1];
      const float sc = 1.0f / sqrtf(float(PI.PL));
      float t[na];
      static_for<te - tb>([&](auto ti) {
        constexpr tab::Term T = tab::kTerms[tb + ti];
        const float xy = x[o1 + T.b1] * y[o2 + T.b2];
        if constexpr (T.fa) t[T.a] = T.c * xy;
        else t[T.a] = fmaf(T.c, xy, t[T.a]);
      });
      float dot = 0.f;
      static_for<na>([&](auto a) { dot = fmaf(g[oL + a], t[a], dot); });
      aacc[p] = fmaf(sc, dot, aacc[p]);
      const float sa = sc * aq[p];
      static_for<te - tb>([&](auto ti) {
        constexpr tab::Term T = tab::kTerms[tb + ti];
        const float cg = (T.c * sa) * g[oL + T.a];
        gp[o1 + T.b1] = fmaf(cg, y[o2 + T.b2], gp[o1 + T.b1]);
        ab[o2 + T.b2] = fmaf(cg, x[o1 + T.b1], ab[o2 + T.b2]);
      });
    });
    if constexpr (FIRST) {
      // phi^1_l = a1[l] A_l
      static_for<LP + 1>([&](auto lc) {
        constexpr int l = lc;
        const float a = a1[(size_t)l * C + k];
        float d = 0.f;
        static_for<ncomp(l)>([&](auto c) {
          ab[rank_off(l) + c] = fmaf(a, gp[rank_off(l) + c], ab[rank_off(l) + c]);
          d = fmaf(gp[rank_off(l) + c], y[rank_off(l) + c], d);
        });
        a1acc[l] += d;
      });
    } else {
      static_for<NP>([&](auto c) { Gprev[((size_t)u * NP + c) * C + k] = gp[c]; });
    }
    static_for<NA>([&](auto c) {
      float* d = Abar + ((size_t)u * NA + c) * C + k;
      *d = acc_abar ? *d + ab[c] : ab[c];
    });
  }
  if (wave > 0) {
    static_for<Cfg::P>([&](auto i) { red[wave - 1][i][lane] = aacc[i]; });
    if constexpr (FIRST) static_for<LP + 1>([&](auto i) { red[wave - 1][Cfg::P + i][lane] = a1acc[i]; });
  }
  __syncthreads();
  if (wave == 0 && active) {
    for (int w = 0; w < kRedWaves - 1; ++w) {
      static_for<Cfg::P>([&](auto i) { aacc[i] += red[w][i][lane]; });
      if constexpr (FIRST) static_for<LP + 1>([&](auto i) { a1acc[i] += red[w][Cfg::P + i][lane]; });
    }
    static_for<Cfg::P>([&](auto i) { apart[((size_t)blockIdx.x * Cfg::P + i) * C + k] = aacc[i]; });
    if constexpr (FIRST)
      static_for<LP + 1>([&](auto i) { a1part[((size_t)blockIdx.x * (LP + 1) + i) * C + k] = a1acc[i]; });
  }
}

// Path-reduced ladder of order 1: z = W (a1 A), so A_bar = a1 Sbar and the
// a1 gradient is <Sbar, A> per rank (ranks <= l_out only).
__global__ __launch_bounds__(kWave) void ladder_reduced_first_kernel(int N, int C, int ntile, int lout, int a_rows,
                                                                     const float* __restrict__ Sbar,
                                                                     const float* __restrict__ A,
                                                                     const float* __restrict__ a1,
                                                                     float* __restrict__ Abar,
                                                                     float* __restrict__ a1part) {
  const int k = blockIdx.y * kWave + threadIdx.x;
  if (k >= C) return;
  const int ro = (lout + 1) * (lout + 1);
  float acc[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
  const int u0 = blockIdx.x * ntile, u1 = min(N, u0 + ntile);
  for (int u = u0; u < u1; ++u)
    for (int c = 0; c < ro; ++c) {
      int l = 0;
      while ((l + 1) * (l + 1) <= c) ++l;
      const float sb = Sbar[((size_t)u * ro + c) * C + k];
      Abar[((size_t)u * a_rows + c) * C + k] += a1[(size_t)l * C + k] * sb;
      acc[l] = fmaf(sb, A[((size_t)u * a_rows + c) * C + k], acc[l]);
    }
  for (int l = 0; l <= lout; ++l) a1part[((size_t)blockIdx.x * (lout + 1) + l) * C + k] = acc[l];
}

// ---------------------------------- path-reduced steps on a product buffer --
// The path-reduced VJP-of-VJP runs a step on the full ladder's product
// buffer (layout of ladder_prod_kernel) with the per-path channel weights:
//   mix:      out_L = s_L sum_{eta -> L} (a_eta X_eta + b_eta Y_eta)
//   mix VJP:  B_bar_eta = s_L (a_eta X_L + b_eta Y_L)
//   weights:  part[blk][eta][k] = s_L sum_{u in tile, c} (X_L B1_eta + Y_L B2_eta)
// with s_L = P_L^{-1/2}, a, b [P][C] (either term nullable).

// out (state rows `orows`, nullable) = or += the mix; dS (rows `srows`,
// ranks <= lout, nullable) += or = it as well.
template <int LP, int LA, int LQ>
__global__ __launch_bounds__(kWave) void ladder_mix_kernel(int N, int C, const float* __restrict__ X,
                                                           const float* __restrict__ a,
                                                           const float* __restrict__ Y,
                                                           const float* __restrict__ b, float* __restrict__ out,
                                                           int orows, float* __restrict__ dS, int srows, int lout,
                                                           int acc_s) {
  using Cfg = ConvCfg<LP, LA, LQ>;
  const int u = blockIdx.x;
  const int k = blockIdx.y * kWave + threadIdx.x;
  if (k >= C) return;
  static_for<LQ + 1>([&](auto Lc) {
    constexpr int L = Lc, PL = Cfg::count_L(L), na = ncomp(L);
    if constexpr (PL > 0) {
      constexpr int p0 = Cfg::first_path_of(L), off = Cfg::paths[p0].off;
      const float sL = 1.0f / sqrtf(float(PL));
      const size_t ld = (size_t)PL * C;
      float t[na];
      static_for<na>([&](auto c) { t[c] = 0.f; });
      static_for<PL>([&](auto e) {
        constexpr int eta = e;
        const size_t base = (size_t)N * off * C + (size_t)eta * C + k;
        if (X) {
          const float w = a[(size_t)(p0 + eta) * C + k];
          static_for<na>([&](auto c) { t[c] = fmaf(w, X[base + ((size_t)u * na + c) * ld], t[c]); });
        }
        if (Y) {
          const float w = b[(size_t)(p0 + eta) * C + k];
          static_for<na>([&](auto c) { t[c] = fmaf(w, Y[base + ((size_t)u * na + c) * ld], t[c]); });
        }
      });
      static_for<na>([&](auto c) {
        const float v = sL * t[c];
        if (out) out[((size_t)u * orows + L * L + c) * C + k] = v;
        if (dS && L <= lout) {
          float* d = dS + ((size_t)u * srows + L * L + c) * C + k;
          *d = acc_s ? *d + v : v;
        }
      });
    }
  });
}

template <int LP, int LA, int LQ>
__global__ __launch_bounds__(kWave) void ladder_mix_vjp_kernel(int N, int C, const float* __restrict__ X, int xrows,
                                                               const float* __restrict__ a,
                                                               const float* __restrict__ Y, int yrows,
                                                               const float* __restrict__ b,
                                                               float* __restrict__ Bbar) {
  using Cfg = ConvCfg<LP, LA, LQ>;
  const int u = blockIdx.x;
  const int k = blockIdx.y * kWave + threadIdx.x;
  if (k >= C) return;
  static_for<LQ + 1>([&](auto Lc) {
    constexpr int L = Lc, PL = Cfg::count_L(L), na = ncomp(L);
    if constexpr (PL > 0) {
      constexpr int p0 = Cfg::first_path_of(L), off = Cfg::paths[p0].off;
      const float sL = 1.0f / sqrtf(float(PL));
      const size_t ld = (size_t)PL * C;
      float xv[na], yv[na];
      static_for<na>([&](auto c) {
        xv[c] = X ? X[((size_t)u * xrows + L * L + c) * C + k] : 0.f;
        yv[c] = Y ? Y[((size_t)u * yrows + L * L + c) * C + k] : 0.f;
      });
      static_for<PL>([&](auto e) {
        constexpr int eta = e;
        const float wa = X ? sL * a[(size_t)(p0 + eta) * C + k] : 0.f;
        const float wb = Y ? sL * b[(size_t)(p0 + eta) * C + k] : 0.f;
        float* dst = Bbar + (size_t)N * off * C + (size_t)eta * C + k;
        static_for<na>([&](auto c) { dst[((size_t)u * na + c) * ld] = fmaf(wa, xv[c], wb * yv[c]); });
      });
    }
  });
}

template <int LP, int LA, int LQ>
__global__ __launch_bounds__(kWave) void ladder_mix_wgrad_kernel(int N, int C, int ntile,
                                                                 const float* __restrict__ X, int xrows,
                                                                 const float* __restrict__ B1,
                                                                 const float* __restrict__ Y, int yrows,
                                                                 const float* __restrict__ B2,
                                                                 float* __restrict__ part) {
  using Cfg = ConvCfg<LP, LA, LQ>;
  const int k = blockIdx.y * kWave + threadIdx.x;
  if (k >= C) return;
  const int u0 = blockIdx.x * ntile, u1 = min(N, u0 + ntile);
  static_for<LQ + 1>([&](auto Lc) {
    constexpr int L = Lc, PL = Cfg::count_L(L), na = ncomp(L);
    if constexpr (PL > 0) {
      constexpr int p0 = Cfg::first_path_of(L), off = Cfg::paths[p0].off;
      const float sL = 1.0f / sqrtf(float(PL));
      const size_t ld = (size_t)PL * C;
      float acc[PL];
      static_for<PL>([&](auto e) { acc[e] = 0.f; });
      for (int u = u0; u < u1; ++u) {
        float xv[na], yv[na];
        static_for<na>([&](auto c) {
          xv[c] = X ? X[((size_t)u * xrows + L * L + c) * C + k] : 0.f;
          yv[c] = Y ? Y[((size_t)u * yrows + L * L + c) * C + k] : 0.f;
        });
        static_for<PL>([&](auto e) {
          constexpr int eta = e;
          const size_t base = (size_t)N * off * C + (size_t)eta * C + k;
          float t = acc[eta];
          static_for<na>([&](auto c) {
            if (X) t = fmaf(xv[c], B1[base + ((size_t)u * na + c) * ld], t);
            if (Y) t = fmaf(yv[c], B2[base + ((size_t)u * na + c) * ld], t);
          });
          acc[eta] = t;
        });
      }
      static_for<PL>([&](auto e) {
        part[((size_t)blockIdx.x * Cfg::P + p0 + e) * C + k] = sL * acc[e];
      });
    }
  });
}

// phi'^1 = a1 v_A + b1 A for ranks l <= lq1 (either term nullable) into the
// state dphi (rows `prows`, nullable) and dS (ranks <= lout, stored).
__global__ __launch_bounds__(kWave) void ladder_first_tangent_kernel(int N, int C, int lq1, int lout, int a_rows,
                                                                     int prows, int srows,
                                                                     const float* __restrict__ vA,
                                                                     const float* __restrict__ a1,
                                                                     const float* __restrict__ A,
                                                                     const float* __restrict__ b1,
                                                                     float* __restrict__ dphi,
                                                                     float* __restrict__ dS) {
  const int u = blockIdx.x;
  const int k = blockIdx.y * kWave + threadIdx.x;
  if (k >= C) return;
  const int rows = (lq1 + 1) * (lq1 + 1);
  for (int c = 0; c < rows; ++c) {
    int l = 0;
    while ((l + 1) * (l + 1) <= c) ++l;
    float v = 0.f;
    if (vA) v = a1[(size_t)l * C + k] * vA[((size_t)u * a_rows + c) * C + k];
    if (b1) v = fmaf(b1[(size_t)l * C + k], A[((size_t)u * a_rows + c) * C + k], v);
    if (dphi) dphi[((size_t)u * prows + c) * C + k] = v;
    if (dS && l <= lout) dS[((size_t)u * srows + c) * C + k] = v;
  }
}

// Reverse of phi^1 = a1 A with tangents: A_hat += a1 G' + b1 G (nullable
// terms), part[blk][l][k] = sum_{u in tile, c} (G' A + G v_A).  Eight waves
// per block share the rows of a tile of nodes (wave w takes rows w, w + 8,
// ...), each walking the tile's nodes with independent loads; the per-rank
// sums meet in LDS in a fixed order.
constexpr int kRevWaves = 8;
__global__ __launch_bounds__(kRevWaves * kWave) void ladder_first_reverse_kernel(
    int N, int C, int ntile, int lq1, int a_rows, int grows, const float* __restrict__ G,
    const float* __restrict__ dG, const float* __restrict__ A, const float* __restrict__ vA,
    const float* __restrict__ a1, const float* __restrict__ b1, float* __restrict__ A_hat, float* __restrict__ part) {
  __shared__ float red[kRevWaves][5][kWave];
  const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int k = blockIdx.y * kWave + lane;
  const bool act = k < C;
  const int rows = (lq1 + 1) * (lq1 + 1);
  float acc[5] = {0.f, 0.f, 0.f, 0.f, 0.f};
  const int u0 = blockIdx.x * ntile, u1 = min(N, u0 + ntile);
  if (act) {
    for (int c = wv; c < rows; c += kRevWaves) {
      int l = 0;
      while ((l + 1) * (l + 1) <= c) ++l;
      const float al = a1[(size_t)l * C + k];
      const float bl = b1 ? b1[(size_t)l * C + k] : 0.f;
      float t = 0.f;
#pragma unroll 4
      for (int u = u0; u < u1; ++u) {
        const size_t gi = ((size_t)u * grows + c) * C + k, ai = ((size_t)u * a_rows + c) * C + k;
        const float g = G[gi];
        const float dg = dG ? dG[gi] : 0.f;
        if (A_hat) A_hat[ai] += fmaf(bl, g, al * dg);
        float tt = dg * A[ai];
        if (vA) tt = fmaf(g, vA[ai], tt);
        t += tt;
      }
#pragma unroll
      for (int li = 0; li < 5; ++li)
        if (li == l) acc[li] += t;
    }
  }
  if (!part) return;
#pragma unroll
  for (int li = 0; li < 5; ++li) red[wv][li][lane] = acc[li];
  __syncthreads();
  if (wv == 0 && act)
    for (int l = 0; l <= lq1; ++l) {
      float s = 0.f;
      for (int w = 0; w < kRevWaves; ++w) s += red[w][l][lane];
      part[((size_t)blockIdx.x * (lq1 + 1) + l) * C + k] = s;
    }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(size_t n, float* __restrict__ p) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// ----------------------------------------------------------------- host --

namespace {

int nr(int l) { return (l + 1) * (l + 1); }

}  // namespace

int LadderPlan::lq(int q) const {
  if (q == 1) return order == 1 ? lout : lprod;
  return q == order ? lout : lprod;
}

int LadderPlan::paths(int q, int L) const {
  int c = 0;
  for (int l1 = 0; l1 <= lq(q - 1); ++l1)
    for (int l2 = 0; l2 <= la; ++l2)
      if (admissible(l1, l2, L)) ++c;
  return c;
}

int LadderPlan::paths(int q) const {
  int c = 0;
  for (int L = 0; L <= lq(q); ++L) c += paths(q, L);
  return c;
}

// rows of the product buffer of step q: sum_L (2L+1) P_{q,L}
int LadderPlan::prod_rows(int q) const {
  int r = 0;
  for (int L = 0; L <= lq(q); ++L) r += (2 * L + 1) * paths(q, L);
  return r;
}

size_t LadderPlan::weight_floats() const {
  const size_t C2 = (size_t)C * C;
  size_t n = 0;
  if (variant == 0) {
    n += (size_t)(lq(1) + 1) * C2;
    for (int q = 2; q <= order; ++q)
      for (int L = 0; L <= lq(q); ++L) n += (size_t)paths(q, L) * C2;
  } else {
    n += (size_t)(lq(1) + 1) * C;
    for (int q = 2; q <= order; ++q) n += (size_t)paths(q) * C;
    n += (size_t)(lout + 1) * C2;
  }
  return n;
}

// the states phi^1 .. phi^(order-1) and, path-reduced, the final state S
// that the output maps read (kept so that the VJP need not recompute it)
size_t LadderPlan::saved_floats() const {
  return (size_t)(order - 1) * N * nr(lprod) * C + (variant == 1 ? (size_t)N * nr(lout) * C : 0);
}

size_t LadderPlan::state_floats() const { return (size_t)N * nr(lprod) * C; }

size_t LadderPlan::fwd_ws_floats() const {
  if (variant == 1) return (size_t)N * nr(lout) * C + gemm_small_split_floats((size_t)N * nr(lout) * C);
  size_t b = 0;
  for (int q = 2; q <= order; ++q) b = std::max(b, (size_t)N * prod_rows(q) * C);
  return b + 2 * state_floats();
}

namespace {
// Nodes per block of the path-reduced reverse kernels: a power of two from 16
// down to the waves per block, the largest for which about 512 blocks (two
// waves per SIMD) still cover the nodes and channel tiles.  A larger tile
// amortises the per-block path weights and partial sums; a smaller one keeps
// a small graph spread over the chip.
int red_ntile(int N, int C) {
  const int ct = (C + kWave - 1) / kWave;
  int t = 16;
  while (t > kRedWaves && (long long)((N + t - 1) / t) * ct < 512) t /= 2;
  return t;
}
constexpr int kMixTile = 2;         // nodes per wave in the path-weight gradient on a product buffer
constexpr int kSplitTarget = 512;   // blocks per split-K weight-gradient GEMM
}  // namespace

size_t LadderPlan::vjp_ws_floats() const {
  const size_t st = state_floats();
  const size_t C2 = (size_t)C * C;
  size_t part = 0;
  if (variant == 0) {
    size_t b = 0;
    for (int q = 2; q <= order; ++q) {
      b = std::max(b, (size_t)N * prod_rows(q) * C);
      size_t g = 0;
      for (int L = 0; L <= lq(q); ++L) {
        const int P = paths(q, L);
        if (P) g += (size_t)gemm_ksplit(C, P * C, N * (2 * L + 1), kSplitTarget) * P * C2;
      }
      part = std::max(part, g);
    }
    size_t g1 = 0;
    for (int l = 0; l <= lq(1); ++l) g1 += (size_t)gemm_ksplit(C, C, N * (2 * l + 1), kSplitTarget) * C2;
    part = std::max(part, g1);
    return 2 * b + 2 * st + part;
  }
  const int nt = red_ntile(N, C);
  const int nblk = (N + nt - 1) / nt;
  int pmax = 0;
  for (int q = 2; q <= order; ++q) pmax = std::max(pmax, paths(q));
  for (int L = 0; L <= lout; ++L) part += (size_t)gemm_ksplit(C, C, N * (2 * L + 1), kSplitTarget) * C2;
  return 2 * (size_t)N * nr(lout) * C + 2 * st + (size_t)nblk * (pmax + lprod + 1) * C + part +
         gemm_small_split_floats((size_t)N * nr(lout) * C);
}

// B, B', B_bar, B_bar' (largest step), G and G' double buffers, phi'^q for
// q < order, split-K partials of the weight gradients
size_t LadderPlan::vv_ws_floats() const {
  const size_t st = state_floats();
  const size_t C2 = (size_t)C * C;
  size_t b = 0, part = 0;
  if (variant == 1) {   // + S, S', S_bar, S_bar' and the path-weight partials
    const int nblk = (N + kMixTile - 1) / kMixTile;
    int pmax = lq(1) + 1;
    for (int q = 2; q <= order; ++q) {
      b = std::max(b, (size_t)N * prod_rows(q) * C);
      pmax = std::max(pmax, paths(q));
    }
    size_t g = 0;
    for (int L = 0; L <= lout; ++L) g += (size_t)gemm_ksplit(C, C, N * (2 * L + 1), kSplitTarget) * C2;
    part = std::max(g, (size_t)nblk * pmax * C);
    return 4 * b + 4 * st + (size_t)(order - 1) * st + 4 * (size_t)N * nr(lout) * C + part;
  }
  for (int q = 2; q <= order; ++q) {
    b = std::max(b, (size_t)N * prod_rows(q) * C);
    size_t g = 0;
    for (int L = 0; L <= lq(q); ++L) {
      const int P = paths(q, L);
      if (P) g += (size_t)gemm_ksplit(C, P * C, N * (2 * L + 1), kSplitTarget) * P * C2;
    }
    part = std::max(part, g);
  }
  size_t g1 = 0;
  for (int l = 0; l <= lq(1); ++l) g1 += (size_t)gemm_ksplit(C, C, N * (2 * l + 1), kSplitTarget) * C2;
  part = std::max(part, g1);
  return 4 * b + 4 * st + (size_t)(order - 1) * st + part;
}

// offset (floats) of W^q_L (full) in the flat weights
size_t LadderPlan::w_full(int q, int L) const {
  const size_t C2 = (size_t)C * C;
  if (q == 1) return (size_t)L * C2;
  size_t n = (size_t)(lq(1) + 1) * C2;
  for (int qq = 2; qq <= order; ++qq)
    for (int LL = 0; LL <= lq(qq); ++LL) {
      if (qq == q && LL == L) return n;
      n += (size_t)paths(qq, LL) * C2;
    }
  return n;
}

size_t LadderPlan::w_a(int q) const {
  if (q == 1) return 0;
  size_t n = (size_t)(lq(1) + 1) * C;
  for (int qq = 2; qq < q; ++qq) n += (size_t)paths(qq) * C;
  return n;
}

size_t LadderPlan::w_final(int L) const {
  size_t n = w_a(order + 1);
  return n + (size_t)L * C * C;
}

namespace {

template <int LP, int LQ>
void launch_prod(const LadderPlan& p, const float* phi, const float* A, float* B, int acc, const float* phi2,
                 const float* A2, hipStream_t st) {
  dim3 grid(p.N, (p.C + kWave - 1) / kWave);
  if (phi2)
    hipLaunchKernelGGL((ladder_prod_kernel<LP, LP, LQ, true>), grid, dim3(kWave), 0, st, p.N, p.C, phi,
                       nr(p.lprod), A, nr(p.la), B, acc, phi2, A2);
  else
    hipLaunchKernelGGL((ladder_prod_kernel<LP, LP, LQ, false>), grid, dim3(kWave), 0, st, p.N, p.C, phi,
                       nr(p.lprod), A, nr(p.la), B, acc, (const float*)nullptr, (const float*)nullptr);
}

template <int LP>
void dispatch_prod(const LadderPlan& p, int LQ, const float* phi, const float* A, float* B, int acc,
                   const float* phi2, const float* A2, hipStream_t st) {
  switch (LQ) {
    case 0: launch_prod<LP, 0>(p, phi, A, B, acc, phi2, A2, st); break;
    case 1: if constexpr (LP >= 1) launch_prod<LP, 1>(p, phi, A, B, acc, phi2, A2, st); break;
    case 2: if constexpr (LP >= 2) launch_prod<LP, 2>(p, phi, A, B, acc, phi2, A2, st); break;
    case 3: if constexpr (LP >= 3) launch_prod<LP, 3>(p, phi, A, B, acc, phi2, A2, st); break;
    case 4: if constexpr (LP >= 4) launch_prod<LP, 4>(p, phi, A, B, acc, phi2, A2, st); break;
  }
}

// B (=, or += with acc) prod(phi, A) [+ prod(phi2, A2) when phi2 is given]
void prod(const LadderPlan& p, int LQ, const float* phi, const float* A, float* B, hipStream_t st, int acc = 0,
          const float* phi2 = nullptr, const float* A2 = nullptr) {
  switch (p.lprod) {
    case 1: dispatch_prod<1>(p, LQ, phi, A, B, acc, phi2, A2, st); break;
    case 2: dispatch_prod<2>(p, LQ, phi, A, B, acc, phi2, A2, st); break;
    case 3: dispatch_prod<3>(p, LQ, phi, A, B, acc, phi2, A2, st); break;
    case 4: dispatch_prod<4>(p, LQ, phi, A, B, acc, phi2, A2, st); break;
  }
}

// The fused step (product tile formed in LDS) covers C = 64 or 128 (one
// column block per MFMA wave and an even number of channel blocks; more
// columns, or l_prod = 4, would not fit the held phi and A rows or the
// accumulators in the register budget) and 16-byte aligned phi, A and
// weights, states and z; other shapes write the product buffer and run the
// grouped GEMM.
bool step_fused_ok(const LadderPlan& p, const float* phi, const float* A, const float* w, const float* out,
                   const float* z) {
  auto al = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
  return (p.C == 64 || p.C == 128) && p.lprod <= 3 && p.la == p.lprod && al(phi) && al(A) && al(w) && al(out) &&
         al(z);
}

template <int LP, int LQ>
void launch_step(const LadderPlan& p, const StepPlan& sp, const float* phi, const float* A, const float* w,
                 float* out, float* z, hipStream_t st) {
  hipLaunchKernelGGL((ladder_step_kernel<LP, LQ>), dim3(sp.count * sp.tiles), dim3(512), 0, st, p.N, p.C, phi, A,
                     w, out, z, nr(p.lout), p.lout, sp);
}

template <int LP>
void dispatch_step(const LadderPlan& p, int LQ, const StepPlan& sp, const float* phi, const float* A,
                   const float* w, float* out, float* z, hipStream_t st) {
  switch (LQ) {
    case 0: launch_step<LP, 0>(p, sp, phi, A, w, out, z, st); break;
    case 1: if constexpr (LP >= 1) launch_step<LP, 1>(p, sp, phi, A, w, out, z, st); break;
    case 2: if constexpr (LP >= 2) launch_step<LP, 2>(p, sp, phi, A, w, out, z, st); break;
    case 3: if constexpr (LP >= 3) launch_step<LP, 3>(p, sp, phi, A, w, out, z, st); break;
  }
}

// Step q >= 2 of the full ladder: phi^q (out, when not NULL) and z += phi^q
// for the ranks <= l_out.  One item per output rank with paths; the items
// with the most MFMA work come first in the grid.
void step_fused(const LadderPlan& p, int q, const float* phi, const float* A, const float* w, float* out,
                float* z, hipStream_t st) {
  StepPlan sp{};
  sp.tiles = (p.N + kStepNodes - 1) / kStepNodes;
  std::vector<std::pair<int, StepItem>> items;   // (MFMA work, item)
  for (int L = 0; L <= p.lq(q); ++L) {
    const int P = p.paths(q, L);
    if (P > 0) items.push_back({(2 * L + 1) * P, StepItem{L, (long long)p.w_full(q, L)}});
  }
  std::stable_sort(items.begin(), items.end(), [](const auto& a, const auto& b) { return a.first > b.first; });
  sp.count = (int)items.size();
  for (int i = 0; i < sp.count; ++i) sp.item[i] = items[i].second;
  switch (p.lprod) {
    case 1: dispatch_step<1>(p, p.lq(q), sp, phi, A, w, out, z, st); break;
    case 2: dispatch_step<2>(p, p.lq(q), sp, phi, A, w, out, z, st); break;
    case 3: dispatch_step<3>(p, p.lq(q), sp, phi, A, w, out, z, st); break;
  }
}

template <int LP, int LO>
void launch_reduced(const LadderPlan& p, const float* A, const float* w, float* S, float* saved, hipStream_t st) {
  dim3 grid(p.N, (p.C + kWave - 1) / kWave);
  const float* amid = w + p.w_a(2);
  const int pmid = p.order > 2 ? p.paths(2) : 0;
  const float* alast = w + p.w_a(p.order);
  hipLaunchKernelGGL((ladder_reduced_kernel<LP, LO>), grid, dim3(kWave), 0, st, p.N, p.C, p.order, A, w, amid,
                     pmid, alast, S, saved);
}

template <int LP>
void dispatch_reduced(const LadderPlan& p, const float* A, const float* w, float* S, float* saved, hipStream_t st) {
  switch (p.lout) {
    case 0: launch_reduced<LP, 0>(p, A, w, S, saved, st); break;
    case 1: if constexpr (LP >= 1) launch_reduced<LP, 1>(p, A, w, S, saved, st); break;
    case 2: if constexpr (LP >= 2) launch_reduced<LP, 2>(p, A, w, S, saved, st); break;
    case 3: if constexpr (LP >= 3) launch_reduced<LP, 3>(p, A, w, S, saved, st); break;
    case 4: if constexpr (LP >= 4) launch_reduced<LP, 4>(p, A, w, S, saved, st); break;
  }
}

// Rank block L of a node array [N][rows][C] as a matrix: row (u, c), column k.
GView node_view(const float* base, int rows, int L, int C) {
  return GView{base + (size_t)L * L * C, 2 * L + 1, (long long)rows * C, (long long)C, 1, 1, 0, 0, 0};
}
// Its transpose: element (k, m) with m = (u, c) the reduction index.
GView node_view_t(const float* base, int rows, int L, int C) {
  return GView{base + (size_t)L * L * C, 1, 1, 0, 2 * L + 1, (long long)rows * C, (long long)C, 0, 0};
}
GOut node_out(float* base, int rows, int L, int C, int acc) {
  if (!base) return no_out();
  return GOut{base + (size_t)L * L * C, 2 * L + 1, (long long)rows * C, (long long)C, acc, 0};
}

}  // namespace

void ladder_forward(const LadderPlan& p, const float* A, const float* w, float* z, float* saved, float* ws,
                    hipStream_t st) {
  const int C = p.C;
  const int ra = nr(p.la), rp = nr(p.lprod), ro = nr(p.lout);
  if (p.variant == 1) {
    float* S = saved ? saved + (size_t)(p.order - 1) * p.state_floats() : ws;
    switch (p.lprod) {
      case 1: dispatch_reduced<1>(p, A, w, S, saved, st); break;
      case 2: dispatch_reduced<2>(p, A, w, S, saved, st); break;
      case 3: dispatch_reduced<3>(p, A, w, S, saved, st); break;
      case 4: dispatch_reduced<4>(p, A, w, S, saved, st); break;
    }
    GemmGroup g{};
    if (S != ws) {   // the final state went to the saved states: ws is free
      g.scratch = ws;
      g.scratch_floats = p.fwd_ws_floats();
    } else {
      g.scratch = ws + (size_t)p.N * ro * C;
      g.scratch_floats = gemm_small_split_floats((size_t)p.N * ro * C);
    }
    for (int L = 0; L <= p.lout; ++L) {
      GemmProblem& pr = g.prob[g.count++];
      pr.M = p.N * (2 * L + 1);
      pr.N = C;
      pr.K = C;
      pr.alpha = 1.f;
      pr.A = node_view(S, ro, L, C);
      pr.Bt = plain_view(w + p.w_final(L), C);
      pr.C = node_out(z, ro, L, C, 0);
      pr.C2 = no_out();
    }
    gemm_group(g, st);
    return;
  }
  // full ladder
  float* B = ws;
  size_t bmax = 0;
  for (int q = 2; q <= p.order; ++q) bmax = std::max(bmax, (size_t)p.N * p.prod_rows(q) * C);
  float* tmp[2] = {ws + bmax, ws + bmax + p.state_floats()};
  auto state = [&](int q) -> float* {
    if (q >= p.order) return nullptr;
    return saved ? saved + (size_t)(q - 1) * p.state_floats() : tmp[q % 2];
  };
  // step 1: phi^1_l = W1_l A_l
  {
    GemmGroup g{};
    for (int L = 0; L <= p.lq(1); ++L) {
      GemmProblem& pr = g.prob[g.count++];
      pr.M = p.N * (2 * L + 1);
      pr.N = C;
      pr.K = C;
      pr.alpha = 1.f;
      pr.A = node_view(A, ra, L, C);
      pr.Bt = plain_view(w + p.w_full(1, L), C);
      pr.C = node_out(state(1), rp, L, C, 0);
      pr.C2 = L <= p.lout ? node_out(z, ro, L, C, 0) : no_out();
    }
    gemm_group(g, st);
  }
  for (int q = 2; q <= p.order; ++q) {
    const float* phi = state(q - 1);
    if (step_fused_ok(p, phi, A, w, state(q), z)) {
      step_fused(p, q, phi, A, w, state(q), z, st);
      continue;
    }
    prod(p, p.lq(q), phi, A, B, st);
    GemmGroup g{};
    size_t boff = 0;
    for (int L = 0; L <= p.lq(q); ++L) {
      const int P = p.paths(q, L);
      if (P == 0) continue;
      GemmProblem& pr = g.prob[g.count++];
      pr.M = p.N * (2 * L + 1);
      pr.N = C;
      pr.K = P * C;
      pr.alpha = 1.f;
      pr.A = plain_view(B + boff, (long long)P * C);
      pr.Bt = plain_view(w + p.w_full(q, L), (long long)P * C);
      pr.C = node_out(state(q), rp, L, C, 0);
      pr.C2 = L <= p.lout ? node_out(z, ro, L, C, 1) : no_out();
      boff += (size_t)p.N * (2 * L + 1) * P * C;
    }
    gemm_group(g, st);
  }
}


namespace {

template <int LP, int LQ>
void launch_prod_vjp(const LadderPlan& p, const float* Bbar, const float* phi, const float* A, const float* gz,
                     float* Gprev, float* Abar, hipStream_t st, int acc_g = 0) {
  dim3 grid(p.N, (p.C + kWave - 1) / kWave);
  hipLaunchKernelGGL((ladder_prod_vjp_kernel<LP, LP, LQ>), grid, dim3(kWave), 0, st, p.N, p.C, Bbar, phi, A, gz,
                     gz ? nr(p.lout) : 0, Gprev, acc_g, Abar);
}

template <int LP, int LQ>
void launch_red_vjp(const LadderPlan& p, bool first, const float* G, int g_rows, const float* phi, const float* A,
                    const float* Sbar, const float* aw, const float* a1, float* Gprev, float* Abar, float* apart,
                    float* a1part, int acc_abar, hipStream_t st) {
  const int nt = red_ntile(p.N, p.C);
  dim3 grid((p.N + nt - 1) / nt, (p.C + kWave - 1) / kWave);
  if (first)
    hipLaunchKernelGGL((ladder_reduced_vjp_kernel<LP, LP, LQ, true>), grid, dim3(kRedWaves * kWave), 0, st, p.N, p.C, nt,
                       G, g_rows, phi, A, Sbar, nr(p.lout), aw, a1, Gprev, Abar, apart, a1part, acc_abar);
  else
    hipLaunchKernelGGL((ladder_reduced_vjp_kernel<LP, LP, LQ, false>), grid, dim3(kRedWaves * kWave), 0, st, p.N, p.C, nt,
                       G, g_rows, phi, A, Sbar, nr(p.lout), aw, a1, Gprev, Abar, apart, a1part, acc_abar);
}

// dispatch (lprod, LQ) -> F<LP, LQ>
template <template <int, int> class F, class... Args>
void by_ranks(int lp, int lq, Args&&... args) {
#define FC_LQ(LPV)                                                   \
  switch (lq) {                                                      \
    case 0: F<LPV, 0>::run(args...); break;                          \
    case 1: if constexpr (LPV >= 1) F<LPV, 1>::run(args...); break;  \
    case 2: if constexpr (LPV >= 2) F<LPV, 2>::run(args...); break;  \
    case 3: if constexpr (LPV >= 3) F<LPV, 3>::run(args...); break;  \
    case 4: if constexpr (LPV >= 4) F<LPV, 4>::run(args...); break;  \
  }
  switch (lp) {
    case 1: FC_LQ(1) break;
    case 2: FC_LQ(2) break;
    case 3: FC_LQ(3) break;
    case 4: FC_LQ(4) break;
  }
#undef FC_LQ
}

template <int LP, int LQ>
struct ProdVjp {
  template <class... A>
  static void run(A&&... a) { launch_prod_vjp<LP, LQ>(a...); }
};
template <int LP, int LQ>
struct RedVjp {
  template <class... A>
  static void run(A&&... a) { launch_red_vjp<LP, LQ>(a...); }
};
template <int LP, int LQ>
struct Mix {
  static void run(const LadderPlan& p, const float* X, const float* a, const float* Y, const float* b, float* out,
                  float* dS, int acc_s, hipStream_t st) {
    dim3 grid(p.N, (p.C + kWave - 1) / kWave);
    hipLaunchKernelGGL((ladder_mix_kernel<LP, LP, LQ>), grid, dim3(kWave), 0, st, p.N, p.C, X, a, Y, b, out,
                       nr(p.lprod), dS, nr(p.lout), p.lout, acc_s);
  }
};
template <int LP, int LQ>
struct MixVjp {
  static void run(const LadderPlan& p, const float* X, int xrows, const float* a, const float* Y, int yrows,
                  const float* b, float* Bbar, hipStream_t st) {
    dim3 grid(p.N, (p.C + kWave - 1) / kWave);
    hipLaunchKernelGGL((ladder_mix_vjp_kernel<LP, LP, LQ>), grid, dim3(kWave), 0, st, p.N, p.C, X, xrows, a, Y,
                       yrows, b, Bbar);
  }
};
template <int LP, int LQ>
struct MixWgrad {
  static void run(const LadderPlan& p, const float* X, int xrows, const float* B1, const float* Y, int yrows,
                  const float* B2, float* part, hipStream_t st) {
    dim3 grid((p.N + kMixTile - 1) / kMixTile, (p.C + kWave - 1) / kWave);
    hipLaunchKernelGGL((ladder_mix_wgrad_kernel<LP, LP, LQ>), grid, dim3(kWave), 0, st, p.N, p.C, kMixTile, X, xrows,
                       B1, Y, yrows, B2, part);
  }
};

void fill_zero(float* p, size_t n, hipStream_t st) {
  if (n) hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, n, p);
}

void block_sum(int nblk, int n, const float* part, float* out, hipStream_t st) {
  launch_block_sum(nblk, n, part, out, st);
}

// element (n, k) = W[k * ld + n]: the weight matrix used untransposed
GView weight_t(const float* W, long long ld) { return GView{W, 1, 1, 0, 1, ld, 0, 0, 0}; }

}  // namespace

void ladder_vjp(const LadderPlan& p, const float* A, const float* w, const float* saved, const float* gz,
                float* A_grad, float* w_grad, float* ws, hipStream_t st) {
  const int C = p.C;
  const int ra = nr(p.la), rp = nr(p.lprod), ro = nr(p.lout);
  const size_t stf = p.state_floats();
  // the path-reduced steps store A_grad at the first reverse step (q = order)
  // and add to it after; the other paths accumulate from zero
  if (p.variant == 0 || p.order == 1) fill_zero(A_grad, (size_t)p.N * ra * C, st);
  if (p.variant == 0) {
    size_t bmax = 0;
    for (int q = 2; q <= p.order; ++q) bmax = std::max(bmax, (size_t)p.N * p.prod_rows(q) * C);
    float* B = ws;
    float* Bbar = B + bmax;
    float* Gbuf[2] = {Bbar + bmax, Bbar + bmax + stf};
    float* part = Gbuf[1] + stf;
    const float* G = gz;
    int grows = ro;
    for (int q = p.order; q >= 2; --q) {
      const float* phi = saved + (size_t)(q - 2) * stf;
      prod(p, p.lq(q), phi, A, B, st);
      GemmGroup g{};
      size_t boff = 0, poff = 0;
      for (int L = 0; L <= p.lq(q); ++L) {
        const int P = p.paths(q, L);
        if (P == 0) continue;
        const long long PC = (long long)P * C;
        const float* W = w + p.w_full(q, L);
        GemmProblem& b = g.prob[g.count++];
        b.M = p.N * (2 * L + 1);
        b.N = (int)PC;
        b.K = C;
        b.alpha = 1.f;
        b.A = node_view(G, grows, L, C);
        b.Bt = weight_t(W, PC);
        b.C = plain_out(Bbar + boff, PC, 0);
        b.C2 = no_out();
        if (w_grad) {
          GemmProblem& d = g.prob[g.count++];
          d.M = C;
          d.N = (int)PC;
          d.K = p.N * (2 * L + 1);
          d.alpha = 1.f;
          d.A = node_view_t(G, grows, L, C);
          d.Bt = weight_t(B + boff, PC);
          d.C = plain_out(w_grad + p.w_full(q, L), PC, 0);
          d.C2 = no_out();
          d.ksplit = gemm_ksplit(d.M, d.N, d.K, kSplitTarget);
          d.part = part + poff;
          poff += (size_t)d.ksplit * d.M * d.N;
        }
        boff += (size_t)p.N * (2 * L + 1) * PC;
      }
      gemm_group(g, st);
      float* Gprev = Gbuf[q % 2];
      by_ranks<ProdVjp>(p.lprod, p.lq(q), p, (const float*)Bbar, phi, A, gz, Gprev, A_grad, st);
      G = Gprev;
      grows = rp;
    }
    GemmGroup g{};
    size_t poff = 0;
    for (int l = 0; l <= p.lq(1); ++l) {
      const float* W1 = w + p.w_full(1, l);
      GemmProblem& b = g.prob[g.count++];
      b.M = p.N * (2 * l + 1);
      b.N = C;
      b.K = C;
      b.alpha = 1.f;
      b.A = node_view(G, grows, l, C);
      b.Bt = weight_t(W1, C);
      b.C = node_out(A_grad, ra, l, C, 1);
      b.C2 = no_out();
      if (w_grad) {
        GemmProblem& d = g.prob[g.count++];
        d.M = C;
        d.N = C;
        d.K = p.N * (2 * l + 1);
        d.alpha = 1.f;
        d.A = node_view_t(G, grows, l, C);
        d.Bt = node_view_t(A, ra, l, C);
        d.C = plain_out(w_grad + p.w_full(1, l), C, 0);
        d.C2 = no_out();
        d.ksplit = gemm_ksplit(d.M, d.N, d.K, kSplitTarget);
        d.part = part + poff;
        poff += (size_t)d.ksplit * d.M * d.N;
      }
    }
    gemm_group(g, st);
    return;
  }
  // path-reduced
  float* S = ws;
  float* Sbar = S + (size_t)p.N * ro * C;
  float* Gbuf[2] = {Sbar + (size_t)p.N * ro * C, Sbar + (size_t)p.N * ro * C + stf};
  const int ntile = red_ntile(p.N, p.C);
  const int nblk = (p.N + ntile - 1) / ntile;
  int pmax = 0;
  for (int q = 2; q <= p.order; ++q) pmax = std::max(pmax, p.paths(q));
  float* apart = Gbuf[1] + stf;
  float* a1part = apart + (size_t)nblk * pmax * C;
  float* part = a1part + (size_t)nblk * (p.lprod + 1) * C;
  // the final state the output maps read: kept by the forward in the saved
  // states, else (order 1 without them) recomputed
  const float* Sf = S;
  if (saved) {
    Sf = saved + (size_t)(p.order - 1) * stf;
  } else {
    switch (p.lprod) {
      case 1: dispatch_reduced<1>(p, A, w, S, nullptr, st); break;
      case 2: dispatch_reduced<2>(p, A, w, S, nullptr, st); break;
      case 3: dispatch_reduced<3>(p, A, w, S, nullptr, st); break;
      case 4: dispatch_reduced<4>(p, A, w, S, nullptr, st); break;
    }
  }
  {
    GemmGroup g{};
    size_t poff = 0, pfl = 0;
    for (int L = 0; L <= p.lout; ++L) pfl += (size_t)gemm_ksplit(C, C, p.N * (2 * L + 1), kSplitTarget) * C * C;
    g.scratch = part + pfl;
    g.scratch_floats = gemm_small_split_floats((size_t)p.N * ro * C);
    for (int L = 0; L <= p.lout; ++L) {
      const float* WL = w + p.w_final(L);
      GemmProblem& b = g.prob[g.count++];
      b.M = p.N * (2 * L + 1);
      b.N = C;
      b.K = C;
      b.alpha = 1.f;
      b.A = node_view(gz, ro, L, C);
      b.Bt = weight_t(WL, C);
      b.C = node_out(Sbar, ro, L, C, 0);
      b.C2 = no_out();
      if (w_grad) {
        GemmProblem& d = g.prob[g.count++];
        d.M = C;
        d.N = C;
        d.K = p.N * (2 * L + 1);
        d.alpha = 1.f;
        d.A = node_view_t(gz, ro, L, C);
        d.Bt = node_view_t(Sf, ro, L, C);
        d.C = plain_out(w_grad + p.w_final(L), C, 0);
        d.C2 = no_out();
        d.ksplit = gemm_ksplit(d.M, d.N, d.K, kSplitTarget);
        d.part = part + poff;
        poff += (size_t)d.ksplit * d.M * d.N;
      }
    }
    gemm_group(g, st);
  }
  const float* a1 = w + p.w_a(1);
  if (p.order == 1) {
    dim3 grid(nblk, (C + kWave - 1) / kWave);
    hipLaunchKernelGGL(ladder_reduced_first_kernel, grid, dim3(kWave), 0, st, p.N, C, ntile, p.lout, ra,
                       (const float*)Sbar, A, a1, A_grad, a1part);
    if (w_grad) block_sum(nblk, (p.lout + 1) * C, a1part, w_grad + p.w_a(1), st);
    return;
  }
  const float* G = Sbar;
  int grows = ro;
  for (int q = p.order; q >= 2; --q) {
    const float* phi = saved + (size_t)(q - 2) * stf;
    float* Gprev = Gbuf[q % 2];
    by_ranks<RedVjp>(p.lprod, p.lq(q), p, q == 2, G, grows, phi, A, (const float*)Sbar,
                     (const float*)(w + p.w_a(q)), a1, Gprev, A_grad, apart, a1part, q != p.order, st);
    if (w_grad) {
      block_sum(nblk, p.paths(q) * C, apart, w_grad + p.w_a(q), st);
      if (q == 2) block_sum(nblk, (p.lprod + 1) * C, a1part, w_grad + p.w_a(1), st);
    }
    G = Gprev;
    grows = rp;
  }
}

namespace {

// Path-reduced ladder, VJP-of-VJP: the same forward-over-reverse scheme as
// the full ladder below, with each step run on the product buffer (B, B')
// and the channel-diagonal path weights a^q in place of the GEMM (the
// register-fused kernels of the forward and VJP have no tangent form).
void ladder_vjp_vjp_reduced(const LadderPlan& p, const float* A, const float* w, const float* saved,
                            const float* gz, const float* vA, const float* vw, float* g_hat, float* A_hat,
                            float* w_hat, float* ws, hipStream_t st) {
  const int C = p.C;
  const int ra = nr(p.la), rp = nr(p.lprod), ro = nr(p.lout);
  const size_t stf = p.state_floats(), so = (size_t)p.N * ro * C;
  size_t bmax = 0;
  for (int q = 2; q <= p.order; ++q) bmax = std::max(bmax, (size_t)p.N * p.prod_rows(q) * C);
  float* B = ws;
  float* dB = B + bmax;
  float* Bb = dB + bmax;
  float* dBb = Bb + bmax;
  float* Gb[2] = {dBb + bmax, dBb + bmax + stf};
  float* dGb[2] = {Gb[1] + stf, Gb[1] + 2 * stf};
  float* dphi = dGb[1] + stf;
  float* S = dphi + (size_t)(p.order - 1) * stf;
  float* dS = S + so;
  float* Sb = dS + so;
  float* dSb = Sb + so;
  float* part = dSb + so;
  auto phi_of = [&](int q) -> const float* { return saved + (size_t)(q - 1) * stf; };
  auto dphi_of = [&](int q) -> float* { return q < p.order ? dphi + (size_t)(q - 1) * stf : nullptr; };
  auto aw = [&](const float* base, int q) -> const float* { return base ? base + p.w_a(q) : nullptr; };
  const int ntile = red_ntile(p.N, p.C);
  const int nblk = (p.N + ntile - 1) / ntile;
  const dim3 ngrid(p.N, (C + kWave - 1) / kWave), tgrid(nblk, (C + kWave - 1) / kWave);
  const bool rev = A_hat || w_hat;
  if (A_hat) fill_zero(A_hat, (size_t)p.N * ra * C, st);
  if (w_hat) fill_zero(w_hat, p.weight_floats(), st);
  if (!vA && !vw) {
    if (g_hat) fill_zero(g_hat, so, st);
    return;
  }
  // ---- forward tangent: S' = sum_q Pi phi'^q
  hipLaunchKernelGGL(ladder_first_tangent_kernel, ngrid, dim3(kWave), 0, st, p.N, C, p.lq(1), p.lout, ra, rp, ro,
                     vA, aw(w, 1), A, aw(vw, 1), dphi_of(1), dS);
  for (int q = 2; q <= p.order; ++q) {
    const float* phi = phi_of(q - 1);
    prod(p, p.lq(q), dphi_of(q - 1), A, dB, st, 0, vA ? phi : nullptr, vA);
    if (vw) prod(p, p.lq(q), phi, A, B, st, 0);
    by_ranks<Mix>(p.lprod, p.lq(q), p, (const float*)dB, aw(w, q), vw ? (const float*)B : nullptr, aw(vw, q),
                  dphi_of(q), dS, 1, st);
  }
  if (vw) {   // S, for the cotangent of the final maps
    switch (p.lprod) {
      case 1: dispatch_reduced<1>(p, A, w, S, nullptr, st); break;
      case 2: dispatch_reduced<2>(p, A, w, S, nullptr, st); break;
      case 3: dispatch_reduced<3>(p, A, w, S, nullptr, st); break;
      case 4: dispatch_reduced<4>(p, A, w, S, nullptr, st); break;
    }
  }
  // g_hat = W_L S'_L + V_L S_L
  for (int pass = 0; g_hat && pass < 2; ++pass) {
    if (pass == 1 && !vw) continue;
    GemmGroup g{};
    for (int L = 0; L <= p.lout; ++L) {
      GemmProblem& pr = g.prob[g.count++];
      pr.M = p.N * (2 * L + 1);
      pr.N = C;
      pr.K = C;
      pr.alpha = 1.f;
      pr.A = node_view(pass == 0 ? dS : S, ro, L, C);
      pr.Bt = plain_view((pass == 0 ? w : vw) + p.w_final(L), C);
      pr.C = node_out(g_hat, ro, L, C, pass);
      pr.C2 = no_out();
    }
    gemm_group(g, st);
  }
  if (!rev) return;
  // ---- reverse: S_bar = g W_L, S_bar' = g V_L;  w_hat(W_L) += g^T S'
  {
    GemmGroup g{};
    for (int L = 0; L <= p.lout; ++L)
      for (int t = 0; t < 2; ++t) {
        if (t == 1 && !vw) continue;
        GemmProblem& b = g.prob[g.count++];
        b.M = p.N * (2 * L + 1);
        b.N = C;
        b.K = C;
        b.alpha = 1.f;
        b.A = node_view(gz, ro, L, C);
        b.Bt = weight_t((t == 0 ? w : vw) + p.w_final(L), C);
        b.C = node_out(t == 0 ? Sb : dSb, ro, L, C, 0);
        b.C2 = no_out();
      }
    gemm_group(g, st);
  }
  if (w_hat) {
    GemmGroup g{};
    size_t poff = 0;
    for (int L = 0; L <= p.lout; ++L) {
      GemmProblem& d = g.prob[g.count++];
      d.M = C;
      d.N = C;
      d.K = p.N * (2 * L + 1);
      d.alpha = 1.f;
      d.A = node_view_t(gz, ro, L, C);
      d.Bt = node_view_t(dS, ro, L, C);
      d.C = plain_out(w_hat + p.w_final(L), C, 1);
      d.C2 = no_out();
      d.ksplit = gemm_ksplit(d.M, d.N, d.K, kSplitTarget);
      d.part = part + poff;
      poff += (size_t)d.ksplit * d.M * d.N;
    }
    gemm_group(g, st);
  }
  const float* G = Sb;
  const float* dG = vw ? dSb : nullptr;
  const float* dSbar = vw ? dSb : nullptr;
  int grows = ro;
  for (int q = p.order; q >= 2; --q) {
    const float* phi = phi_of(q - 1);
    const float* dph = dphi_of(q - 1);
    const float* aq = aw(w, q);
    const float* vaq = aw(vw, q);
    prod(p, p.lq(q), phi, A, B, st, 0);
    prod(p, p.lq(q), dph, A, dB, st, 0, vA ? phi : nullptr, vA);
    by_ranks<MixVjp>(p.lprod, p.lq(q), p, G, grows, aq, (const float*)nullptr, 0, (const float*)nullptr, Bb, st);
    const bool have_dBb = dG || vaq;
    if (have_dBb)
      by_ranks<MixVjp>(p.lprod, p.lq(q), p, dG, grows, aq, vaq ? G : nullptr, grows, vaq, dBb, st);
    if (w_hat) {
      by_ranks<MixWgrad>(p.lprod, p.lq(q), p, dG, grows, (const float*)B, G, grows, (const float*)dB, part, st);
      block_sum((p.N + kMixTile - 1) / kMixTile, p.paths(q) * C, part, w_hat + p.w_a(q), st);
    }
    float* Gn = Gb[q % 2];
    float* dGn = dGb[q % 2];
    by_ranks<ProdVjp>(p.lprod, p.lq(q), p, (const float*)Bb, phi, A, (const float*)Sb, Gn, (float*)nullptr, st, 0);
    if (have_dBb)
      by_ranks<ProdVjp>(p.lprod, p.lq(q), p, (const float*)dBb, phi, A, dSbar, dGn, A_hat, st, 0);
    by_ranks<ProdVjp>(p.lprod, p.lq(q), p, (const float*)Bb, dph, vA, have_dBb ? nullptr : dSbar, dGn, A_hat, st,
                      have_dBb ? 1 : 0);
    G = Gn;
    dG = dGn;
    grows = rp;
  }
  hipLaunchKernelGGL(ladder_first_reverse_kernel, tgrid, dim3(kRevWaves * kWave), 0, st, p.N, C, ntile, p.lq(1), ra, grows, G,
                     dG, A, vA, aw(w, 1), aw(vw, 1), A_hat, w_hat ? part : nullptr);
  if (w_hat) block_sum(nblk, (p.lq(1) + 1) * C, part, w_hat + p.w_a(1), st);
}

}  // namespace

// Full ladder, VJP-of-VJP by forward-over-reverse: every map of the ladder is
// linear in each operand, so the tangent of a product step is two product
// launches (prod(phi', A) + prod(phi, v_A)), the tangent of a GEMM two GEMMs
// (X' W + X V), and the tangent of a reverse product step two reverse
// launches (G' from VJP1(B_bar', A) + VJP1(B_bar, v_A), A_hat from
// VJP2(B_bar', phi) + VJP2(B_bar, phi')).  The forward tangent gives
// g_hat = z' and phi'^q; the reverse sweep recomputes G^q = dL/dphi^q beside
// its tangent G'^q, and A_hat and w_hat collect the tangents of A_bar and
// w_bar (zero-filled, then accumulated: the GEMM groups that add to the same
// output run one after another).
void ladder_vjp_vjp(const LadderPlan& p, const float* A, const float* w, const float* saved, const float* gz,
                    const float* vA, const float* vw, float* g_hat, float* A_hat, float* w_hat, float* ws,
                    hipStream_t st) {
  if (p.variant == 1) {
    ladder_vjp_vjp_reduced(p, A, w, saved, gz, vA, vw, g_hat, A_hat, w_hat, ws, st);
    return;
  }
  const int C = p.C;
  const int ra = nr(p.la), rp = nr(p.lprod), ro = nr(p.lout);
  const size_t stf = p.state_floats();
  size_t bmax = 0;
  for (int q = 2; q <= p.order; ++q) bmax = std::max(bmax, (size_t)p.N * p.prod_rows(q) * C);
  float* B = ws;
  float* dB = B + bmax;
  float* Bb = dB + bmax;
  float* dBb = Bb + bmax;
  float* Gb[2] = {dBb + bmax, dBb + bmax + stf};
  float* dGb[2] = {Gb[1] + stf, Gb[1] + 2 * stf};
  float* dphi = dGb[1] + stf;
  float* part = dphi + (size_t)(p.order - 1) * stf;
  auto phi_of = [&](int q) -> const float* { return saved + (size_t)(q - 1) * stf; };
  auto dphi_of = [&](int q) -> float* { return q < p.order ? dphi + (size_t)(q - 1) * stf : nullptr; };
  const bool rev = A_hat || w_hat;
  if (A_hat) fill_zero(A_hat, (size_t)p.N * ra * C, st);
  if (w_hat) fill_zero(w_hat, p.weight_floats(), st);
  if (!vA && !vw) {   // zero cotangents
    if (g_hat) fill_zero(g_hat, (size_t)p.N * ro * C, st);
    return;
  }

  // ---- forward tangent: phi'^1 = W1 v_A + V1 A, phi'^q = W^q B' + V^q B
  {
    for (int pass = 0; pass < 2; ++pass) {
      const float* X = pass == 0 ? vA : A;
      const float* Wt = pass == 0 ? w : vw;
      if (!X || !Wt) continue;
      const int acc = (pass == 1 && vA) ? 1 : 0;
      GemmGroup g{};
      for (int L = 0; L <= p.lq(1); ++L) {
        GemmProblem& pr = g.prob[g.count++];
        pr.M = p.N * (2 * L + 1);
        pr.N = C;
        pr.K = C;
        pr.alpha = 1.f;
        pr.A = node_view(X, ra, L, C);
        pr.Bt = plain_view(Wt + p.w_full(1, L), C);
        pr.C = node_out(dphi_of(1), rp, L, C, acc);
        pr.C2 = L <= p.lout ? node_out(g_hat, ro, L, C, acc) : no_out();
      }
      gemm_group(g, st);
    }
  }
  for (int q = 2; q <= p.order; ++q) {
    float* out = dphi_of(q);
    if (!out && !g_hat) break;
    const float* phi = phi_of(q - 1);
    prod(p, p.lq(q), dphi_of(q - 1), A, dB, st, 0, vA ? phi : nullptr, vA);
    if (vw) prod(p, p.lq(q), phi, A, B, st, 0);
    for (int pass = 0; pass < 2; ++pass) {
      if (pass == 1 && !vw) continue;
      const float* X = pass == 0 ? dB : B;
      const float* Wt = pass == 0 ? w : vw;
      GemmGroup g{};
      size_t boff = 0;
      for (int L = 0; L <= p.lq(q); ++L) {
        const int P = p.paths(q, L);
        if (P == 0) continue;
        GemmProblem& pr = g.prob[g.count++];
        pr.M = p.N * (2 * L + 1);
        pr.N = C;
        pr.K = P * C;
        pr.alpha = 1.f;
        pr.A = plain_view(X + boff, (long long)P * C);
        pr.Bt = plain_view(Wt + p.w_full(q, L), (long long)P * C);
        pr.C = node_out(out, rp, L, C, pass);
        pr.C2 = L <= p.lout ? node_out(g_hat, ro, L, C, 1) : no_out();
        boff += (size_t)p.N * (2 * L + 1) * P * C;
      }
      gemm_group(g, st);
    }
  }
  if (!rev) return;

  // ---- reverse sweep with tangents
  const float* G = gz;
  const float* dG = nullptr;
  int grows = ro;
  for (int q = p.order; q >= 2; --q) {
    const float* phi = phi_of(q - 1);
    const float* dph = dphi_of(q - 1);
    prod(p, p.lq(q), phi, A, B, st, 0);
    prod(p, p.lq(q), dph, A, dB, st, 0, vA ? phi : nullptr, vA);
    const bool have_dBb = dG || vw;
    // B_bar = G W, B_bar' = G' W (+ G V below)
    {
      GemmGroup g{};
      size_t boff = 0;
      for (int L = 0; L <= p.lq(q); ++L) {
        const int P = p.paths(q, L);
        if (P == 0) continue;
        const long long PC = (long long)P * C;
        for (int t = 0; t < 2; ++t) {
          const float* X = t == 0 ? G : dG;
          if (!X) continue;
          GemmProblem& b = g.prob[g.count++];
          b.M = p.N * (2 * L + 1);
          b.N = (int)PC;
          b.K = C;
          b.alpha = 1.f;
          b.A = node_view(X, grows, L, C);
          b.Bt = weight_t(w + p.w_full(q, L), PC);
          b.C = plain_out((t == 0 ? Bb : dBb) + boff, PC, 0);
          b.C2 = no_out();
        }
        boff += (size_t)p.N * (2 * L + 1) * PC;
      }
      gemm_group(g, st);
    }
    // B_bar' += G V;  w_hat^q += G^T B'  (then += G'^T B)
    for (int pass = 0; pass < 2; ++pass) {
      GemmGroup g{};
      size_t boff = 0, poff = 0;
      for (int L = 0; L <= p.lq(q); ++L) {
        const int P = p.paths(q, L);
        if (P == 0) continue;
        const long long PC = (long long)P * C;
        if (pass == 0 && vw) {
          GemmProblem& b = g.prob[g.count++];
          b.M = p.N * (2 * L + 1);
          b.N = (int)PC;
          b.K = C;
          b.alpha = 1.f;
          b.A = node_view(G, grows, L, C);
          b.Bt = weight_t(vw + p.w_full(q, L), PC);
          b.C = plain_out(dBb + boff, PC, dG ? 1 : 0);
          b.C2 = no_out();
        }
        const float* Gx = pass == 0 ? G : dG;
        const float* Bx = pass == 0 ? dB : B;
        if (w_hat && Gx) {
          GemmProblem& d = g.prob[g.count++];
          d.M = C;
          d.N = (int)PC;
          d.K = p.N * (2 * L + 1);
          d.alpha = 1.f;
          d.A = node_view_t(Gx, grows, L, C);
          d.Bt = weight_t(Bx + boff, PC);
          d.C = plain_out(w_hat + p.w_full(q, L), PC, 1);
          d.C2 = no_out();
          d.ksplit = gemm_ksplit(d.M, d.N, d.K, kSplitTarget);
          d.part = part + poff;
          poff += (size_t)d.ksplit * d.M * d.N;
        }
        boff += (size_t)p.N * (2 * L + 1) * PC;
      }
      if (g.count) gemm_group(g, st);
    }
    float* Gn = Gb[q % 2];
    float* dGn = dGb[q % 2];
    by_ranks<ProdVjp>(p.lprod, p.lq(q), p, (const float*)Bb, phi, A, gz, Gn, (float*)nullptr, st, 0);
    if (have_dBb)
      by_ranks<ProdVjp>(p.lprod, p.lq(q), p, (const float*)dBb, phi, A, (const float*)nullptr, dGn, A_hat, st, 0);
    by_ranks<ProdVjp>(p.lprod, p.lq(q), p, (const float*)Bb, dph, vA, (const float*)nullptr, dGn, A_hat, st,
                      have_dBb ? 1 : 0);
    G = Gn;
    dG = dGn;
    grows = rp;
  }
  // step 1: A_hat += G' W1 + G V1;  w_hat^1 += G^T v_A + G'^T A
  for (int pass = 0; pass < 2; ++pass) {
    GemmGroup g{};
    size_t poff = 0;
    for (int l = 0; l <= p.lq(1); ++l) {
      const float* Gx = pass == 0 ? dG : G;
      const float* Wt = pass == 0 ? w : vw;
      if (A_hat && Gx && Wt) {
        GemmProblem& b = g.prob[g.count++];
        b.M = p.N * (2 * l + 1);
        b.N = C;
        b.K = C;
        b.alpha = 1.f;
        b.A = node_view(Gx, grows, l, C);
        b.Bt = weight_t(Wt + p.w_full(1, l), C);
        b.C = node_out(A_hat, ra, l, C, 1);
        b.C2 = no_out();
      }
      const float* Gy = pass == 0 ? G : dG;
      const float* Xy = pass == 0 ? vA : A;
      if (w_hat && Gy && Xy) {
        GemmProblem& d = g.prob[g.count++];
        d.M = C;
        d.N = C;
        d.K = p.N * (2 * l + 1);
        d.alpha = 1.f;
        d.A = node_view_t(Gy, grows, l, C);
        d.Bt = node_view_t(Xy, ra, l, C);
        d.C = plain_out(w_hat + p.w_full(1, l), C, 1);
        d.C2 = no_out();
        d.ksplit = gemm_ksplit(d.M, d.N, d.K, kSplitTarget);
        d.part = part + poff;
        poff += (size_t)d.ksplit * d.M * d.N;
      }
    }
    if (g.count) gemm_group(g, st);
  }
}

}  // namespace fc
