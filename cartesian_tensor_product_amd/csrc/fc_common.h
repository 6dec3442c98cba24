// Shared device helpers for the FlashCart gfx950 kernels.
//
// * compile-time path configuration of a convolution (path list, output rows);
// * direction tensors T_l(n) and their n-gradients from the generated
//   monomial tables (FlashCart paper, App. B direction-tensor formula);
// * the Bessel radial basis with cosine cutoff and its r-derivatives;
// * static_for, so that every register-array index is a compile-time constant.
#pragma once

#include <hip/hip_runtime.h>

#include <array>
#include <cstdint>
#include <type_traits>
#include <utility>

#include "generated/fc_tables.h"

namespace fc {

inline constexpr int kWave = 64;
inline constexpr int kNB = 8;          // radial basis functions
inline constexpr float kPi = 3.14159265358979323846f;

// ---------------------------------------------------------------- static_for
template <class F, int... Is>
__host__ __device__ __forceinline__ constexpr void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, class F>
__host__ __device__ __forceinline__ constexpr void static_for(F&& f) {
  if constexpr (N > 0) static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------ rank bookkeeping
__host__ __device__ constexpr int ncomp(int l) { return 2 * l + 1; }
__host__ __device__ constexpr int nrank(int l) { return (l + 1) * (l + 1); }   // sum_{l'<=l} (2l'+1)
__host__ __device__ constexpr int rank_off(int l) { return l * l; }         // sum_{l'<l} (2l'+1)
__host__ __device__ constexpr bool admissible(int l1, int l2, int L) {
  int d = l1 > l2 ? l1 - l2 : l2 - l1;
  return d <= L && L <= l1 + l2 && ((l1 + l2 + L) % 2 == 0);
}
// every triangle-allowed path, odd J included (the Levi-Civita extension)
__host__ __device__ constexpr bool triangle(int l1, int l2, int L) {
  int d = l1 > l2 ? l1 - l2 : l2 - l1;
  return d <= L && L <= l1 + l2;
}
// Output-rank key of a configuration: l_out, plus kAllParities to keep every
// triangle-allowed path, plus kSumPaths to sum the outputs of the paths of
// each output rank into one block.
inline constexpr int kAllParities = 8;
inline constexpr int kSumPaths = 16;
__host__ __device__ constexpr int path_type(int l1, int l2, int L) {
  for (int t = 0; t < tab::kNumPathTypes; ++t)
    if (tab::kPathL1[t] == l1 && tab::kPathL2[t] == l2 && tab::kPathL[t] == L) return t;
  return -1;
}

struct PathInfo {
  int type, l1, l2, L;
  int eta;   // position among the paths with the same L
  int PL;    // number of paths with this L
  int off;   // first row of the L block
};

// Paths (l1 <= LIN, l2 <= LEDGE, L <= LOUT), ordered by L then (l1, l2);
// natural parity, or every triangle-allowed path with kAllParities in the
// output-rank key.  Output rows: path-separated (component c of path eta of
// rank L at off(L) + c P_L + eta), or with kSumPaths one block of 2L+1 rows
// per output rank that has a path, into which all its paths add.
template <int LIN, int LEDGE, int LOUT_KEY>
struct ConvCfg {
  static constexpr int LOUT = LOUT_KEY % kAllParities;
  static constexpr bool ALL_PARITIES = (LOUT_KEY / kAllParities) % 2 == 1;
  static constexpr bool SUM = LOUT_KEY >= kSumPaths;
  static constexpr int NIN = nrank(LIN);
  static constexpr int NE = nrank(LEDGE);
  static constexpr bool path_ok(int l1, int l2, int L) {
    return ALL_PARITIES ? triangle(l1, l2, L) : admissible(l1, l2, L);
  }

  static constexpr int count_L(int L) {
    int c = 0;
    for (int l1 = 0; l1 <= LIN; ++l1)
      for (int l2 = 0; l2 <= LEDGE; ++l2)
        if (path_ok(l1, l2, L)) ++c;
    return c;
  }
  static constexpr int count_all() {
    int c = 0;
    for (int L = 0; L <= LOUT; ++L) c += count_L(L);
    return c;
  }
  static constexpr int P = count_all();
  static constexpr int off_L(int L) {
    int o = 0;
    for (int l = 0; l < L; ++l) o += SUM ? (count_L(l) > 0 ? ncomp(l) : 0) : ncomp(l) * count_L(l);
    return o;
  }
  static constexpr int NOUT = off_L(LOUT + 1);

  static constexpr std::array<PathInfo, (P > 0 ? P : 1)> build() {
    std::array<PathInfo, (P > 0 ? P : 1)> a{};
    int i = 0;
    for (int L = 0; L <= LOUT; ++L) {
      int eta = 0;
      for (int l1 = 0; l1 <= LIN; ++l1)
        for (int l2 = 0; l2 <= LEDGE; ++l2)
          if (path_ok(l1, l2, L)) {
            a[i] = PathInfo{path_type(l1, l2, L), l1, l2, L, eta, count_L(L), off_L(L)};
            ++eta;
            ++i;
          }
    }
    return a;
  }
  static constexpr std::array<PathInfo, (P > 0 ? P : 1)> paths = build();

  static constexpr int row(int p, int c) {
    return SUM ? paths[p].off + c : paths[p].off + c * paths[p].PL + paths[p].eta;
  }
  static constexpr int first_path_of(int L) {
    int i = 0;
    for (int l = 0; l < L; ++l) i += count_L(l);
    return i;
  }
};

// A path group: the contiguous paths [P0, P1) of a configuration, handled by
// one kernel launch (forward) or one sweep over the edges (VJP).  The rows of
// the group's paths are held path-major in registers: component c of path p
// sits at loff(p) + c; its row in the node-feature layout is Cfg::row(p, c).
// With summed outputs the paths of one rank share their registers (loff is
// that of the group's first path of the rank, the owner), and a group whose
// first rank began in an earlier group adds to that group's output (carry).
template <class Cfg, int P0, int P1>
struct PathGroup {
  static constexpr int p0 = P0, p1 = P1, NP = P1 - P0;
  // first path of the group with this path's output rank
  static constexpr bool owner(int p) { return !Cfg::SUM || p == P0 || Cfg::paths[p - 1].L != Cfg::paths[p].L; }
  static constexpr int loff(int p) {
    int o = 0;
    for (int q = P0; q < p; ++q)
      if (owner(q) && !(Cfg::SUM && Cfg::paths[q].L == Cfg::paths[p].L)) o += ncomp(Cfg::paths[q].L);
    return o;
  }
  static constexpr int nregs() {
    int o = 0;
    for (int q = P0; q < P1; ++q)
      if (owner(q)) o += ncomp(Cfg::paths[q].L);
    return o;
  }
  static constexpr int NR = nregs();
  // the rank block of path p was begun by an earlier group (summed outputs)
  static constexpr bool carry(int p) { return Cfg::SUM && P0 > 0 && Cfg::paths[P0 - 1].L == Cfg::paths[p].L; }
  // whether some path of the group has edge rank l2
  static constexpr bool uses_l2(int l2) {
    for (int q = P0; q < P1; ++q)
      if (Cfg::paths[q].l2 == l2) return true;
    return false;
  }
  // whether stored direction component g (= l2^2 + c) enters the group
  static constexpr bool uses_comp(int g) {
    int l = 0;
    while ((l + 1) * (l + 1) <= g) ++l;
    return uses_l2(l);
  }
  // bit g set for every direction component that enters the group
  static constexpr uint64_t comp_mask() {
    uint64_t m = 0;
    for (int g = 0; g < Cfg::NE; ++g)
      if (uses_comp(g)) m |= uint64_t(1) << g;
    return m;
  }
};

// Split of the paths into groups whose register cost stays within BUDGET:
// every path costs its 2L+1 output rows (with summed outputs only the first
// path of each rank in the group) plus its kNB radial weights.  Greedy in
// path order; a group holds at least one path.
template <class Cfg, int BUDGET>
struct PathGroups {
  static constexpr int cost(int p, bool shares) { return (shares ? 0 : ncomp(Cfg::paths[p].L)) + kNB; }
  static constexpr std::array<int, Cfg::P + 1> build() {
    std::array<int, Cfg::P + 1> s{};
    int n = 0, used = 0;
    s[0] = 0;
    for (int p = 0; p < Cfg::P; ++p) {
      const bool shares = Cfg::SUM && p > s[n] && Cfg::paths[p - 1].L == Cfg::paths[p].L;
      if (p > s[n] && used + cost(p, shares) > BUDGET) {
        s[++n] = p;
        used = 0;
        used += cost(p, false);
        continue;
      }
      used += cost(p, shares);
    }
    s[++n] = Cfg::P;
    return s;
  }
  static constexpr std::array<int, Cfg::P + 1> start = build();
  static constexpr int count() {
    int n = 0;
    while (start[n] != Cfg::P) ++n;
    return n;
  }
  static constexpr int n = count();
  template <int I>
  using group = PathGroup<Cfg, start[I], start[I + 1]>;
};

// ----------------------------------------------------------- direction tensors
// y[g], g = l^2 + c, for all ranks l <= LE; n is a unit vector.
template <int LE>
__device__ __forceinline__ void direction_tensors(float nx, float ny, float nz, float* y) {
  float px[LE + 1], py[LE + 1], pz[LE + 1];
  px[0] = py[0] = pz[0] = 1.f;
  static_for<LE>([&](auto i) {
    px[i + 1] = px[i] * nx;
    py[i + 1] = py[i] * ny;
    pz[i + 1] = pz[i] * nz;
  });
  static_for<nrank(LE)>([&](auto gi) {
    constexpr int g = gi;
    constexpr int mb = tab::kMonoBegin[g], me = tab::kMonoBegin[g + 1];
    float v = 0.f;
    static_for<me - mb>([&](auto mi) {
      constexpr tab::Mono m = tab::kMono[mb + mi];
      v = fmaf(m.c, px[m.ex] * py[m.ey] * pz[m.ez], v);
    });
    y[g] = v;
  });
}

// d y[g] / d n_j as polynomials (n treated as free variables).
template <int LE>
__device__ __forceinline__ void direction_tensor_grads(float nx, float ny, float nz, float* dy /*[NE][3]*/) {
  float px[LE + 1], py[LE + 1], pz[LE + 1];
  px[0] = py[0] = pz[0] = 1.f;
  static_for<LE>([&](auto i) {
    px[i + 1] = px[i] * nx;
    py[i + 1] = py[i] * ny;
    pz[i + 1] = pz[i] * nz;
  });
  static_for<nrank(LE)>([&](auto gi) {
    constexpr int g = gi;
    constexpr int mb = tab::kMonoBegin[g], me = tab::kMonoBegin[g + 1];
    float gx = 0.f, gy = 0.f, gz = 0.f;
    static_for<me - mb>([&](auto mi) {
      constexpr tab::Mono m = tab::kMono[mb + mi];
      if constexpr (m.ex > 0) gx = fmaf(m.c * float(m.ex), px[m.ex - 1] * py[m.ey] * pz[m.ez], gx);
      if constexpr (m.ey > 0) gy = fmaf(m.c * float(m.ey), px[m.ex] * py[m.ey - 1] * pz[m.ez], gy);
      if constexpr (m.ez > 0) gz = fmaf(m.c * float(m.ez), px[m.ex] * py[m.ey] * pz[m.ez - 1], gz);
    });
    dy[3 * g + 0] = gx;
    dy[3 * g + 1] = gy;
    dy[3 * g + 2] = gz;
  });
}

// ------------------------------------------------------------------- radial
// R_b(r) = sin(b pi r/rc)/r * (1 + cos(pi r/rc))/2, b = 1..8, 0 for r >= rc
// (and for r == 0, where no direction exists).  sin(b t) and cos(b t) follow
// from sin t, cos t by the angle-addition recurrences.
struct Radial {
  float R[kNB];
  float dR[kNB];   // dR_b/dr (only when requested)
};

template <bool DERIV>
__device__ __forceinline__ void radial(float r, float rc, float* R, float* dR) {
  if (!(r < rc) || !(r > 0.f)) {
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      R[b] = 0.f;
      if constexpr (DERIV) dR[b] = 0.f;
    }
    return;
  }
  const float th = kPi * r / rc;
  float s1, c1;
  sincosf(th, &s1, &c1);
  const float inv_r = 1.f / r;
  const float env = 0.5f * (1.f + c1);
  const float denv = -0.5f * s1 * (kPi / rc);
  float sp = 0.f, s = s1;      // sin((b-1)t), sin(b t)
  float cp = 1.f, c = c1;      // cos((b-1)t), cos(b t)
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    R[b] = s * inv_r * env;
    if constexpr (DERIV) {
      const float kb = float(b + 1) * (kPi / rc);
      dR[b] = (kb * c * inv_r - s * inv_r * inv_r) * env + s * inv_r * denv;
    }
    const float sn = 2.f * c1 * s - sp;
    const float cn = 2.f * c1 * c - cp;
    sp = s;
    s = sn;
    cp = c;
    c = cn;
  }
}

// R_b, R'_b and R''_b (second derivatives for the VJP-of-VJP).
__device__ __forceinline__ void radial2(float r, float rc, float* R, float* dR, float* d2R) {
  if (!(r < rc) || !(r > 0.f)) {
#pragma unroll
    for (int b = 0; b < kNB; ++b) R[b] = dR[b] = d2R[b] = 0.f;
    return;
  }
  const float a = kPi / rc;
  float s1, c1;
  sincosf(a * r, &s1, &c1);
  const float ir = 1.f / r;
  const float e = 0.5f * (1.f + c1), de = -0.5f * a * s1, d2e = -0.5f * a * a * c1;
  float sp = 0.f, s = s1, cp = 1.f, c = c1;
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const float k = float(b + 1) * a;
    const float h = s * ir;
    const float dh = (k * c - h) * ir;                               // (k cos)/r - s/r^2
    const float d2h = (-k * k * s - 2.f * dh) * ir;                  // -k^2 s/r - 2k cos/r^2 + 2 s/r^3
    R[b] = h * e;
    dR[b] = dh * e + h * de;
    d2R[b] = d2h * e + 2.f * dh * de + h * d2e;
    const float sn = 2.f * c1 * s - sp, cn = 2.f * c1 * c - cp;
    sp = s;
    s = sn;
    cp = c;
    c = cn;
  }
}

// Gradient g = dG/dn and Hessian H (xx, yy, zz, xy, xz, yz) of the
// polynomial G(n) = sum_c coef[c] y_c(n) over all ranks <= LE; components
// whose bit is clear in MASK are taken as zero.
template <int LE, uint64_t MASK = ~uint64_t(0)>
__device__ __forceinline__ void direction_contract_d2(const float* coef, float nx, float ny, float nz, float* g,
                                                      float* H) {
  float px[LE + 1], py[LE + 1], pz[LE + 1];
  px[0] = py[0] = pz[0] = 1.f;
  static_for<LE>([&](auto i) {
    px[i + 1] = px[i] * nx;
    py[i + 1] = py[i] * ny;
    pz[i + 1] = pz[i] * nz;
  });
  auto P = [&](int a, int b, int c) -> float { return (a < 0 || b < 0 || c < 0) ? 0.f : px[a] * py[b] * pz[c]; };
  g[0] = g[1] = g[2] = 0.f;
  for (int i = 0; i < 6; ++i) H[i] = 0.f;
  static_for<nrank(LE)>([&](auto gi) {
    constexpr int gg = gi;
    constexpr int mb = tab::kMonoBegin[gg], me = tab::kMonoBegin[gg + 1];
    if constexpr (((MASK >> gg) & 1) == 0) return;
    const float cf = coef[gg];
    static_for<me - mb>([&](auto mi) {
      constexpr tab::Mono m = tab::kMono[mb + mi];
      constexpr int a = m.ex, b = m.ey, c = m.ez;
      const float w = cf * m.c;
      if constexpr (a > 0) g[0] = fmaf(w * a, P(a - 1, b, c), g[0]);
      if constexpr (b > 0) g[1] = fmaf(w * b, P(a, b - 1, c), g[1]);
      if constexpr (c > 0) g[2] = fmaf(w * c, P(a, b, c - 1), g[2]);
      if constexpr (a > 1) H[0] = fmaf(w * (a * (a - 1)), P(a - 2, b, c), H[0]);
      if constexpr (b > 1) H[1] = fmaf(w * (b * (b - 1)), P(a, b - 2, c), H[1]);
      if constexpr (c > 1) H[2] = fmaf(w * (c * (c - 1)), P(a, b, c - 2), H[2]);
      if constexpr (a > 0 && b > 0) H[3] = fmaf(w * (a * b), P(a - 1, b - 1, c), H[3]);
      if constexpr (a > 0 && c > 0) H[4] = fmaf(w * (a * c), P(a - 1, b, c - 1), H[4]);
      if constexpr (b > 0 && c > 0) H[5] = fmaf(w * (b * c), P(a, b - 1, c - 1), H[5]);
    });
  });
}

// ------------------------------------------------------------- misc device
__device__ __forceinline__ int uniform_int(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Raw buffer access: a row gather becomes one buffer_load with the row
// offset in an SGPR (soffset) and the lane's channel offset in a VGPR
// (voffset), so no per-load 64-bit address arithmetic runs on the VALU.
// Out-of-range offsets read 0.  dword3 0x00020000 is the gfx9-family
// (CDNA) raw-buffer format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// Descriptor of one node's rows ([row_floats] floats) of a node array.  The
// base is formed in 64 bits from a wave-uniform node index, so node arrays
// may exceed the 2 GiB reach of a 32-bit buffer offset; row offsets inside
// the node (at most n_rows * C * 4 bytes) stay small.  Loads past the node's
// rows (lanes beyond the last channel of the last row) return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t node_rsrc(const float* base, int u, int row_floats) {
  return make_rsrc(base + (size_t)u * (size_t)row_floats, (uint32_t)row_floats * 4u);
}
__device__ __forceinline__ float buf_load(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

}  // namespace fc
