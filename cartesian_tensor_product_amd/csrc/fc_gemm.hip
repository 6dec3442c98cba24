// Grouped FP32 GEMM on the gfx950 matrix cores.
//
// Block tile 128 (M) x 128 (N) x 32 (K), four waves in a 2 x 2 grid; each
// wave owns a 64 x 64 sub-tile held as 2 x 2 accumulators of
// v_mfma_f32_32x32x2f32.  Problems with N <= 64 take a narrow layout
// instead: four waves stacked along M, each 32 x 64 (1 x 2 accumulators),
// so that no wave computes columns past N.  Operand layout of that instruction: lane l
// supplies A[l % 32][l / 32] and B[l / 32][l % 32]; the sixteen accumulator
// registers r of lane l hold D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
//
// Reduction order inside a K tile: at MFMA step s (0..15) the lanes of half
// h = l / 32 supply reduction index k = 16 h + s for both operands, so a
// lane's sixteen A (or B) values of the tile are contiguous in a k-major
// LDS row and come in four 128-bit LDS reads.
//
// Staging: K tiles go through registers into two LDS buffers; a tile is
// loaded two steps ahead of its use and stored one step ahead, so global
// loads stay in flight while the matrix cores work on the current tile and
// one barrier per K tile suffices.  Each operand is staged in one of three ways, chosen per problem
// on the host from its strides:
//   kK  k contiguous:    128-bit loads along k, LDS rows [row][BK + 4];
//   kR  rows contiguous: 128-bit loads along rows, LDS [k][rows + 4];
//   kG  anything else:   scalar loads into the kK layout.
// The paddings make the 128-bit LDS writes and the operand reads
// conflict-free.
#include "fc_gemm.h"

namespace fc {

namespace {

constexpr int BM = 128, BN = 128, BK = 32, NT = 256;
constexpr int kMinSplitTiles = 16;   // K tiles per split-K block, at least
constexpr int KPAD = BK + 4;     // kK / kG row length (floats)
constexpr int RPAD = BM + 4;     // kR row length (floats)
constexpr int SMEM = (BM * KPAD > BK * RPAD ? BM * KPAD : BK * RPAD);
constexpr int TPAD = BN + 4;     // epilogue tile row length (floats)
static_assert(BM * TPAD <= 4 * SMEM, "the epilogue tile reuses the operand buffers");

enum StageMode { kK = 0, kR = 1, kG = 2 };
constexpr int kNarrow = 16;   // added to a problem's mode: N <= 64, narrow wave layout
constexpr int kNLoop = 32;    // added to a problem's mode: K <= 2 BK, one block walks every N tile

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// x / d for d <= 64, x < 2^26: q = umulhi(x, ceil(2^32 / d)) is exact.
__device__ __forceinline__ int fdiv(int x, int d, uint32_t m) {
  return d == 1 ? x : (int)__umulhi((uint32_t)x, m);
}

__device__ __forceinline__ long long two_level(int i, int d, uint32_t m, long long s1, long long s2) {
  if (d == 1) return (long long)i * s1;
  const int q = fdiv(i, d, m);
  return (long long)q * s1 + (long long)(i - q * d) * s2;
}

__device__ __forceinline__ long long row_off(const GView& v, int r) { return two_level(r, v.div, v.mdiv, v.s1, v.s2); }
__device__ __forceinline__ long long col_off(const GView& v, int k) {
  return two_level(k, v.kdiv, v.mkdiv, v.sk1, v.sk2);
}

// Per-thread staging state of one operand (rows [r0, r0 + 128) of a view).
// Elements per thread per K tile: 4 x float4 (kK, kR) or 16 scalars (kG).
template <int MODE>
struct Stager {
  floatx4 reg[4];
  long long base[4];   // kK: row offsets of the thread's four rows
  bool rok[4];

  __device__ __forceinline__ void init(const GView& v, int rows, int r0) {
    if constexpr (MODE == kK) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = threadIdx.x + i * NT;
        const int r = r0 + e / (BK / 4);
        rok[i] = r < rows;
        base[i] = rok[i] ? row_off(v, r) : 0;
      }
    } else if constexpr (MODE == kR) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = threadIdx.x + i * NT;
        const int r = r0 + 4 * (e % (BM / 4));
        rok[i] = r < rows;   // rows is a multiple of 4
        base[i] = r;
      }
    }
  }

  __device__ __forceinline__ void load(const GView& v, int rows, int r0, int k0, int k_hi) {
    if constexpr (MODE == kK) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = threadIdx.x + i * NT;
        const int k = k0 + 4 * (e % (BK / 4));
        if (rok[i] && k < k_hi) reg[i] = *reinterpret_cast<const floatx4*>(v.p + base[i] + k);
        else reg[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    } else if constexpr (MODE == kR) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = threadIdx.x + i * NT;
        const int k = k0 + e / (BM / 4);
        if (rok[i] && k < k_hi) reg[i] = *reinterpret_cast<const floatx4*>(v.p + col_off(v, k) + base[i]);
        else reg[i] = floatx4{0.f, 0.f, 0.f, 0.f};
      }
    } else {
      // consecutive threads walk k of one row
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = threadIdx.x + i * NT;
        const int r = r0 + e / BK, k = k0 + e % BK;
        float val = 0.f;
        if (r < rows && k < k_hi) val = v.p[row_off(v, r) + col_off(v, k)];
        reg[i / 4][i % 4] = val;
      }
    }
  }

  __device__ __forceinline__ void store(float* S) const {
    if constexpr (MODE == kK) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = threadIdx.x + i * NT;
        *reinterpret_cast<floatx4*>(S + (e / (BK / 4)) * KPAD + 4 * (e % (BK / 4))) = reg[i];
      }
    } else if constexpr (MODE == kR) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = threadIdx.x + i * NT;
        *reinterpret_cast<floatx4*>(S + (e / (BM / 4)) * RPAD + 4 * (e % (BM / 4))) = reg[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int e = threadIdx.x + i * NT;
        S[(e / BK) * KPAD + e % BK] = reg[i / 4][i % 4];
      }
    }
  }
};

// The sixteen operand values (s = 0..15) of lane l for the 32-row block at
// row offset t0 of the staged tile.
template <int MODE>
__device__ __forceinline__ void fetch(const float* S, int t0, int lane, float* o) {
  const int m = t0 + lane % 32, h = lane / 32;
  if constexpr (MODE == kR) {
#pragma unroll
    for (int s = 0; s < 16; ++s) o[s] = S[(16 * h + s) * RPAD + m];
  } else {
    const floatx4* src = reinterpret_cast<const floatx4*>(S + m * KPAD + 16 * h);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const floatx4 q = src[j];
      o[4 * j] = q[0];
      o[4 * j + 1] = q[1];
      o[4 * j + 2] = q[2];
      o[4 * j + 3] = q[3];
    }
  }
}

// Problem fields pinned in scalar registers: read once from the kernel
// arguments (the problem index is only known at run time, and reloading the
// fields inside the K loop would make every step wait on scalar loads).
__device__ __forceinline__ int sreg(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint32_t sreg(uint32_t v) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)v); }
__device__ __forceinline__ float sreg(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ long long sreg(long long v) {
  const uint32_t lo = sreg((uint32_t)(unsigned long long)v), hi = sreg((uint32_t)((unsigned long long)v >> 32));
  return (long long)(((unsigned long long)hi << 32) | lo);
}
template <class T>
__device__ __forceinline__ T* sreg(T* p) {
  return reinterpret_cast<T*>(sreg((long long)reinterpret_cast<uintptr_t>(p)));
}
__device__ __forceinline__ GView pin(const GView& v) {
  return GView{sreg(v.p), sreg(v.div), sreg(v.s1), sreg(v.s2), sreg(v.kdiv), sreg(v.sk1), sreg(v.sk2),
               sreg(v.mdiv), sreg(v.mkdiv)};
}
__device__ __forceinline__ GOut pin(const GOut& o) {
  return GOut{sreg(o.p), sreg(o.div), sreg(o.s1), sreg(o.s2), sreg(o.accumulate), sreg(o.mdiv)};
}
__device__ __forceinline__ GemmProblem pin(const GemmProblem& q) {
  GemmProblem r;
  r.M = sreg(q.M);
  r.N = sreg(q.N);
  r.K = sreg(q.K);
  r.alpha = sreg(q.alpha);
  r.A = pin(q.A);
  r.Bt = pin(q.Bt);
  r.C = pin(q.C);
  r.C2 = pin(q.C2);
  r.ksplit = sreg(q.ksplit);
  r.part = sreg(q.part);
  return r;
}

__device__ __forceinline__ void store_out(const GOut& o, int m, int n, float val) {
  if (!o.p) return;
  float* dst = o.p + two_level(m, o.div, o.mdiv, o.s1, o.s2) + n;
  if (o.accumulate) *dst += val;
  else *dst = val;
}

// NI: 32-row accumulator blocks per wave, 2 (2 x 2 waves of 64 x 64) or 1
// (narrow: 4 x 1 waves of 32 x 64, for N <= 64).
template <int MA, int MB, int NI>
__device__ __forceinline__ void gemm_tile(const GemmProblem& P, int m0, int n0, int k_lo, int k_hi, int ks, float* As,
                                          float* Bs, bool vec_out) {
  const int wv = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int wm = NI == 2 ? wv % 2 : wv, wn = NI == 2 ? wv / 2 : 0;
  const int row0 = wm * 32 * NI;   // first row of the wave's sub-tile
  Stager<MA> sa;
  Stager<MB> sb;
  sa.init(P.A, P.M, m0);
  sb.init(P.Bt, P.N, n0);
  floatx16 acc[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // Two LDS buffers: step t computes on buffer t % 2 while the registers
  // holding tile t + 1 go to the other buffer and tile t + 2 is loaded.  The
  // single barrier per step orders both the stores (read next step) and the
  // reads of this step (overwritten by the next step's stores).
  if (k_lo < k_hi) {
    sa.load(P.A, P.M, m0, k_lo, k_hi);
    sb.load(P.Bt, P.N, n0, k_lo, k_hi);
    sa.store(As);
    sb.store(Bs);
    if (k_lo + BK < k_hi) {
      sa.load(P.A, P.M, m0, k_lo + BK, k_hi);
      sb.load(P.Bt, P.N, n0, k_lo + BK, k_hi);
    }
    __syncthreads();
  }
  int buf = 0;
  for (int k0 = k_lo; k0 < k_hi; k0 += BK) {
    const float* Ac = As + buf * SMEM;
    const float* Bc = Bs + buf * SMEM;
    float a[NI][16], b[2][16];
#pragma unroll
    for (int i = 0; i < NI; ++i) fetch<MA>(Ac, row0 + i * 32, lane, a[i]);
#pragma unroll
    for (int j = 0; j < 2; ++j) fetch<MB>(Bc, wn * 64 + j * 32, lane, b[j]);
#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s], acc[i][j], 0, 0, 0);
    if (k0 + BK < k_hi) {
      sa.store(As + (buf ^ 1) * SMEM);
      sb.store(Bs + (buf ^ 1) * SMEM);
      if (k0 + 2 * BK < k_hi) {
        sa.load(P.A, P.M, m0, k0 + 2 * BK, k_hi);
        sb.load(P.Bt, P.N, n0, k0 + 2 * BK, k_hi);
      }
    }
    __syncthreads();
    buf ^= 1;
  }

  // Epilogue: the 128 x 128 tile goes through LDS (the operand buffers are
  // free after the loop's last barrier), then every thread writes rows of
  // it as float4 (or scalars when the output is not 16-byte aligned or N is
  // not a multiple of 4): one two-level row offset per row instead of one
  // per element, and whole 512-byte row segments per wave.
  float* T = As;   // [BM][TPAD]
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + i * 32 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
        T[row * TPAD + wn * 64 + j * 32 + lane % 32] = acc[i][j][r];
      }
  __syncthreads();
  const int c4 = 4 * (threadIdx.x % 32);
  const int n = n0 + c4;
  const bool split = P.ksplit > 1;
#pragma unroll 1
  for (int it = 0; it < BM / 8; ++it) {
    const int row = it * 8 + threadIdx.x / 32;
    const int m = m0 + row;
    if (m >= P.M || n >= P.N) continue;
    floatx4 v = *reinterpret_cast<const floatx4*>(T + row * TPAD + c4);
    if (split) {
      float* dst = P.part + (size_t)ks * P.M * P.N + (size_t)m * P.N + n;
      if (vec_out) *reinterpret_cast<floatx4*>(dst) = v;
      else
        for (int e = 0; e < 4 && n + e < P.N; ++e) dst[e] = v[e];
      continue;
    }
    v *= P.alpha;
    auto put = [&](const GOut& O) {
      if (!O.p) return;
      float* dst = O.p + two_level(m, O.div, O.mdiv, O.s1, O.s2) + n;
      if (vec_out) {
        floatx4 w = v;
        if (O.accumulate) w += *reinterpret_cast<const floatx4*>(dst);
        *reinterpret_cast<floatx4*>(dst) = w;
      } else {
        for (int e = 0; e < 4 && n + e < P.N; ++e) dst[e] = O.accumulate ? dst[e] + v[e] : v[e];
      }
    };
    put(P.C);
    put(P.C2);
  }
}

// Short reductions (K <= 2 BK, e.g. the radial network's output layer,
// K = 64) with several N tiles: one block per M tile keeps its A tile (both
// K tiles) in LDS and walks every N tile; after a tile's products it loads
// the next tile's B operand, and stores the result straight from the
// accumulators (two 128-byte row segments per wave store) while those loads
// are in flight.  Plain outputs only (one row stride, no accumulation, no
// second output).  The general path's per-tile prologue and LDS epilogue
// dominated there: two K tiles of products per block.
template <int MA, int MB>
__device__ __forceinline__ void gemm_tile_nloop(const GemmProblem& P, int m0, int ntiles, float* As, float* Bs) {
  const int wv = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int wm = wv % 2, wn = wv / 2;
  const int nkt = (P.K + BK - 1) / BK;   // 1 or 2
  {
    Stager<MA> sa;
    sa.init(P.A, P.M, m0);
    for (int kt = 0; kt < nkt; ++kt) {
      sa.load(P.A, P.M, m0, kt * BK, P.K);
      sa.store(As + kt * SMEM);
    }
  }
  {
    Stager<MB> sb;
    sb.init(P.Bt, P.N, 0);
    for (int kt = 0; kt < nkt; ++kt) {
      sb.load(P.Bt, P.N, 0, kt * BK, P.K);
      sb.store(Bs + kt * SMEM);
    }
  }
  __syncthreads();
  for (int tn = 0; tn < ntiles; ++tn) {
    const int n0 = tn * BN;
    floatx16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    for (int kt = 0; kt < nkt; ++kt) {
      float a[2][16], b[2][16];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        fetch<MA>(As + kt * SMEM, wm * 64 + i * 32, lane, a[i]);
        fetch<MB>(Bs + kt * SMEM, wn * 64 + i * 32, lane, b[i]);
      }
#pragma unroll
      for (int st = 0; st < 16; ++st)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][st], b[j][st], acc[i][j], 0, 0, 0);
    }
    __syncthreads();   // every wave is done reading this tile's B
    Stager<MB> sb;
    if (tn + 1 < ntiles) {
      sb.init(P.Bt, P.N, n0 + BN);
      sb.load(P.Bt, P.N, n0 + BN, 0, P.K);
    }
    // plain output (one row stride, no second output, no accumulation)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int mr = m0 + wm * 64 + i * 32 + 4 * (lane / 32);
      float* rowp = P.C.p + (long long)mr * P.C.s1 + n0 + wn * 64 + lane % 32;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dm = 8 * (r / 4) + r % 4;
        if (mr + dm < P.M) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if (n0 + wn * 64 + j * 32 + lane % 32 < P.N) rowp[(long long)dm * P.C.s1 + j * 32] = P.alpha * acc[i][j][r];
          }
        }
      }
    }
    if (tn + 1 < ntiles) {
      sb.store(Bs);
      for (int kt = 1; kt < nkt; ++kt) {
        sb.load(P.Bt, P.N, n0 + BN, kt * BK, P.K);
        sb.store(Bs + kt * SMEM);
      }
    }
    __syncthreads();   // the next tile's B is in LDS
  }
}

__global__ __launch_bounds__(NT, 2) void gemm_kernel(GemmGroup g) {
  __shared__ __attribute__((aligned(16))) float smem[4 * SMEM];   // A and B, two buffers each
  float* As = smem;
  float* Bs = smem + 2 * SMEM;
  int b = blockIdx.x, pi = 0;
  while (pi < g.count - 1 && b >= g.blocks[pi]) {
    b -= g.blocks[pi];
    ++pi;
  }
  const GemmProblem P = pin(g.prob[pi]);
  if (g.mode[pi] >= kNLoop) {   // one block per M tile, every N tile
    const int m0 = b * BM;
    switch (g.mode[pi] - kNLoop) {
      case kK * 3 + kK: gemm_tile_nloop<kK, kK>(P, m0, g.tiles_n[pi], As, Bs); break;
      case kK * 3 + kR: gemm_tile_nloop<kK, kR>(P, m0, g.tiles_n[pi], As, Bs); break;
      case kR * 3 + kR: gemm_tile_nloop<kR, kR>(P, m0, g.tiles_n[pi], As, Bs); break;
      case kR * 3 + kK: gemm_tile_nloop<kR, kK>(P, m0, g.tiles_n[pi], As, Bs); break;
      default: gemm_tile_nloop<kG, kG>(P, m0, g.tiles_n[pi], As, Bs); break;
    }
    return;
  }
  const int tiles = g.tiles_m[pi] * g.tiles_n[pi];
  const int ks = b / tiles;
  b %= tiles;
  const int tm = b % g.tiles_m[pi], tn = b / g.tiles_m[pi];
  const int m0 = tm * BM, n0 = tn * BN;
  const int k_lo = ks * g.kchunk[pi];
  const int k_hi = min(P.K, k_lo + g.kchunk[pi]);
  const bool vec_out = g.vec_out[pi] != 0;
  switch (g.mode[pi]) {
    case kK * 3 + kK: gemm_tile<kK, kK, 2>(P, m0, n0, k_lo, k_hi, ks, As, Bs, vec_out); break;
    case kK * 3 + kR: gemm_tile<kK, kR, 2>(P, m0, n0, k_lo, k_hi, ks, As, Bs, vec_out); break;
    case kR * 3 + kR: gemm_tile<kR, kR, 2>(P, m0, n0, k_lo, k_hi, ks, As, Bs, vec_out); break;
    case kR * 3 + kK: gemm_tile<kR, kK, 2>(P, m0, n0, k_lo, k_hi, ks, As, Bs, vec_out); break;
    case kNarrow + kK * 3 + kK: gemm_tile<kK, kK, 1>(P, m0, n0, k_lo, k_hi, ks, As, Bs, vec_out); break;
    case kNarrow + kK * 3 + kR: gemm_tile<kK, kR, 1>(P, m0, n0, k_lo, k_hi, ks, As, Bs, vec_out); break;
    case kNarrow + kR * 3 + kR: gemm_tile<kR, kR, 1>(P, m0, n0, k_lo, k_hi, ks, As, Bs, vec_out); break;
    case kNarrow + kR * 3 + kK: gemm_tile<kR, kK, 1>(P, m0, n0, k_lo, k_hi, ks, As, Bs, vec_out); break;
    case kNarrow + kG * 3 + kG: gemm_tile<kG, kG, 1>(P, m0, n0, k_lo, k_hi, ks, As, Bs, vec_out); break;
    default: gemm_tile<kG, kG, 2>(P, m0, n0, k_lo, k_hi, ks, As, Bs, vec_out); break;
  }
}

// Sum the ksplit partial tiles in split order, then store/add.  Loads are
// issued eight at a time; the additions stay in split order.
__global__ __launch_bounds__(256) void split_reduce_kernel(GemmProblem P) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t MN = (size_t)P.M * P.N;
  if (i >= MN) return;
  const float* src = P.part + i;
  float t = 0.f;
  int s = 0;
  for (; s + 8 <= P.ksplit; s += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[(size_t)(s + j) * MN];
#pragma unroll
    for (int j = 0; j < 8; ++j) t += v[j];
  }
  for (; s < P.ksplit; ++s) t += src[(size_t)s * MN];
  const int m = (int)(i / P.N), n = (int)(i % P.N);
  store_out(P.C, m, n, P.alpha * t);
  store_out(P.C2, m, n, P.alpha * t);
}

uint32_t magic(int d) { return d <= 1 ? 0u : (uint32_t)((0x100000000ull + d - 1) / d); }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Staging mode of a view with `rows` rows and reduction length K.
int stage_mode(const GView& v, int rows, int K) {
  if (!aligned16(v.p)) return kG;
  if (v.kdiv == 1 && v.sk1 == 1 && K % 4 == 0 && v.s1 % 4 == 0 && (v.div == 1 || v.s2 % 4 == 0)) return kK;
  if (v.div == 1 && v.s1 == 1 && rows % 4 == 0 && v.sk1 % 4 == 0 && (v.kdiv == 1 || v.sk2 % 4 == 0)) return kR;
  return kG;
}

}  // namespace

int gemm_ksplit(int M, int N, int K, int target) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  int s = target / (tiles > 0 ? tiles : 1);
  // every split covers at least kMinSplitTiles K tiles: short splits would
  // spend more on writing their partial tile than on the products
  const int kt = (K + BK - 1) / BK;
  const int smax = (kt + kMinSplitTiles - 1) / kMinSplitTiles;
  if (s > smax) s = smax;
  return s < 1 ? 1 : s;
}

void gemm_group(const GemmGroup& g0, hipStream_t st) {
  GemmGroup g = g0;
  // A group too small to fill the chip (e.g. a 1000-row map: 8 tiles) splits
  // K over up to four blocks when the caller lent scratch for the partials:
  // four times the blocks, each a quarter of the products, summed in split
  // order by split_reduce_kernel.
  if (g.scratch && g.scratch_floats) {
    long long tiles = 0;
    for (int i = 0; i < g.count; ++i) {
      const GemmProblem& P = g.prob[i];
      tiles += (long long)((P.M + BM - 1) / BM) * ((P.N + BN - 1) / BN) * (P.ksplit > 1 ? P.ksplit : 1);
    }
    if (tiles > 0 && tiles < 64) {
      size_t used = 0;
      for (int i = 0; i < g.count; ++i) {
        GemmProblem& P = g.prob[i];
        if (P.ksplit > 1) continue;
        const long long kt = (P.K + BK - 1) / BK;
        long long sp = 128 / tiles;
        if (sp > 4) sp = 4;
        if (sp > kt) sp = kt;
        const size_t need = (size_t)sp * P.M * P.N;
        if (sp > 1 && used + need <= g.scratch_floats) {
          P.ksplit = (int)sp;
          P.part = g.scratch + used;
          used += need;
        }
      }
    }
  }
  int total = 0;
  for (int i = 0; i < g.count; ++i) {
    GemmProblem& P = g.prob[i];
    if (P.ksplit < 1) P.ksplit = 1;
    g.tiles_m[i] = (P.M + BM - 1) / BM;
    g.tiles_n[i] = (P.N + BN - 1) / BN;
    const int kt = (P.K + BK - 1) / BK;
    g.kchunk[i] = ((kt + P.ksplit - 1) / P.ksplit) * BK;
    P.A.mdiv = magic(P.A.div);
    P.A.mkdiv = magic(P.A.kdiv);
    P.Bt.mdiv = magic(P.Bt.div);
    P.Bt.mkdiv = magic(P.Bt.kdiv);
    P.C.mdiv = magic(P.C.div);
    P.C2.mdiv = magic(P.C2.div);
    const int ma = stage_mode(P.A, P.M, P.K), mb = stage_mode(P.Bt, P.N, P.K);
    g.mode[i] = ((ma == kG || mb == kG) ? kG * 3 + kG : ma * 3 + mb) + (P.N <= BN / 2 ? kNarrow : 0);
    const bool nloop = P.K <= 2 * BK && g.tiles_n[i] > 1 && P.ksplit == 1 && !P.C2.p && P.C.p && P.C.div == 1 &&
                       !P.C.accumulate;
    if (nloop) g.mode[i] = ((ma == kG || mb == kG) ? kG * 3 + kG : ma * 3 + mb) + kNLoop;
    g.blocks[i] = nloop ? g.tiles_m[i] : g.tiles_m[i] * g.tiles_n[i] * P.ksplit;
    auto out_vec = [&](const GOut& o) {
      return !o.p || (aligned16(o.p) && o.s1 % 4 == 0 && (o.div == 1 || o.s2 % 4 == 0));
    };
    g.vec_out[i] = P.N % 4 == 0 && (P.ksplit > 1 ? aligned16(P.part) : (out_vec(P.C) && out_vec(P.C2)));
    total += g.blocks[i];
  }
  if (total == 0) return;
  hipLaunchKernelGGL(gemm_kernel, dim3(total), dim3(NT), 0, st, g);
  for (int i = 0; i < g.count; ++i) {
    const GemmProblem& P = g.prob[i];
    if (P.ksplit > 1) {
      const size_t MN = (size_t)P.M * P.N;
      hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, st, P);
    }
  }
}

}  // namespace fc
