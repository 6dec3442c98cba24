// Grouped FP32 GEMM on the gfx950 matrix cores.
//
// Block tile 32 (M) x 128 (N) x 32 (K), four waves; wave w owns output
// columns [32w, 32w + 32) of the block tile and accumulates one 32x32 tile
// with v_mfma_f32_32x32x2f32 (K = 2 per instruction).  Operand layout of that
// instruction: lane l supplies A[l % 32][l / 32] and B[l / 32][l % 32]; the
// sixteen accumulator registers r of lane l hold
// D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].  Tiles are staged through LDS
// k-major, so both operand reads are bank-conflict free.
#include "fc_gemm.h"

namespace fc {

namespace {

constexpr int BM = 32, BN = 128, BK = 32, NT = 256;

typedef float floatx16 __attribute__((ext_vector_type(16)));

// x / d for d <= 64, x < 2^26: q = umulhi(x, ceil(2^32 / d)) is exact.
__device__ __forceinline__ int fdiv(int x, int d, uint32_t m) {
  return d == 1 ? x : (int)__umulhi((uint32_t)x, m);
}

__device__ __forceinline__ long long two_level(int i, int d, uint32_t m, long long s1, long long s2) {
  if (d == 1) return (long long)i * s1;
  const int q = fdiv(i, d, m);
  return (long long)q * s1 + (long long)(i - q * d) * s2;
}

// Stage rows [r0, r0 + R) x cols [k0, k0 + BK) of a view into S[BK][R]
// (k-major), zero outside [0, rows) x [k_lo, k_hi).
template <int R>
__device__ __forceinline__ void stage(const GView& v, int rows, int k_hi, int r0, int k0, float* S) {
  constexpr int ELEMS = R * BK;
  const bool k_contig = v.kdiv == 1 && v.sk1 == 1;
  if (k_contig) {
    // consecutive threads walk k of one row (contiguous in memory)
#pragma unroll
    for (int i = 0; i < ELEMS / NT; ++i) {
      const int e = threadIdx.x + i * NT;
      const int r = e / BK, kk = e % BK;
      const int gr = r0 + r, gk = k0 + kk;
      float val = 0.f;
      if (gr < rows && gk < k_hi) val = v.p[two_level(gr, v.div, v.mdiv, v.s1, v.s2) + gk];
      S[kk * R + r] = val;
    }
  } else {
    // consecutive threads walk rows
#pragma unroll
    for (int i = 0; i < ELEMS / NT; ++i) {
      const int e = threadIdx.x + i * NT;
      const int kk = e / R, r = e % R;
      const int gr = r0 + r, gk = k0 + kk;
      float val = 0.f;
      if (gr < rows && gk < k_hi)
        val = v.p[two_level(gr, v.div, v.mdiv, v.s1, v.s2) + two_level(gk, v.kdiv, v.mkdiv, v.sk1, v.sk2)];
      S[kk * R + r] = val;
    }
  }
}

__device__ __forceinline__ void store_out(const GOut& o, int m, int n, float val) {
  if (!o.p) return;
  float* dst = o.p + two_level(m, o.div, o.mdiv, o.s1, o.s2) + n;
  if (o.accumulate) *dst += val;
  else *dst = val;
}

__global__ __launch_bounds__(NT) void gemm_kernel(GemmGroup g) {
  __shared__ float As[BK * BM];
  __shared__ float Bs[BK * BN];
  int b = blockIdx.x, pi = 0;
  while (pi < g.count - 1 && b >= g.tiles_m[pi] * g.tiles_n[pi] * g.prob[pi].ksplit) {
    b -= g.tiles_m[pi] * g.tiles_n[pi] * g.prob[pi].ksplit;
    ++pi;
  }
  const GemmProblem& P = g.prob[pi];
  const int tiles = g.tiles_m[pi] * g.tiles_n[pi];
  const int ks = b / tiles;
  b %= tiles;
  const int tm = b % g.tiles_m[pi], tn = b / g.tiles_m[pi];
  const int m0 = tm * BM, n0 = tn * BN;
  const int k_lo = ks * g.kchunk[pi];
  const int k_hi = min(P.K, k_lo + g.kchunk[pi]);
  const int wv = threadIdx.x / 64, lane = threadIdx.x % 64;
  floatx16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;

  for (int k0 = k_lo; k0 < k_hi; k0 += BK) {
    stage<BM>(P.A, P.M, k_hi, m0, k0, As);
    stage<BN>(P.Bt, P.N, k_hi, n0, k0, Bs);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 2) {
      const float a = As[(kk + lane / 32) * BM + lane % 32];
      const float bb = Bs[(kk + lane / 32) * BN + wv * 32 + lane % 32];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bb, acc, 0, 0, 0);
    }
    __syncthreads();
  }
  const int n = n0 + wv * 32 + lane % 32;
  if (n >= P.N) return;
  if (P.ksplit > 1) {
    float* part = P.part + (size_t)ks * P.M * P.N;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
      if (m < P.M) part[(size_t)m * P.N + n] = acc[r];
    }
    return;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + 8 * (r / 4) + 4 * (lane / 32) + r % 4;
    if (m < P.M) {
      const float val = P.alpha * acc[r];
      store_out(P.C, m, n, val);
      store_out(P.C2, m, n, val);
    }
  }
}

// Sum the ksplit partial tiles in split order, then store/add.
__global__ __launch_bounds__(256) void split_reduce_kernel(GemmProblem P) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t MN = (size_t)P.M * P.N;
  if (i >= MN) return;
  float t = 0.f;
  for (int s = 0; s < P.ksplit; ++s) t += P.part[(size_t)s * MN + i];
  const int m = (int)(i / P.N), n = (int)(i % P.N);
  store_out(P.C, m, n, P.alpha * t);
  store_out(P.C2, m, n, P.alpha * t);
}

uint32_t magic(int d) { return d <= 1 ? 0u : (uint32_t)((0x100000000ull + d - 1) / d); }

}  // namespace

int gemm_ksplit(int M, int N, int K, int target) {
  const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  int s = target / (tiles > 0 ? tiles : 1);
  const int kt = (K + BK - 1) / BK;
  if (s > kt) s = kt;
  return s < 1 ? 1 : s;
}

void gemm_group(const GemmGroup& g0, hipStream_t st) {
  GemmGroup g = g0;
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
    total += g.tiles_m[i] * g.tiles_n[i] * P.ksplit;
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
