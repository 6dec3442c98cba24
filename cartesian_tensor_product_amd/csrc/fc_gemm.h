// Grouped FP32 GEMM on the gfx950 matrix cores (v_mfma_f32_32x32x2f32),
// used for the correlation ladder's path/channel mixing (FlashCart paper,
// §5 Eq. 2 and App. E "Path-reduced products") and its gradients.
//
//   C[m, n] (=|+=) alpha * sum_k A(m, k) * Bt(n, k)
//
// Operands are strided views so that node-feature arrays [N][rows][C] can be
// read and written in place: element (r, k) of a view lives at
//   (r / div) * s1 + (r % div) * s2 + (k / kdiv) * sk1 + (k % kdiv) * sk2,
// divisors at most 64 (they are 2l+1 or 1), indices below 2^26.
// Long reductions (weight gradients, where K runs over all node rows) are
// split over ksplit blocks writing partial tiles to a scratch buffer, summed
// afterwards in a fixed order (deterministic).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fc {

struct GView {
  const float* p;
  int div;             // >= 1
  long long s1, s2;    // row offset = (r / div) * s1 + (r % div) * s2
  int kdiv;            // >= 1
  long long sk1, sk2;  // column offset = (k / kdiv) * sk1 + (k % kdiv) * sk2
  uint32_t mdiv, mkdiv;  // multiply-high reciprocals (filled by gemm_group)
};

struct GOut {
  float* p;            // nullptr: no output
  int div;
  long long s1, s2;    // row offset as in GView; columns are contiguous
  int accumulate;      // 0: store, 1: add to the existing value
  uint32_t mdiv;
};

struct GemmProblem {
  int M, N, K;
  float alpha;
  GView A, Bt;
  GOut C, C2;          // C2 (optional) receives the same values (store/add)
  int ksplit;          // >= 1; > 1 needs part (ksplit * M * N floats)
  float* part;
};

inline constexpr int kMaxGemmGroup = 10;

struct GemmGroup {
  int count;
  // optional scratch (floats): a group of fewer than 64 tiles splits its
  // unsplit problems' K over up to four blocks with partials here (set by the
  // caller; zero-initialised groups have none)
  float* scratch;
  size_t scratch_floats;
  int tiles_m[kMaxGemmGroup];
  int tiles_n[kMaxGemmGroup];
  int kchunk[kMaxGemmGroup];
  int mode[kMaxGemmGroup];   // operand staging modes (filled by gemm_group)
  int blocks[kMaxGemmGroup];   // workgroups of each problem (filled by gemm_group)
  int vec_out[kMaxGemmGroup];   // float4 output rows allowed (filled by gemm_group)
  GemmProblem prob[kMaxGemmGroup];
};

// Launches all problems of the group in one grid (block tile 128 x 128),
// then the split-K reductions if any problem uses them.
void gemm_group(const GemmGroup& g, hipStream_t st);

// Split count for a long reduction: about `target` blocks in total.
int gemm_ksplit(int M, int N, int K, int target);

// Scratch floats that lets a group of these problems (M, N per problem)
// split when small: four partial tiles per problem.
inline size_t gemm_small_split_floats(size_t sum_MN) { return 4 * sum_MN; }

inline GView plain_view(const float* p, long long ld) { return GView{p, 1, ld, 0, 1, 1, 0, 0, 0}; }
// element (r, k) = p[k * ld + r] (a transposed plain matrix)
inline GView plain_view_t(const float* p, long long ld) { return GView{p, 1, 1, 0, 1, ld, 0, 0, 0}; }
inline GOut plain_out(float* p, long long ld, int acc) { return GOut{p, 1, ld, 0, acc, 0}; }
inline GOut no_out() { return GOut{nullptr, 1, 0, 0, 0, 0}; }

}  // namespace fc
