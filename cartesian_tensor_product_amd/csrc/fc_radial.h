// The pages' radial network: per-edge Chebyshev features with a polynomial
// envelope and a bias-free SiLU MLP whose output layer (one weight per
// path and channel) runs on the matrix cores (launch interface).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace fc {

inline constexpr int kRadFeat = 8;     // Chebyshev functions
inline constexpr int kRadHidden = 64;  // width of both hidden layers
inline constexpr int kRadRow = 2 * kRadHidden;  // floats per edge of launch_radial_hidden_rows: h2, dh2/dr

// Flat weights: W1 [8][64], W2 [64][64], W3 [64][P C].
inline size_t radial_weight_floats(int P, int C) {
  return (size_t)kRadFeat * kRadHidden + (size_t)kRadHidden * kRadHidden + (size_t)kRadHidden * P * C;
}

struct RadialArgs {
  int N, E, P, C;
  float r_max;
  const int *rowptr, *sender, *receiver, *t_rowptr, *t_edge;
  const float *pos, *shift, *weights;
};

// Row stride of the edge-minor hidden layer: E rounded up to a multiple of 4
// (128-bit loads of the GEMM operand).
inline int radial_ld(int E) { return (E + 3) / 4 * 4; }

// h2t [64][radial_ld(E)] = second hidden layer, edge-minor.
void launch_radial_hidden(const RadialArgs& a, float* h2t, hipStream_t st);
// w [E][P C] = h2 W3.
void launch_radial_out(const RadialArgs& a, const float* h2t, float* w, hipStream_t st);
// hh [E][2][64]: the second hidden layer of every edge and its derivative
// with respect to the edge length (edge-major rows, for the convolution
// with the output layer fused into its lanes).
void launch_radial_hidden_rows(const RadialArgs& a, float* hh, hipStream_t st);
// Backward from w_bar [E][P C]: q [E][3] = dL/dr_vec per edge, then
// pos_grad[v] += sum_{e out of v} q_e - sum_{e into v} q_e; with w_grad
// (flat layout) the weight gradients.  Scratch: hbar [E][64], then (w_grad)
// a2bt, h1t, a1bt [64][E] and phit [8][E], and split-K partials.
size_t radial_vjp_scratch_floats(int E, int P, int C);
void launch_radial_vjp(const RadialArgs& a, const float* h2t, const float* w_bar, float* q, float* pos_grad,
                       float* w_grad, float* scratch, hipStream_t st);

}  // namespace fc
