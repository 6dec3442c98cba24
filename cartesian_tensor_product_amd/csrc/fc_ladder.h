// Host-side plan of the node-local correlation ladder (FlashCart paper §5
// Eq. 2 and App. E "Path-reduced products").
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>

namespace fc {

struct LadderPlan {
  int N, C, la, lprod, lout, order, variant;   // variant 0 full, 1 path-reduced

  int lq(int q) const;                 // highest rank kept at step q
  int paths(int q, int L) const;       // paths of step q >= 2 with output rank L
  int paths(int q) const;              // all paths of step q >= 2
  int prod_rows(int q) const;          // sum_L (2L+1) P_{q,L}
  size_t weight_floats() const;
  size_t saved_floats() const;         // phi^q, q = 1 .. order-1, [N][(l_prod+1)^2][C] each
  size_t state_floats() const;
  size_t fwd_ws_floats() const;
  size_t vjp_ws_floats() const;
  size_t vv_ws_floats() const;         // VJP-of-VJP
  // offsets (floats) into the flat weight buffer
  size_t w_full(int q, int L) const;   // full: W1_L (q = 1) or W^q_L
  size_t w_a(int q) const;             // reduced: a1 (q = 1) or a^q
  size_t w_final(int L) const;         // reduced: W_L
};

void ladder_forward(const LadderPlan& p, const float* A, const float* w, float* z, float* saved, float* ws,
                    hipStream_t st);
void ladder_vjp(const LadderPlan& p, const float* A, const float* w, const float* saved, const float* gz,
                float* A_grad, float* w_grad, float* ws, hipStream_t st);
// Derivatives of s = <v_A, A_bar> + <v_w, w_bar> (cotangents
// nullable) with respect to g_z (g_hat), A (A_hat) and the weights (w_hat).
void ladder_vjp_vjp(const LadderPlan& p, const float* A, const float* w, const float* saved, const float* gz,
                    const float* vA, const float* vw, float* g_hat, float* A_hat, float* w_hat, float* ws,
                    hipStream_t st);

}  // namespace fc
