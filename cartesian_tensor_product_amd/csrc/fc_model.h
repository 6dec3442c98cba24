// Pieces of a full message-passing block (launch interface): scalar SiLU
// gates and the readout MLP.
#pragma once

#include <hip/hip_runtime.h>

namespace fc {

inline constexpr int kReadoutHidden = 64;

// y_0 = SiLU(n_0), y_l = SiLU(n_0) n_l (l >= 1); A = n (copied).
void launch_gate_fwd(int N, int C, int l_max, const float* n, float* y, float* A, hipStream_t st);
// n_bar = A_bar + the gate terms of y_bar: n_bar_0 += SiLU'(n_0) (y_bar_0 +
// sum_{l>=1} <y_bar_l, n_l>), n_bar_l += SiLU(n_0) y_bar_l.
void launch_gate_vjp(int N, int C, int l_max, const float* n, const float* Abar, const float* ybar, float* nbar,
                     hipStream_t st);
// e[u] = SiLU(SiLU(f_u Wr1) Wr2) . wr3 for f [N][C] (bias-free MLP
// C -> 64 -> 64 -> 1), and its VJP f_bar [N][C] for e_bar = 1.
void launch_readout_fwd(int N, int C, const float* f, const float* Wr1, const float* Wr2, const float* wr3, float* e,
                        hipStream_t st);
void launch_readout_vjp(int N, int C, const float* f, const float* Wr1, const float* Wr2, const float* wr3,
                        float* fbar, hipStream_t st);

}  // namespace fc
