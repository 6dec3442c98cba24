// Edge-convolution launch interface shared by the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "fc_common.h"
#include "fc_reduce.h"

namespace fc {

struct ConvArgs {
  int N, E, C;
  float rc;
  const int *rowptr, *sender, *receiver, *t_rowptr, *t_edge;
  const float *pos, *shift, *x, *W, *g;
  float *z, *x_bar, *pos_bar, *rbar;
  // VJP-of-VJP: cotangents of x_bar / pos_bar (nullable) and the g_hat output;
  // x_hat and pos_hat reuse x_bar and pos_bar, the per-edge term reuses rbar
  const float *v_x, *v_pos;
  float* g_hat;
  // VJP: gradient of the radial weights W [8][P][C] (nullable)
  float* W_bar;
  // explicit per-edge weights w [E][P][C] (replacing R W when non-null) and
  // their gradient (VJP, nullable)
  const float* w_edge;
  float* w_edge_bar;
  // VJP-of-VJP with explicit weights: the weight cotangent [E][P][C]
  // (nullable); w_hat reuses w_edge_bar
  const float* v_w_edge;
  // radial network fused into the lanes (conv_mlp_dispatch): the second
  // hidden layer and its r-derivative per edge, [E][2][64]; W is then W3
  // [64][P][C]
  const float* mlp_h;
};

// l_out is the output-rank key: l_out + kAllParities keeps every
// triangle-allowed path
bool conv_supported(int l_in, int l_edge, int l_out);
// whether the VJP-of-VJP (op 2) is instantiated for these ranks
bool conv_vv_supported(int l_in, int l_edge, int l_out);
// op 0: forward (needs rowptr, sender, pos, shift, x, W, z);
// op 1: VJP (additionally receiver, t_rowptr, t_edge, g, rbar, and x_bar
//       and/or pos_bar);
// op 2: VJP-of-VJP (g, v_x / v_pos, and g_hat, x_bar (= x_hat) and/or
//       pos_bar (= pos_hat)).
// Outgoing edges of a sender are split into S contiguous slices (about 32
// edges each on average) processed by separate blocks.
inline int vjp_slices(int N, int E) {
  const int avg = N > 0 ? E / N : 0;
  int s = (avg + 16) / 32;
  return s < 1 ? 1 : (s > 8 ? 8 : s);
}

inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Receivers (one per wave) of a block of the radial-weight gradient pass.
inline constexpr int kWgWaves = 4;
inline int wgrad_blocks(int N) { return (N + kWgWaves - 1) / kWgWaves; }

// VJP workspace: per-edge position cotangents, then (S > 1) per-slice
// partial position sums and partial x_bar, then (with_w) the per-block
// partial radial-weight gradients [wgrad_blocks(N)][8][P][C].
struct VjpWorkspace {
  int S;
  float *rbar, *p_part, *x_part, *w_part;
  size_t bytes;
  VjpWorkspace(int N, int E, int C, int nin, int P, bool with_w, void* base) {
    S = vjp_slices(N, E);
    char* p = static_cast<char*>(base);
    size_t off = 0;
    rbar = reinterpret_cast<float*>(p + off);
    off += align256((size_t)3 * E * sizeof(float));
    p_part = reinterpret_cast<float*>(p + off);
    if (S > 1) off += align256((size_t)3 * N * S * sizeof(float));
    x_part = reinterpret_cast<float*>(p + off);
    if (S > 1) off += align256((size_t)N * S * nin * C * sizeof(float));
    w_part = reinterpret_cast<float*>(p + off);
    if (with_w) off += align256((size_t)wgrad_blocks(N) * kNB * P * C * sizeof(float));
    bytes = off;
    if (!base) rbar = p_part = x_part = w_part = nullptr;
  }
};

void launch_vjp_combine(const ConvArgs& a, const VjpWorkspace& w, int nin, hipStream_t st);
// pos_bar[v] = sum over v's out-edges of rbar - sum over its in-edges (the
// receiver-side VJP's position gradient; needs rowptr, t_rowptr, t_edge)
void launch_pos_from_edges(const ConvArgs& a, const float* rbar, hipStream_t st);

// The launch sequences of one configuration's VJP-of-VJP passes (g_hat,
// W_hat, and the sender pass without / with a feature cotangent).
struct VVParts {
  void (*recv)(const ConvArgs&, hipStream_t);
  void (*wgrad)(const ConvArgs&, hipStream_t);
  void (*sender)(const ConvArgs&, hipStream_t);
  void (*sender_vx)(const ConvArgs&, hipStream_t);
};
// g_hat, W_hat (args.W_bar), then x_hat / pos_hat with the combine pass,
// each when requested; nin input rows and P paths size the workspace.
void run_vjp_vjp(const VVParts& parts, int nin, int P, const ConvArgs& a, hipStream_t st);
bool conv_dispatch(int op, int l_in, int l_edge, int l_out, const ConvArgs& args, hipStream_t stream);
// VJP-of-VJP with explicit per-edge weights (w_edge, v_w_edge; w_hat in
// w_edge_bar); false when not instantiated (the configurations of
// conv_vv_supported)
bool conv_vv_w_dispatch(int l_in, int l_edge, int l_out, const ConvArgs& args, hipStream_t stream);
bool conv_vv_w_supported(int l_in, int l_edge, int l_out);
// The convolution weighted by the radial network with its output layer
// fused into the lanes (args.W = W3, args.mlp_h): op 0 forward (z), op 1
// VJP (x_bar and/or pos_bar, the latter through w(r) as well); false when
// not instantiated for these ranks.
bool conv_mlp_dispatch(int op, int l_in, int l_edge, int l_out, const ConvArgs& args, hipStream_t stream);
bool conv_mlp_supported(int l_in, int l_edge, int l_out);
// whether the fused forward is the default for these ranks (measured faster
// than the materialised one; the VJP is materialised by default)
bool conv_mlp_fwd_fused(int l_in, int l_edge, int l_out);

}  // namespace fc
