// C ABI of the FlashCart gfx950 library: argument checks on the host, then
// stream-ordered kernel launches.  See include/flashcart.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/flashcart.h"
#include "fc_conv.h"
#include "fc_graph.h"
#include "fc_block.h"
#include "fc_ladder.h"
#include "fc_norm.h"
#include "fc_radial.h"
#include "fc_model.h"
#include "fc_gemm.h"

// Scratch of the allocation-free VJP (fc_edge_conv_vjp_noalloc): the VJP
// workspace of one call, in device memory the library owns.  Each GPU the
// library runs on holds its own copy from module load until the process
// ends; all calls on one GPU share it.
constexpr size_t kNoAllocScratchBytes = FC_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

thread_local std::string g_msg;

fc_status fail(fc_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_msg = buf;
  return s;
}

fc_status ok() {
  g_msg.clear();
  return FC_OK;
}

fc_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(FC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool misaligned(const void* p, size_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) != 0; }

bool all_parities(const fc_conv_desc* d) { return (d->flags & FC_CONV_ALL_PARITIES) != 0; }
bool sum_paths(const fc_conv_desc* d) { return (d->flags & FC_CONV_SUM_PATHS) != 0; }

bool path_ok(const fc_conv_desc* d, int l1, int l2, int L) {
  return all_parities(d) ? fc::triangle(l1, l2, L) : fc::admissible(l1, l2, L);
}

// output-rank key of the configuration (kAllParities set for every path,
// kSumPaths for path-summed outputs)
int lout_key(const fc_conv_desc* d) {
  return d->l_out + (all_parities(d) ? fc::kAllParities : 0) + (sum_paths(d) ? fc::kSumPaths : 0);
}

int conv_paths_L(const fc_conv_desc* d, int L) {
  int c = 0;
  for (int l1 = 0; l1 <= d->l_in; ++l1)
    for (int l2 = 0; l2 <= d->l_edge; ++l2)
      if (path_ok(d, l1, l2, L)) ++c;
  return c;
}

fc_status check_desc(const fc_conv_desc* d) {
  if (!d) return fail(FC_ERR_INVALID_ARGUMENT, "descriptor is NULL");
  if (d->n_nodes < 1) return fail(FC_ERR_INVALID_ARGUMENT, "n_nodes must be >= 1 (got %d)", d->n_nodes);
  if (d->n_edges < 0) return fail(FC_ERR_INVALID_ARGUMENT, "n_edges must be >= 0 (got %d)", d->n_edges);
  if (d->channels < 1) return fail(FC_ERR_INVALID_ARGUMENT, "channels must be >= 1 (got %d)", d->channels);
  if (d->l_in < 0 || d->l_edge < 0 || d->l_out < 0)
    return fail(FC_ERR_INVALID_ARGUMENT, "ranks must be >= 0");
  if (d->l_in > 5 || d->l_edge > 5 || d->l_out > 5)
    return fail(FC_ERR_UNSUPPORTED, "ranks above 5 are not supported (l_in=%d l_edge=%d l_out=%d)", d->l_in,
                d->l_edge, d->l_out);
  if (!(d->r_cut > 0.f) || !std::isfinite(d->r_cut))
    return fail(FC_ERR_INVALID_ARGUMENT, "r_cut must be positive and finite");
  if (d->n_basis != fc::kNB) return fail(FC_ERR_UNSUPPORTED, "n_basis must be 8 (got %d)", d->n_basis);
  if ((d->flags & ~uint32_t(FC_CONV_ALL_PARITIES | FC_CONV_SUM_PATHS | FC_CONV_MLP_MATERIALIZE | FC_CONV_MLP_FUSE)) != 0)
    return fail(FC_ERR_UNSUPPORTED,
                "unknown flags 0x%x (FC_CONV_ALL_PARITIES, FC_CONV_SUM_PATHS, FC_CONV_MLP_MATERIALIZE and "
                "FC_CONV_MLP_FUSE are defined)", d->flags);
  if ((d->flags & FC_CONV_MLP_MATERIALIZE) && (d->flags & FC_CONV_MLP_FUSE))
    return fail(FC_ERR_INVALID_ARGUMENT, "FC_CONV_MLP_MATERIALIZE and FC_CONV_MLP_FUSE exclude each other");
  int P = 0;
  for (int L = 0; L <= d->l_out; ++L) P += conv_paths_L(d, L);
  if (P == 0) return fail(FC_ERR_INVALID_ARGUMENT, "no admissible path for these ranks");
  if (d->channels > 256) return fail(FC_ERR_UNSUPPORTED, "channels above 256 are not supported");
  if (!fc::conv_supported(d->l_in, d->l_edge, lout_key(d)))
    return fail(FC_ERR_UNSUPPORTED,
                "(l_in, l_edge, l_out) = (%d, %d, %d) with flags 0x%x is not instantiated in this library", d->l_in,
                d->l_edge, d->l_out, d->flags);
  return FC_OK;
}

void layout(const fc_conv_desc* d, int* P, int* nin, int* nout) {
  int p = 0, o = 0;
  for (int L = 0; L <= d->l_out; ++L) {
    const int c = conv_paths_L(d, L);
    p += c;
    o += (2 * L + 1) * (sum_paths(d) ? (c > 0 ? 1 : 0) : c);
  }
  *P = p;
  *nin = (d->l_in + 1) * (d->l_in + 1);
  *nout = o;
}

fc::ConvArgs make_args(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                       const float* x, const float* W) {
  fc::ConvArgs a{};
  a.N = d->n_nodes;
  a.E = d->n_edges;
  a.C = d->channels;
  a.rc = d->r_cut;
  a.rowptr = g->rowptr;
  a.sender = g->sender;
  a.receiver = g->receiver;
  a.t_rowptr = g->t_rowptr;
  a.t_edge = g->t_edge;
  a.pos = pos;
  a.shift = shift;
  a.x = x;
  a.W = W;
  return a;
}


// Where the radial network's output layer runs fused in the convolution's
// lanes (w = h2 W3 never stored), for rank sets instantiated for it: the
// forward where it was measured faster (conv_mlp_fwd_fused) or with
// FC_CONV_MLP_FUSE; the VJP with FC_CONV_MLP_FUSE only; neither with
// FC_CONV_MLP_MATERIALIZE.
bool mlp_fusable(const fc_conv_desc* d) {
  return !(d->flags & FC_CONV_MLP_MATERIALIZE) && fc::conv_mlp_supported(d->l_in, d->l_edge, lout_key(d));
}
bool mlp_fuse_fwd(const fc_conv_desc* d) {
  return mlp_fusable(d) &&
         ((d->flags & FC_CONV_MLP_FUSE) || fc::conv_mlp_fwd_fused(d->l_in, d->l_edge, lout_key(d)));
}
bool mlp_fuse_vjp(const fc_conv_desc* d) { return mlp_fusable(d) && (d->flags & FC_CONV_MLP_FUSE); }

// Workspace of the convolution weighted by the radial network, for op 0
// (forward), 1 (VJP, any outputs) or 2 (VJP without the network's weight
// gradient; a forward on this layout follows the VJP's choice, so that the
// VJP can reuse what it leaves).  Fused (op 0 where mlp_fuse_fwd, op 2
// where mlp_fuse_vjp): (op 2) the
// convolution's VJP workspace, then the per-edge hidden rows hh [E][2][64].
// Materialised: (ops 1, 2) the VJP workspace, then h2 [64][E], w [E][P C],
// (ops 1, 2) w_bar [E][P C], the per-edge position terms [E][3] and the
// radial VJP scratch.
struct MlpWorkspace {
  bool fused;
  size_t conv_bytes;
  float *hh, *h2t, *w, *wbar, *q, *scratch;
  size_t bytes;
  MlpWorkspace(const fc_conv_desc* d, int op, void* base) {
    int P, nin, nout;
    layout(d, &P, &nin, &nout);
    const size_t E = d->n_edges, PC = (size_t)P * d->channels;
    fused = op == 0 ? mlp_fuse_fwd(d) : op == 2 && mlp_fuse_vjp(d);
    const bool vjp = op != 0;
    conv_bytes = vjp ? fc::VjpWorkspace(d->n_nodes, d->n_edges, d->channels, nin, P, false, nullptr).bytes : 0;
    char* p = static_cast<char*>(base);
    size_t off = conv_bytes;
    auto take = [&](size_t floats) {
      float* r = reinterpret_cast<float*>(p + off);
      off += fc::align256(floats * sizeof(float));
      return r;
    };
    hh = h2t = w = wbar = q = scratch = nullptr;
    if (fused) {
      // (at least h2 [64][E] of fc_radial_mlp, which takes the op 0 bytes)
      hh = take(std::max(E * fc::kRadRow, (size_t)fc::radial_ld(d->n_edges) * fc::kRadHidden));
    } else {
      h2t = take((size_t)fc::radial_ld(d->n_edges) * fc::kRadHidden);
      w = take(E * PC);
      wbar = vjp ? take(E * PC) : nullptr;
      q = vjp ? take(E * 3) : nullptr;
      scratch = vjp ? take(fc::radial_vjp_scratch_floats(d->n_edges, P, d->channels)) : nullptr;
    }
    bytes = off;
  }
};

const float* mlp_w3(const float* mlp_w) {
  return mlp_w + (size_t)fc::kRadFeat * fc::kRadHidden + (size_t)fc::kRadHidden * fc::kRadHidden;
}

fc::RadialArgs radial_args(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                           const float* mlp_w) {
  int P, nin, nout;
  layout(d, &P, &nin, &nout);
  return fc::RadialArgs{d->n_nodes, d->n_edges, P, d->channels, d->r_cut, g->rowptr, g->sender, g->receiver,
                        g->t_rowptr, g->t_edge, pos, shift, mlp_w};
}

// The convolution weighted by the radial network, forward and VJP, on a
// workspace laid out by MlpWorkspace; with have_w the VJP reuses the hidden
// rows (fused) or h2 and w (materialised) left in it by a forward on the
// same workspace.  The fused VJP gives no network weight gradient (the
// caller asks for the op 1 layout, which is materialised, to get one).
void mlp_conv_forward(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift, const float* x,
                      const float* mlp_w, float* z, const MlpWorkspace& ws, hipStream_t stream) {
  const fc::RadialArgs ra = radial_args(d, g, pos, shift, mlp_w);
  if (ws.fused) {
    fc::launch_radial_hidden_rows(ra, ws.hh, stream);
    fc::ConvArgs a = make_args(d, g, pos, shift, x, mlp_w3(mlp_w));
    a.mlp_h = ws.hh;
    a.z = z;
    fc::conv_mlp_dispatch(0, d->l_in, d->l_edge, lout_key(d), a, stream);
    return;
  }
  fc::launch_radial_hidden(ra, ws.h2t, stream);
  fc::launch_radial_out(ra, ws.h2t, ws.w, stream);
  fc::ConvArgs a = make_args(d, g, pos, shift, x, nullptr);
  a.w_edge = d->n_edges > 0 ? ws.w : x;   // never read without edges
  a.z = z;
  fc::conv_dispatch(0, d->l_in, d->l_edge, lout_key(d), a, stream);
}

void mlp_conv_vjp(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift, const float* x,
                  const float* mlp_w, const float* g_z, float* x_grad, float* pos_grad, float* mlp_w_grad,
                  const MlpWorkspace& ws, void* conv_ws, bool have_w, hipStream_t stream) {
  const fc::RadialArgs ra = radial_args(d, g, pos, shift, mlp_w);
  if (ws.fused) {
    if (!have_w) fc::launch_radial_hidden_rows(ra, ws.hh, stream);
    fc::ConvArgs a = make_args(d, g, pos, shift, x, mlp_w3(mlp_w));
    a.mlp_h = ws.hh;
    a.g = g_z;
    a.x_bar = x_grad;
    a.pos_bar = pos_grad;
    a.rbar = static_cast<float*>(conv_ws);
    fc::conv_mlp_dispatch(1, d->l_in, d->l_edge, lout_key(d), a, stream);
    return;
  }
  const bool radial = pos_grad || mlp_w_grad;
  if (!have_w) {
    fc::launch_radial_hidden(ra, ws.h2t, stream);
    fc::launch_radial_out(ra, ws.h2t, ws.w, stream);
  }
  fc::ConvArgs a = make_args(d, g, pos, shift, x, nullptr);
  a.w_edge = d->n_edges > 0 ? ws.w : x;
  a.w_edge_bar = (radial && d->n_edges > 0) ? ws.wbar : nullptr;
  a.g = g_z;
  a.x_bar = x_grad;
  a.pos_bar = pos_grad;
  a.rbar = static_cast<float*>(conv_ws);
  if (x_grad || pos_grad || a.w_edge_bar) fc::conv_dispatch(1, d->l_in, d->l_edge, lout_key(d), a, stream);
  if (radial) fc::launch_radial_vjp(ra, ws.h2t, ws.wbar, ws.q, pos_grad, mlp_w_grad, ws.scratch, stream);
}

fc_status check_norm(const fc_norm_desc* d) {
  if (!d) return fail(FC_ERR_INVALID_ARGUMENT, "norm descriptor is NULL");
  if (d->n_nodes < 1) return fail(FC_ERR_INVALID_ARGUMENT, "norm: n_nodes must be >= 1 (got %d)", d->n_nodes);
  if (d->channels < 1) return fail(FC_ERR_INVALID_ARGUMENT, "norm: channels must be >= 1 (got %d)", d->channels);
  if (d->channels > fc::kNormMaxChannels)
    return fail(FC_ERR_UNSUPPORTED, "norm: channels above %d are not supported", fc::kNormMaxChannels);
  if (d->l_max < 0) return fail(FC_ERR_INVALID_ARGUMENT, "norm: l_max must be >= 0");
  if (d->l_max > fc::kNormMaxRank) return fail(FC_ERR_UNSUPPORTED, "norm: l_max above 5 is not supported");
  if (!(d->eps >= 0.f) || !std::isfinite(d->eps))
    return fail(FC_ERR_INVALID_ARGUMENT, "norm: eps must be >= 0 and finite");
  return FC_OK;
}

fc_status ladder_plan(const fc_ladder_desc* d, fc::LadderPlan* p) {
  if (!d) return fail(FC_ERR_INVALID_ARGUMENT, "ladder descriptor is NULL");
  if (d->n_nodes < 1) return fail(FC_ERR_INVALID_ARGUMENT, "ladder: n_nodes must be >= 1");
  if (d->channels < 32 || d->channels > 512 || d->channels % 32 != 0)
    return fail(FC_ERR_UNSUPPORTED, "ladder: channels must be a multiple of 32 in [32, 512] (got %d)", d->channels);
  if (d->variant != FC_LADDER_FULL && d->variant != FC_LADDER_PATH_REDUCED)
    return fail(FC_ERR_INVALID_ARGUMENT, "ladder: unknown variant %d", d->variant);
  if (d->order < 1) return fail(FC_ERR_INVALID_ARGUMENT, "ladder: order must be >= 1");
  if (d->order > 8) return fail(FC_ERR_UNSUPPORTED, "ladder: order above 8 is not supported");
  if (d->l_a < 0 || d->l_prod < 0 || d->l_out < 0) return fail(FC_ERR_INVALID_ARGUMENT, "ladder: negative rank");
  if (d->l_a != d->l_prod || d->l_prod < 1 || d->l_prod > 4 || d->l_out > d->l_prod)
    return fail(FC_ERR_UNSUPPORTED, "ladder: the library needs l_a == l_prod in 1..4 and l_out <= l_prod");
  // the mixing GEMMs index node rows n (2l + 1) + c, divided exactly by
  // 2l + 1 with a multiply-high reciprocal, which holds below 2^26
  if ((int64_t)d->n_nodes * (2 * d->l_prod + 1) >= (int64_t(1) << 26))
    return fail(FC_ERR_UNSUPPORTED, "ladder: n_nodes * (2 l_prod + 1) = %lld reaches 2^26, the GEMM row index range",
                (long long)d->n_nodes * (2 * d->l_prod + 1));
  *p = fc::LadderPlan{d->n_nodes, d->channels, d->l_a, d->l_prod, d->l_out, d->order, d->variant};
  return FC_OK;
}

fc_status check_vjp_args(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                         const float* x, const float* radial_w, const float* g_z, const float* x_grad,
                         const float* pos_grad, const float* radial_w_grad) {
  if (fc_status s = check_desc(d)) return s;
  if (!g || !g->rowptr || !g->t_rowptr || (d->n_edges > 0 && (!g->sender || !g->receiver || !g->t_edge)))
    return fail(FC_ERR_INVALID_ARGUMENT, "VJP needs the full graph (run fc_graph_transpose first)");
  if (!pos || !x || !radial_w || !g_z) return fail(FC_ERR_INVALID_ARGUMENT, "VJP: NULL pos, x, radial_w or g_z");
  if (!x_grad && !pos_grad && !radial_w_grad) return fail(FC_ERR_INVALID_ARGUMENT, "VJP: no output requested");
  if (misaligned(pos, 4) || misaligned(x, 4) || misaligned(radial_w, 4) || misaligned(g_z, 4) ||
      misaligned(x_grad, 4) || misaligned(pos_grad, 4) || misaligned(radial_w_grad, 4) || misaligned(shift, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "VJP: arrays must be 4-byte aligned");
  return FC_OK;
}

// The VJP launches on a checked request; `workspace` holds at least the
// VjpWorkspace layout (its radial-weight partials only when radial_w_grad is
// requested).  The kernels write every workspace slot they later read, so
// its initial contents do not matter.
fc_status run_vjp(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift, const float* x,
                  const float* radial_w, const float* g_z, float* x_grad, float* pos_grad, float* radial_w_grad,
                  void* workspace, hipStream_t stream) {
  fc::ConvArgs a = make_args(d, g, pos, shift, x, radial_w);
  a.g = g_z;
  a.x_bar = x_grad;
  a.pos_bar = pos_grad;
  a.W_bar = radial_w_grad;
  a.rbar = static_cast<float*>(workspace);
  fc::conv_dispatch(1, d->l_in, d->l_edge, lout_key(d), a, stream);
  return check_launch("edge conv VJP");
}

// Device address of this GPU's copy of `scratch`, looked up once per device
// (with that device current) and kept.  In host code the array's name is
// only a stand-in for the symbol: kernels get this address, never the name.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

fc_status device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(FC_ERR_HIP, "allocation-free VJP: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(FC_ERR_UNSUPPORTED, "allocation-free VJP: device %d is beyond the %d the library tracks", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(FC_ERR_HIP, "allocation-free VJP: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FC_OK;
}

}  // namespace

extern "C" {

const char* fc_status_string(fc_status s) {
  switch (s) {
    case FC_OK: return "FC_OK";
    case FC_ERR_INVALID_ARGUMENT: return "FC_ERR_INVALID_ARGUMENT";
    case FC_ERR_UNSUPPORTED: return "FC_ERR_UNSUPPORTED";
    case FC_ERR_WORKSPACE: return "FC_ERR_WORKSPACE";
    case FC_ERR_HIP: return "FC_ERR_HIP";
  }
  return "FC_UNKNOWN_STATUS";
}

const char* fc_last_error_message(void) { return g_msg.c_str(); }

int32_t fc_abi_version(void) { return FC_ABI_VERSION; }

fc_status fc_conv_layout(const fc_conv_desc* d, int32_t* n_paths, int32_t* in_rows, int32_t* out_rows) {
  if (fc_status s = check_desc(d)) return s;
  int P, nin, nout;
  layout(d, &P, &nin, &nout);
  if (n_paths) *n_paths = P;
  if (in_rows) *in_rows = nin;
  if (out_rows) *out_rows = nout;
  return ok();
}

fc_status fc_conv_path(const fc_conv_desc* d, int32_t i, int32_t* l1, int32_t* l2, int32_t* L) {
  if (fc_status s = check_desc(d)) return s;
  int idx = 0;
  for (int LL = 0; LL <= d->l_out; ++LL)
    for (int a = 0; a <= d->l_in; ++a)
      for (int b = 0; b <= d->l_edge; ++b)
        if (path_ok(d, a, b, LL)) {
          if (idx == i) {
            if (l1) *l1 = a;
            if (l2) *l2 = b;
            if (L) *L = LL;
            return ok();
          }
          ++idx;
        }
  return fail(FC_ERR_INVALID_ARGUMENT, "path index %d out of range [0, %d)", i, idx);
}

size_t fc_graph_transpose_workspace_bytes(int32_t n_nodes) {
  return n_nodes > 0 ? fc::graph_transpose_ws(n_nodes) : 0;
}

fc_status fc_graph_transpose(int32_t n_nodes, int32_t n_edges, const int32_t* rowptr, const int32_t* sender,
                             int32_t* receiver, int32_t* t_rowptr, int32_t* t_edge, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  if (n_nodes < 1 || n_edges < 0) return fail(FC_ERR_INVALID_ARGUMENT, "need n_nodes >= 1, n_edges >= 0");
  if (!rowptr || !t_rowptr || (n_edges > 0 && (!sender || !receiver || !t_edge)))
    return fail(FC_ERR_INVALID_ARGUMENT, "graph transpose: NULL array");
  if (!workspace || workspace_bytes < fc::graph_transpose_ws(n_nodes))
    return fail(FC_ERR_WORKSPACE, "graph transpose needs %zu workspace bytes", fc::graph_transpose_ws(n_nodes));
  fc::graph_transpose(n_nodes, n_edges, rowptr, sender, receiver, t_rowptr, t_edge, workspace, stream);
  return check_launch("graph transpose");
}

fc_status fc_graph_validate(int32_t n_nodes, int32_t n_edges, const int32_t* h_rowptr, const int32_t* h_sender) {
  if (n_nodes < 1 || n_edges < 0) return fail(FC_ERR_INVALID_ARGUMENT, "need n_nodes >= 1, n_edges >= 0");
  if (!h_rowptr || (n_edges > 0 && !h_sender)) return fail(FC_ERR_INVALID_ARGUMENT, "NULL array");
  if (h_rowptr[0] != 0) return fail(FC_ERR_INVALID_ARGUMENT, "rowptr[0] = %d, expected 0", h_rowptr[0]);
  for (int u = 0; u < n_nodes; ++u)
    if (h_rowptr[u + 1] < h_rowptr[u])
      return fail(FC_ERR_INVALID_ARGUMENT, "rowptr decreases at node %d", u);
  if (h_rowptr[n_nodes] != n_edges)
    return fail(FC_ERR_INVALID_ARGUMENT, "rowptr[N] = %d, expected E = %d", h_rowptr[n_nodes], n_edges);
  for (int e = 0; e < n_edges; ++e)
    if (h_sender[e] < 0 || h_sender[e] >= n_nodes)
      return fail(FC_ERR_INVALID_ARGUMENT, "sender[%d] = %d out of range", e, h_sender[e]);
  return ok();
}

namespace {
// VJP-of-VJP workspace: the VJP workspace, then (weight cotangent given
// with x / pos cotangents) the forward and VJP taken with the weight
// cotangent as weights, [N][out_rows][C], [N][in_rows][C] and [N][3].
struct VVWorkspace {
  fc::VjpWorkspace vjp;
  float *g_lin, *x_lin, *p_lin;
  size_t bytes;
  VVWorkspace(const fc_conv_desc* d, int P, int nin, int nout, void* base)
      : vjp(d->n_nodes, d->n_edges, d->channels, nin, P, true, base) {
    const size_t N = d->n_nodes, C = d->channels;
    char* p = static_cast<char*>(base);
    size_t off = vjp.bytes;
    g_lin = reinterpret_cast<float*>(p + off);
    off += fc::align256(N * nout * C * sizeof(float));
    x_lin = reinterpret_cast<float*>(p + off);
    off += fc::align256(N * nin * C * sizeof(float));
    p_lin = reinterpret_cast<float*>(p + off);
    off += fc::align256(N * 3 * sizeof(float));
    bytes = off;
    if (!base) g_lin = x_lin = p_lin = nullptr;
  }
};
}  // namespace

size_t fc_edge_conv_workspace_bytes(const fc_conv_desc* d, int32_t op) {
  if (check_desc(d) != FC_OK) return 0;
  if (op == 1 || op == 2) {
    int P, nin, nout;
    layout(d, &P, &nin, &nout);
    if (op == 2) return VVWorkspace(d, P, nin, nout, nullptr).bytes;
    const fc::VjpWorkspace w(d->n_nodes, d->n_edges, d->channels, nin, P, true, nullptr);
    return w.bytes;
  }
  return 0;
}

fc_status fc_edge_conv_fwd(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                           const float* x, const float* radial_w, float* z, hipStream_t stream) {
  if (fc_status s = check_desc(d)) return s;
  if (!g || !g->rowptr || (d->n_edges > 0 && !g->sender))
    return fail(FC_ERR_INVALID_ARGUMENT, "forward needs graph rowptr and sender");
  if (!pos || !x || !radial_w || !z) return fail(FC_ERR_INVALID_ARGUMENT, "forward: NULL pos, x, radial_w or z");
  if (misaligned(pos, 4) || misaligned(x, 4) || misaligned(radial_w, 4) || misaligned(z, 4) ||
      misaligned(shift, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "forward: arrays must be 4-byte aligned");
  fc::ConvArgs a = make_args(d, g, pos, shift, x, radial_w);
  a.z = z;
  fc::conv_dispatch(0, d->l_in, d->l_edge, lout_key(d), a, stream);
  return check_launch("edge conv forward");
}

fc_status fc_edge_conv_vjp(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                           const float* x, const float* radial_w, const float* g_z, float* x_grad,
                           float* pos_grad, float* radial_w_grad, void* workspace, size_t workspace_bytes,
                           hipStream_t stream) {
  if (fc_status s = check_vjp_args(d, g, pos, shift, x, radial_w, g_z, x_grad, pos_grad, radial_w_grad)) return s;
  const size_t need = fc_edge_conv_workspace_bytes(d, 1);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(FC_ERR_WORKSPACE, "VJP needs %zu workspace bytes", need);
  return run_vjp(d, g, pos, shift, x, radial_w, g_z, x_grad, pos_grad, radial_w_grad, workspace, stream);
}

fc_status fc_edge_conv_vjp_noalloc(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                                   const float* x, const float* radial_w, const float* g_z, float* x_grad,
                                   float* pos_grad, float* radial_w_grad, hipStream_t stream) {
  if (fc_status s = check_vjp_args(d, g, pos, shift, x, radial_w, g_z, x_grad, pos_grad, radial_w_grad)) return s;
  int P, nin, nout;
  layout(d, &P, &nin, &nout);
  // the partial radial-weight gradients come last in the layout: without
  // radial_w_grad the call needs only the part before them
  const size_t need = fc::VjpWorkspace(d->n_nodes, d->n_edges, d->channels, nin, P, radial_w_grad != nullptr,
                                       nullptr).bytes;
  if (need > kNoAllocScratchBytes)
    return fail(FC_ERR_WORKSPACE,
                "allocation-free VJP: this call needs %zu scratch bytes, above the %zu bytes the library holds per "
                "GPU (use fc_edge_conv_vjp with a caller workspace)",
                need, kNoAllocScratchBytes);
  void* ptr = nullptr;
  if (fc_status s = device_scratch(&ptr)) return s;
  return run_vjp(d, g, pos, shift, x, radial_w, g_z, x_grad, pos_grad, radial_w_grad, ptr, stream);
}

fc_status fc_edge_conv_fwd_w(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                             const float* x, const float* w, float* z, hipStream_t stream) {
  if (fc_status s = check_desc(d)) return s;
  if (!g || !g->rowptr || (d->n_edges > 0 && !g->sender))
    return fail(FC_ERR_INVALID_ARGUMENT, "explicit-weight forward needs graph rowptr and sender");
  if (!pos || !x || !z || (d->n_edges > 0 && !w))
    return fail(FC_ERR_INVALID_ARGUMENT, "explicit-weight forward: NULL pos, x, w or z");
  if (misaligned(pos, 4) || misaligned(x, 4) || misaligned(w, 4) || misaligned(z, 4) || misaligned(shift, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "explicit-weight forward: arrays must be 4-byte aligned");
  fc::ConvArgs a = make_args(d, g, pos, shift, x, nullptr);
  a.w_edge = w;
  a.z = z;
  if (d->n_edges == 0) {
    // no edge: z is zero (launch with a dummy weight pointer, nothing reads it)
    a.w_edge = x;
  }
  fc::conv_dispatch(0, d->l_in, d->l_edge, lout_key(d), a, stream);
  return check_launch("explicit-weight edge conv forward");
}

fc_status fc_edge_conv_vjp_w(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                             const float* x, const float* w, const float* g_z, float* x_grad, float* pos_grad,
                             float* w_grad, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (fc_status s = check_desc(d)) return s;
  if (!g || !g->rowptr || !g->t_rowptr || (d->n_edges > 0 && (!g->sender || !g->receiver || !g->t_edge)))
    return fail(FC_ERR_INVALID_ARGUMENT, "VJP needs the full graph (run fc_graph_transpose first)");
  if (!pos || !x || !g_z || (d->n_edges > 0 && !w))
    return fail(FC_ERR_INVALID_ARGUMENT, "explicit-weight VJP: NULL pos, x, w or g_z");
  if (!x_grad && !pos_grad && !w_grad) return fail(FC_ERR_INVALID_ARGUMENT, "explicit-weight VJP: no output requested");
  if (misaligned(pos, 4) || misaligned(x, 4) || misaligned(w, 4) || misaligned(g_z, 4) || misaligned(x_grad, 4) ||
      misaligned(pos_grad, 4) || misaligned(w_grad, 4) || misaligned(shift, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "explicit-weight VJP: arrays must be 4-byte aligned");
  const size_t need = fc_edge_conv_workspace_bytes(d, 1);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(FC_ERR_WORKSPACE, "explicit-weight VJP needs %zu workspace bytes", need);
  fc::ConvArgs a = make_args(d, g, pos, shift, x, nullptr);
  a.w_edge = d->n_edges > 0 ? w : x;   // never read without edges
  a.w_edge_bar = d->n_edges > 0 ? w_grad : nullptr;
  a.g = g_z;
  a.x_bar = x_grad;
  a.pos_bar = pos_grad;
  a.rbar = static_cast<float*>(workspace);
  fc::conv_dispatch(1, d->l_in, d->l_edge, lout_key(d), a, stream);
  return check_launch("explicit-weight edge conv VJP");
}

fc_status fc_edge_conv_vjp_vjp(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                               const float* x, const float* radial_w, const float* g_z, const float* v_x,
                               const float* v_pos, const float* v_radial_w, float* g_hat, float* x_hat,
                               float* pos_hat, float* radial_w_hat, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  if (fc_status s = check_desc(d)) return s;
  if (!fc::conv_vv_supported(d->l_in, d->l_edge, lout_key(d)))
    return fail(FC_ERR_UNSUPPORTED, "VJP-of-VJP is not instantiated for (l_in, l_edge, l_out) = (%d, %d, %d)",
                d->l_in, d->l_edge, d->l_out);
  if (!g_hat && !x_hat && !pos_hat && !radial_w_hat)
    return fail(FC_ERR_INVALID_ARGUMENT, "VJP-of-VJP: no output requested");
  if (!g || !g->rowptr || (d->n_edges > 0 && !g->sender))
    return fail(FC_ERR_INVALID_ARGUMENT, "VJP-of-VJP needs graph rowptr and sender");
  if ((x_hat || pos_hat) && (!g->t_rowptr || (d->n_edges > 0 && (!g->receiver || !g->t_edge))))
    return fail(FC_ERR_INVALID_ARGUMENT, "VJP-of-VJP: x_hat/pos_hat need the graph transpose");
  if (!pos || !x || !radial_w || ((x_hat || pos_hat || radial_w_hat) && !g_z))
    return fail(FC_ERR_INVALID_ARGUMENT, "VJP-of-VJP: NULL pos, x, radial_w or g_z");
  if (misaligned(pos, 4) || misaligned(x, 4) || misaligned(radial_w, 4) || misaligned(g_z, 4) ||
      misaligned(v_x, 4) || misaligned(v_pos, 4) || misaligned(v_radial_w, 4) || misaligned(g_hat, 4) ||
      misaligned(x_hat, 4) || misaligned(pos_hat, 4) || misaligned(radial_w_hat, 4) || misaligned(shift, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "VJP-of-VJP: arrays must be 4-byte aligned");
  // second-order part (x / pos cotangents) and the part linear in the
  // weight cotangent
  const bool second = v_x || v_pos || !v_radial_w;
  const bool lin = v_radial_w && (g_hat || x_hat || pos_hat);
  const size_t need = fc_edge_conv_workspace_bytes(d, 2);
  if ((x_hat || pos_hat || radial_w_hat || (lin && second)) && need > 0 && (!workspace || workspace_bytes < need))
    return fail(FC_ERR_WORKSPACE, "VJP-of-VJP needs %zu workspace bytes", need);
  int P, nin, nout;
  layout(d, &P, &nin, &nout);
  const VVWorkspace ws(d, P, nin, nout, workspace);
  const size_t N = d->n_nodes, C = d->channels;
  if (second) {
    fc::ConvArgs a = make_args(d, g, pos, shift, x, radial_w);
    a.g = g_z;
    a.v_x = v_x;
    a.v_pos = v_pos;
    a.g_hat = g_hat;
    a.x_bar = x_hat;
    a.pos_bar = pos_hat;
    a.W_bar = radial_w_hat;
    a.rbar = static_cast<float*>(workspace);
    fc::conv_dispatch(2, d->l_in, d->l_edge, lout_key(d), a, stream);
  } else if (radial_w_hat) {
    // W_bar does not depend on the radial weights: no x / pos cotangent, no W_hat
    fc::launch_zero((size_t)d->n_basis * P * C, radial_w_hat, stream);
  }
  if (lin) {
    // z, x_bar and pos_bar are linear in the radial weights: the weight
    // cotangent adds the forward and the VJP taken with v_radial_w as the
    // weights (written straight to the outputs when there is no
    // second-order part, else added to it)
    if (g_hat) {
      fc::ConvArgs a = make_args(d, g, pos, shift, x, v_radial_w);
      a.z = second ? ws.g_lin : g_hat;
      fc::conv_dispatch(0, d->l_in, d->l_edge, lout_key(d), a, stream);
      if (second) fc::launch_add(N * nout * C, ws.g_lin, g_hat, stream);
    }
    if (x_hat || pos_hat) {
      fc::ConvArgs a = make_args(d, g, pos, shift, x, v_radial_w);
      a.g = g_z;
      a.x_bar = x_hat ? (second ? ws.x_lin : x_hat) : nullptr;
      a.pos_bar = pos_hat ? (second ? ws.p_lin : pos_hat) : nullptr;
      a.rbar = static_cast<float*>(workspace);
      fc::conv_dispatch(1, d->l_in, d->l_edge, lout_key(d), a, stream);
      if (second && x_hat) fc::launch_add(N * nin * C, ws.x_lin, x_hat, stream);
      if (second && pos_hat) fc::launch_add(N * 3, ws.p_lin, pos_hat, stream);
    }
  }
  return check_launch("edge conv VJP-of-VJP");
}

fc_status fc_edge_conv_vjp_vjp_w(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                                 const float* x, const float* w, const float* g_z, const float* v_x,
                                 const float* v_pos, const float* v_w, float* g_hat, float* x_hat, float* pos_hat,
                                 float* w_hat, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (fc_status s = check_desc(d)) return s;
  if (!fc::conv_vv_w_supported(d->l_in, d->l_edge, lout_key(d)))
    return fail(FC_ERR_UNSUPPORTED, "VJP-of-VJP is not instantiated for (l_in, l_edge, l_out) = (%d, %d, %d)",
                d->l_in, d->l_edge, d->l_out);
  if (!g_hat && !x_hat && !pos_hat && !w_hat)
    return fail(FC_ERR_INVALID_ARGUMENT, "explicit-weight VJP-of-VJP: no output requested");
  if (!g || !g->rowptr || (d->n_edges > 0 && !g->sender))
    return fail(FC_ERR_INVALID_ARGUMENT, "explicit-weight VJP-of-VJP needs graph rowptr and sender");
  const bool back = x_hat || pos_hat || w_hat;
  if (back && (!g->t_rowptr || (d->n_edges > 0 && (!g->receiver || !g->t_edge))))
    return fail(FC_ERR_INVALID_ARGUMENT, "explicit-weight VJP-of-VJP: x_hat/pos_hat/w_hat need the graph transpose");
  if (!pos || !x || (d->n_edges > 0 && !w) || (back && !g_z))
    return fail(FC_ERR_INVALID_ARGUMENT, "explicit-weight VJP-of-VJP: NULL pos, x, w or g_z");
  if (misaligned(pos, 4) || misaligned(x, 4) || misaligned(w, 4) || misaligned(g_z, 4) || misaligned(v_x, 4) ||
      misaligned(v_pos, 4) || misaligned(v_w, 4) || misaligned(g_hat, 4) || misaligned(x_hat, 4) ||
      misaligned(pos_hat, 4) || misaligned(w_hat, 4) || misaligned(shift, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "explicit-weight VJP-of-VJP: arrays must be 4-byte aligned");
  const size_t need = fc_edge_conv_workspace_bytes(d, 1);
  if (back && need > 0 && (!workspace || workspace_bytes < need))
    return fail(FC_ERR_WORKSPACE, "explicit-weight VJP-of-VJP needs %zu workspace bytes", need);
  fc::ConvArgs a = make_args(d, g, pos, shift, x, nullptr);
  const bool edges = d->n_edges > 0;
  a.w_edge = edges ? w : x;   // never read without edges
  a.v_w_edge = edges ? v_w : nullptr;
  a.w_edge_bar = edges ? w_hat : nullptr;
  a.g = g_z;
  a.v_x = v_x;
  a.v_pos = v_pos;
  a.g_hat = g_hat;
  a.x_bar = x_hat;
  a.pos_bar = pos_hat;
  a.rbar = static_cast<float*>(workspace);
  fc::conv_vv_w_dispatch(d->l_in, d->l_edge, lout_key(d), a, stream);
  return check_launch("explicit-weight edge conv VJP-of-VJP");
}

fc_status fc_ladder_layout(const fc_ladder_desc* d, size_t* n_weight_floats, size_t* n_saved_floats) {
  fc::LadderPlan p;
  if (fc_status s = ladder_plan(d, &p)) return s;
  if (n_weight_floats) *n_weight_floats = p.weight_floats();
  if (n_saved_floats) *n_saved_floats = p.saved_floats();
  return ok();
}

fc_status fc_ladder_weight_block(const fc_ladder_desc* d, int32_t i, size_t* offset, int32_t* rows, int32_t* cols,
                                 int32_t* kind) {
  fc::LadderPlan p;
  if (fc_status s = ladder_plan(d, &p)) return s;
  struct Blk { size_t off; int r, c, k; };
  Blk blk[64];
  int n = 0;
  const int C = p.C;
  if (p.variant == FC_LADDER_FULL) {
    for (int l = 0; l <= p.lq(1); ++l) blk[n++] = {p.w_full(1, l), C, C, 0};
    for (int q = 2; q <= p.order; ++q)
      for (int L = 0; L <= p.lq(q); ++L)
        if (p.paths(q, L)) blk[n++] = {p.w_full(q, L), C, p.paths(q, L) * C, 0};
  } else {
    blk[n++] = {p.w_a(1), p.lq(1) + 1, C, 1};
    for (int q = 2; q <= p.order; ++q) blk[n++] = {p.w_a(q), p.paths(q), C, 1};
    for (int L = 0; L <= p.lout; ++L) blk[n++] = {p.w_final(L), C, C, 0};
  }
  if (i < 0 || i >= n) return fail(FC_ERR_INVALID_ARGUMENT, "weight block %d out of range [0, %d)", i, n);
  if (offset) *offset = blk[i].off;
  if (rows) *rows = blk[i].r;
  if (cols) *cols = blk[i].c;
  if (kind) *kind = blk[i].k;
  return ok();
}

size_t fc_ladder_workspace_bytes(const fc_ladder_desc* d, int32_t op) {
  fc::LadderPlan p;
  if (ladder_plan(d, &p) != FC_OK) return 0;
  if (op == 2) return sizeof(float) * p.vv_ws_floats();
  return sizeof(float) * (op == 1 ? p.vjp_ws_floats() : p.fwd_ws_floats());
}

fc_status fc_node_ladder_fwd(const fc_ladder_desc* d, const float* A, const float* weights, float* z,
                             float* saved, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  fc::LadderPlan p;
  if (fc_status s = ladder_plan(d, &p)) return s;
  if (!A || !weights || !z) return fail(FC_ERR_INVALID_ARGUMENT, "ladder forward: NULL A, weights or z");
  if (misaligned(A, 4) || misaligned(weights, 4) || misaligned(z, 4) || misaligned(saved, 4) ||
      misaligned(workspace, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "ladder forward: arrays must be 4-byte aligned");
  const size_t need = fc_ladder_workspace_bytes(d, 0);
  if (!workspace || workspace_bytes < need)
    return fail(FC_ERR_WORKSPACE, "ladder forward needs %zu workspace bytes", need);
  fc::ladder_forward(p, A, weights, z, saved, static_cast<float*>(workspace), stream);
  return check_launch("ladder forward");
}

fc_status fc_node_ladder_vjp(const fc_ladder_desc* d, const float* A, const float* weights, const float* saved,
                             const float* g_z, float* A_grad, float* weights_grad, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  fc::LadderPlan p;
  if (fc_status s = ladder_plan(d, &p)) return s;
  if (!A || !weights || !g_z || !A_grad)
    return fail(FC_ERR_INVALID_ARGUMENT, "ladder VJP: NULL A, weights, g_z or A_grad");
  if (p.order > 1 && !saved) return fail(FC_ERR_INVALID_ARGUMENT, "ladder VJP: saved states required (order > 1)");
  if (misaligned(A, 4) || misaligned(weights, 4) || misaligned(saved, 4) || misaligned(g_z, 4) ||
      misaligned(A_grad, 4) || misaligned(weights_grad, 4) || misaligned(workspace, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "ladder VJP: arrays must be 4-byte aligned");
  const size_t need = fc_ladder_workspace_bytes(d, 1);
  if (!workspace || workspace_bytes < need)
    return fail(FC_ERR_WORKSPACE, "ladder VJP needs %zu workspace bytes", need);
  fc::ladder_vjp(p, A, weights, saved, g_z, A_grad, weights_grad, static_cast<float*>(workspace), stream);
  return check_launch("ladder VJP");
}

fc_status fc_node_ladder_vjp_vjp(const fc_ladder_desc* d, const float* A, const float* weights, const float* saved,
                                 const float* g_z, const float* v_A, const float* v_weights, float* g_hat,
                                 float* A_hat, float* weights_hat, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  fc::LadderPlan p;
  if (fc_status s = ladder_plan(d, &p)) return s;
  if (!g_hat && !A_hat && !weights_hat) return fail(FC_ERR_INVALID_ARGUMENT, "ladder VJP-of-VJP: no output requested");
  if (!A || !weights || ((A_hat || weights_hat) && !g_z))
    return fail(FC_ERR_INVALID_ARGUMENT, "ladder VJP-of-VJP: NULL A, weights or g_z");
  if (p.order > 1 && !saved)
    return fail(FC_ERR_INVALID_ARGUMENT, "ladder VJP-of-VJP: saved states required (order > 1)");
  if (misaligned(A, 4) || misaligned(weights, 4) || misaligned(saved, 4) || misaligned(g_z, 4) ||
      misaligned(v_A, 4) || misaligned(v_weights, 4) || misaligned(g_hat, 4) || misaligned(A_hat, 4) ||
      misaligned(weights_hat, 4) || misaligned(workspace, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "ladder VJP-of-VJP: arrays must be 4-byte aligned");
  const size_t need = fc_ladder_workspace_bytes(d, 2);
  if (!workspace || workspace_bytes < need)
    return fail(FC_ERR_WORKSPACE, "ladder VJP-of-VJP needs %zu workspace bytes", need);
  fc::ladder_vjp_vjp(p, A, weights, saved, g_z, v_A, v_weights, g_hat, A_hat, weights_hat,
                     static_cast<float*>(workspace), stream);
  return check_launch("ladder VJP-of-VJP");
}

}  // extern "C"

namespace {

struct BlockLayout {
  size_t A, z, saved, lws, gz, Ab, wsc, cws, parts, total;   // byte offsets / total
  size_t n_w;   // radial weight floats (wsc holds a scaled and a negated copy)
};

fc_status block_layout(const fc_conv_desc* cd, const fc_ladder_desc* ld, BlockLayout* L) {
  if (fc_status s = check_desc(cd)) return s;
  fc::LadderPlan p;
  if (fc_status s = ladder_plan(ld, &p)) return s;
  if (cd->l_in != 0) return fail(FC_ERR_UNSUPPORTED, "block: the convolution needs scalar senders (l_in == 0)");
  if (cd->l_out != ld->l_a || cd->channels != ld->channels || cd->n_nodes != ld->n_nodes)
    return fail(FC_ERR_INVALID_ARGUMENT, "block: conv l_out/channels/nodes must match ladder l_a/channels/nodes");
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  const size_t N = cd->n_nodes, C = cd->channels;
  const size_t nA = (size_t)(cd->l_out + 1) * (cd->l_out + 1), nz = (size_t)(ld->l_out + 1) * (ld->l_out + 1);
  size_t o = 0;
  L->A = o;      o += al(N * nA * C * 4);
  L->z = o;      o += al(N * nz * C * 4);
  L->saved = o;  o += al(p.saved_floats() * 4);
  L->lws = o;    o += al(std::max(p.fwd_ws_floats(), p.vjp_ws_floats()) * 4);
  L->gz = o;     o += al(N * nz * C * 4);
  L->Ab = o;     o += al(N * nA * C * 4);
  int P, nin, nout;
  layout(cd, &P, &nin, &nout);
  L->n_w = (size_t)cd->n_basis * P * C;
  L->wsc = o;    o += al(2 * L->n_w * 4);
  L->cws = o;    o += al(fc_edge_conv_workspace_bytes(cd, 1));
  L->parts = o;  o += al((size_t)fc::block_energy_parts(cd->n_nodes) * 8);
  L->total = o;
  return FC_OK;
}

// A full message-passing block: flat weight offsets (floats) and workspace
// (bytes), in the order
//   radial network | Mpre [C][C] | M [l+1][C][C] | R0 [C][C] |
//   gamma1 [l+1][C] | O [l+1][C][C] | ladder | R2 [C][C] | gamma2 [C] |
//   Wr1 [C][64] | Wr2 [64][64] | wr3 [64]
struct MsgLayout {
  size_t w_mlp, w_pre, w_M, w_R0, w_g1, w_O, w_lad, w_R2, w_g2, w_r1, w_r2, w_r3, n_weights;
  size_t a, m, n, y, A, Ab, nb, mb, hb, z, f, fb, ob, inv1, inv2, ea, saved, lws, cws, cws_bytes, parts, total;
};

fc_status msg_layout(const fc_conv_desc* cd, const fc_ladder_desc* ld, MsgLayout* L) {
  if (fc_status s = check_desc(cd)) return s;
  fc::LadderPlan p;
  if (fc_status s = ladder_plan(ld, &p)) return s;
  if (cd->l_in != 0 || cd->l_edge != cd->l_out ||
      (cd->flags & ~uint32_t(FC_CONV_MLP_MATERIALIZE | FC_CONV_MLP_FUSE)) != 0)
    return fail(FC_ERR_UNSUPPORTED,
                "message block: the convolution needs scalar senders, l_edge == l_out, natural parity, paths apart");
  if (ld->l_a != cd->l_out || ld->l_out != 0 || ld->channels != cd->channels || ld->n_nodes != cd->n_nodes)
    return fail(FC_ERR_INVALID_ARGUMENT,
                "message block: ladder l_a must equal the conv l_out, ladder l_out 0, equal channels and nodes");
  const size_t N = cd->n_nodes, C = cd->channels, le = cd->l_edge, R = (le + 1) * (le + 1);
  const size_t C2 = C * C, H = fc::kReadoutHidden;
  size_t o = 0;
  L->w_mlp = o; o += fc::radial_weight_floats((int)le + 1, (int)C);
  L->w_pre = o; o += C2;
  L->w_M = o;   o += (le + 1) * C2;
  L->w_R0 = o;  o += C2;
  L->w_g1 = o;  o += (le + 1) * C;
  L->w_O = o;   o += (le + 1) * C2;
  L->w_lad = o; o += p.weight_floats();
  L->w_R2 = o;  o += C2;
  L->w_g2 = o;  o += C;
  L->w_r1 = o;  o += C * H;
  L->w_r2 = o;  o += H * H;
  L->w_r3 = o;  o += H;
  L->n_weights = o;
  auto al = [](size_t floats) { return (floats * 4 + 255) / 256 * 256; };
  o = 0;
  size_t* big[] = {&L->a, &L->m, &L->n, &L->y, &L->A, &L->Ab, &L->nb, &L->mb};
  for (size_t* b : big) { *b = o; o += al(N * R * C); }
  size_t* small[] = {&L->hb, &L->z, &L->f, &L->fb, &L->ob};
  for (size_t* b : small) { *b = o; o += al(N * C); }
  L->inv1 = o;  o += al(N);
  L->inv2 = o;  o += al(N);
  L->ea = o;    o += al(N);
  L->saved = o; o += al(p.saved_floats());
  L->lws = o;   o += al(std::max(p.fwd_ws_floats(), p.vjp_ws_floats()));
  L->cws_bytes = fc_edge_conv_mlp_workspace_bytes(cd, 2);   // the VJP reuses the forward's rows in it
  L->cws = o;   o += (L->cws_bytes + 255) / 256 * 256;
  L->parts = o; o += (size_t)fc::block_energy_parts(cd->n_nodes) * 8;
  L->total = o;
  return FC_OK;
}

// Rank block l of [N][rows][C] as a GEMM view / output, and a [out][in]
// channel matrix applied to it (y = M x) or its transpose (x_bar = M^T y_bar).
fc::GView rank_view(const float* base, int rows, int l, int C) {
  return fc::GView{base + (size_t)l * l * C, 2 * l + 1, (long long)rows * C, (long long)C, 1, 1, 0, 0, 0};
}
fc::GOut rank_out(float* base, int rows, int l, int C, int acc) {
  return fc::GOut{base + (size_t)l * l * C, 2 * l + 1, (long long)rows * C, (long long)C, acc, 0};
}
fc::GemmProblem channel_map(int N, int C, const float* X, int xrows, int l, const float* Mat, bool transpose,
                            float* Y, int yrows, int yl, int acc) {
  fc::GemmProblem p{};
  p.M = N * (2 * l + 1);
  p.N = C;
  p.K = C;
  p.alpha = 1.f;
  p.A = rank_view(X, xrows, l, C);
  p.Bt = transpose ? fc::plain_view_t(Mat, C) : fc::plain_view(Mat, C);
  p.C = rank_out(Y, yrows, yl, C, acc);
  p.C2 = fc::no_out();
  p.ksplit = 1;
  return p;
}

}  // namespace

extern "C" {

size_t fc_block_workspace_bytes(const fc_conv_desc* conv, const fc_ladder_desc* lad) {
  BlockLayout L;
  return block_layout(conv, lad, &L) == FC_OK ? L.total : 0;
}

fc_status fc_block_energy_forces(const fc_conv_desc* cd, const fc_graph* g, const float* pos, const float* shift,
                                 const float* x, const float* radial_w, const fc_ladder_desc* ld,
                                 const float* ladder_w, float conv_scale, double* energy, float* e_atom,
                                 float* forces, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  BlockLayout L;
  if (fc_status s = block_layout(cd, ld, &L)) return s;
  if (!energy || !ladder_w) return fail(FC_ERR_INVALID_ARGUMENT, "block: NULL energy or ladder weights");
  if (!workspace || workspace_bytes < L.total)
    return fail(FC_ERR_WORKSPACE, "block needs %zu workspace bytes", L.total);
  char* w = static_cast<char*>(workspace);
  float* A = reinterpret_cast<float*>(w + L.A);
  float* z = reinterpret_cast<float*>(w + L.z);
  float* saved = reinterpret_cast<float*>(w + L.saved);
  float* lws = reinterpret_cast<float*>(w + L.lws);
  float* gz = reinterpret_cast<float*>(w + L.gz);
  float* Ab = reinterpret_cast<float*>(w + L.Ab);
  double* parts = reinterpret_cast<double*>(w + L.parts);
  fc::LadderPlan p;
  ladder_plan(ld, &p);
  const int N = cd->n_nodes, C = cd->channels;
  const int nz = (ld->l_out + 1) * (ld->l_out + 1);
  // the convolution is linear in its radial weights: the scale (and, for
  // the backward pass, the sign of F = -dE/dpos) goes into a copy of them
  float* Wpos = reinterpret_cast<float*>(w + L.wsc);
  float* Wneg = Wpos + L.n_w;
  if (!radial_w) return fail(FC_ERR_INVALID_ARGUMENT, "block: NULL radial weights");
  fc::block_scaled_weights(radial_w, L.n_w, conv_scale, Wpos, forces ? Wneg : nullptr, stream);
  if (fc_status s = fc_edge_conv_fwd(cd, g, pos, shift, x, Wpos, A, stream)) return s;
  fc::ladder_forward(p, A, ladder_w, z, saved, lws, stream);
  fc::block_energy(z, N, nz, C, e_atom, parts, energy, stream);
  if (forces) {
    fc::block_unit_cotangent(gz, N, nz, C, stream);
    fc::ladder_vjp(p, A, ladder_w, saved, gz, Ab, nullptr, lws, stream);
    if (fc_status s = fc_edge_conv_vjp(cd, g, pos, shift, x, Wneg, Ab, nullptr, forces, nullptr,
                                       w + L.cws, L.parts - L.cws, stream))
      return s;
  }
  return check_launch("block energy/forces");
}

fc_status fc_rms_norm_fwd(const fc_norm_desc* d, const float* x, const float* gamma, float* y, float* inv_scale,
                          hipStream_t stream) {
  if (fc_status s = check_norm(d)) return s;
  if (!x || !y) return fail(FC_ERR_INVALID_ARGUMENT, "norm forward: NULL x or y");
  if (misaligned(x, 4) || misaligned(gamma, 4) || misaligned(y, 4) || misaligned(inv_scale, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "norm forward: arrays must be 4-byte aligned");
  fc::launch_rms_norm_fwd(d->l_max, d->n_nodes, d->channels, d->eps, x, gamma, y, inv_scale, stream);
  return check_launch("RMS norm forward");
}

size_t fc_rms_norm_workspace_bytes(const fc_norm_desc* d) {
  if (check_norm(d) != FC_OK) return 0;
  return (size_t)fc::rms_norm_vjp_blocks(d->n_nodes) * (d->l_max + 1) * d->channels * sizeof(float);
}

fc_status fc_rms_norm_vjp(const fc_norm_desc* d, const float* x, const float* gamma, const float* inv_scale,
                          const float* g_y, float* x_grad, float* gamma_grad, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  if (fc_status s = check_norm(d)) return s;
  if (!x || !inv_scale || !g_y) return fail(FC_ERR_INVALID_ARGUMENT, "norm VJP: NULL x, inv_scale or g_y");
  if (!x_grad && !gamma_grad) return fail(FC_ERR_INVALID_ARGUMENT, "norm VJP: no output requested");
  if (misaligned(x, 4) || misaligned(gamma, 4) || misaligned(inv_scale, 4) || misaligned(g_y, 4) ||
      misaligned(x_grad, 4) || misaligned(gamma_grad, 4) || misaligned(workspace, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "norm VJP: arrays must be 4-byte aligned");
  const size_t need = fc_rms_norm_workspace_bytes(d);
  if (gamma_grad && (!workspace || workspace_bytes < need))
    return fail(FC_ERR_WORKSPACE, "norm VJP needs %zu workspace bytes for gamma_grad", need);
  fc::launch_rms_norm_vjp(d->l_max, d->n_nodes, d->channels, x, gamma, inv_scale, g_y, x_grad,
                          gamma_grad ? static_cast<float*>(workspace) : nullptr, gamma_grad, stream);
  return check_launch("RMS norm VJP");
}

size_t fc_radial_mlp_weight_floats(const fc_conv_desc* d) {
  if (check_desc(d) != FC_OK) return 0;
  int P, nin, nout;
  layout(d, &P, &nin, &nout);
  return fc::radial_weight_floats(P, d->channels);
}

size_t fc_edge_conv_mlp_workspace_bytes(const fc_conv_desc* d, int32_t op) {
  if (check_desc(d) != FC_OK || op < 0 || op > 2) return 0;
  return MlpWorkspace(d, op, nullptr).bytes;
}

fc_status fc_radial_mlp(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                        const float* mlp_w, float* w, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (fc_status s = check_desc(d)) return s;
  if (!g || (d->n_edges > 0 && (!g->sender || !g->receiver)))
    return fail(FC_ERR_INVALID_ARGUMENT, "radial MLP needs graph sender and receiver");
  if (!pos || !mlp_w || (d->n_edges > 0 && !w))
    return fail(FC_ERR_INVALID_ARGUMENT, "radial MLP: NULL pos, mlp_w or w");
  if (misaligned(pos, 4) || misaligned(shift, 4) || misaligned(mlp_w, 4) || misaligned(w, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "radial MLP: arrays must be 4-byte aligned");
  // h2 [64][E] at the start of the workspace (within the op 0 size, fused or not)
  const size_t need = fc::align256((size_t)fc::radial_ld(d->n_edges) * fc::kRadHidden * sizeof(float));
  if (!workspace || workspace_bytes < need)
    return fail(FC_ERR_WORKSPACE, "radial MLP needs %zu workspace bytes", need);
  float* h2t = static_cast<float*>(workspace);
  const fc::RadialArgs ra = radial_args(d, g, pos, shift, mlp_w);
  fc::launch_radial_hidden(ra, h2t, stream);
  fc::launch_radial_out(ra, h2t, w, stream);
  return check_launch("radial MLP");
}

fc_status fc_edge_conv_mlp_fwd(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                               const float* x, const float* mlp_w, float* z, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  if (fc_status s = check_desc(d)) return s;
  if (!g || !g->rowptr || (d->n_edges > 0 && (!g->sender || !g->receiver)))
    return fail(FC_ERR_INVALID_ARGUMENT, "MLP-weighted forward needs graph rowptr, sender and receiver");
  if (!pos || !x || !mlp_w || !z) return fail(FC_ERR_INVALID_ARGUMENT, "MLP-weighted forward: NULL pos, x, mlp_w or z");
  if (misaligned(pos, 4) || misaligned(shift, 4) || misaligned(x, 4) || misaligned(mlp_w, 4) || misaligned(z, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "MLP-weighted forward: arrays must be 4-byte aligned");
  const MlpWorkspace ws(d, 0, workspace);
  if (!workspace || workspace_bytes < ws.bytes)
    return fail(FC_ERR_WORKSPACE, "MLP-weighted forward needs %zu workspace bytes", ws.bytes);
  mlp_conv_forward(d, g, pos, shift, x, mlp_w, z, ws, stream);
  return check_launch("MLP-weighted edge conv forward");
}

fc_status fc_edge_conv_mlp_vjp(const fc_conv_desc* d, const fc_graph* g, const float* pos, const float* shift,
                               const float* x, const float* mlp_w, const float* g_z, float* x_grad, float* pos_grad,
                               float* mlp_w_grad, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (fc_status s = check_desc(d)) return s;
  if (!g || !g->rowptr || !g->t_rowptr || (d->n_edges > 0 && (!g->sender || !g->receiver || !g->t_edge)))
    return fail(FC_ERR_INVALID_ARGUMENT, "MLP-weighted VJP needs the full graph (run fc_graph_transpose first)");
  if (!pos || !x || !mlp_w || !g_z)
    return fail(FC_ERR_INVALID_ARGUMENT, "MLP-weighted VJP: NULL pos, x, mlp_w or g_z");
  if (!x_grad && !pos_grad && !mlp_w_grad) return fail(FC_ERR_INVALID_ARGUMENT, "MLP-weighted VJP: no output requested");
  if (misaligned(pos, 4) || misaligned(shift, 4) || misaligned(x, 4) || misaligned(mlp_w, 4) || misaligned(g_z, 4) ||
      misaligned(x_grad, 4) || misaligned(pos_grad, 4) || misaligned(mlp_w_grad, 4))
    return fail(FC_ERR_INVALID_ARGUMENT, "MLP-weighted VJP: arrays must be 4-byte aligned");
  const int op = mlp_w_grad ? 1 : 2;
  const MlpWorkspace ws(d, op, workspace);
  if (!workspace || workspace_bytes < ws.bytes)
    return fail(FC_ERR_WORKSPACE, "MLP-weighted VJP needs %zu workspace bytes (fc_edge_conv_mlp_workspace_bytes op %d)",
                ws.bytes, op);
  mlp_conv_vjp(d, g, pos, shift, x, mlp_w, g_z, x_grad, pos_grad, mlp_w_grad, ws, workspace, false, stream);
  return check_launch("MLP-weighted edge conv VJP");
}

size_t fc_message_block_weight_floats(const fc_conv_desc* conv, const fc_ladder_desc* lad) {
  MsgLayout L;
  return msg_layout(conv, lad, &L) == FC_OK ? L.n_weights : 0;
}

size_t fc_message_block_workspace_bytes(const fc_conv_desc* conv, const fc_ladder_desc* lad) {
  MsgLayout L;
  return msg_layout(conv, lad, &L) == FC_OK ? L.total : 0;
}

fc_status fc_message_block_energy_forces(const fc_conv_desc* cd, const fc_graph* g, const float* pos,
                                         const float* shift, const float* h0, const fc_ladder_desc* ld,
                                         const float* weights, float conv_scale, float eps, double* energy,
                                         float* e_atom, float* forces, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream) {
  MsgLayout L;
  if (fc_status s = msg_layout(cd, ld, &L)) return s;
  if (!g || !energy || !weights || !h0 || !pos)
    return fail(FC_ERR_INVALID_ARGUMENT, "message block: NULL graph, input or energy");
  if (!(eps >= 0.f) || !std::isfinite(eps) || !std::isfinite(conv_scale))
    return fail(FC_ERR_INVALID_ARGUMENT, "message block: eps must be >= 0 and finite");
  if (misaligned(pos, 4) || misaligned(shift, 4) || misaligned(h0, 4) || misaligned(weights, 4) ||
      misaligned(e_atom, 4) || misaligned(forces, 4) || misaligned(energy, 8))
    return fail(FC_ERR_INVALID_ARGUMENT, "message block: misaligned array");
  if (!workspace || workspace_bytes < L.total)
    return fail(FC_ERR_WORKSPACE, "message block needs %zu workspace bytes", L.total);
  if (forces && (!g->t_rowptr || (cd->n_edges > 0 && (!g->receiver || !g->t_edge))))
    return fail(FC_ERR_INVALID_ARGUMENT, "message block: forces need the full graph (run fc_graph_transpose first)");
  char* wb = static_cast<char*>(workspace);
  auto buf = [&](size_t off) { return reinterpret_cast<float*>(wb + off); };
  float *a = buf(L.a), *m = buf(L.m), *n = buf(L.n), *y = buf(L.y), *A = buf(L.A), *Ab = buf(L.Ab);
  float *nb = buf(L.nb), *mb = buf(L.mb), *hb = buf(L.hb), *z = buf(L.z), *f = buf(L.f), *fb = buf(L.fb);
  float* ob = buf(L.ob);
  float *inv1 = buf(L.inv1), *inv2 = buf(L.inv2), *ea = buf(L.ea), *saved = buf(L.saved), *lws = buf(L.lws);
  double* parts = reinterpret_cast<double*>(wb + L.parts);
  const float* W = weights;
  fc::LadderPlan p;
  ladder_plan(ld, &p);
  const int N = cd->n_nodes, C = cd->channels, le = cd->l_edge, R = (le + 1) * (le + 1);
  const float* lw = W + L.w_lad;
  auto chan = [&](const float* M, int l) { return M + (size_t)l * C * C; };

  if (cd->n_edges > 0 && (!g->rowptr || !g->sender || !g->receiver))
    return fail(FC_ERR_INVALID_ARGUMENT, "message block needs graph rowptr, sender and receiver");
  const MlpWorkspace mws(cd, 2, wb + L.cws);

  // ---- forward
  {  // hb = Mpre h0: the channel map of the sender features before the convolution
    fc::GemmGroup gg{};
    gg.prob[gg.count++] = channel_map(N, C, h0, 1, 0, W + L.w_pre, false, hb, 1, 0, 0);
    fc::gemm_group(gg, stream);
  }
  mlp_conv_forward(cd, g, pos, shift, hb, W + L.w_mlp, a, mws, stream);
  {  // m_l = conv_scale M_l a_l (the scale rides on the GEMM) + R0 h0 for l = 0
    fc::GemmGroup gg{};
    for (int l = 0; l <= le; ++l) {
      gg.prob[gg.count] = channel_map(N, C, a, R, l, chan(W + L.w_M, l), false, m, R, l, 0);
      gg.prob[gg.count++].alpha = conv_scale;
    }
    fc::gemm_group(gg, stream);
    fc::GemmGroup gr{};
    gr.prob[gr.count++] = channel_map(N, C, h0, 1, 0, W + L.w_R0, false, m, R, 0, 1);
    fc::gemm_group(gr, stream);
  }
  fc::launch_rms_norm_fwd(le, N, C, eps, m, W + L.w_g1, n, inv1, stream);
  fc::launch_gate_fwd(N, C, le, n, y, A, stream);
  {
    fc::GemmGroup gg{};
    for (int l = 0; l <= le; ++l) gg.prob[gg.count++] = channel_map(N, C, y, R, l, chan(W + L.w_O, l), false, A, R, l, 1);
    fc::gemm_group(gg, stream);
  }
  fc::ladder_forward(p, A, lw, z, saved, lws, stream);
  {  // o = z + R2 A_0 (in place in z)
    fc::GemmGroup gg{};
    gg.prob[gg.count++] = channel_map(N, C, A, R, 0, W + L.w_R2, false, z, 1, 0, 1);
    fc::gemm_group(gg, stream);
  }
  fc::launch_rms_norm_fwd(0, N, C, eps, z, W + L.w_g2, f, inv2, stream);
  fc::launch_readout_fwd(N, C, f, W + L.w_r1, W + L.w_r2, W + L.w_r3, ea, stream);
  fc::block_energy(ea, N, 1, 1, e_atom, parts, energy, stream);
  if (!forces) return check_launch("message block energy");

  // ---- backward for the forces
  fc::launch_readout_vjp(N, C, f, W + L.w_r1, W + L.w_r2, W + L.w_r3, fb, stream);
  fc::launch_rms_norm_vjp(0, N, C, z, W + L.w_g2, inv2, fb, ob, nullptr, nullptr, stream);
  fc::ladder_vjp(p, A, lw, saved, ob, Ab, nullptr, lws, stream);
  {  // A_bar_0 += R2^T o_bar;  y_bar_l = O_l^T A_bar_l (into y)
    fc::GemmGroup gg{};
    gg.prob[gg.count++] = channel_map(N, C, ob, 1, 0, W + L.w_R2, true, Ab, R, 0, 1);
    fc::gemm_group(gg, stream);
    fc::GemmGroup gy{};
    for (int l = 0; l <= le; ++l) gy.prob[gy.count++] = channel_map(N, C, Ab, R, l, chan(W + L.w_O, l), true, y, R, l, 0);
    fc::gemm_group(gy, stream);
  }
  fc::launch_gate_vjp(N, C, le, n, Ab, y, nb, stream);
  fc::launch_rms_norm_vjp(le, N, C, m, W + L.w_g1, inv1, nb, mb, nullptr, nullptr, stream);
  {  // a_bar_l = conv_scale M_l^T m_bar_l (into a), negated: the convolution's
     // VJP is linear in its cotangent, so its position gradient is then the force
    fc::GemmGroup gg{};
    for (int l = 0; l <= le; ++l) {
      gg.prob[gg.count] = channel_map(N, C, mb, R, l, chan(W + L.w_M, l), true, a, R, l, 0);
      gg.prob[gg.count++].alpha = -conv_scale;
    }
    fc::gemm_group(gg, stream);
  }
  mlp_conv_vjp(cd, g, pos, shift, hb, W + L.w_mlp, a, nullptr, forces, nullptr, mws, wb + L.cws, true, stream);
  return check_launch("message block energy/forces");
}

}  // extern "C"
