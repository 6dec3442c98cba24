/*
 * flashcart.h -- C ABI of the MI355X (gfx950) FlashCart hot path.
 *
 * Operations follow "FlashCart: Fast Cartesian Tensor Products for
 * Equivariant Interatomic Potentials" (arXiv 2610.06409):
 *   - edge convolution, §4 Eq. 1 (receiver-sorted sum over incoming edges),
 *     with path-separated outputs and the layout of App. D ("Data layout",
 *     Fig. D1);
 *   - its VJP, App. C Eq. C1, carried through the direction tensors and the
 *     radial weights to the positions (forces);
 *   - its VJP-of-VJP for position cotangents, App. C Eq. C2;
 *   - the node-local correlation ladder, §5 Eq. 2 (full) and App. E
 *     "Path-reduced products", and its VJP.
 *
 * Conventions shared by every call
 * --------------------------------
 * Precision: fp32 storage and arithmetic.
 * Memory: every array argument is a DEVICE pointer into caller-owned memory.
 *   The library allocates nothing inside any call and keeps no pointer after
 *   return; scratch comes from a caller workspace sized by the matching
 *   *_workspace_bytes query.  Inputs and outputs must not alias.
 * Streams: calls are asynchronous and ordered on the given hipStream_t
 *   (pass 0 for the null stream).  Host-side argument checks happen before
 *   any launch; on error nothing is launched.
 * Outputs are overwritten, never accumulated into.
 * Determinism: no atomics touch floating-point data; results are bitwise
 *   reproducible for fixed inputs and launch configuration.
 * Errors: every call returns an fc_status; fc_last_error_message() gives a
 *   thread-local detail string for the last failing call on this thread.
 * Sizes: node and edge counts are int32.  Every kernel forms node and edge
 *   offsets in 64 bits, so arrays may exceed 2 GiB (e.g. [N][230][128] at
 *   rank 4 beyond 18 k nodes).  The correlation ladder, and the blocks that
 *   contain it, need n_nodes * (2 l_prod + 1) < 2^26 (the row index range of
 *   its matrix-core GEMMs); larger requests return FC_ERR_UNSUPPORTED.
 * Graph contents are not checked by the device calls: a graph must satisfy
 *   fc_graph_validate (rowptr monotone from 0 to E, senders in [0, N)),
 *   otherwise kernels read and write out of bounds.
 *
 * Layouts (row-major, channels contiguous)
 * ----------------------------------------
 * Stored components of a rank-l tensor: the 2l+1 entries with at most one z
 * index, ordered (p_x descending with p_z = 0), then (p_x descending with
 * p_z = 1); e.g. l = 2: xx, xy, yy, xz, yz (§3 "Symbolic construction").
 * Node features x: [N][(l_in+1)^2][C]; rank block l starts at row l^2.
 * Path-separated outputs z (and g, g_hat): [N][n_out][C] with
 *   row(path p, component c) = off(L) + c * P_L + eta_L,
 *   off(L) = sum_{L'<L} (2L'+1) P_L',
 * where P_L counts the paths with output rank L and eta_L is the position of
 * p among them.  Paths are the natural-parity triples (l1, l2, L),
 * l1 <= l_in, l2 <= l_edge, L <= l_out, |l1-l2| <= L <= l1+l2, l1+l2+L even,
 * ordered by L and then (l1, l2) lexicographically (fc_conv_path).
 * Radial weights W: [n_basis][P][C]; the weight of edge e, path p, channel k
 *   is w = sum_b R_b(r_e) W[b][p][k] with
 *   R_b(r) = sin(b pi r / r_cut) / r * (1 + cos(pi r / r_cut)) / 2 for
 *   r < r_cut and 0 beyond, b = 1..n_basis (n_basis = 8 supported).
 * Graph: receiver-sorted CSR (rowptr[N+1], sender[E]); edge e has receiver
 *   u_e (rowptr[u] <= e < rowptr[u+1]), sender v_e = sender[e] and vector
 *   r_e = pos[v_e] - pos[u_e] + shift[e] (shift may be NULL), pointing from
 *   the receiver to its neighbour (§2).  The sender-sorted transpose
 *   (t_rowptr[N+1], t_edge[E], with receiver[E]) is built by
 *   fc_graph_transpose and lets the VJP run without atomics.
 */
#ifndef FLASHCART_H_
#define FLASHCART_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FC_ABI_VERSION 3

typedef enum {
  FC_OK = 0,
  FC_ERR_INVALID_ARGUMENT = 1, /* bad descriptor, NULL required pointer, bad size */
  FC_ERR_UNSUPPORTED = 2,      /* valid request the library does not implement   */
  FC_ERR_WORKSPACE = 3,        /* workspace NULL or smaller than required        */
  FC_ERR_HIP = 4               /* a HIP runtime call or launch failed            */
} fc_status;

/* Human-readable name of a status code (static string). */
const char* fc_status_string(fc_status s);
/* Detail of the last failing call on the calling thread ("" if none). */
const char* fc_last_error_message(void);
/* Returns FC_ABI_VERSION. */
int32_t fc_abi_version(void);

/* ------------------------------------------------------------------------
 * Edge convolution descriptor.
 * n_nodes >= 1, n_edges >= 0, 1 <= channels <= 256,
 * 0 <= l_in, l_edge, l_out <= 5 with at least one admissible path and the
 * rank set instantiated in the build: equal ranks 0..5, and (l_prop, l_e, l_e)
 * with l_prop <= min(l_e, 3), l_e <= 4 (FC_ERR_UNSUPPORTED otherwise);
 * n_basis == 8, r_cut > 0.  flags:
 *   0: natural parity (even l1+l2+L, the pages' method), paths separate;
 *   FC_CONV_ALL_PARITIES: every triangle-allowed path (the odd-J couplings
 *     are STF_L(Sym_L(E)) with one index of each operand contracted through
 *     the Levi-Civita symbol, constant 1, so (1,1)->1 is the cross product
 *     x × y); instantiated for equal ranks 1..4, the VJP-of-VJP for 1..3;
 *   FC_CONV_SUM_PATHS: the outputs of all paths with the same output rank L
 *     are summed into one block of 2L+1 rows (App. D, "Executing Cartesian
 *     tensor products": the kernel option of summing path outputs; weights
 *     stay per path, and the cotangents g_z / g_hat use the same rows);
 *     natural parity, instantiated for equal ranks 1..4, the VJP-of-VJP
 *     for 1..3.
 * ---------------------------------------------------------------------- */
#define FC_CONV_ALL_PARITIES 1u
#define FC_CONV_SUM_PATHS 2u
/* FC_CONV_MLP_MATERIALIZE / FC_CONV_MLP_FUSE (exclusive): how the calls
 * weighted by the radial network (fc_edge_conv_mlp_*, the message blocks)
 * apply its output layer -- materialised (w [E][P][C] written by an MFMA
 * GEMM and streamed through the explicit-weight kernels) or fused into the
 * convolution's lanes (see fc_edge_conv_mlp_workspace_bytes for the
 * default); every other call ignores them. */
#define FC_CONV_MLP_MATERIALIZE 4u
#define FC_CONV_MLP_FUSE 8u

typedef struct {
  int32_t n_nodes, n_edges, channels;
  int32_t l_in, l_edge, l_out;
  int32_t n_basis;
  float r_cut;
  uint32_t flags;
} fc_conv_desc;

typedef struct {
  const int32_t* rowptr;   /* [N+1] receiver-sorted row pointer              */
  const int32_t* sender;   /* [E]   sender of each receiver-sorted edge       */
  const int32_t* receiver; /* [E]   receiver of each edge (fc_graph_transpose) */
  const int32_t* t_rowptr; /* [N+1] sender-sorted row pointer                 */
  const int32_t* t_edge;   /* [E]   edge ids grouped by sender, ascending     */
} fc_graph;

/* Number of paths and row counts (in units of C floats) of x and z.
 * Implements the path enumeration of §2 "Irreducible Cartesian tensors"
 * (admissible = triangle + even J).  out_rows is sum_L (2L+1) P_L with paths
 * separate, and the sum of 2L+1 over the ranks L that have a path with
 * FC_CONV_SUM_PATHS: block L starts after the blocks of the lower ranks.
 * Host only. */
fc_status fc_conv_layout(const fc_conv_desc* d, int32_t* n_paths, int32_t* in_rows,
                         int32_t* out_rows);
/* The i-th path (l1, l2, L) in storage order.  Host only. */
fc_status fc_conv_path(const fc_conv_desc* d, int32_t i, int32_t* l1, int32_t* l2,
                       int32_t* L);

/* Builds receiver[E], t_rowptr[N+1] and t_edge[E] on the device from the
 * receiver-sorted CSR.  Within each sender, edge ids are ascending, so the
 * result is unique.  Workspace: fc_graph_transpose_workspace_bytes(N). */
size_t fc_graph_transpose_workspace_bytes(int32_t n_nodes);
fc_status fc_graph_transpose(int32_t n_nodes, int32_t n_edges, const int32_t* rowptr,
                             const int32_t* sender, int32_t* receiver, int32_t* t_rowptr,
                             int32_t* t_edge, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);
/* Host-side check of a receiver-sorted CSR given in HOST memory: rowptr[0]
 * == 0, non-decreasing, rowptr[N] == E, 0 <= sender < N. */
fc_status fc_graph_validate(int32_t n_nodes, int32_t n_edges, const int32_t* h_rowptr,
                            const int32_t* h_sender);

/* Workspace bytes for op = 0 (forward), 1 (VJP), 2 (VJP-of-VJP). */
size_t fc_edge_conv_workspace_bytes(const fc_conv_desc* d, int32_t op);

/* Forward, Eq. 1: z[u, eta, k] = sum_{e: u_e = u} w[e, eta, k] f_eta(x[v_e, k], T(r_hat_e)).
 * pos [N][3], shift [E][3] or NULL, x [N][in_rows][C], radial_w [8][P][C],
 * z [N][out_rows][C] (written).  Needs rowptr and sender of g. */
fc_status fc_edge_conv_fwd(const fc_conv_desc* d, const fc_graph* g, const float* pos,
                           const float* shift, const float* x, const float* radial_w,
                           float* z, hipStream_t stream);

/* VJP of L = <g_z, z> (Eq. C1 and the chain rule through T_l and R_b).
 * x_grad [N][in_rows][C] and pos_grad [N][3] are written when non-NULL;
 * radial_w_grad [8][P][C] is written when non-NULL: the weight-gradient
 * line of Eq. C1 carried through w = R W, i.e.
 * radial_w_grad[b, eta, k] = sum_e R_b(r_e) <g_z[u_e, eta, k], f_eta(x[v_e, k], T(r_hat_e))>,
 * computed by a separate receiver-sorted pass and reduced in a fixed order.
 * At least one output must be requested.  Needs the full graph (transpose
 * included) and a workspace of fc_edge_conv_workspace_bytes(d, 1) bytes. */
fc_status fc_edge_conv_vjp(const fc_conv_desc* d, const fc_graph* g, const float* pos,
                           const float* shift, const float* x, const float* radial_w,
                           const float* g_z, float* x_grad, float* pos_grad,
                           float* radial_w_grad, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * VJP as fc_edge_conv_vjp (same kernels, same results) with its workspace
 * taken from a device array the library owns, FC_NOALLOC_SCRATCH_BYTES
 * (64 MiB) on each GPU it runs on, held until the process ends.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine);
 * the caller still passes inputs and outputs.  A call needs the VJP
 * workspace of fc_edge_conv_workspace_bytes(d, 1), less its per-block
 * radial-weight partials when radial_w_grad is NULL (at 1024 nodes x 128
 * neighbours x 128 channels, ranks <= 2: 20.5 MB, or 32.0 MB with
 * radial_w_grad; ranks <= 3: 35.2 MB / 59.3 MB); a larger request returns
 * FC_ERR_WORKSPACE before any launch.  All calls on one GPU share its array
 * and leave the last call's partial sums in it (nothing in it needs to start
 * at zero): calls that overlap on one GPU (different streams or threads)
 * race, so order them on one stream or with events.  The first call on a
 * device looks up that device's copy of the array with the device current. */
#define FC_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
fc_status fc_edge_conv_vjp_noalloc(const fc_conv_desc* d, const fc_graph* g, const float* pos,
                                   const float* shift, const float* x, const float* radial_w,
                                   const float* g_z, float* x_grad, float* pos_grad,
                                   float* radial_w_grad, hipStream_t stream);

/* Forward of Eq. 1 with the per-edge weights given, as the pages state it:
 * w [E][P][C] in receiver-sorted edge order (w[e, eta, k] weights path eta,
 * channel k of edge e) replaces the radial basis; r_cut and n_basis of d are
 * not used.  An edge of zero length has no direction and takes no part.
 * Other arguments and layouts as fc_edge_conv_fwd. */
fc_status fc_edge_conv_fwd_w(const fc_conv_desc* d, const fc_graph* g, const float* pos,
                             const float* shift, const float* x, const float* w, float* z,
                             hipStream_t stream);

/* VJP of L = <g_z, z> for fc_edge_conv_fwd_w with w held fixed (Eq. C1):
 * x_grad [N][in_rows][C]; pos_grad [N][3] through the direction tensors
 * only; w_grad [E][P][C] = <g_z[u_e, eta, k], f_eta(x[v_e, k], T(r_hat_e))>
 * (0 for an edge of zero length).  Each output is written when non-NULL; at
 * least one.  Needs the full graph (transpose included) and a workspace of
 * fc_edge_conv_workspace_bytes(d, 1) bytes. */
fc_status fc_edge_conv_vjp_w(const fc_conv_desc* d, const fc_graph* g, const float* pos,
                             const float* shift, const float* x, const float* w,
                             const float* g_z, float* x_grad, float* pos_grad, float* w_grad,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* VJP-of-VJP (Eq. C2 with the position derivatives of T_l and R_b): for
 * s = <v_x, x_grad> + <v_pos, pos_grad> + <v_radial_w, radial_w_grad>
 * (v_x [N][in_rows][C], v_pos [N][3], v_radial_w [8][P][C]; a NULL
 * cotangent is zero), writes g_hat = ds/dg_z [N][out_rows][C],
 * x_hat = ds/dx [N][in_rows][C], pos_hat = ds/dpos [N][3] and
 * radial_w_hat = ds/dradial_w [8][P][C] (each when non-NULL; at least one).
 * z is linear in radial_w, so the weight cotangent adds the forward and
 * the VJP evaluated with v_radial_w as the weights to g_hat, x_hat and
 * pos_hat and leaves radial_w_hat unchanged.  Needs g_z unless only g_hat
 * is requested, the graph transpose for x_hat and pos_hat, and a workspace
 * of fc_edge_conv_workspace_bytes(d, 2) bytes unless only g_hat is
 * requested with v_radial_w NULL (or v_radial_w the only cotangent).
 * Instantiated for ranks <= 4 (FC_ERR_UNSUPPORTED at rank 5). */
fc_status fc_edge_conv_vjp_vjp(const fc_conv_desc* d, const fc_graph* g, const float* pos,
                               const float* shift, const float* x, const float* radial_w,
                               const float* g_z, const float* v_x, const float* v_pos,
                               const float* v_radial_w, float* g_hat, float* x_hat,
                               float* pos_hat, float* radial_w_hat, void* workspace,
                               size_t workspace_bytes, hipStream_t stream);

/* VJP-of-VJP of the explicit-weight convolution (App. C Eq. C2; the inputs
 * and outputs of Alg. 3, with the direction cotangent carried on to the
 * positions): for s = <v_x, x_grad> + <v_pos, pos_grad> + <v_w, w_grad> of
 * fc_edge_conv_vjp_w (v_x [N][in_rows][C], v_pos [N][3], v_w [E][P][C] in
 * receiver-sorted edge order; a NULL cotangent is zero), writes
 * g_hat = ds/dg_z [N][out_rows][C], x_hat = ds/dx [N][in_rows][C],
 * pos_hat = ds/dpos [N][3] and w_hat = ds/dw [E][P][C], i.e.
 * w_hat[e, eta, k] = <g_z[u_e], f_eta(v_x[v_e], y_e) + f_eta(x[v_e], J_y dv_e)>
 * (each when non-NULL; at least one).  An edge of zero length takes no part
 * (its w_hat is 0).  Needs g_z, the graph transpose and a workspace of
 * fc_edge_conv_workspace_bytes(d, 1) bytes unless only g_hat is requested.
 * Ranks as fc_edge_conv_vjp_vjp. */
fc_status fc_edge_conv_vjp_vjp_w(const fc_conv_desc* d, const fc_graph* g, const float* pos,
                                 const float* shift, const float* x, const float* w,
                                 const float* g_z, const float* v_x, const float* v_pos,
                                 const float* v_w, float* g_hat, float* x_hat, float* pos_hat,
                                 float* w_hat, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * The pages' radial network (App. E "Model architecture", the weights
 * w_{eta k}(r) of Eq. E1; App. F "Model architecture and training"):
 *   phi_n(r) = T_n(cos(pi r / r_cut)) u(r / r_cut), n = 0..7, with the p = 6
 *   envelope u(d) = 1 - 28 d^6 + 48 d^7 - 21 d^8 (0 for d >= 1; value and
 *   first two derivatives vanish at d = 1; the pages fix the property, this
 *   polynomial is the reading),
 *   w[e, eta, k] = (SiLU(SiLU(phi(r_e) W1) W2) W3)[eta C + k], bias-free.
 * Flat weights mlp_w: W1 [8][64], W2 [64][64], W3 [64][P][C]
 * (fc_radial_mlp_weight_floats(d) floats).  r_cut of d is r_max; n_basis
 * must be 8 (the Chebyshev count).  An edge of zero length gets w = 0.
 * ---------------------------------------------------------------------- */
size_t fc_radial_mlp_weight_floats(const fc_conv_desc* d);
/* How w is applied.  Fused: a pre-pass stores each edge's second hidden
 * layer and its r-derivative (512 bytes per edge), and the convolution's
 * lanes form w = h2 W3 (and dw/dr) for batches of edges without storing
 * them; available for natural parity, paths apart and ranks <= 3, in the
 * forward and in a VJP without mlp_w_grad.  Materialised: w [E][P][C] is
 * written to the workspace by an MFMA GEMM and streamed through the
 * explicit-weight kernels, and the VJP carries w_bar back through the
 * network.  Default (measured): the forward fused where l_in <= 1 or every
 * rank is <= 2, materialised at (2,3,3) and (3,3,3); the VJP materialised
 * (the fused VJP needs 2 x 64 P FMAs per edge and channel on the vector
 * units and was slower or within 4 %, but takes a far smaller workspace).
 * FC_CONV_MLP_FUSE / FC_CONV_MLP_MATERIALIZE override.  A forward on an op 2
 * workspace (the message blocks) follows the VJP's choice.
 * Workspace of the calls below: op 0 forward (and fc_radial_mlp), op 1 VJP
 * with mlp_w_grad, op 2 VJP without it (op 1 bytes serve both VJPs). */
size_t fc_edge_conv_mlp_workspace_bytes(const fc_conv_desc* d, int32_t op);

/* w [E][P][C] (receiver-sorted edges): the per-edge weights alone, for
 * fc_edge_conv_fwd_w.  Needs sender and receiver of g. */
fc_status fc_radial_mlp(const fc_conv_desc* d, const fc_graph* g, const float* pos,
                        const float* shift, const float* mlp_w, float* w, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* Eq. 1 / E1 with w from the radial network: z [N][out_rows][C].  Needs
 * rowptr, sender and receiver of g. */
fc_status fc_edge_conv_mlp_fwd(const fc_conv_desc* d, const fc_graph* g, const float* pos,
                               const float* shift, const float* x, const float* mlp_w, float* z,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* VJP of L = <g_z, z> through the convolution and the radial network:
 * x_grad [N][in_rows][C], pos_grad [N][3] (through the direction tensors
 * and through w(r)), mlp_w_grad (flat, as mlp_w); each when non-NULL, at
 * least one.  Needs the full graph. */
fc_status fc_edge_conv_mlp_vjp(const fc_conv_desc* d, const fc_graph* g, const float* pos,
                               const float* shift, const float* x, const float* mlp_w,
                               const float* g_z, float* x_grad, float* pos_grad, float* mlp_w_grad,
                               void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Node-local correlation ladder (§5 Eq. 2; App. E "Path-reduced products").
 * A [N][(l_a+1)^2][C]; z [N][(l_out+1)^2][C].  Steps q = 1..order; the
 * product at step q >= 2 couples phi^{q-1} (ranks <= l_{q-1}) with A (ranks
 * <= l_a) to ranks <= l_q, with l_q = l_prod for q < order and l_q = l_out
 * for q = order (phi^1 keeps ranks <= min(l_a, l_1)).  Paths of a step are
 * ordered like the convolution paths.
 * variant FC_LADDER_FULL: phi^1_l = W1_l A_l; phi^q_L = W^q_L B^q_L with
 *   B^q_L [(2L+1) rows][P_{q,L} * C] the path-separated products;
 *   z = sum_q Pi_{<= l_out} phi^q.
 *   Flat weights: W1_l [C][C] for l = 0..l_1, then for q = 2..order and
 *   L = 0..l_q with P_{q,L} > 0: W^q_L [C][P_{q,L} C], element
 *   [k_out][eta * C + k_in].
 * variant FC_LADDER_PATH_REDUCED: phi^1_l = a1[l][k] A_l;
 *   phi^q_L = P_{q,L}^{-1/2} sum_{eta -> L} a^q[eta][k] (phi^{q-1} (x) A)_eta;
 *   z_L = W_L sum_q phi^q_L.
 *   Flat weights: a1 [l_1+1][C], a^q [P_q][C] for q = 2..order,
 *   W_L [C][C] for L = 0..l_out.
 * Constraints: 1 <= order <= 8, ranks <= 4, C a multiple of 32 and <= 512.
 * ---------------------------------------------------------------------- */
enum { FC_LADDER_FULL = 0, FC_LADDER_PATH_REDUCED = 1 };

typedef struct {
  int32_t n_nodes, channels;
  int32_t l_a, l_prod, l_out, order;
  int32_t variant;
} fc_ladder_desc;

/* Sizes in floats of the flat weight buffer and of the saved-state buffer
 * the forward fills for the VJP.  Host only. */
fc_status fc_ladder_layout(const fc_ladder_desc* d, size_t* n_weight_floats,
                           size_t* n_saved_floats);
size_t fc_ladder_workspace_bytes(const fc_ladder_desc* d, int32_t op /*0 fwd, 1 vjp, 2 vjp-of-vjp*/);
/* Block i (0-based, in flat order) of the weight buffer: its offset in
 * floats, its shape rows x cols, and kind 0 (a mixing matrix, fan-in =
 * cols) or 1 (per-rank or per-path channel weights a, shape [rows][C]).
 * FC_ERR_INVALID_ARGUMENT past the last block.  Host only. */
fc_status fc_ladder_weight_block(const fc_ladder_desc* d, int32_t i, size_t* offset, int32_t* rows,
                                 int32_t* cols, int32_t* kind);

/* Forward.  saved may be NULL when no VJP follows; otherwise it receives
 * n_saved_floats floats of intermediate states. */
fc_status fc_node_ladder_fwd(const fc_ladder_desc* d, const float* A, const float* weights,
                             float* z, float* saved, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* VJP of L = <g_z, z>: A_grad [N][(l_a+1)^2][C] and, when non-NULL, the
 * weight gradient in the flat weight layout.  saved must come from
 * fc_node_ladder_fwd with the same A and weights. */
fc_status fc_node_ladder_vjp(const fc_ladder_desc* d, const float* A, const float* weights,
                             const float* saved, const float* g_z, float* A_grad,
                             float* weights_grad, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* VJP-of-VJP of the ladder (App. C Eq. C2 carried through Eq. 2): for
 * s = <v_A, A_grad> + <v_weights, weights_grad> (NULL cotangent = zero),
 * writes g_hat = ds/dg_z [N][(l_out+1)^2][C], A_hat = ds/dA and
 * weights_hat = ds/dweights (flat weight layout), each when non-NULL (at
 * least one).  Needs the forward's saved states (order > 1), g_z unless only
 * g_hat is requested, and a workspace of fc_ladder_workspace_bytes(d, 2)
 * bytes (op 2: the largest step's product buffer four times, four states,
 * order - 1 tangent states, split-K partials and, path-reduced, four
 * output-sized sums).  Both variants. */
fc_status fc_node_ladder_vjp_vjp(const fc_ladder_desc* d, const float* A, const float* weights,
                                 const float* saved, const float* g_z, const float* v_A,
                                 const float* v_weights, float* g_hat, float* A_hat,
                                 float* weights_hat, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * One message-passing block for energy and forces (App. E "Model
 * architecture" and Eq. E1; §2 for F = -grad E):
 *   A = conv_scale * edge_conv(x) ,  z = ladder(A),
 *   E = sum_u sum_k z[u, 0, k],      forces = -dE/dpos.
 * Needs conv.l_in == 0 (scalar senders: one path per output rank, so the
 * convolution output has the node-feature layout), conv.l_out == lad.l_a,
 * equal channels and node counts.  energy: DEVICE double[1] (summed in
 * fp64 in a fixed order); e_atom: DEVICE float[N] or NULL (per-atom sums);
 * forces: DEVICE float[N][3] or NULL (skips the backward pass).  Residual
 * updates, normalisation, gates and the readout are not included.
 * ---------------------------------------------------------------------- */
size_t fc_block_workspace_bytes(const fc_conv_desc* conv, const fc_ladder_desc* lad);
fc_status fc_block_energy_forces(const fc_conv_desc* conv, const fc_graph* g, const float* pos,
                                 const float* shift, const float* x, const float* radial_w,
                                 const fc_ladder_desc* lad, const float* ladder_w, float conv_scale,
                                 double* energy, float* e_atom, float* forces, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * A full message-passing block for energy and forces (App. E "Model
 * architecture"; App. F for the radial network, SiLU gates and the readout
 * width), one final block with scalar senders in and scalars out, with the
 * caller's (random) weights.  Readings where the pages leave a step open:
 *   hb  = Mpre h0 (the d x d channel map of the sender features before the
 *         convolution; one rank with scalar senders);
 *   a   = conv_scale * conv(hb), weights from the radial network (Eq. E1);
 *   m_l = M_l a_l (rank-wise map of the paths and channels; one path per
 *         rank with scalar senders), m_0 += R0 h0 (residual update);
 *   n   = RMSnorm(m; gamma1, eps) (fc_rms_norm_fwd);
 *   y_0 = SiLU(n_0), y_l = SiLU(n_0) n_l (scalar SiLU gates);
 *   A_l = n_l + O_l y_l (the output map added to the gated layer's input);
 *   z   = ladder(A) with l_out = 0;  o = z + R2 A_0 (residual update);
 *   f   = RMSnorm(o; gamma2, eps);  E_u = SiLU(SiLU(f Wr1) Wr2) . wr3
 *         (bias-free readout MLP C -> 64 -> 64 -> 1);
 *   E   = sum_u E_u (fp64, fixed order), forces = -dE/dpos.
 * Matrices act on channels as [out][in].  Flat weights, in order: radial
 * network (fc_radial_mlp_weight_floats layout, P = l_edge + 1), Mpre
 * [C][C], M [l+1][C][C], R0 [C][C], gamma1 [l+1][C], O [l+1][C][C], ladder weights
 * (fc_ladder_layout), R2 [C][C], gamma2 [C], Wr1 [C][64], Wr2 [64][64],
 * wr3 [64] (fc_message_block_weight_floats floats).  conv: l_in = 0,
 * l_edge = l_out = l, flags 0; lad: l_a = l_prod = l, l_out = 0, equal
 * nodes and channels.  h0 [N][1][C]; energy: DEVICE double[1]; e_atom
 * DEVICE float[N] or NULL; forces DEVICE float[N][3] or NULL (then no
 * backward pass; otherwise the full graph is needed).
 * ---------------------------------------------------------------------- */
size_t fc_message_block_weight_floats(const fc_conv_desc* conv, const fc_ladder_desc* lad);
size_t fc_message_block_workspace_bytes(const fc_conv_desc* conv, const fc_ladder_desc* lad);
fc_status fc_message_block_energy_forces(const fc_conv_desc* conv, const fc_graph* g,
                                         const float* pos, const float* shift, const float* h0,
                                         const fc_ladder_desc* lad, const float* weights,
                                         float conv_scale, float eps, double* energy, float* e_atom,
                                         float* forces, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/* ------------------------------------------------------------------------
 * Equivariant RMS normalisation of node features (App. E "Model
 * architecture": scalar invariants from the generated (l,l)->0 couplings,
 * combined over ranks and channels into one scale per atom, no batch
 * statistics).  The combination is read as the root mean square:
 *   q[u,l,k] = f_(l,l)->0(x[u,l,k], x[u,l,k]),
 *   s[u] = sqrt(sum_{l,k} q[u,l,k] / ((l_max+1) C) + eps),
 *   y[u,l,k] = gamma[l,k] x[u,l,k] / s[u].
 * x, y [N][(l_max+1)^2][C] (ranks 0..l_max, stored components);
 * gamma [l_max+1][C] or NULL (all ones); inv_scale [N] = 1/s (written by
 * the forward when non-NULL, read by the VJP).  Constraints: n_nodes >= 1,
 * 1 <= channels <= 512, 0 <= l_max <= 5, eps >= 0 and finite (with eps = 0
 * a node of zeros gives non-finite outputs).
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t n_nodes, channels, l_max;
  float eps;
} fc_norm_desc;

fc_status fc_rms_norm_fwd(const fc_norm_desc* d, const float* x, const float* gamma, float* y,
                          float* inv_scale, hipStream_t stream);

/* VJP of L = <g_y, y> at the forward's inv_scale: x_grad [N][rows][C] and
 * gamma_grad [l_max+1][C] (summed over nodes in a fixed order), each when
 * non-NULL (at least one).  gamma_grad needs a workspace of
 * fc_rms_norm_workspace_bytes(d) bytes. */
size_t fc_rms_norm_workspace_bytes(const fc_norm_desc* d);
fc_status fc_rms_norm_vjp(const fc_norm_desc* d, const float* x, const float* gamma,
                          const float* inv_scale, const float* g_y, float* x_grad,
                          float* gamma_grad, void* workspace, size_t workspace_bytes,
                          hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FLASHCART_H_ */
