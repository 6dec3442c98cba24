"""Oracle for the equivariant edge convolution, its VJP and its VJP-of-VJP.

TEST INFRASTRUCTURE ONLY.  Plain fp64 numpy, chunked over edges; follows the
FlashCart paper:

* forward: Eq. 1 (§4 "Receiver-sorted forward"),
      z[u, eta, k] = sum_{e: u_e = u} w[e, eta, k] f_eta(x[v_e, k], y_e),
  with y_e = T(r_hat_e) (App. B) and r_e = pos[v_e] - pos[u_e] + shift_e
  pointing from the receiver u to its neighbour v (§2).  Paths are kept
  separate (Eq. 1 and App. D "Data layout").
* radial weights (reading of the workload, not printed on the pages): eight
  Bessel functions sin(b pi r / r_c)/r, b = 1..8, times the cosine cutoff
  (1 + cos(pi r / r_c))/2 for r < r_c and 0 beyond, contracted with a weight
  W[b, path, channel]: w[e, p, k] = sum_b R_b(r_e) W[b, p, k].
* VJP: Eq. C1 (App. C) applied edge by edge -- because f is bilinear the
  input VJPs are transposed contractions of the same bilinear form -- and the
  chain rule through T_l(r_hat) and R_b(r) to the positions (App. C
  "Symbolic derivatives": direction-tensor derivatives).  Gradients are taken
  with respect to the stored independent components (§3).
* explicit per-edge weights (the pages' own interface of Eq. 1 and Eq. C1):
  the same forward and VJP with w [E, P, C] given instead of formed from the
  radial basis; its gradient w_bar [E, P, C] is returned per edge and the
  position gradient runs through the direction tensors only (w held fixed).
* path-summed outputs (ConvSpec(sum_paths=True)): the kernel option of
  summing the outputs of all paths with the same output rank L into one
  (2L+1)-row block instead of keeping them separate (App. D "Executing
  Cartesian tensor products"; weights stay per path).  The VJPs read the same g
  block for every path of rank L.
* VJP-of-VJP: with s = <v_x, x_bar> + <v_pos, pos_bar>, g_hat = ds/dg is the
  directional derivative of the forward along (v_x, v_pos), and
  (x_hat, pos_hat, W_hat) is the directional derivative of the VJP along the
  same direction (a Hessian-vector product of <g, z>).  Both are computed by
  complex-step differentiation (derivative = Im f(p + i h v) / h, exact to
  rounding for h = 1e-20), which needs the forward and the VJP to be written
  without conjugation; Eq. C2 (App. C) is then checked against these
  derivatives in the tests.

Parity pins (tests/test_oracle_*.py): explicit full-tensor mode against the
probed bilinear mode; O(3) equivariance of z; central finite differences and
complex-step derivatives against the hand-written VJP; the identities
<g, f(x,y)> = <x, VJP1(g,y)> = <y, VJP2(g,x)>; translation invariance
(sum of position gradients = 0); rotation covariance of the position gradient;
symmetry of the Hessian-vector products; zero forces in the perfect diamond
cell.
"""

from __future__ import annotations

import numpy as np
import scipy.sparse as sp

from . import tensors as T


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------

def receivers(rowptr: np.ndarray) -> np.ndarray:
    return np.repeat(np.arange(len(rowptr) - 1), np.diff(rowptr))


def segment_sum(vals: np.ndarray, seg: np.ndarray, nseg: int) -> np.ndarray:
    """out[s] = sum of vals[e] over e with seg[e] = s (sparse incidence matmul)."""
    E = vals.shape[0]
    m = sp.csr_matrix((np.ones(E), (seg, np.arange(E))), shape=(nseg, E))
    flat = vals.reshape(E, int(np.prod(vals.shape[1:])))
    if np.iscomplexobj(flat):
        out = (m @ flat.real) + 1j * (m @ flat.imag)
    else:
        out = m @ flat
    return np.asarray(out).reshape((nseg,) + vals.shape[1:])


def radial(r, n_basis: int, r_cut: float):
    """R_b(r) = sin(b pi r/r_c)/r * (1 + cos(pi r/r_c))/2 for r < r_c, else 0."""
    b = np.arange(1, n_basis + 1)
    th = np.pi * r / r_cut
    env = 0.5 * (1.0 + np.cos(th))
    val = np.sin(b[None, :] * th[:, None]) / r[:, None] * env[:, None]
    return np.where((np.real(r) < r_cut)[:, None], val, 0.0)


def radial_deriv(r, n_basis: int, r_cut: float):
    """d R_b / d r for the radial functions above (0 beyond the cutoff)."""
    b = np.arange(1, n_basis + 1)[None, :]
    th = (np.pi * r / r_cut)[:, None]
    rr = r[:, None]
    env = 0.5 * (1.0 + np.cos(th))
    denv = -0.5 * np.sin(th) * np.pi / r_cut
    s = np.sin(b * th)
    ds = np.cos(b * th) * b * np.pi / r_cut
    val = (ds / rr - s / rr ** 2) * env + s / rr * denv
    return np.where((np.real(r) < r_cut)[:, None], val, 0.0)


class ConvSpec:
    """Ranks, paths and layouts of one edge-convolution problem."""

    def __init__(self, l_in: int, l_edge: int, l_out: int, r_cut: float,
                 n_basis: int = 8, all_parities: bool = False, sum_paths: bool = False):
        self.l_in, self.l_edge, self.l_out = l_in, l_edge, l_out
        self.r_cut, self.n_basis = r_cut, n_basis
        self.paths = T.conv_paths(l_in, l_edge, l_out, all_parities)
        # path-separated rows (Eq. 1), or one block per output rank into which
        # every path of that rank adds (the summed-output option); the
        # forward adds each path into its rows and the VJPs read g from them,
        # so both layouts run through the same code below
        layout = T.summed_out_layout if sum_paths else T.out_layout
        self.rows, self.n_out = layout(self.paths, l_out)
        self.in_off = T.rank_offsets(l_in)
        self.n_in = self.in_off[-1]

    @property
    def n_paths(self) -> int:
        return len(self.paths)


def _geometry(pos, shift, s, u, idx):
    rv = pos[s] - pos[u]
    if shift is not None:
        rv = rv + shift[idx]
    rn = np.sqrt(np.sum(rv * rv, axis=-1))
    return rv, rn


def _chunks(idx: np.ndarray, chunk: int):
    for i in range(0, len(idx), chunk):
        yield idx[i:i + chunk]


# ----------------------------------------------------------------------------
# forward (Eq. 1)
# ----------------------------------------------------------------------------

def edge_conv_fwd(spec: ConvSpec, pos, rowptr, sender, x, W, shift=None,
                  edges=None, chunk: int = 4096, mode: str = "probed"):
    """z [N, n_out, C] (path-separated rows, App. D layout).

    ``edges`` restricts the sum to a subset of edge ids (used to sample
    receivers at full size).  ``mode='explicit'`` evaluates every product on
    full 3^l tensors (symmetrise, contract, detrace) instead of the probed
    bilinear tensor; it is slow and meant for the tiny workload.
    """
    N, C = pos.shape[0], x.shape[-1]
    recv = receivers(rowptr)
    idx = np.arange(len(sender)) if edges is None else np.asarray(edges)
    dt = np.result_type(pos.dtype, x.dtype, W.dtype, np.float64)
    z = np.zeros((N, spec.n_out, C), dtype=dt)
    for ch in _chunks(idx, chunk):
        s, u = sender[ch], recv[ch]
        rv, rn = _geometry(pos, shift, s, u, ch)
        n = rv / rn[:, None]
        R = radial(rn, spec.n_basis, spec.r_cut)
        w = np.einsum('eb,bpk->epk', R, W)
        ys = [T.direction_tensor(l, n) for l in range(spec.l_edge + 1)]
        for p, (l1, l2, L) in enumerate(spec.paths):
            xs = x[s, spec.in_off[l1]:spec.in_off[l1 + 1], :]
            if mode == "probed":
                K = T.coupling_tensor(l1, l2, L)
                M = np.einsum('abc,ec->eab', K, ys[l2])
                f = np.matmul(M, xs)
            elif mode == "explicit":
                xe = np.transpose(xs, (0, 2, 1))                  # (Ec, C, n1)
                ye = np.broadcast_to(ys[l2][:, None, :], xe.shape[:2] + (ys[l2].shape[-1],))
                f = np.transpose(T.coupling(l1, l2, L, xe, ye), (0, 2, 1))
            else:
                raise ValueError(mode)
            z[:, spec.rows[p], :] += segment_sum(w[:, p, None, :] * f, u, N)
    return z


# ----------------------------------------------------------------------------
# VJP (Eq. C1 + chain rule to positions)
# ----------------------------------------------------------------------------

def edge_conv_vjp(spec: ConvSpec, pos, rowptr, sender, x, W, g, shift=None,
                  edges=None, chunk: int = 4096, want_W: bool = False):
    """Gradients of L = <g, z>: x_bar [N, n_in, C], pos_bar [N, 3], W_bar.

    W_bar [n_basis, P, C] is returned only when ``want_W``.
    """
    N, C = pos.shape[0], x.shape[-1]
    recv = receivers(rowptr)
    idx = np.arange(len(sender)) if edges is None else np.asarray(edges)
    dt = np.result_type(pos.dtype, x.dtype, W.dtype, g.dtype, np.float64)
    x_bar = np.zeros((N, spec.n_in, C), dtype=dt)
    pos_bar = np.zeros((N, 3), dtype=dt)
    W_bar = np.zeros(W.shape, dtype=dt) if want_W else None
    for ch in _chunks(idx, chunk):
        s, u = sender[ch], recv[ch]
        Ec = len(ch)
        rv, rn = _geometry(pos, shift, s, u, ch)
        n = rv / rn[:, None]
        R = radial(rn, spec.n_basis, spec.r_cut)
        dR = radial_deriv(rn, spec.n_basis, spec.r_cut)
        w = np.einsum('eb,bpk->epk', R, W)
        ys = [T.direction_tensor(l, n) for l in range(spec.l_edge + 1)]
        jac = [T.direction_tensor_jac(l, rv) for l in range(spec.l_edge + 1)]
        y_bar = [np.zeros((Ec, T.n_comp(l)), dtype=dt) for l in range(spec.l_edge + 1)]
        w_bar = np.zeros((Ec, spec.n_paths, C), dtype=dt)
        xb_edge = np.zeros((Ec, spec.n_in, C), dtype=dt)
        for p, (l1, l2, L) in enumerate(spec.paths):
            K = T.coupling_tensor(l1, l2, L)
            gp = g[u][:, spec.rows[p], :]                         # (Ec, a, C)
            xs = x[s, spec.in_off[l1]:spec.in_off[l1 + 1], :]     # (Ec, b1, C)
            # VJP_1(g, y): sum_a g_a df_a/dx_b1 (unweighted)
            v1 = np.einsum('abc,eak,ec->ebk', K, gp, ys[l2], optimize=True)
            xb_edge[:, spec.in_off[l1]:spec.in_off[l1 + 1], :] += w[:, p, None, :] * v1
            # VJP_2(g, x) per channel: sum_a g_a df_a/dy_b2
            v2 = np.einsum('abc,eak,ebk->eck', K, gp, xs, optimize=True)
            y_bar[l2] += np.einsum('eck,ek->ec', v2, w[:, p, :])
            # weight gradient <g, f(x, y)> = <VJP_2(g, x), y>
            w_bar[:, p, :] = np.einsum('eck,ec->ek', v2, ys[l2])
        x_bar += segment_sum(xb_edge, s, N)
        rho = np.einsum('epk,bpk->eb', w_bar, W)
        r_bar = np.sum(dR * rho, axis=1)[:, None] * n
        for l in range(spec.l_edge + 1):
            r_bar = r_bar + np.einsum('ec,ecj->ej', y_bar[l], jac[l])
        pos_bar += segment_sum(r_bar, s, N) - segment_sum(r_bar, u, N)
        if want_W:
            W_bar += np.einsum('eb,epk->bpk', R, w_bar)
    return x_bar, pos_bar, W_bar


# ----------------------------------------------------------------------------
# explicit per-edge weights (Eq. 1 and Eq. C1 as the pages state them)
# ----------------------------------------------------------------------------

def edge_conv_fwd_w(spec: ConvSpec, pos, rowptr, sender, x, w, shift=None,
                    edges=None, chunk: int = 4096):
    """Eq. 1 with the per-edge weights given: w [E, P, C] in receiver-sorted
    edge order; z [N, n_out, C] as in edge_conv_fwd.  Edges of zero length
    take no part (their direction is undefined)."""
    N, C = pos.shape[0], x.shape[-1]
    recv = receivers(rowptr)
    idx = np.arange(len(sender)) if edges is None else np.asarray(edges)
    dt = np.result_type(pos.dtype, x.dtype, w.dtype, np.float64)
    z = np.zeros((N, spec.n_out, C), dtype=dt)
    for ch in _chunks(idx, chunk):
        s, u = sender[ch], recv[ch]
        rv, rn = _geometry(pos, shift, s, u, ch)
        keep = np.real(rn) > 0          # an edge of zero length has no direction
        n = rv / np.where(keep, rn, 1.0)[:, None]
        ys = [T.direction_tensor(l, n) for l in range(spec.l_edge + 1)]
        wc = w[ch] * keep[:, None, None]
        for p, (l1, l2, L) in enumerate(spec.paths):
            K = T.coupling_tensor(l1, l2, L)
            xs = x[s, spec.in_off[l1]:spec.in_off[l1 + 1], :]
            f = np.matmul(np.einsum('abc,ec->eab', K, ys[l2]), xs)
            z[:, spec.rows[p], :] += segment_sum(wc[:, p, None, :] * f, u, N)
    return z


def edge_conv_vjp_w(spec: ConvSpec, pos, rowptr, sender, x, w, g, shift=None,
                    edges=None, chunk: int = 4096):
    """Gradients of L = <g, z> for the explicit-weight forward, with w held
    fixed: x_bar [N, n_in, C], w_bar [E, P, C] (Eq. C1: w_bar = <g, f>), and
    pos_bar [N, 3] through the direction tensors only.  Edges of zero length
    take no part (their direction is undefined; w_bar is 0 there)."""
    N, C = pos.shape[0], x.shape[-1]
    recv = receivers(rowptr)
    idx = np.arange(len(sender)) if edges is None else np.asarray(edges)
    dt = np.result_type(pos.dtype, x.dtype, w.dtype, g.dtype, np.float64)
    x_bar = np.zeros((N, spec.n_in, C), dtype=dt)
    pos_bar = np.zeros((N, 3), dtype=dt)
    w_bar = np.zeros(w.shape, dtype=dt)
    for ch in _chunks(idx, chunk):
        s, u = sender[ch], recv[ch]
        Ec = len(ch)
        rv, rn = _geometry(pos, shift, s, u, ch)
        keep = np.real(rn) > 0          # an edge of zero length has no direction
        rv = np.where(keep[:, None], rv, 1.0)
        n = rv / np.where(keep, rn, np.sqrt(3.0))[:, None]
        ys = [T.direction_tensor(l, n) for l in range(spec.l_edge + 1)]
        jac = [T.direction_tensor_jac(l, rv) for l in range(spec.l_edge + 1)]
        y_bar = [np.zeros((Ec, T.n_comp(l)), dtype=dt) for l in range(spec.l_edge + 1)]
        xb_edge = np.zeros((Ec, spec.n_in, C), dtype=dt)
        wc = w[ch] * keep[:, None, None]
        for p, (l1, l2, L) in enumerate(spec.paths):
            K = T.coupling_tensor(l1, l2, L)
            gp = g[u][:, spec.rows[p], :]
            xs = x[s, spec.in_off[l1]:spec.in_off[l1 + 1], :]
            v1 = np.einsum('abc,eak,ec->ebk', K, gp, ys[l2], optimize=True)
            xb_edge[:, spec.in_off[l1]:spec.in_off[l1 + 1], :] += wc[:, p, None, :] * v1
            v2 = np.einsum('abc,eak,ebk->eck', K, gp, xs, optimize=True)
            y_bar[l2] += np.einsum('eck,ek->ec', v2, wc[:, p, :])
            w_bar[ch, p, :] = np.einsum('eck,ec->ek', v2, ys[l2]) * keep[:, None]
        x_bar += segment_sum(xb_edge, s, N)
        r_bar = np.zeros((Ec, 3), dtype=dt)
        for l in range(spec.l_edge + 1):
            r_bar = r_bar + np.einsum('ec,ecj->ej', y_bar[l], jac[l])
        pos_bar += segment_sum(r_bar, s, N) - segment_sum(r_bar, u, N)
    return x_bar, pos_bar, w_bar


# ----------------------------------------------------------------------------
# VJP-of-VJP (complex step through the forward and the VJP)
# ----------------------------------------------------------------------------

CSTEP = 1e-20


def edge_conv_vjp_vjp(spec: ConvSpec, pos, rowptr, sender, x, W, g, v_x=None,
                      v_pos=None, shift=None, edges=None, chunk: int = 4096,
                      want_W: bool = False, outputs=("g", "x", "pos"), v_W=None):
    """(g_hat, x_hat, pos_hat, W_hat) for s = <v_x, x_bar> + <v_pos, pos_bar> + <v_W, W_bar>.

    App. C Eq. C2 (second-order term) with the weight cotangent carried
    through w = R W: s is the derivative of <g, z> along (v_x, v_pos, v_W),
    so g_hat = d z / d eps and (x_hat, pos_hat, W_hat) = d (x_bar, pos_bar,
    W_bar) / d eps at (x + eps v_x, pos + eps v_pos, W + eps v_W), by
    complex step.  Each missing cotangent is zero.
    """
    h = CSTEP
    xc = x.astype(np.complex128)
    pc = pos.astype(np.complex128)
    if v_x is not None:
        xc = xc + 1j * h * v_x
    if v_pos is not None:
        pc = pc + 1j * h * v_pos
    if v_W is not None:
        W = W.astype(np.complex128) + 1j * h * v_W
    g_hat = x_hat = pos_hat = W_hat = None
    if "g" in outputs:
        g_hat = edge_conv_fwd(spec, pc, rowptr, sender, xc, W, shift, edges, chunk).imag / h
    if "x" in outputs or "pos" in outputs or want_W:
        xb, pb, Wb = edge_conv_vjp(spec, pc, rowptr, sender, xc, W, g, shift,
                                   edges, chunk, want_W)
        x_hat, pos_hat = xb.imag / h, pb.imag / h
        W_hat = Wb.imag / h if want_W else None
    return g_hat, x_hat, pos_hat, W_hat


def edge_conv_vjp_vjp_w(spec: ConvSpec, pos, rowptr, sender, x, w, g, v_x=None,
                        v_pos=None, v_w=None, shift=None, edges=None, chunk: int = 4096,
                        outputs=("g", "x", "pos", "w")):
    """(g_hat, x_hat, pos_hat, w_hat) of the explicit-weight convolution for
    s = <v_x, x_bar> + <v_pos, pos_bar> + <v_w, w_bar> (App. C Eq. C2 and
    Alg. 3 with the per-edge weights as inputs; the direction cotangent of
    Alg. 3 carried to the positions): g_hat = d z / d eps and (x_hat,
    pos_hat, w_hat) = d (x_bar, pos_bar, w_bar) / d eps of edge_conv_fwd_w
    and edge_conv_vjp_w at (x + eps v_x, pos + eps v_pos, w + eps v_w), by
    complex step.  A missing cotangent is zero.
    """
    h = CSTEP
    xc = x.astype(np.complex128)
    pc = pos.astype(np.complex128)
    wc = w.astype(np.complex128)
    if v_x is not None:
        xc = xc + 1j * h * v_x
    if v_pos is not None:
        pc = pc + 1j * h * v_pos
    if v_w is not None:
        wc = wc + 1j * h * v_w
    g_hat = x_hat = pos_hat = w_hat = None
    if "g" in outputs:
        g_hat = edge_conv_fwd_w(spec, pc, rowptr, sender, xc, wc, shift, edges, chunk).imag / h
    if "x" in outputs or "pos" in outputs or "w" in outputs:
        xb, pb, wb = edge_conv_vjp_w(spec, pc, rowptr, sender, xc, wc, g, shift, edges, chunk)
        x_hat, pos_hat, w_hat = xb.imag / h, pb.imag / h, wb.imag / h
    return g_hat, x_hat, pos_hat, w_hat
