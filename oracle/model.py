"""Oracle for the diamond-cell composition: one edge convolution, then an
order-5 path-reduced ladder; energy = sum of rank-0 outputs; forces = -dE/dpos.

TEST INFRASTRUCTURE ONLY.  Follows the FlashCart paper, App. E (a message-
passing block is a convolution followed by the product ladder; the first
convolution has scalar sender features and four paths; Eq. E1 scales the
convolution by 1/sqrt(N_bar); the final block returns scalars), and §2
(F_u = -grad_{r_u} E).  Residual updates, normalisation, gates and the
readout MLP are left out (they carry trained weights).

Pins (tests/test_oracle_model.py): perfect diamond gives zero forces and
equal per-atom energies (every site is equivalent, with tetrahedral site
symmetry); complex-step derivatives of E reproduce the forces on the
rattled cell.

The full message-passing block at the end of this file adds the pages'
channel map before the convolution, the radial network, the rank-wise
path/channel map, residual updates, the
equivariant RMS normalisation, scalar SiLU gates with their output map and
a readout MLP (random weights); its pins are the same three properties,
plus a two-atom walkthrough (one channel, ranks <= 3, ladder of order 2)
whose energy is evaluated step by step in scalar code and whose forces are
central differences of that energy (tests/test_oracle_hand.py).
"""

from __future__ import annotations

import numpy as np

from . import conv, ladder


def diamond_specs(channels: int = 128, r_cut: float = 5.0, order: int = 5):
    cspec = conv.ConvSpec(0, 3, 3, r_cut)
    lspec = ladder.LadderSpec(3, 3, 0, order, "reduced", channels)
    return cspec, lspec


def energy_forces(cspec, lspec, pos, rowptr, sender, shift, x, W, lws, n_bar: float):
    """Returns (E, per-atom energies, forces [N,3], A)."""
    s = 1.0 / np.sqrt(n_bar)
    A = s * conv.edge_conv_fwd(cspec, pos, rowptr, sender, x, W, shift=shift)
    z = ladder.ladder_fwd(lspec, A, lws)
    e_atom = z[:, 0, :].sum(axis=1)
    gz = np.zeros(z.shape)
    gz[:, 0, :] = 1.0
    A_bar, _ = ladder.ladder_vjp(lspec, A, lws, gz)
    _, pos_bar, _ = conv.edge_conv_vjp(cspec, pos, rowptr, sender, x, W, s * A_bar, shift=shift)
    return float(np.sum(e_atom)) if not np.iscomplexobj(e_atom) else np.sum(e_atom), e_atom, -pos_bar, A


def energy(cspec, lspec, pos, rowptr, sender, shift, x, W, lws, n_bar: float):
    s = 1.0 / np.sqrt(n_bar)
    A = s * conv.edge_conv_fwd(cspec, pos, rowptr, sender, x, W, shift=shift)
    z = ladder.ladder_fwd(lspec, A, lws)
    return np.sum(z[:, 0, :])


# ----------------------------------------------------------------------------
# A full message-passing block (App. E "Model architecture")
# ----------------------------------------------------------------------------
#
# The block as the pages describe it, with random weights, for one final block
# (scalar senders in, scalars out).  Readings where the pages leave a step
# open:
#   hb  = Mpre h0 (the d x d channel map applied to the sender features of
#         each rank before the convolution; scalars only here);
#   a   = N_bar^{-1/2} conv(hb) with the radial network's weights (Eq. E1);
#   m_l = M_l a_l (rank-wise map of the paths -- one per rank with scalar
#         senders -- and channels), m_0 += R0 h0 (residual: a learned linear
#         map of the block input);
#   n   = RMSnorm(m; gamma1);  gates y_0 = SiLU(n_0), y_l = SiLU(n_0) * n_l;
#   A_l = n_l + O_l y_l (the learned output map added to the gated layer's
#         input);  z = ladder(A) (l_out = 0);  o = z + R2 A_0 (residual);
#   f   = RMSnorm(o; gamma2);  E_u = readout(f_0), a bias-free MLP
#         C -> 64 -> 64 -> 1 with SiLU;  E = sum_u E_u;  F = -dE/dpos.
# Matrices act on the channel index as [out][in].

BLOCK_HIDDEN = 64


def block_weight_shapes(C: int, l_e: int, n_paths: int, lspec):
    """(name, shape) of the block's flat weights, in order."""
    out = [("mlp", (8 * 64 + 64 * 64 + 64 * n_paths * C,)), ("Mpre", (C, C)), ("M", (l_e + 1, C, C)), ("R0", (C, C)),
           ("gamma1", (l_e + 1, C)), ("O", (l_e + 1, C, C))]
    out += [(f"ladder{i}", s[1]) for i, s in enumerate(lspec.weight_shapes())]
    out += [("R2", (C, C)), ("gamma2", (1, C)), ("Wr1", (C, BLOCK_HIDDEN)), ("Wr2", (BLOCK_HIDDEN, BLOCK_HIDDEN)),
            ("wr3", (BLOCK_HIDDEN,))]
    return out


def _rank_map(X, M, l_e):
    """Y_l[u, c, j] = sum_k M[l][j, k] X_l[u, c, k] for every rank l <= l_e."""
    off = [l * l for l in range(l_e + 2)]
    Y = np.empty(X.shape, dtype=np.result_type(X, M))
    for l in range(l_e + 1):
        Y[:, off[l]:off[l + 1], :] = np.einsum('uck,jk->ucj', X[:, off[l]:off[l + 1], :], M[l])
    return Y


def _rank_map_t(G, M, l_e):
    """Adjoint of _rank_map: X_bar_l = G_l M_l."""
    off = [l * l for l in range(l_e + 2)]
    Y = np.empty(G.shape, dtype=np.result_type(G, M))
    for l in range(l_e + 1):
        Y[:, off[l]:off[l + 1], :] = np.einsum('ucj,jk->uck', G[:, off[l]:off[l + 1], :], M[l])
    return Y


def _block_forward(cspec, lspec, w, pos, rowptr, sender, shift, h0, n_bar, eps):
    from . import norm, radial
    C, l_e = h0.shape[-1], cspec.l_edge
    P = cspec.n_paths
    mlp = w["mlp"]
    W1, W2, W3 = mlp[:512].reshape(8, 64), mlp[512:4608].reshape(64, 64), mlp[4608:].reshape(64, P * C)
    s = 1.0 / np.sqrt(n_bar)
    hb = np.einsum('uk,jk->uj', h0[:, 0, :], w["Mpre"])[:, None, :]
    a = s * radial.edge_conv_fwd_mlp(cspec, pos, rowptr, sender, hb, W1, W2, W3, shift=shift)
    m = _rank_map(a, w["M"], l_e)
    m[:, 0, :] = m[:, 0, :] + np.einsum('uk,jk->uj', h0[:, 0, :], w["R0"])
    n, _ = norm.rms_norm_fwd(m, l_e, eps, w["gamma1"])
    sg = radial.silu(n[:, 0, :])
    y = n * sg[:, None, :]
    y[:, 0, :] = sg
    A = n + _rank_map(y, w["O"], l_e)
    lws = [w[f"ladder{i}"] for i in range(len(lspec.weight_shapes()))]
    from . import ladder as lad
    z = lad.ladder_fwd(lspec, A, lws)
    o = z + np.einsum('uk,jk->uj', A[:, 0, :], w["R2"])[:, None, :]
    f, _ = norm.rms_norm_fwd(o, 0, eps, w["gamma2"])
    h1 = radial.silu(f[:, 0, :] @ w["Wr1"])
    h2 = radial.silu(h1 @ w["Wr2"])
    e_atom = h2 @ w["wr3"]
    return dict(hb=hb, a=a, m=m, n=n, sg=sg, y=y, A=A, z=z, o=o, f=f, h1=h1, e_atom=e_atom, W=(W1, W2, W3),
                lws=lws)


def block_energy(cspec, lspec, w, pos, rowptr, sender, shift, h0, n_bar, eps=1e-5):
    st = _block_forward(cspec, lspec, w, pos, rowptr, sender, shift, h0, n_bar, eps)
    return np.sum(st["e_atom"]), st["e_atom"]


def block_energy_forces(cspec, lspec, w, pos, rowptr, sender, shift, h0, n_bar, eps=1e-5):
    """(E, e_atom [N], forces [N, 3]); the backward written out by hand from
    the oracles of each step."""
    from . import norm, radial
    from . import ladder as lad
    C, l_e = h0.shape[-1], cspec.l_edge
    st = _block_forward(cspec, lspec, w, pos, rowptr, sender, shift, h0, n_bar, eps)
    f0 = st["f"][:, 0, :]
    a1 = f0 @ w["Wr1"]
    a2 = st["h1"] @ w["Wr2"]
    a2b = w["wr3"][None, :] * radial.silu_grad(a2)
    a1b = (a2b @ w["Wr2"].T) * radial.silu_grad(a1)
    fb = np.zeros(st["f"].shape)
    fb[:, 0, :] = a1b @ w["Wr1"].T
    ob, _ = norm.rms_norm_vjp(st["o"], 0, eps, fb, w["gamma2"])
    Ab, _ = lad.ladder_vjp(lspec, st["A"], st["lws"], ob)
    Ab[:, 0, :] = Ab[:, 0, :] + np.einsum('uj,jk->uk', ob[:, 0, :], w["R2"])
    yb = _rank_map_t(Ab, w["O"], l_e)
    n, sg = st["n"], st["sg"]
    dsg = radial.silu_grad(n[:, 0, :])
    nb = Ab.copy()
    nb[:, 1:, :] += sg[:, None, :] * yb[:, 1:, :]
    nb[:, 0, :] += dsg * (yb[:, 0, :] + np.sum(yb[:, 1:, :] * n[:, 1:, :], axis=1))
    mb, _ = norm.rms_norm_vjp(st["m"], l_e, eps, nb, w["gamma1"])
    ab = _rank_map_t(mb, w["M"], l_e)
    s = 1.0 / np.sqrt(n_bar)
    W1, W2, W3 = st["W"]
    _, pb, _, _, _ = radial.edge_conv_vjp_mlp(cspec, pos, rowptr, sender, st["hb"], W1, W2, W3, s * ab, shift=shift)
    return float(np.sum(st["e_atom"])), st["e_atom"], -pb
