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
