"""Pins of the diamond-cell composition oracle."""
import numpy as np
import pytest

from cartesian_tensor_product_amd import inputs
from oracle import model


def load(rattle, channels=8, ncell=2, r_cut=3.0):
    cspec, lspec = model.diamond_specs(channels, r_cut)
    shapes = [(s[1], s[2], s[3]) for s in lspec.weight_shapes()]
    d = inputs.diamond_inputs(channels=channels, r_cut=r_cut, rattle=rattle, ncell=ncell,
                              n_paths=cspec.n_paths, ladder_weight_shapes=shapes)
    f = lambda a: a.astype(np.float64)
    return cspec, lspec, d, (f(d["pos"]), d["rowptr"], d["sender"], f(d["shift"]), f(d["x"]),
                             f(d["W"]), [f(w) for w in d["ladder_weights"]])


def test_perfect_diamond_symmetry():
    cspec, lspec, d, args = load(0.0)
    nbar = float(np.mean(np.diff(d["rowptr"])))
    E, e_atom, F, A = model.energy_forces(cspec, lspec, *args, n_bar=nbar)
    _, _, Fr, _ = model.energy_forces(*load(0.05)[:2], *load(0.05)[3], n_bar=nbar)
    scale = np.abs(Fr).max()
    assert scale > 1e-3
    # positions are rounded to fp32 (~1e-6 A), which breaks the lattice
    # symmetry at that level; exact symmetry would give exact zeros
    assert np.abs(F).max() < 1e-5 * scale
    assert np.allclose(e_atom, e_atom[0], rtol=1e-4)
    # tetrahedral sites: the rank-1 and rank-2 blocks of the atomic basis vanish
    assert np.abs(A[:, 1:9, :]).max() < 1e-5 * np.abs(A).max()
    assert np.abs(A[:, 9:16, :]).max() > 1e-3 * np.abs(A).max()


def test_rattled_forces_complex_step():
    cspec, lspec, d, args = load(0.05)
    nbar = float(np.mean(np.diff(d["rowptr"])))
    E, _, F, _ = model.energy_forces(cspec, lspec, *args, n_bar=nbar)
    pos = args[0]
    for (i, j) in [(0, 0), (3, 1), (17, 2), (40, 0)]:
        pc = pos.astype(complex)
        pc[i, j] += 1e-20j
        dE = model.energy(cspec, lspec, pc, *args[1:], n_bar=nbar).imag / 1e-20
        assert -dE == pytest.approx(F[i, j], rel=1e-8, abs=1e-10 * np.abs(F).max())
    assert np.abs(F.sum(0)).max() < 1e-9 * np.abs(F).max()
