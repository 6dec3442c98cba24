"""GPU parity of the diamond-cell block (edge convolution with scalar
senders, 1/sqrt(N_bar), order-5 path-reduced ladder, energy and forces)."""
import numpy as np
import pytest

from cartesian_tensor_product_amd import inputs
from oracle import model
from tests.gpu_common import assert_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run(rattle, channels=128, ncell=5):
    from cartesian_tensor_product_amd import flashcart as fc
    cspec, lspec = model.diamond_specs(channels, 5.0)
    shapes = [(s[1], s[2], s[3]) for s in lspec.weight_shapes()]
    d = inputs.diamond_inputs(channels=channels, r_cut=5.0, rattle=rattle, ncell=ncell,
                              n_paths=cspec.n_paths, ladder_weight_shapes=shapes)
    N, E = d["pos"].shape[0], len(d["sender"])
    nbar = E / N
    dev = "cuda"
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    cd = fc.conv_desc(N, E, channels, 0, 3, 3, 5.0)
    ld = fc.ladder_desc(N, channels, 3, 3, 0, 5, fc.FC_LADDER_PATH_REDUCED)
    graph = fc.DeviceGraph(d["rowptr"], d["sender"], N, device=dev)
    lw = t(np.concatenate([w.ravel() for w in d["ladder_weights"]]))
    energy = torch.zeros(1, dtype=torch.float64, device=dev)
    e_atom = torch.empty(N, device=dev)
    forces = torch.empty((N, 3), device=dev)
    ws = fc.workspace(fc.fc_block_workspace_bytes(cd, ld), dev)
    fc.fc_block_energy_forces(cd, graph, t(d["pos"]), t(d["shift"]), t(d["x"]), t(d["W"]), ld, lw,
                              1.0 / np.sqrt(nbar), energy, e_atom, forces, ws)
    torch.cuda.synchronize()
    f = lambda a: a.astype(np.float64)
    E0, ea0, F0, _ = model.energy_forces(cspec, lspec, f(d["pos"]), d["rowptr"], d["sender"], f(d["shift"]),
                                         f(d["x"]), f(d["W"]), [f(w) for w in d["ladder_weights"]], n_bar=nbar)
    return (energy.item(), e_atom.cpu().numpy(), forces.cpu().numpy()), (E0, ea0, F0), nbar


def test_diamond_rattled():
    (E, ea, F), (E0, ea0, F0), nbar = run(0.05)
    assert nbar > 80
    assert_close("e_atom", ea, ea0)
    assert abs(E - E0) <= 1e-4 * np.abs(ea0).sum()
    assert_close("forces", F, F0)


def test_diamond_perfect_cell():
    """1000 atoms, 86 neighbours each.  Forces vanish by symmetry, so their
    tolerance uses the rattled cell's force scale (the fp32-rounded lattice is
    symmetric only to about 1e-6 A)."""
    (E, ea, F), (E0, ea0, F0), nbar = run(0.0)
    assert nbar == 86
    _, (_, _, Fr), _ = run(0.05)
    assert_close("e_atom", ea, ea0)
    assert abs(E - E0) <= 1e-4 * np.abs(ea0).sum()
    assert_close("forces", F, F0, floor=np.abs(Fr).max())
