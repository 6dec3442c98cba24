"""GPU parity of the full message-passing block (radial network, rank-wise
map, residuals, RMS norms, SiLU gates, ladder, readout) for energy and
forces on the diamond cell against the oracle."""
import numpy as np
import pytest

from oracle import model
from tests.gpu_common import assert_close
from tests.test_oracle_block import args, block_setup

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def gpu_block(cspec, lspec, w, d, entries, C, order, variant, forces=True):
    from cartesian_tensor_product_amd import flashcart as fc
    N, E = d["pos"].shape[0], len(d["sender"])
    cd = fc.conv_desc(N, E, C, 0, cspec.l_edge, cspec.l_edge, 5.0)
    ld = fc.ladder_desc(N, C, cspec.l_edge, cspec.l_edge, 0, order,
                        fc.FC_LADDER_FULL if variant == "full" else fc.FC_LADDER_PATH_REDUCED)
    flat = np.concatenate([w[name].astype(np.float32).ravel() for name, *_ in entries])
    assert fc.fc_message_block_weight_floats(cd, ld) == flat.size
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    graph = fc.DeviceGraph(d["rowptr"], d["sender"], N, device="cuda")
    en = torch.zeros(1, dtype=torch.float64, device="cuda")
    ea = torch.empty(N, device="cuda")
    F = torch.empty((N, 3), device="cuda") if forces else None
    ws = fc.workspace(fc.fc_message_block_workspace_bytes(cd, ld), "cuda")
    fc.fc_message_block_energy_forces(cd, graph, t(d["pos"]), t(d["shift"]), t(d["x"]), ld, t(flat),
                                      1.0 / np.sqrt(E / N), 1e-5, en, ea, F, ws)
    torch.cuda.synchronize()
    return float(en.item()), ea.cpu().numpy(), None if F is None else F.cpu().numpy()


@pytest.mark.parametrize("variant,order,C", [("reduced", 3, 32), ("full", 3, 32), ("reduced", 5, 32),
                                             ("reduced", 3, 96)])
def test_message_block_rattled(variant, order, C):
    """C = 32 and 96 leave lanes of the readout's channel chunks idle."""
    cspec, lspec, w, d, entries = block_setup(C=C, order=order, variant=variant)
    E, ea, F = gpu_block(cspec, lspec, w, d, entries, C, order, variant)
    Eo, eao, Fo = model.block_energy_forces(*args(cspec, lspec, w, d))
    assert abs(E - Eo) <= 1e-4 * np.abs(eao).sum()
    assert_close("e_atom", ea, eao)
    assert_close("forces", F, Fo)


def test_message_block_perfect_cell_and_energy_only():
    C = 32
    cspec, lspec, w, d, entries = block_setup(C=C, rattle=0.0)
    E, ea, F = gpu_block(cspec, lspec, w, d, entries, C, 3, "reduced")
    E2, ea2, _ = gpu_block(cspec, lspec, w, d, entries, C, 3, "reduced", forces=False)
    assert E2 == E and np.array_equal(ea, ea2)
    _, _, Fr = gpu_block(*block_setup(C=C, rattle=0.05), C, 3, "reduced")
    assert np.abs(F).max() < 1e-3 * np.abs(Fr).max()
    assert np.ptp(ea) < 1e-4 * np.abs(ea).max()


def test_message_block_without_edges():
    """r_cut below the nearest-neighbour distance: no edge, so the block is
    node-local (residual, norms, gates, ladder, readout of the embedding);
    the energy matches the oracle and the forces are zero."""
    from cartesian_tensor_product_amd import inputs
    C = 32
    cspec, lspec, w, d, entries = block_setup(C=C)
    d = inputs.diamond_inputs(channels=C, r_cut=1.0, rattle=0.05, ncell=3, n_paths=cspec.n_paths)
    assert len(d["sender"]) == 0
    from cartesian_tensor_product_amd import flashcart as fc
    N = d["pos"].shape[0]
    cd = fc.conv_desc(N, 0, C, 0, 3, 3, 1.0)
    ld = fc.ladder_desc(N, C, 3, 3, 0, 3, fc.FC_LADDER_PATH_REDUCED)
    flat = np.concatenate([w[name].astype(np.float32).ravel() for name, *_ in entries])
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    graph = fc.DeviceGraph(d["rowptr"], d["sender"], N, device="cuda")
    en = torch.zeros(1, dtype=torch.float64, device="cuda")
    F = torch.empty((N, 3), device="cuda")
    ws = fc.workspace(fc.fc_message_block_workspace_bytes(cd, ld), "cuda")
    fc.fc_message_block_energy_forces(cd, graph, t(d["pos"]), t(d["shift"]), t(d["x"]), ld, t(flat), 1.0, 1e-5, en,
                                      None, F, ws)
    torch.cuda.synchronize()
    from oracle import conv as cv
    cs1 = cv.ConvSpec(0, 3, 3, 1.0)
    Eo, eao, Fo = model.block_energy_forces(cs1, lspec, w, d["pos"].astype(np.float64), d["rowptr"], d["sender"],
                                            d["shift"].astype(np.float64), d["x"].astype(np.float64), 1.0)
    assert abs(float(en.item()) - Eo) <= 1e-4 * np.abs(eao).sum()
    assert float(F.abs().max()) == 0.0 and np.abs(Fo).max() == 0.0


def test_message_block_bitwise_deterministic():
    """No floating-point atomics anywhere: two runs give the same bits."""
    C = 32
    cspec, lspec, w, d, entries = block_setup(C=C)
    a = gpu_block(cspec, lspec, w, d, entries, C, 3, "reduced")
    b = gpu_block(cspec, lspec, w, d, entries, C, 3, "reduced")
    assert a[0] == b[0] and np.array_equal(a[1], b[1]) and np.array_equal(a[2], b[2])
