"""GPU parity of the node-local correlation ladder (full Eq. 2 and
path-reduced products) and its VJP against the oracle."""
import numpy as np
import pytest

from cartesian_tensor_product_amd import inputs
from oracle import ladder
from tests.gpu_common import assert_close

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


class GpuLadder:
    def __init__(self, l, l_out, order, variant, C, N, seed=3):
        from cartesian_tensor_product_amd import flashcart as fc
        self.fc = fc
        self.spec = ladder.LadderSpec(l, l, l_out, order, variant, C)
        shapes = [(s[1], s[2], s[3]) for s in self.spec.weight_shapes()]
        rng, A, ws = inputs.ladder_inputs(seed, N, C, self.spec.a_off[-1], shapes)
        self.gz = inputs.ladder_cotangent(rng, N, self.spec.n_out_rows(), C)
        self.A, self.ws = A, ws
        self.desc = fc.ladder_desc(N, C, l, l, l_out, order,
                                   fc.FC_LADDER_FULL if variant == "full" else fc.FC_LADDER_PATH_REDUCED)
        nw, ns = fc.fc_ladder_layout(self.desc)
        assert nw == sum(w.size for w in ws), (nw, [w.shape for w in ws])
        dev = "cuda"
        self.dA = torch.from_numpy(A).to(dev)
        self.dW = torch.from_numpy(np.concatenate([w.ravel() for w in ws])).to(dev)
        self.saved = torch.empty(max(ns, 1), device=dev)
        self.z = torch.empty((N, self.spec.n_out_rows(), C), device=dev)
        self.wsf = fc.workspace(fc.fc_ladder_workspace_bytes(self.desc, 0), dev)
        self.wsb = fc.workspace(fc.fc_ladder_workspace_bytes(self.desc, 1), dev)
        self.N, self.C = N, C

    def fwd(self):
        self.fc.fc_node_ladder_fwd(self.desc, self.dA, self.dW, self.z, self.saved, self.wsf)
        return self.z

    def vjp(self, gz=None):
        gz = self.gz if gz is None else gz
        dg = torch.from_numpy(np.ascontiguousarray(gz)).to("cuda")
        Ab = torch.empty_like(self.dA)
        Wb = torch.empty_like(self.dW)
        self.fc.fc_node_ladder_vjp(self.desc, self.dA, self.dW, self.saved, dg, Ab, Wb, self.wsb)
        return Ab, Wb

    def split(self, flat):
        out, o = [], 0
        for w in self.ws:
            out.append(flat[o:o + w.size].reshape(w.shape))
            o += w.size
        return out


CASES = [(l, lo, order, var) for var in ("full", "reduced") for (l, lo, order) in
         [(1, 1, 1), (1, 0, 3), (2, 2, 2), (2, 1, 4), (3, 3, 4), (3, 0, 5), (3, 2, 1), (4, 4, 3), (4, 0, 2)]]


@pytest.mark.parametrize("l,l_out,order,variant", CASES)
def test_ladder_small(l, l_out, order, variant):
    g = GpuLadder(l, l_out, order, variant, C=64, N=37)
    z = g.fwd()
    Ab, Wb = g.vjp()
    torch.cuda.synchronize()
    f = lambda a: a.astype(np.float64)
    zo = ladder.ladder_fwd(g.spec, f(g.A), [f(w) for w in g.ws])
    Ao, Wo = ladder.ladder_vjp(g.spec, f(g.A), [f(w) for w in g.ws], f(g.gz))
    assert_close("z", z.cpu().numpy(), zo)
    assert_close("A_grad", Ab.cpu().numpy(), Ao)
    for i, (got, want) in enumerate(zip(g.split(Wb.cpu().numpy()), Wo)):
        assert_close(f"w_grad[{i}]", got, want)


@pytest.mark.parametrize("variant", ["full", "reduced"])
def test_ladder_workload_sampled(variant):
    """4096 nodes, 128 channels, ranks <= 3, order 4; 24 sampled nodes for z
    and A_grad, and weight gradients of a cotangent restricted to 48 nodes
    (the weight gradient is a sum over nodes, so the oracle needs only those)."""
    g = GpuLadder(3, 3, 4, variant, C=128, N=4096)
    z = g.fwd()
    Ab, _ = g.vjp()
    torch.cuda.synchronize()
    rng = np.random.default_rng(123)
    nodes = np.sort(rng.choice(4096, size=24, replace=False))
    f = lambda a: a.astype(np.float64)
    W64 = [f(w) for w in g.ws]
    zo = ladder.ladder_fwd(g.spec, f(g.A), W64, nodes=nodes)
    assert_close("z", z.cpu().numpy()[nodes], zo)
    Ao, _ = ladder.ladder_vjp(g.spec, f(g.A), W64, f(g.gz), nodes=nodes)
    assert_close("A_grad", Ab.cpu().numpy()[nodes], Ao)
    wn = np.sort(rng.choice(4096, size=48, replace=False))
    gm = np.zeros_like(g.gz)
    gm[wn] = g.gz[wn]
    _, Wb = g.vjp(gm)
    torch.cuda.synchronize()
    _, Wo = ladder.ladder_vjp(g.spec, f(g.A), W64, f(gm), nodes=wn)
    for i, (got, want) in enumerate(zip(g.split(Wb.cpu().numpy()), Wo)):
        assert_close(f"w_grad[{i}]", got, want)


def test_ladder_determinism():
    g = GpuLadder(3, 3, 4, "full", C=128, N=512)
    a = [g.fwd().clone(), *g.vjp()]
    b = [g.fwd().clone(), *g.vjp()]
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


@pytest.mark.parametrize("C", [32, 160, 288])
@pytest.mark.parametrize("l,l_out,order,variant", [(2, 2, 3, "full"), (3, 3, 2, "reduced")])
def test_ladder_channel_tiles(l, l_out, order, variant, C):
    """Channel counts that leave the 128-wide GEMM tiles partly filled (32),
    or add a ragged last tile (160, 288), with a ragged node count."""
    g = GpuLadder(l, l_out, order, variant, C=C, N=45, seed=11)
    z = g.fwd()
    Ab, Wb = g.vjp()
    torch.cuda.synchronize()
    f = lambda a: a.astype(np.float64)
    zo = ladder.ladder_fwd(g.spec, f(g.A), [f(w) for w in g.ws])
    Ao, Wo = ladder.ladder_vjp(g.spec, f(g.A), [f(w) for w in g.ws], f(g.gz))
    assert_close("z", z.cpu().numpy(), zo)
    assert_close("A_grad", Ab.cpu().numpy(), Ao)
    for i, (got, want) in enumerate(zip(g.split(Wb.cpu().numpy()), Wo)):
        assert_close(f"w_grad[{i}]", got, want)


@pytest.mark.parametrize("l,l_out", [(2, 2), (3, 1)])
def test_ladder_reduced_order1_without_saved_states(l, l_out):
    """Order 1 needs no saved states: without them the path-reduced VJP forms
    the final state again instead of reading the forward's copy."""
    g = GpuLadder(l, l_out, 1, "reduced", C=64, N=37)
    g.fc.fc_node_ladder_fwd(g.desc, g.dA, g.dW, g.z, None, g.wsf)
    dg = torch.from_numpy(np.ascontiguousarray(g.gz)).to("cuda")
    Ab, Wb = torch.empty_like(g.dA), torch.empty_like(g.dW)
    g.fc.fc_node_ladder_vjp(g.desc, g.dA, g.dW, None, dg, Ab, Wb, g.wsb)
    torch.cuda.synchronize()
    f = lambda a: a.astype(np.float64)
    zo = ladder.ladder_fwd(g.spec, f(g.A), [f(w) for w in g.ws])
    Ao, Wo = ladder.ladder_vjp(g.spec, f(g.A), [f(w) for w in g.ws], f(g.gz))
    assert_close("z", g.z.cpu().numpy(), zo)
    assert_close("A_grad", Ab.cpu().numpy(), Ao)
    for i, (got, want) in enumerate(zip(g.split(Wb.cpu().numpy()), Wo)):
        assert_close(f"w_grad[{i}]", got, want)
