"""GPU parity of the ladder's VJP-of-VJP, full and path-reduced (cotangents
on A_grad and on the weight gradients), against the oracle's complex-step
derivatives."""
import numpy as np
import pytest

from cartesian_tensor_product_amd import inputs
from oracle import ladder
from tests.gpu_common import assert_close
from tests.test_gpu_ladder import GpuLadder

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run_vv(g, vA, vw, want=("g", "A", "W")):
    fc = g.fc
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dvw = None if vw is None else t(np.concatenate([v.ravel() for v in vw]))
    gh = torch.empty_like(g.z) if "g" in want else None
    Ah = torch.empty_like(g.dA) if "A" in want else None
    Wh = torch.empty_like(g.dW) if "W" in want else None
    ws = fc.workspace(fc.fc_ladder_workspace_bytes(g.desc, 2), "cuda")
    fc.fc_node_ladder_vjp_vjp(g.desc, g.dA, g.dW, g.saved, t(g.gz), t(vA), dvw, gh, Ah, Wh, ws)
    torch.cuda.synchronize()
    return gh, Ah, Wh


def check(g, vA, vw, want=("g", "A", "W")):
    f = lambda a: None if a is None else a.astype(np.float64)
    go, Ao, Wo = ladder.ladder_vjp_vjp(g.spec, f(g.A), [f(w) for w in g.ws], f(g.gz), v_A=f(vA),
                                       v_ws=None if vw is None else [f(v) for v in vw])
    gh, Ah, Wh = run_vv(g, vA, vw, want)
    if gh is not None:
        assert_close("g_hat", gh.cpu().numpy(), go)
    if Ah is not None:
        assert_close("A_hat", Ah.cpu().numpy(), Ao)
    if Wh is not None:
        for i, (got, wo) in enumerate(zip(g.split(Wh.cpu().numpy()), Wo)):
            # each weight block (W^q, path weights a^q, final maps) at its own scale
            assert_close(f"w_hat[{i}]", got, wo)


def cotangents(g, seed, with_A=True, with_w=True):
    rng = np.random.default_rng(seed)
    vA = inputs.normal(rng, g.A.shape) if with_A else None
    vw = [inputs.normal(rng, w.shape, std=float(np.std(w)) or 1.0) for w in g.ws] if with_w else None
    return vA, vw


@pytest.mark.parametrize("variant", ["full", "reduced"])
@pytest.mark.parametrize("l,l_out,order", [(1, 1, 1), (1, 0, 3), (2, 2, 2), (2, 1, 4), (3, 3, 4), (3, 2, 1),
                                           (4, 4, 3)])
def test_ladder_vjp_vjp_small(l, l_out, order, variant):
    g = GpuLadder(l, l_out, order, variant, C=64, N=37)
    g.fwd()
    vA, vw = cotangents(g, 40 + order)
    check(g, vA, vw)


@pytest.mark.parametrize("variant", ["full", "reduced"])
@pytest.mark.parametrize("which", ["A", "w"])
def test_ladder_vjp_vjp_one_cotangent(which, variant):
    g = GpuLadder(3, 3, 4, variant, C=32, N=29)
    g.fwd()
    vA, vw = cotangents(g, 7, with_A=which == "A", with_w=which == "w")
    check(g, vA, vw)


@pytest.mark.parametrize("variant", ["full", "reduced"])
def test_ladder_vjp_vjp_single_outputs(variant):
    g = GpuLadder(2, 2, 3, variant, C=32, N=21)
    g.fwd()
    vA, vw = cotangents(g, 8)
    for want in (("g",), ("A",), ("W",)):
        check(g, vA, vw, want)


@pytest.mark.parametrize("variant", ["full", "reduced"])
def test_ladder_vjp_vjp_workload_sampled(variant):
    """4096 nodes, 128 channels, ranks <= 3, order 4 (the ladder workload),
    position-free training derivative with v_A only (as the pages time it);
    g_hat and A_hat compared on 24 sampled nodes (the ladder is node-local)."""
    g = GpuLadder(3, 3, 4, variant, C=128, N=4096)
    g.fwd()
    vA, _ = cotangents(g, 10, with_w=False)
    gh, Ah, _ = run_vv(g, vA, None, want=("g", "A"))
    nodes = np.random.default_rng(11).choice(4096, size=24, replace=False)
    f = lambda a: a.astype(np.float64)
    go, Ao, _ = ladder.ladder_vjp_vjp(g.spec, f(g.A[nodes]), [f(w) for w in g.ws], f(g.gz[nodes]), v_A=f(vA[nodes]))
    assert_close("g_hat", gh.cpu().numpy()[nodes], go)
    assert_close("A_hat", Ah.cpu().numpy()[nodes], Ao)


@pytest.mark.parametrize("variant", ["full", "reduced"])
def test_ladder_vjp_vjp_bitwise_deterministic(variant):
    g = GpuLadder(2, 2, 3, variant, C=32, N=300)
    g.fwd()
    vA, vw = cotangents(g, 13)
    a = [x.cpu().numpy() for x in run_vv(g, vA, vw)]
    b = [x.cpu().numpy() for x in run_vv(g, vA, vw)]
    for p, q in zip(a, b):
        assert np.array_equal(p, q)
