"""GPU parity of the path-summed convolution (FC_CONV_SUM_PATHS: the outputs
of all paths of one output rank added into one block, the kernel option of
App. D "Executing Cartesian tensor products") against the oracle: forward,
VJP, explicit per-edge weights and VJP-of-VJP."""
import numpy as np
import pytest

from cartesian_tensor_product_amd import inputs
from oracle import conv
from tests.gpu_common import GpuConv, assert_close, f64, sample_edges
from tests.test_gpu_conv_w import GpuConvW
from tests.test_gpu_conv_w import oracle as oracle_w

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def summed(ranks, rc=6.0):
    return conv.ConvSpec(*ranks, rc, sum_paths=True)


def flags():
    from cartesian_tensor_product_amd import flashcart as fc
    return fc.FC_CONV_SUM_PATHS


def oracle_all(spec, d, edges=None, g=None):
    a = (spec, f64(d["pos"]), d["rowptr"], d["sender"], f64(d["x"]), f64(d["W"]))
    z = conv.edge_conv_fwd(*a, shift=f64(d.get("shift")), edges=edges)
    g = d["g"] if g is None else g
    xb, pb, Wb = conv.edge_conv_vjp(*a, f64(g), shift=f64(d.get("shift")), edges=edges, want_W=True)
    return z, xb, pb, Wb


def check_full(ranks, d, C, rc=6.0):
    spec = summed(ranks, rc)
    gc = GpuConv(ranks, rc, d, C, flags=flags())
    assert gc.nout == spec.n_out
    z = gc.fwd()
    xb, pb, Wb = gc.vjp(want_W=True)
    torch.cuda.synchronize()
    zo, xo, po, Wo = oracle_all(spec, d)
    assert_close("z", z.cpu().numpy(), zo)
    assert_close("x_grad", xb.cpu().numpy(), xo)
    assert_close("pos_grad", pb.cpu().numpy(), po)
    assert_close("radial_w_grad", Wb.cpu().numpy(), Wo)


def summed_inputs(ranks, C, seed=21, n=40, k=12, box=5.0, rc=6.0, **kw):
    spec = summed(ranks, rc)
    return spec, inputs.edge_conv_inputs(seed, n, k, box, C, spec.n_in, spec.n_paths, spec.n_out, **kw)


@pytest.mark.parametrize("ranks", [(1, 1, 1), (2, 2, 2), (3, 3, 3), (4, 4, 4)])
def test_summed_every_rank(ranks):
    """Ranks 3 and 4 split the paths of one output rank over two path groups,
    the second adding to the first's output."""
    _, d = summed_inputs(ranks, 40)
    check_full(ranks, d, 40)


@pytest.mark.parametrize("C", [1, 65, 256])
def test_summed_channel_tiles(C):
    _, d = summed_inputs((2, 2, 2), C, seed=22, n=48, k=20, box=8.0)
    check_full((2, 2, 2), d, C)


@pytest.mark.parametrize("ranks", [(2, 2, 2), (3, 3, 3)])
def test_summed_explicit_weights(ranks):
    spec = summed(ranks)
    d = inputs.edge_conv_inputs(23, 40, 12, 5.0, 40, spec.n_in, spec.n_paths, spec.n_out, with_edge_w=True)
    gc = GpuConvW(ranks, d, 40, 6.0, flags=flags())
    z = gc.fwd()
    xb, pb, wb = gc.vjp()
    torch.cuda.synchronize()
    zo, xo, po, wo = oracle_w(spec, d)
    assert_close("z", z.cpu().numpy(), zo)
    assert_close("x_grad", xb.cpu().numpy(), xo)
    assert_close("pos_grad", pb.cpu().numpy(), po)
    assert_close("w_grad", wb.cpu().numpy(), wo)


@pytest.mark.parametrize("ranks", [(1, 1, 1), (2, 2, 2), (3, 3, 3), (4, 4, 4)])
def test_summed_vjp_vjp(ranks):
    spec, d = summed_inputs(ranks, 24, seed=24, with_vpos=True)
    rng = np.random.default_rng(25)
    v_x = inputs.normal(rng, d["x"].shape)
    v_W = inputs.normal(rng, d["W"].shape)
    gc = GpuConv(ranks, 6.0, d, 24, flags=flags())
    gh, xh, ph, Wh = gc.vjp_vjp(v_x=v_x, v_pos=d["v_pos"], v_W=v_W, want=("g", "x", "pos", "W"))
    torch.cuda.synchronize()
    go, xo, po, Wo = conv.edge_conv_vjp_vjp(spec, f64(d["pos"]), d["rowptr"], d["sender"], f64(d["x"]),
                                            f64(d["W"]), f64(d["g"]), v_x=f64(v_x), v_pos=f64(d["v_pos"]),
                                            v_W=f64(v_W), want_W=True)
    assert_close("g_hat", gh.cpu().numpy(), go)
    assert_close("x_hat", xh.cpu().numpy(), xo)
    assert_close("pos_hat", ph.cpu().numpy(), po)
    assert_close("radial_w_hat", Wh.cpu().numpy(), Wo)


def test_summed_microbenchmark_sampled():
    """1024 nodes x 128 neighbours x 128 channels at rank 2, 12 sampled
    nodes compared element by element."""
    spec = summed((2, 2, 2), 5.0)
    d = inputs.edge_conv_inputs(1, 1024, 128, 20.0, 128, spec.n_in, spec.n_paths, spec.n_out)
    gc = GpuConv((2, 2, 2), 5.0, d, 128, flags=flags())
    z = gc.fwd()
    xb, pb = gc.vjp()
    torch.cuda.synchronize()
    nodes = np.random.default_rng(98).choice(1024, size=12, replace=False)
    zo, xo, po, _ = oracle_all(spec, d, edges=sample_edges(d["rowptr"], d["sender"], nodes))
    assert_close("z", z.cpu().numpy()[nodes], zo[nodes])
    assert_close("x_grad", xb.cpu().numpy()[nodes], xo[nodes])
    assert_close("pos_grad", pb.cpu().numpy()[nodes], po[nodes])
