"""GPU parity of the edge-convolution VJP-of-VJP (position and feature
cotangents) against the oracle's complex-step second derivatives."""
import numpy as np
import pytest

from cartesian_tensor_product_amd import inputs
from oracle import conv
from tests.gpu_common import GpuConv, assert_close, f64, sample_edges

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def oracle_vv(spec, d, v_x, v_pos, edges=None, g=None, v_W=None):
    g = d["g"] if g is None else g
    return conv.edge_conv_vjp_vjp(spec, f64(d["pos"]), d["rowptr"], d["sender"], f64(d["x"]), f64(d["W"]),
                                  f64(g), v_x=f64(v_x), v_pos=f64(v_pos), shift=f64(d.get("shift")),
                                  edges=edges, want_W=True, v_W=f64(v_W))


@pytest.mark.parametrize("ranks", [(1, 1, 1), (2, 2, 2), (3, 3, 3), (4, 4, 4), (5, 5, 5), (0, 3, 3), (2, 3, 3)])
@pytest.mark.parametrize("with_vx", [False, True])
def test_vjp_vjp_small(ranks, with_vx):
    spec = conv.ConvSpec(*ranks, 6.0)
    C = 24
    d = inputs.edge_conv_inputs(7, 40, 12, 5.0, C, spec.n_in, spec.n_paths, spec.n_out, with_vpos=True)
    rng = np.random.default_rng(8)
    v_x = inputs.normal(rng, d["x"].shape) if with_vx else None
    gc = GpuConv(ranks, 6.0, d, C)
    gh, xh, ph, Wh = gc.vjp_vjp(v_x=v_x, v_pos=d["v_pos"], want=("g", "x", "pos", "W"))
    torch.cuda.synchronize()
    go, xo, po, Wo = oracle_vv(spec, d, v_x, d["v_pos"])
    assert_close("g_hat", gh.cpu().numpy(), go)
    assert_close("x_hat", xh.cpu().numpy(), xo)
    assert_close("pos_hat", ph.cpu().numpy(), po)
    assert_close("radial_w_hat", Wh.cpu().numpy(), Wo)


@pytest.mark.parametrize("ranks", [(1, 1, 1), (2, 2, 2), (3, 3, 3), (4, 4, 4)])
@pytest.mark.parametrize("with_vx", [False, True])
def test_vjp_vjp_all_parities(ranks, with_vx):
    """Every triangle-allowed path (odd J through the Levi-Civita reading)."""
    from cartesian_tensor_product_amd import flashcart as fc
    spec = conv.ConvSpec(*ranks, 6.0, all_parities=True)
    C = 24
    d = inputs.edge_conv_inputs(7, 40, 12, 5.0, C, spec.n_in, spec.n_paths, spec.n_out, with_vpos=True)
    rng = np.random.default_rng(8)
    v_x = inputs.normal(rng, d["x"].shape) if with_vx else None
    gc = GpuConv(ranks, 6.0, d, C, flags=fc.FC_CONV_ALL_PARITIES)
    gh, xh, ph, Wh = gc.vjp_vjp(v_x=v_x, v_pos=d["v_pos"], want=("g", "x", "pos", "W"))
    torch.cuda.synchronize()
    go, xo, po, Wo = oracle_vv(spec, d, v_x, d["v_pos"])
    assert_close("g_hat", gh.cpu().numpy(), go)
    assert_close("x_hat", xh.cpu().numpy(), xo)
    assert_close("pos_hat", ph.cpu().numpy(), po)
    assert_close("radial_w_hat", Wh.cpu().numpy(), Wo)


@pytest.mark.parametrize("ranks", [(3, 3, 3), (4, 4, 4)])
@pytest.mark.parametrize("with_vx", [False, True])
def test_vjp_vjp_256_channels(ranks, with_vx):
    """Four channel waves per sender block: the VJP-of-VJP then stages fewer
    edges per chunk (32 or 16 at rank 4) so its row sums fit in LDS; senders
    of about 40 edges span several chunks."""
    spec = conv.ConvSpec(*ranks, 6.0)
    C = 256
    d = inputs.edge_conv_inputs(13, 60, 40, 5.0, C, spec.n_in, spec.n_paths, spec.n_out, with_vpos=True)
    rng = np.random.default_rng(14)
    v_x = inputs.normal(rng, d["x"].shape) if with_vx else None
    gc = GpuConv(ranks, 6.0, d, C)
    gh, xh, ph, _ = gc.vjp_vjp(v_x=v_x, v_pos=d["v_pos"])
    torch.cuda.synchronize()
    go, xo, po, _ = oracle_vv(spec, d, v_x, d["v_pos"])
    assert_close("g_hat", gh.cpu().numpy(), go)
    assert_close("x_hat", xh.cpu().numpy(), xo)
    assert_close("pos_hat", ph.cpu().numpy(), po)


@pytest.mark.parametrize("ranks", [(2, 2, 2), (4, 4, 4)])
def test_radial_w_hat_ragged_receivers(ranks):
    """Receiver counts that leave the last four-receiver block partly empty,
    degrees above one 32-edge chunk, radial_w_hat requested alone."""
    spec = conv.ConvSpec(*ranks, 6.0)
    C = 40
    d = inputs.edge_conv_inputs(9, 43, 37, 6.0, C, spec.n_in, spec.n_paths, spec.n_out, with_vpos=True)
    rng = np.random.default_rng(10)
    v_x = inputs.normal(rng, d["x"].shape)
    gc = GpuConv(ranks, 6.0, d, C)
    Wh = gc.vjp_vjp(v_x=v_x, v_pos=d["v_pos"], want=("W",))[3]
    torch.cuda.synchronize()
    Wo = oracle_vv(spec, d, v_x, d["v_pos"])[3]
    assert_close("radial_w_hat", Wh.cpu().numpy(), Wo)


@pytest.mark.parametrize("ranks", [(3, 3, 3), (4, 4, 4)])
@pytest.mark.parametrize("rc", [5.0, 35.0])
def test_vjp_vjp_microbenchmark_sampled(ranks, rc):
    """1024 nodes x 128 neighbours x 128 channels, position cotangent only
    (v_x = 0), 10 sampled nodes compared element by element; r_c = 35 A
    keeps every edge of the 20 A cube inside the cutoff (at 5 A about 95 %
    of them carry zero weight)."""
    spec = conv.ConvSpec(*ranks, rc)
    d = inputs.edge_conv_inputs(2, 1024, 128, 20.0, 128, spec.n_in, spec.n_paths, spec.n_out, with_vpos=True)
    gc = GpuConv(ranks, rc, d, 128)
    gh, xh, ph, _ = gc.vjp_vjp(v_pos=d["v_pos"])
    # radial_w_hat through a cotangent that vanishes off the sampled
    # receivers: only their incoming edges contribute
    nodes = np.random.default_rng(5).choice(1024, size=10, replace=False)
    gm = np.zeros_like(d["g"])
    gm[nodes] = d["g"][nodes]
    Wh = gc.vjp_vjp(v_pos=d["v_pos"], want=("W",), g=gm)[3]
    torch.cuda.synchronize()
    edges = sample_edges(d["rowptr"], d["sender"], nodes)
    go, xo, po, _ = oracle_vv(spec, d, None, d["v_pos"], edges=edges)
    recv = np.repeat(np.arange(1024), np.diff(d["rowptr"]))
    Wo = oracle_vv(spec, d, None, d["v_pos"], edges=np.nonzero(np.isin(recv, nodes))[0], g=gm)[3]
    assert_close("g_hat", gh.cpu().numpy()[nodes], go[nodes])
    assert_close("x_hat", xh.cpu().numpy()[nodes], xo[nodes])
    assert_close("pos_hat", ph.cpu().numpy()[nodes], po[nodes])
    assert_close("radial_w_hat", Wh.cpu().numpy(), Wo)


def test_vjp_vjp_periodic_and_subsets():
    """Diamond cell with shifts; each output requested on its own."""
    spec = conv.ConvSpec(0, 3, 3, 5.0)
    d = inputs.diamond_inputs(channels=32, r_cut=5.0, rattle=0.05, ncell=3, n_paths=spec.n_paths)
    rng = np.random.default_rng(2)
    d["g"] = inputs.normal(rng, (d["pos"].shape[0], spec.n_out, 32))
    vp = inputs.normal(rng, d["pos"].shape)
    gc = GpuConv((0, 3, 3), 5.0, d, 32)
    go, xo, po, Wo = oracle_vv(spec, d, None, vp)
    for want, ref, idx in ((("g",), go, 0), (("x",), xo, 1), (("pos",), po, 2), (("W",), Wo, 3)):
        out = gc.vjp_vjp(v_pos=vp, want=want)
        torch.cuda.synchronize()
        assert_close(want[0], out[idx].cpu().numpy(), ref)


@pytest.mark.parametrize("ranks", [(1, 1, 1), (2, 2, 2), (3, 3, 3), (0, 3, 3)])
@pytest.mark.parametrize("cot", ["W", "W+pos", "W+x+pos"])
def test_vjp_vjp_weight_cotangent(ranks, cot):
    """A cotangent on the radial-weight gradient, alone or with the x and
    position cotangents (the linear part is then added to the second-order
    part)."""
    spec = conv.ConvSpec(*ranks, 6.0)
    C = 40
    d = inputs.edge_conv_inputs(17, 40, 12, 5.0, C, spec.n_in, spec.n_paths, spec.n_out, with_vpos=True)
    rng = np.random.default_rng(18)
    v_W = inputs.normal(rng, d["W"].shape)
    v_x = inputs.normal(rng, d["x"].shape) if "x" in cot else None
    v_pos = d["v_pos"] if "pos" in cot else None
    gc = GpuConv(ranks, 6.0, d, C)
    gh, xh, ph, Wh = gc.vjp_vjp(v_x=v_x, v_pos=v_pos, v_W=v_W, want=("g", "x", "pos", "W"))
    torch.cuda.synchronize()
    go, xo, po, Wo = oracle_vv(spec, d, v_x, v_pos, v_W=v_W)
    assert_close("g_hat", gh.cpu().numpy(), go)
    assert_close("x_hat", xh.cpu().numpy(), xo)
    assert_close("pos_hat", ph.cpu().numpy(), po)
    if cot == "W":
        assert float(Wh.abs().max()) == 0.0 and np.abs(Wo).max() == 0.0
    else:
        assert_close("radial_w_hat", Wh.cpu().numpy(), Wo)


@pytest.mark.parametrize("with_pos", [False, True])
def test_vjp_vjp_weight_cotangent_subsets(with_pos):
    """Each output requested on its own with the weight cotangent; g_hat
    alone without a workspace when the weight cotangent is the only one."""
    spec = conv.ConvSpec(2, 2, 2, 6.0)
    C = 24
    d = inputs.edge_conv_inputs(19, 36, 10, 5.0, C, spec.n_in, spec.n_paths, spec.n_out, with_vpos=True)
    rng = np.random.default_rng(20)
    v_W = inputs.normal(rng, d["W"].shape)
    v_pos = d["v_pos"] if with_pos else None
    gc = GpuConv((2, 2, 2), 6.0, d, C)
    ref = oracle_vv(spec, d, None, v_pos, v_W=v_W)
    for idx, want in enumerate(("g", "x", "pos", "W")):
        out = gc.vjp_vjp(v_pos=v_pos, v_W=v_W, want=(want,))
        torch.cuda.synchronize()
        if want == "W" and not with_pos:
            assert float(out[idx].abs().max()) == 0.0
        else:
            assert_close(want, out[idx].cpu().numpy(), ref[idx])
    if not with_pos:
        gh = torch.empty((gc.N, gc.nout, gc.C), device=gc.device)
        gc.fc.fc_edge_conv_vjp_vjp(gc.desc, gc.graph, gc.pos, gc.shift, gc.x, gc.W, None, None, None,
                                   torch.from_numpy(v_W).to(gc.device), gh, None, None, None, None)
        torch.cuda.synchronize()
        assert_close("g_hat", gh.cpu().numpy(), ref[0])
