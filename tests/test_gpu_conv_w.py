"""GPU parity of the explicit-weight edge convolution (per-edge weights
w [E, P, C] given, as in the pages' statement of Eq. 1 and Eq. C1) against
the oracle: forward, feature and position gradients (w held fixed) and the
per-edge weight gradient."""
import numpy as np
import pytest

from cartesian_tensor_product_amd import inputs
from oracle import conv
from tests.gpu_common import assert_close, f64, sample_edges

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


class GpuConvW:
    def __init__(self, ranks, d, C, rc=6.0, flags=0):
        from cartesian_tensor_product_amd import flashcart as fc
        self.fc = fc
        self.N, self.E, self.C = d["pos"].shape[0], int(len(d["sender"])), C
        self.desc = fc.conv_desc(self.N, self.E, C, *ranks, rc, flags=flags)
        self.P, self.nin, self.nout = fc.fc_conv_layout(self.desc)
        self.graph = fc.DeviceGraph(d["rowptr"], d["sender"], self.N, device="cuda")
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.pos, self.shift, self.x, self.w, self.g = t(d["pos"]), t(d.get("shift")), t(d["x"]), t(d["w"]), t(d["g"])
        self.ws = fc.workspace(fc.fc_edge_conv_workspace_bytes(self.desc, 1), "cuda")

    def fwd(self):
        z = torch.empty((self.N, self.nout, self.C), device="cuda")
        self.fc.fc_edge_conv_fwd_w(self.desc, self.graph, self.pos, self.shift, self.x, self.w, z)
        return z

    def vjp(self, want=("x", "pos", "w")):
        xb = torch.empty_like(self.x) if "x" in want else None
        pb = torch.empty((self.N, 3), device="cuda") if "pos" in want else None
        wb = torch.empty_like(self.w) if "w" in want else None
        self.fc.fc_edge_conv_vjp_w(self.desc, self.graph, self.pos, self.shift, self.x, self.w, self.g, xb, pb, wb,
                                   self.ws)
        return xb, pb, wb


def oracle(spec, d, edges=None):
    a = (spec, f64(d["pos"]), d["rowptr"], d["sender"], f64(d["x"]), d["w"])
    z = conv.edge_conv_fwd_w(*a, shift=f64(d.get("shift")), edges=edges)
    xb, pb, wb = conv.edge_conv_vjp_w(*a, f64(d["g"]), shift=f64(d.get("shift")), edges=edges)
    return z, xb, pb, wb


def check(ranks, d, C, rc=6.0, allp=False):
    from cartesian_tensor_product_amd import flashcart as fc
    spec = conv.ConvSpec(*ranks, rc, all_parities=allp)
    gc = GpuConvW(ranks, d, C, rc, flags=fc.FC_CONV_ALL_PARITIES if allp else 0)
    z = gc.fwd()
    xb, pb, wb = gc.vjp()
    torch.cuda.synchronize()
    zo, xo, po, wo = oracle(spec, d)
    assert_close("z", z.cpu().numpy(), zo)
    assert_close("x_grad", xb.cpu().numpy(), xo)
    assert_close("pos_grad", pb.cpu().numpy(), po)
    assert_close("w_grad", wb.cpu().numpy(), wo)
    return gc


def small(ranks, C, seed=11, n=40, k=12, box=5.0, rc=6.0, allp=False):
    spec = conv.ConvSpec(*ranks, rc, all_parities=allp)
    return inputs.edge_conv_inputs(seed, n, k, box, C, spec.n_in, spec.n_paths, spec.n_out, with_edge_w=True)


@pytest.mark.parametrize("ranks", [(0, 0, 0), (1, 1, 1), (2, 2, 2), (3, 3, 3), (4, 4, 4), (5, 5, 5), (0, 3, 3),
                                   (1, 2, 2), (2, 4, 4), (3, 4, 4)])
def test_explicit_weights_every_rank_set(ranks):
    check(ranks, small(ranks, 24), 24)


@pytest.mark.parametrize("ranks", [(1, 1, 1), (2, 2, 2), (4, 4, 4)])
def test_explicit_weights_all_parities(ranks):
    check(ranks, small(ranks, 24, allp=True), 24, allp=True)


@pytest.mark.parametrize("C", [1, 65, 200])
def test_explicit_weights_channel_tiles(C):
    check((2, 2, 2), small((2, 2, 2), C, seed=3, n=100, k=70, box=8.0), C)


def test_explicit_weights_zero_length_edge_and_partial_outputs():
    """Coincident atoms give an edge of zero length, which takes no part;
    each output requested on its own."""
    ranks = (2, 2, 2)
    d = small(ranks, 32, seed=5)
    recv = np.repeat(np.arange(40), np.diff(d["rowptr"]))
    e0 = 7
    d["pos"][d["sender"][e0]] = d["pos"][recv[e0]]
    gc = check(ranks, d, 32)
    spec = conv.ConvSpec(*ranks, 6.0)
    _, xo, po, wo = oracle(spec, d)
    for want, ref, i in ((("x",), xo, 0), (("pos",), po, 1), (("w",), wo, 2)):
        out = gc.vjp(want)
        torch.cuda.synchronize()
        assert_close(want[0], out[i].cpu().numpy(), ref)


@pytest.mark.parametrize("ranks,C,mode", [((0, 0, 0), 24, ""), ((1, 1, 1), 24, ""), ((0, 3, 3), 24, ""),
                                          ((3, 3, 3), 24, ""), ((4, 4, 4), 24, ""), ((5, 5, 5), 16, ""),
                                          ((2, 2, 2), 65, ""), ((2, 2, 2), 200, ""), ((2, 2, 2), 24, "allp"),
                                          ((3, 3, 3), 24, "summed")])
def test_explicit_weights_receiver_side_vjp(ranks, C, mode):
    """Without x_grad the VJP walks each receiver's incoming edges (its
    cotangent rows read once) and sums the per-edge position terms per node
    afterwards: positions and w_grad together and each alone, against the
    oracle."""
    from cartesian_tensor_product_amd import flashcart as fc
    allp, summed = mode == "allp", mode == "summed"
    spec = conv.ConvSpec(*ranks, 6.0, all_parities=allp, sum_paths=summed)
    d = inputs.edge_conv_inputs(13, 50, 20, 5.5, C, spec.n_in, spec.n_paths, spec.n_out, with_edge_w=True)
    flags = fc.FC_CONV_ALL_PARITIES if allp else (fc.FC_CONV_SUM_PATHS if summed else 0)
    gc = GpuConvW(ranks, d, C, 6.0, flags=flags)
    _, _, po, wo = oracle(spec, d)
    _, pb, wb = gc.vjp(("pos", "w"))
    torch.cuda.synchronize()
    assert_close("pos_grad", pb.cpu().numpy(), po)
    assert_close("w_grad", wb.cpu().numpy(), wo)
    for want, ref, i in ((("pos",), po, 1), (("w",), wo, 2)):
        out = gc.vjp(want)
        torch.cuda.synchronize()
        assert_close(want[0], out[i].cpu().numpy(), ref)
    again = gc.vjp(("pos", "w"))
    torch.cuda.synchronize()
    assert torch.equal(again[1], pb) and torch.equal(again[2], wb)


def test_explicit_weights_microbenchmark_sampled():
    """1024 nodes x 128 neighbours x 128 channels, ranks <= 2, w [E, 11, 128]
    (738 MB): sampled nodes element by element, and the per-edge weight
    gradient on every edge into or out of them."""
    ranks = (2, 2, 2)
    spec = conv.ConvSpec(*ranks, 5.0)
    d = inputs.edge_conv_inputs(1, 1024, 128, 20.0, 128, spec.n_in, spec.n_paths, spec.n_out, with_edge_w=True)
    gc = GpuConvW(ranks, d, 128, 5.0)
    z = gc.fwd()
    xb, pb, wb = gc.vjp()
    torch.cuda.synchronize()
    nodes = np.random.default_rng(98).choice(1024, size=10, replace=False)
    edges = sample_edges(d["rowptr"], d["sender"], nodes)
    zo, xo, po, wo = oracle(spec, d, edges=edges)
    assert_close("z", z.cpu().numpy()[nodes], zo[nodes])
    assert_close("x_grad", xb.cpu().numpy()[nodes], xo[nodes])
    assert_close("pos_grad", pb.cpu().numpy()[nodes], po[nodes])
    assert_close("w_grad", wb[torch.from_numpy(edges).cuda()].cpu().numpy(), wo[edges])
    # the receiver-side VJP (no x_grad) at the same size
    _, pr, wr = gc.vjp(("pos", "w"))
    torch.cuda.synchronize()
    assert_close("pos_grad (receiver side)", pr.cpu().numpy()[nodes], po[nodes])
    assert_close("w_grad (receiver side)", wr[torch.from_numpy(edges).cuda()].cpu().numpy(), wo[edges])
    a = [gc.fwd(), *gc.vjp()]
    torch.cuda.synchronize()
    for u, v in zip(a, [z, xb, pb, wb]):
        assert torch.equal(u, v)
