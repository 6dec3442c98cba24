"""GPU parity of the pages' radial network (Chebyshev features, envelope,
bias-free SiLU MLP with an MFMA output layer) and of the convolution it
weights (forward; VJP to features, positions and the network's weights)
against the oracle, with the output layer fused into the convolution's
lanes (FC_CONV_MLP_FUSE), with w [E][P][C] stored and streamed
(FC_CONV_MLP_MATERIALIZE), and with the default choice."""
import numpy as np
import pytest

from cartesian_tensor_product_amd import inputs
from oracle import conv, radial
from tests.gpu_common import assert_close, f64, sample_edges

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def split(flat, P, C):
    W1 = flat[:512].reshape(8, 64)
    W2 = flat[512:512 + 4096].reshape(64, 64)
    W3 = flat[512 + 4096:].reshape(64, P * C)
    return W1, W2, W3


MODES = ["fused", "materialized"]
FLAGS = {"fused": "FC_CONV_MLP_FUSE", "materialized": "FC_CONV_MLP_MATERIALIZE", "default": None}


class GpuMlpConv:
    def __init__(self, ranks, d, C, rc, mlp, mode="fused"):
        from cartesian_tensor_product_amd import flashcart as fc
        self.fc = fc
        self.N, self.E, self.C = d["pos"].shape[0], int(len(d["sender"])), C
        flags = getattr(fc, FLAGS[mode]) if FLAGS[mode] else 0
        self.desc = fc.conv_desc(self.N, self.E, C, *ranks, rc, flags=flags)
        self.P, self.nin, self.nout = fc.fc_conv_layout(self.desc)
        assert fc.fc_radial_mlp_weight_floats(self.desc) == mlp.size
        self.graph = fc.DeviceGraph(d["rowptr"], d["sender"], self.N, device="cuda")
        t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
        self.pos, self.shift, self.x, self.g, self.mlp = t(d["pos"]), t(d.get("shift")), t(d["x"]), t(d["g"]), t(mlp)

    def weights(self):
        w = torch.empty((self.E, self.P, self.C), device="cuda")
        ws = self.fc.workspace(self.fc.fc_edge_conv_mlp_workspace_bytes(self.desc, 0), "cuda")
        self.fc.fc_radial_mlp(self.desc, self.graph, self.pos, self.shift, self.mlp, w, ws)
        return w

    def fwd(self):
        z = torch.empty((self.N, self.nout, self.C), device="cuda")
        ws = self.fc.workspace(self.fc.fc_edge_conv_mlp_workspace_bytes(self.desc, 0), "cuda")
        self.fc.fc_edge_conv_mlp_fwd(self.desc, self.graph, self.pos, self.shift, self.x, self.mlp, z, ws)
        return z

    def vjp(self, want=("x", "pos", "w")):
        xb = torch.empty_like(self.x) if "x" in want else None
        pb = torch.empty((self.N, 3), device="cuda") if "pos" in want else None
        wb = torch.empty_like(self.mlp) if "w" in want else None
        op = 1 if "w" in want else 2
        ws = self.fc.workspace(self.fc.fc_edge_conv_mlp_workspace_bytes(self.desc, op), "cuda")
        self.fc.fc_edge_conv_mlp_vjp(self.desc, self.graph, self.pos, self.shift, self.x, self.mlp, self.g, xb, pb,
                                     wb, ws)
        return xb, pb, wb


def setup(ranks, C, seed, n=40, k=12, box=5.0, rc=5.0):
    spec = conv.ConvSpec(*ranks, rc)
    d = inputs.edge_conv_inputs(seed, n, k, box, C, spec.n_in, spec.n_paths, spec.n_out)
    mlp = inputs.radial_mlp_weights(np.random.default_rng(seed + 50), spec.n_paths, C)
    return spec, d, mlp


@pytest.mark.parametrize("mode", MODES + ["default"])
@pytest.mark.parametrize("ranks", [(1, 1, 1), (2, 2, 2), (0, 3, 3), (1, 2, 2), (3, 3, 3)])
def test_mlp_conv_full(ranks, mode):
    """The forward and the VJP to x and positions (fused unless
    materialised), then the VJP with the network's weight gradient (which
    stores w in both modes)."""
    spec, d, mlp = setup(ranks, 40, 31)
    gc = GpuMlpConv(ranks, d, 40, 5.0, mlp, mode)
    w = gc.weights()
    z = gc.fwd()
    xb, pb, _ = gc.vjp(("x", "pos"))
    xb2, pb2, wb = gc.vjp()
    torch.cuda.synchronize()
    W1, W2, W3 = split(f64(mlp), spec.n_paths, 40)
    r, _ = radial.edge_lengths(f64(d["pos"]), d["rowptr"], d["sender"])
    assert_close("w", w.cpu().numpy(), radial.radial_mlp(r, 5.0, W1, W2, W3, spec.n_paths, 40))
    args = (spec, f64(d["pos"]), d["rowptr"], d["sender"], f64(d["x"]), W1, W2, W3)
    assert_close("z", z.cpu().numpy(), radial.edge_conv_fwd_mlp(*args))
    xo, po, W1b, W2b, W3b = radial.edge_conv_vjp_mlp(*args, f64(d["g"]))
    assert_close("x_grad", xb.cpu().numpy(), xo)
    assert_close("pos_grad", pb.cpu().numpy(), po)
    assert_close("x_grad (with the weight gradient)", xb2.cpu().numpy(), xo)
    assert_close("pos_grad (with the weight gradient)", pb2.cpu().numpy(), po)
    wo = np.concatenate([W1b.ravel(), W2b.ravel(), W3b.ravel()])
    assert_close("mlp_w_grad", wb.cpu().numpy(), wo)


@pytest.mark.parametrize("mode", MODES)
def test_mlp_conv_single_outputs_and_channel_tail(mode):
    """C = 65: the second wave has one live lane (the idle lanes must add
    nothing to the per-edge sums over lanes)."""
    spec, d, mlp = setup((2, 2, 2), 65, 32, n=30, k=9)
    gc = GpuMlpConv((2, 2, 2), d, 65, 5.0, mlp, mode)
    W1, W2, W3 = split(f64(mlp), spec.n_paths, 65)
    xo, po, W1b, W2b, W3b = radial.edge_conv_vjp_mlp(spec, f64(d["pos"]), d["rowptr"], d["sender"], f64(d["x"]), W1,
                                                     W2, W3, f64(d["g"]))
    for want, ref in ((("x",), xo), (("pos",), po), (("w",), np.concatenate([W1b.ravel(), W2b.ravel(), W3b.ravel()]))):
        out = gc.vjp(want)
        torch.cuda.synchronize()
        got = out[("x", "pos", "w").index(want[0])]
        assert_close(want[0], got.cpu().numpy(), ref)


def subgraph(rowptr, sender, edges):
    """The receiver-sorted graph of the given (sorted) edge ids over the same nodes."""
    recv = np.repeat(np.arange(len(rowptr) - 1), np.diff(rowptr))
    counts = np.bincount(recv[edges], minlength=len(rowptr) - 1)
    return np.concatenate([[0], np.cumsum(counts)]).astype(rowptr.dtype), sender[edges]


@pytest.mark.parametrize("mode", MODES)
def test_mlp_conv_microbenchmark_sampled(mode):
    """1024 nodes x 128 neighbours x 128 channels, rank 2, r_max 5 A: the
    weights of 2000 sampled edges; z, x_grad and pos_grad on 8 sampled nodes
    (the oracle runs on the edges touching them, which is all these outputs
    read); translation invariance of the forces at full size."""
    spec, d, mlp = setup((2, 2, 2), 128, 1, n=1024, k=128, box=20.0, rc=5.0)
    gc = GpuMlpConv((2, 2, 2), d, 128, 5.0, mlp, mode)
    w = gc.weights()
    z = gc.fwd()
    xb, pb, _ = gc.vjp(("x", "pos"))
    torch.cuda.synchronize()
    W1, W2, W3 = split(f64(mlp), spec.n_paths, 128)
    r, _ = radial.edge_lengths(f64(d["pos"]), d["rowptr"], d["sender"])
    es = np.random.default_rng(3).choice(len(r), size=2000, replace=False)
    assert_close("w", w.cpu().numpy()[es], radial.radial_mlp(r[es], 5.0, W1, W2, W3, spec.n_paths, 128))
    nodes = np.random.default_rng(4).choice(1024, size=8, replace=False)
    rp, sd = subgraph(d["rowptr"], d["sender"], sample_edges(d["rowptr"], d["sender"], nodes))
    args = (spec, f64(d["pos"]), rp, sd, f64(d["x"]), W1, W2, W3)
    zo = radial.edge_conv_fwd_mlp(*args)
    xo, po, _, _, _ = radial.edge_conv_vjp_mlp(*args, f64(d["g"]))
    assert_close("z", z.cpu().numpy()[nodes], zo[nodes])
    assert_close("x_grad", xb.cpu().numpy()[nodes], xo[nodes])
    assert_close("pos_grad", pb.cpu().numpy()[nodes], po[nodes])
    p = pb.double().cpu().numpy()
    assert np.abs(p.sum(0)).max() < 1e-4 * np.abs(p).max() * np.sqrt(1024)


@pytest.mark.parametrize("mode", MODES)
def test_mlp_conv_without_edges(mode):
    """No edge: z and the gradients are zero (the network's weight gradient
    included)."""
    from cartesian_tensor_product_amd import flashcart as fc
    spec = conv.ConvSpec(2, 2, 2, 5.0)
    N, C = 6, 24
    d = dict(pos=inputs.normal(np.random.default_rng(1), (N, 3)), rowptr=np.zeros(N + 1, np.int32),
             sender=np.zeros(0, np.int32), x=inputs.normal(np.random.default_rng(2), (N, spec.n_in, C)),
             g=inputs.normal(np.random.default_rng(3), (N, spec.n_out, C)))
    mlp = inputs.radial_mlp_weights(np.random.default_rng(4), spec.n_paths, C)
    gc = GpuMlpConv((2, 2, 2), d, C, 5.0, mlp, mode)
    z = gc.fwd()
    xb, pb, wb = gc.vjp()
    xf, pf, _ = gc.vjp(("x", "pos"))
    torch.cuda.synchronize()
    for name, a in (("z", z), ("x_grad", xb), ("pos_grad", pb), ("mlp_w_grad", wb), ("x_grad", xf), ("pos_grad", pf)):
        assert float(a.abs().max()) == 0.0, name


@pytest.mark.parametrize("want", [("x", "pos", "w"), ("x", "pos")])
def test_mlp_conv_bitwise_deterministic(want):
    spec, d, mlp = setup((2, 2, 2), 40, 33, n=60, k=20, box=6.0)
    gc = GpuMlpConv((2, 2, 2), d, 40, 5.0, mlp)
    r1 = [t.cpu().numpy() for t in gc.vjp(want) if t is not None]
    r2 = [t.cpu().numpy() for t in gc.vjp(want) if t is not None]
    assert len(r1) == len(want)
    for a, b in zip(r1, r2):
        assert np.array_equal(a, b)


def test_mlp_workspace_sizes():
    """The fused layouts are small (hidden rows, 512 bytes per edge); the
    VJP with the network's weight gradient takes the materialised layout,
    whose size also covers the fused VJP; a VJP asking for the weight
    gradient with the smaller op 2 workspace is refused."""
    from cartesian_tensor_product_amd import flashcart as fc
    spec, d, mlp = setup((2, 2, 2), 128, 1, n=200, k=32, box=10.0)
    gc = GpuMlpConv((2, 2, 2), d, 128, 5.0, mlp, "fused")
    E = gc.E
    b0, b1, b2 = (fc.fc_edge_conv_mlp_workspace_bytes(gc.desc, op) for op in (0, 1, 2))
    mat = fc.conv_desc(gc.N, E, 128, 2, 2, 2, 5.0, flags=fc.FC_CONV_MLP_MATERIALIZE)
    m0 = fc.fc_edge_conv_mlp_workspace_bytes(mat, 0)
    assert b0 < E * 600 and m0 > E * gc.P * 128 * 4 and b2 < b1
    ws = fc.workspace(b2, "cuda")
    with pytest.raises(fc.FlashCartError):
        fc.fc_edge_conv_mlp_vjp(gc.desc, gc.graph, gc.pos, gc.shift, gc.x, gc.mlp, gc.g, None, None,
                                torch.empty_like(gc.mlp), ws)
