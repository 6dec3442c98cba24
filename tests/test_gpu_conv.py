"""GPU parity of the edge convolution (forward and VJP) against the oracle.

Full element-by-element comparison at sizes the oracle finishes quickly
(several 64-edge chunks, ragged channel tiles, empty and high-degree nodes);
sampled comparison at the full microbenchmark sizes (1024 nodes, 128
neighbours, 128 channels) in the launch configuration the benchmark times.
"""
import numpy as np
import pytest

from cartesian_tensor_product_amd import inputs
from oracle import conv
from tests.gpu_common import GpuConv, assert_close, f64, sample_edges

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def oracle_all(spec, d, edges=None, g=None):
    a = (spec, f64(d["pos"]), d["rowptr"], d["sender"], f64(d["x"]), f64(d["W"]))
    z = conv.edge_conv_fwd(*a, shift=f64(d.get("shift")), edges=edges)
    g = d["g"] if g is None else g
    xb, pb, Wb = conv.edge_conv_vjp(*a, f64(g), shift=f64(d.get("shift")), edges=edges, want_W=True)
    return z, xb, pb, Wb


def check_full(ranks, rc, d, C, allp=False):
    from cartesian_tensor_product_amd import flashcart as fc
    spec = conv.ConvSpec(*ranks, rc, all_parities=allp)
    gc = GpuConv(ranks, rc, d, C, flags=fc.FC_CONV_ALL_PARITIES if allp else 0)
    z = gc.fwd()
    xb, pb, Wb = gc.vjp(want_W=True)
    torch.cuda.synchronize()
    zo, xo, po, Wo = oracle_all(spec, d)
    assert_close("z", z.cpu().numpy(), zo)
    assert_close("x_grad", xb.cpu().numpy(), xo)
    assert_close("pos_grad", pb.cpu().numpy(), po)
    assert_close("radial_w_grad", Wb.cpu().numpy(), Wo)


def tiny_inputs(ranks, C, seed=0, n=32, k=8, box=6.0, rc=6.0, allp=False):
    spec = conv.ConvSpec(*ranks, rc, all_parities=allp)
    return spec, inputs.edge_conv_inputs(seed, n, k, box, C, spec.n_in, spec.n_paths, spec.n_out)


def test_tiny_workload():
    """32 nodes, 8 neighbours, 8 channels, ranks <= 1, rc 6 A, seed 0."""
    _, d = tiny_inputs((1, 1, 1), 8)
    check_full((1, 1, 1), 6.0, d, 8)


@pytest.mark.parametrize("ranks", [(0, 0, 0), (1, 1, 1), (2, 2, 2), (3, 3, 3), (4, 4, 4), (5, 5, 5), (0, 1, 1),
                                   (0, 2, 2), (1, 2, 2), (0, 3, 3), (1, 3, 3), (2, 3, 3), (0, 4, 4), (1, 4, 4),
                                   (2, 4, 4), (3, 4, 4)])
def test_every_instantiated_config(ranks):
    _, d = tiny_inputs(ranks, 24, seed=11, n=40, k=12, box=5.0, rc=6.0)
    check_full(ranks, 6.0, d, 24)


def test_tiny_workload_all_triangle_allowed_paths():
    """The tiny workload with every triangle-allowed path of ranks <= 1:
    the odd (1,1)->1 coupling (the cross product) joins the four natural
    paths."""
    _, d = tiny_inputs((1, 1, 1), 8, allp=True)
    check_full((1, 1, 1), 6.0, d, 8, allp=True)


@pytest.mark.parametrize("ranks", [(1, 1, 1), (2, 2, 2), (3, 3, 3), (4, 4, 4)])
def test_all_parities_every_rank(ranks):
    _, d = tiny_inputs(ranks, 40, seed=12, n=40, k=12, box=5.0, rc=6.0, allp=True)
    check_full(ranks, 6.0, d, 40, allp=True)


@pytest.mark.parametrize("C", [1, 63, 64, 65, 128, 200, 256])
def test_channel_tiles(C):
    _, d = tiny_inputs((2, 2, 2), C, seed=3, n=48, k=20, box=8.0, rc=6.0)
    check_full((2, 2, 2), 6.0, d, C)


def test_ragged_degrees_and_chunks():
    """Degrees 0..200: empty receivers/senders and several 64-edge chunks."""
    rng = np.random.default_rng(17)
    N, C = 150, 32
    deg = rng.integers(0, 201, size=N)
    deg[:5] = 0
    deg = np.minimum(deg, N - 1)
    rowptr = np.concatenate([[0], np.cumsum(deg)]).astype(np.int32)
    sender = np.concatenate([np.sort(rng.choice(np.delete(np.arange(N), i), size=deg[i], replace=False))
                             for i in range(N)]).astype(np.int32)
    spec = conv.ConvSpec(2, 2, 2, 9.0)
    d = dict(pos=inputs.f32(rng.uniform(0, 10, (N, 3))), rowptr=rowptr, sender=sender, shift=None,
             x=inputs.normal(rng, (N, spec.n_in, C)), W=inputs.normal(rng, (8, spec.n_paths, C), 0.35),
             g=inputs.normal(rng, (N, spec.n_out, C)))
    check_full((2, 2, 2), 9.0, d, C)


def test_empty_graph():
    N, C = 10, 16
    spec = conv.ConvSpec(2, 2, 2, 5.0)
    rng = np.random.default_rng(0)
    d = dict(pos=inputs.f32(rng.uniform(0, 5, (N, 3))), rowptr=np.zeros(N + 1, np.int32),
             sender=np.zeros(0, np.int32), shift=None, x=inputs.normal(rng, (N, spec.n_in, C)),
             W=inputs.normal(rng, (8, spec.n_paths, C)), g=inputs.normal(rng, (N, spec.n_out, C)))
    gc = GpuConv((2, 2, 2), 5.0, d, C)
    z = gc.fwd()
    xb, pb, Wb = gc.vjp(want_W=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(z) == 0 and torch.count_nonzero(xb) == 0 and torch.count_nonzero(pb) == 0
    assert torch.count_nonzero(Wb) == 0


@pytest.mark.parametrize("ranks", [(1, 1, 1), (2, 2, 2), (0, 3, 3)])
def test_radial_weight_grad_alone(ranks):
    """radial_w_grad requested without x_grad and pos_grad (receiver pass only)."""
    spec, d = tiny_inputs(ranks, 40, seed=8, n=70, k=30, box=7.0, rc=6.0)
    gc = GpuConv(ranks, 6.0, d, 40)
    _, _, Wb = gc.vjp(want_x=False, want_pos=False, want_W=True)
    torch.cuda.synchronize()
    Wo = oracle_all(spec, d)[3]
    assert_close("radial_w_grad", Wb.cpu().numpy(), Wo)


def test_graph_transpose_matches_stable_sort():
    spec, d = tiny_inputs((1, 1, 1), 8, seed=5, n=300, k=40, box=10.0)
    from cartesian_tensor_product_amd import flashcart as fc
    g = fc.DeviceGraph(d["rowptr"], d["sender"], 300)
    torch.cuda.synchronize()
    recv = np.repeat(np.arange(300), np.diff(d["rowptr"]))
    order = np.argsort(d["sender"], kind="stable")
    assert np.array_equal(g.receiver.cpu().numpy(), recv)
    assert np.array_equal(g.t_edge.cpu().numpy(), order)
    assert np.array_equal(g.t_rowptr.cpu().numpy(),
                          np.concatenate([[0], np.cumsum(np.bincount(d["sender"], minlength=300))]))


def test_graph_transpose_skewed_degrees():
    """One sender feeds every receiver, a tenth of the nodes send nothing,
    and senders are unsorted within a receiver: the transpose lists each
    sender's edge ids in ascending order whatever the scatter did."""
    from cartesian_tensor_product_amd import flashcart as fc
    rng = np.random.default_rng(23)
    N = 700
    quiet = rng.choice(np.arange(1, N), size=N // 10, replace=False)
    pool = np.setdiff1d(np.arange(N), quiet)
    rows = []
    for u in range(N):
        k = int(rng.integers(0, 60))
        s = rng.choice(pool[pool != u], size=k, replace=False)
        if u != 0:
            s = np.concatenate([s[s != 0], [0]])
        rows.append(rng.permutation(s))
    rowptr = np.concatenate([[0], np.cumsum([len(r) for r in rows])]).astype(np.int32)
    sender = np.concatenate(rows).astype(np.int32)
    g = fc.DeviceGraph(rowptr, sender, N)
    torch.cuda.synchronize()
    recv = np.repeat(np.arange(N), np.diff(rowptr))
    assert np.count_nonzero(sender == 0) == N - 1
    assert np.array_equal(g.receiver.cpu().numpy(), recv)
    assert np.array_equal(g.t_edge.cpu().numpy(), np.argsort(sender, kind="stable"))
    assert np.array_equal(g.t_rowptr.cpu().numpy(),
                          np.concatenate([[0], np.cumsum(np.bincount(sender, minlength=N))]))


def test_periodic_shifts_diamond():
    """The diamond cell's convolution (scalar senders, ranks <= 3, shifts)."""
    spec = conv.ConvSpec(0, 3, 3, 5.0)
    d = inputs.diamond_inputs(channels=64, r_cut=5.0, rattle=0.05, ncell=3, n_paths=spec.n_paths)
    rng = np.random.default_rng(1)
    d["g"] = inputs.normal(rng, (d["pos"].shape[0], spec.n_out, 64))
    check_full((0, 3, 3), 5.0, d, 64)


# ---------------------------------------------------- full workload sizes --

def micro(ranks, seed, rc):
    spec = conv.ConvSpec(*ranks, rc)
    d = inputs.edge_conv_inputs(seed, 1024, 128, 20.0, 128, spec.n_in, spec.n_paths, spec.n_out)
    return spec, d


@pytest.mark.parametrize("ranks,seed,rc", [((2, 2, 2), 1, 5.0), ((2, 2, 2), 1, 35.0), ((3, 3, 3), 2, 5.0),
                                           ((4, 4, 4), 2, 5.0), ((3, 3, 3), 2, 35.0)])
def test_microbenchmark_sampled(ranks, seed, rc):
    """1024 nodes x 128 neighbours x 128 channels; 12 sampled nodes compared
    element by element (r_c = 35 A keeps every edge inside the cutoff)."""
    spec, d = micro(ranks, seed, rc)
    gc = GpuConv(ranks, rc, d, 128)
    z = gc.fwd()
    xb, pb = gc.vjp()
    # radial-weight gradient of a cotangent that vanishes off the sampled
    # receivers: only their incoming edges contribute, so the oracle sums
    # exactly those
    nodes = np.random.default_rng(99).choice(1024, size=12, replace=False)
    gm = np.zeros_like(d["g"])
    gm[nodes] = d["g"][nodes]
    _, _, Wb = gc.vjp(g=torch.from_numpy(gm).cuda(), want_x=False, want_pos=False, want_W=True)
    torch.cuda.synchronize()
    edges = sample_edges(d["rowptr"], d["sender"], nodes)
    zo, xo, po, _ = oracle_all(spec, d, edges=edges)
    recv = np.repeat(np.arange(1024), np.diff(d["rowptr"]))
    Wo = oracle_all(spec, d, edges=np.nonzero(np.isin(recv, nodes))[0], g=gm)[3]
    assert_close("z", z.cpu().numpy()[nodes], zo[nodes])
    assert_close("x_grad", xb.cpu().numpy()[nodes], xo[nodes])
    assert_close("pos_grad", pb.cpu().numpy()[nodes], po[nodes])
    assert_close("radial_w_grad", Wb.cpu().numpy(), Wo)
    # properties that hold at any size: translation invariance of the forces
    p = pb.double().cpu().numpy()
    assert np.abs(p.sum(0)).max() < 1e-4 * np.abs(p).max() * np.sqrt(1024)


def test_bitwise_determinism():
    spec, d = micro((2, 2, 2), 1, 5.0)
    gc = GpuConv((2, 2, 2), 5.0, d, 128)
    a = [gc.fwd(), *gc.vjp(want_W=True)]
    b = [gc.fwd(), *gc.vjp(want_W=True)]
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u, v)


def test_rank5_256_channels():
    """Rank 5 with four channel waves per sender block: the VJP stages 32
    edges per chunk there so its row sums fit in LDS; senders of about 40
    edges span two chunks."""
    _, d = tiny_inputs((5, 5, 5), 256, seed=21, n=50, k=40, box=6.0, rc=6.0)
    check_full((5, 5, 5), 6.0, d, 256)


def test_rank5_microbenchmark_sampled():
    """Rank 5 (69 paths, 457 output rows per channel) at 1024 nodes x 64
    neighbours x 64 channels (r_c = 35 A: every edge inside the cutoff),
    sampled nodes: forward, VJP and the VJP-of-VJP with a position
    cotangent, whose passes (g_hat, x_hat and the position terms) run as
    separate launches at this rank."""
    ranks = (5, 5, 5)
    spec = conv.ConvSpec(*ranks, 35.0)
    d = inputs.edge_conv_inputs(2, 1024, 64, 20.0, 64, spec.n_in, spec.n_paths, spec.n_out, with_vpos=True)
    gc = GpuConv(ranks, 35.0, d, 64)
    z = gc.fwd()
    xb, pb = gc.vjp()
    gh, xh, ph, _ = gc.vjp_vjp(v_pos=d["v_pos"])
    torch.cuda.synchronize()
    nodes = np.random.default_rng(97).choice(1024, size=4, replace=False)
    edges = sample_edges(d["rowptr"], d["sender"], nodes)
    zo, xo, po, _ = oracle_all(spec, d, edges=edges)
    assert_close("z", z.cpu().numpy()[nodes], zo[nodes])
    assert_close("x_grad", xb.cpu().numpy()[nodes], xo[nodes])
    assert_close("pos_grad", pb.cpu().numpy()[nodes], po[nodes])
    go, xho, pho, _ = conv.edge_conv_vjp_vjp(spec, f64(d["pos"]), d["rowptr"], d["sender"], f64(d["x"]),
                                             f64(d["W"]), f64(d["g"]), v_pos=f64(d["v_pos"]), edges=edges)
    assert_close("g_hat", gh.cpu().numpy()[nodes], go[nodes])
    assert_close("x_hat", xh.cpu().numpy()[nodes], xho[nodes])
    assert_close("pos_hat", ph.cpu().numpy()[nodes], pho[nodes])


@pytest.mark.parametrize("ranks,seed", [((2, 2, 2), 1), ((3, 3, 3), 2)])
def test_all_parities_microbenchmark_sampled(ranks, seed):
    """1024 nodes x 128 neighbours x 128 channels with every triangle-allowed
    path (15 at rank 2, 34 at rank 3), sampled nodes."""
    from cartesian_tensor_product_amd import flashcart as fc
    spec = conv.ConvSpec(*ranks, 5.0, all_parities=True)
    d = inputs.edge_conv_inputs(seed, 1024, 128, 20.0, 128, spec.n_in, spec.n_paths, spec.n_out)
    gc = GpuConv(ranks, 5.0, d, 128, flags=fc.FC_CONV_ALL_PARITIES)
    z = gc.fwd()
    xb, pb = gc.vjp()
    torch.cuda.synchronize()
    nodes = np.random.default_rng(96).choice(1024, size=8, replace=False)
    edges = sample_edges(d["rowptr"], d["sender"], nodes)
    zo, xo, po, _ = oracle_all(spec, d, edges=edges)
    assert_close("z", z.cpu().numpy()[nodes], zo[nodes])
    assert_close("x_grad", xb.cpu().numpy()[nodes], xo[nodes])
    assert_close("pos_grad", pb.cpu().numpy()[nodes], po[nodes])
