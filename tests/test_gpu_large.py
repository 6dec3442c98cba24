"""GPU parity where node arrays pass 2 GiB, so byte offsets of the last nodes'
rows exceed 2^31: rank 4 (230 output rows per channel) at 128 channels and
20 000 nodes (g, z and g_hat are 2.36 GB each).

The oracle evaluates the sampled nodes on the subgraph of the edges that
touch them (renumbered over the nodes those edges reach): the forward at a
receiver needs only its incoming edges, the VJP and VJP-of-VJP at a node
only the edges touching it, so the sampled values are exact.
"""
import numpy as np
import pytest

from cartesian_tensor_product_amd import inputs
from oracle import conv
from tests.gpu_common import GpuConv, assert_close, f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def subgraph(rowptr, sender, nodes):
    """(ids, rowptr', sender') of the edges touching ``nodes``, renumbered
    over ``ids`` (sorted), receiver-sorted as the original."""
    N = len(rowptr) - 1
    recv = np.repeat(np.arange(N), np.diff(rowptr))
    e = np.nonzero(np.isin(recv, nodes) | np.isin(sender, nodes))[0]
    ids = np.unique(np.concatenate([nodes, recv[e], sender[e]]))
    r2 = np.searchsorted(ids, recv[e])
    s2 = np.searchsorted(ids, sender[e])
    assert np.all(np.diff(r2) >= 0)
    rp = np.concatenate([[0], np.cumsum(np.bincount(r2, minlength=len(ids)))]).astype(np.int32)
    return ids, rp, s2.astype(np.int32)


def test_rank4_node_arrays_beyond_2GiB():
    N, K, C, ranks, rc = 20000, 4, 128, (4, 4, 4), 35.0
    spec = conv.ConvSpec(*ranks, rc)
    assert N * spec.n_out * C * 4 > 2 ** 31
    rng, pos, rowptr, sender = inputs.random_cloud(41, N, K, 20.0)
    x = inputs.normal(rng, (N, spec.n_in, C))
    W = inputs.normal(rng, (8, spec.n_paths, C), std=1.0 / np.sqrt(8))
    v_pos = inputs.normal(rng, (N, 3))
    gen = torch.Generator(device="cuda").manual_seed(41)
    g = torch.randn((N, spec.n_out, C), generator=gen, device="cuda")
    d = dict(pos=pos, rowptr=rowptr, sender=sender, shift=None, x=x, W=W, g=None)
    gc = GpuConv(ranks, rc, d, C)
    gc.g = g
    z = gc.fwd()
    xb, pb = gc.vjp()
    gh, xh, ph, _ = gc.vjp_vjp(v_pos=v_pos)
    torch.cuda.synchronize()
    # nodes whose rows start past 2 GiB (node 18 236 onwards) and a few below
    nodes = np.array([N - 1, N - 7, 19000, 18300, 12345, 3])
    ids, rp, sd = subgraph(rowptr, sender, nodes)
    at = np.searchsorted(ids, nodes)
    tid = torch.from_numpy(ids).cuda()
    g_s = f64(g[tid].cpu().numpy())
    a = (spec, f64(pos[ids]), rp, sd, f64(x[ids]), f64(W))
    zo = conv.edge_conv_fwd(*a)
    xo, po, _ = conv.edge_conv_vjp(*a, g_s)
    gho, xho, pho, _ = conv.edge_conv_vjp_vjp(*a, g_s, v_pos=f64(v_pos[ids]))
    tn = torch.from_numpy(nodes).cuda()
    assert_close("z", z[tn].cpu().numpy(), zo[at])
    assert_close("x_grad", xb[tn].cpu().numpy(), xo[at])
    assert_close("pos_grad", pb[tn].cpu().numpy(), po[at])
    assert_close("g_hat", gh[tn].cpu().numpy(), gho[at])
    assert_close("x_hat", xh[tn].cpu().numpy(), xho[at])
    assert_close("pos_hat", ph[tn].cpu().numpy(), pho[at])
