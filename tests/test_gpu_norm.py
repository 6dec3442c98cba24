"""GPU parity of the equivariant RMS normalisation (forward, feature and
scale gradients) against the oracle."""
import numpy as np
import pytest

from cartesian_tensor_product_amd import inputs
from oracle import norm
from tests.gpu_common import assert_close, f64

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def run(l_max, N, C, eps, seed, with_gamma=True, want=("x", "gamma")):
    from cartesian_tensor_product_amd import flashcart as fc
    rng = np.random.default_rng(seed)
    x = inputs.normal(rng, (N, (l_max + 1) ** 2, C))
    gamma = inputs.f32(1.0 + 0.3 * rng.standard_normal((l_max + 1, C))) if with_gamma else None
    g = inputs.normal(rng, x.shape)
    t = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
    d = fc.norm_desc(N, C, l_max, eps)
    dx, dgam, dg = t(x), t(gamma), t(g)
    y = torch.empty_like(dx)
    inv_s = torch.empty(N, device="cuda")
    fc.fc_rms_norm_fwd(d, dx, dgam, y, inv_s)
    xb = torch.empty_like(dx) if "x" in want else None
    gb = torch.empty((l_max + 1, C), device="cuda") if "gamma" in want else None
    ws = fc.workspace(fc.fc_rms_norm_workspace_bytes(d), "cuda")
    fc.fc_rms_norm_vjp(d, dx, dgam, inv_s, dg, xb, gb, ws)
    torch.cuda.synchronize()
    yo, iso = norm.rms_norm_fwd(f64(x), l_max, eps, f64(gamma))
    xo, go = norm.rms_norm_vjp(f64(x), l_max, eps, f64(g), f64(gamma))
    assert_close("y", y.cpu().numpy(), yo)
    assert_close("inv_scale", inv_s.cpu().numpy(), iso)
    if xb is not None:
        assert_close("x_grad", xb.cpu().numpy(), xo)
    if gb is not None:
        assert_close("gamma_grad", gb.cpu().numpy(), go)


@pytest.mark.parametrize("l_max", [0, 1, 2, 3, 4, 5])
def test_every_rank(l_max):
    run(l_max, 37, 40, 1e-3, l_max)


@pytest.mark.parametrize("C", [1, 63, 64, 65, 128, 200, 512])
def test_channel_tiles(C):
    run(3, 19, C, 1e-3, 100 + C)


def test_many_nodes_span_vjp_blocks():
    """More nodes than the VJP grid's waves: each wave sums several nodes'
    scale gradients in order before the fixed-order block sum."""
    run(3, 4096 + 77, 128, 1e-5, 7)


def test_without_gamma_and_single_outputs():
    run(2, 25, 48, 0.1, 8, with_gamma=False)
    run(2, 25, 48, 0.1, 9, want=("x",))
    run(2, 25, 48, 0.1, 10, want=("gamma",))


def test_norm_vjp_bitwise_deterministic():
    from cartesian_tensor_product_amd import flashcart as fc
    rng = np.random.default_rng(12)
    N, C = 3000, 64
    x = torch.from_numpy(inputs.normal(rng, (N, 9, C))).cuda()
    g = torch.from_numpy(inputs.normal(rng, (N, 9, C))).cuda()
    gam = torch.from_numpy(inputs.f32(1 + 0.1 * rng.standard_normal((3, C)))).cuda()
    d = fc.norm_desc(N, C, 2, 1e-5)
    y, s = torch.empty_like(x), torch.empty(N, device="cuda")
    fc.fc_rms_norm_fwd(d, x, gam, y, s)
    ws = fc.workspace(fc.fc_rms_norm_workspace_bytes(d), "cuda")
    outs = []
    for _ in range(2):
        xb, gb = torch.empty_like(x), torch.empty_like(gam)
        fc.fc_rms_norm_vjp(d, x, gam, s, g, xb, gb, ws)
        torch.cuda.synchronize()
        outs.append((xb.cpu().numpy(), gb.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
