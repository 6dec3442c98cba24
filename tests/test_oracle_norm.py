"""Pins of the equivariant RMS normalisation oracle."""
import numpy as np
import pytest

from oracle import norm, tensors as T
from tests.test_oracle_conv import rotate_rows
from tests.test_oracle_tensors import rand_rotation


def feats(l_max, N=6, C=5, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, (l_max + 1) ** 2, C))
    gamma = 1.0 + 0.3 * rng.standard_normal((l_max + 1, C))
    g = rng.standard_normal(x.shape)
    return x, gamma, g


def rank_rows(l_max):
    off = T.rank_offsets(l_max)
    return [(np.arange(off[l], off[l + 1]), l) for l in range(l_max + 1)]


def test_rank0_is_torch_rms_norm():
    """With only scalars the normalisation is the textbook RMS norm over the
    channels (torch.nn.functional.rms_norm)."""
    torch = pytest.importorskip("torch")
    x, gamma, _ = feats(0, N=7, C=9)
    y, inv_s = norm.rms_norm_fwd(x, 0, 1e-3, gamma)
    want = torch.nn.functional.rms_norm(torch.from_numpy(x[:, 0, :]), (9,), torch.from_numpy(gamma[0]), 1e-3)
    assert np.abs(y[:, 0, :] - want.numpy()).max() < 1e-12


def test_rank1_uses_the_dot_product():
    """(1,1)->0 is the dot product: s^2 = (sum_k x0^2 + sum_k |x1|^2) / (2C) + eps."""
    x, gamma, _ = feats(1, N=4, C=3)
    y, inv_s = norm.rms_norm_fwd(x, 1, 0.25, gamma)
    s2 = ((x[:, 0, :] ** 2).sum(1) + (x[:, 1:4, :] ** 2).sum((1, 2))) / (2 * 3) + 0.25
    assert np.allclose(inv_s, 1 / np.sqrt(s2), rtol=1e-14)
    assert np.allclose(y[:, 1:4, :], gamma[1][None, None, :] * x[:, 1:4, :] / np.sqrt(s2)[:, None, None], rtol=1e-14)


@pytest.mark.parametrize("l_max", [2, 3, 4])
def test_invariance_and_equivariance(l_max):
    x, gamma, _ = feats(l_max, seed=l_max)
    rng = np.random.default_rng(40 + l_max)
    y, inv_s = norm.rms_norm_fwd(x, l_max, 1e-2, gamma)
    for reflect in (False, True):
        R = rand_rotation(rng, reflect)
        xr = rotate_rows(rank_rows(l_max), x, R)
        yr, inv_sr = norm.rms_norm_fwd(xr, l_max, 1e-2, gamma)
        assert np.abs(inv_sr - inv_s).max() < 1e-12 * inv_s.max()
        assert np.abs(yr - rotate_rows(rank_rows(l_max), y, R)).max() < 1e-10 * np.abs(y).max()
    # a Euclidean norm of the stored components is not invariant at l >= 2
    euc = lambda a: np.sum(a[:, 4:9, :] ** 2)
    assert abs(euc(rotate_rows(rank_rows(l_max), x, R)) - euc(x)) > 1e-6 * euc(x)


def test_scale_invariance_without_eps():
    x, gamma, _ = feats(3, seed=5)
    y1, _ = norm.rms_norm_fwd(x, 3, 0.0, gamma)
    y2, _ = norm.rms_norm_fwd(7.5 * x, 3, 0.0, gamma)
    assert np.abs(y1 - y2).max() < 1e-12 * np.abs(y1).max()


@pytest.mark.parametrize("l_max", [1, 3])
def test_vjp_against_complex_step(l_max):
    x, gamma, g = feats(l_max, N=3, C=4, seed=9)
    eps = 0.05
    xb, gb = norm.rms_norm_vjp(x, l_max, eps, g, gamma)
    loss = lambda xx, gg: np.sum(g * norm.rms_norm_fwd(xx, l_max, eps, gg)[0])
    h = 1e-20
    for idx in np.ndindex(*x.shape):
        xc = x.astype(complex)
        xc[idx] += 1j * h
        assert abs(loss(xc, gamma).imag / h - xb[idx]) < 1e-12 * max(1.0, np.abs(xb).max())
    for idx in np.ndindex(*gamma.shape):
        gc = gamma.astype(complex)
        gc[idx] += 1j * h
        assert abs(loss(x, gc).imag / h - gb[idx]) < 1e-12 * max(1.0, np.abs(gb).max())
