"""Oracle for the equivariant RMS normalisation of node features.

TEST INFRASTRUCTURE ONLY.  Plain fp64 numpy.  Follows the FlashCart paper,
App. E "Model architecture" (the paragraph on residual updates and
normalisation): scalar invariants of every rank are formed with the
(l, l) -> 0 couplings, combined over ranks and channels into one scale per
atom, without batch statistics.
The pages leave the combination open; the reading here is the root mean
square over the l_max + 1 ranks and the C channels,

    q[u, l, k] = f_(l,l)->0(x[u, l, k], x[u, l, k])       (an invariant, >= 0)
    s[u]       = sqrt( sum_{l, k} q[u, l, k] / ((l_max + 1) C) + eps )
    y[u, l, k] = gamma[l, k] x[u, l, k] / s[u],

with a learned scale gamma [l_max + 1, C] per rank and channel (ones when
absent).  A plain Euclidean norm of the stored components would not be
invariant (the stored coordinates are not orthonormal), which is why the
coupling is used.

The VJP is written out by hand: with B[u] = sum_{l,k} <g_y, gamma x> and
(K_l x) = (1/2) d q / d x (the (l,l)->0 form is symmetric),

    x_bar     = gamma g_y / s - B (K_l x) / (s^3 (l_max + 1) C)
    gamma_bar = sum_u <g_y[u, l, k], x[u, l, k]> / s[u].

Parity pins (tests/test_oracle_norm.py): l_max = 0 is torch's RMS norm over
the channels; l_max = 1 uses the plain dot product x_1 . x_1; invariance of
s and equivariance of y under random rotations and reflections; scale
invariance with eps = 0; the VJP against complex-step derivatives.
"""

from __future__ import annotations

import numpy as np

from . import tensors as T


def invariants(x, l_max: int):
    """q [N, l_max + 1, C] from the (l, l) -> 0 couplings of the stored
    components (§3 "Symbolic construction": the coupling tensor of the
    path (l, l, 0))."""
    off = T.rank_offsets(l_max)
    N, _, C = x.shape
    q = np.zeros((N, l_max + 1, C), dtype=x.dtype)
    for l in range(l_max + 1):
        K = T.coupling_tensor(l, l, 0)[0]                   # (2l+1, 2l+1)
        xl = x[:, off[l]:off[l + 1], :]
        q[:, l, :] = np.einsum('ab,uak,ubk->uk', K, xl, xl)
    return q


def rms_norm_fwd(x, l_max: int, eps: float, gamma=None):
    """(y [N, rows, C], inv_s [N])."""
    off = T.rank_offsets(l_max)
    N, _, C = x.shape
    q = invariants(x, l_max)
    s = np.sqrt(q.sum(axis=(1, 2)) / ((l_max + 1) * C) + eps)
    y = np.empty(x.shape, dtype=np.result_type(x, s, np.float64 if gamma is None else gamma))
    for l in range(l_max + 1):
        gl = np.ones(C) if gamma is None else gamma[l]
        y[:, off[l]:off[l + 1], :] = gl[None, None, :] * x[:, off[l]:off[l + 1], :] / s[:, None, None]
    return y, 1.0 / s


def rms_norm_vjp(x, l_max: int, eps: float, g, gamma=None):
    """(x_bar [N, rows, C], gamma_bar [l_max + 1, C]) of L = <g, y>."""
    off = T.rank_offsets(l_max)
    N, _, C = x.shape
    q = invariants(x, l_max)
    s = np.sqrt(q.sum(axis=(1, 2)) / ((l_max + 1) * C) + eps)
    gam = np.ones((l_max + 1, C)) if gamma is None else gamma
    B = np.zeros(N, dtype=np.result_type(x, g))
    gbar = np.zeros((l_max + 1, C), dtype=np.result_type(x, g))
    for l in range(l_max + 1):
        xl, gl = x[:, off[l]:off[l + 1], :], g[:, off[l]:off[l + 1], :]
        B += np.einsum('uak,uak,k->u', gl, xl, gam[l])
        gbar[l] = np.einsum('uak,uak,u->k', gl, xl, 1.0 / s)
    xb = np.empty_like(g, dtype=np.result_type(x, g))
    for l in range(l_max + 1):
        K = T.coupling_tensor(l, l, 0)[0]
        xl, gl = x[:, off[l]:off[l + 1], :], g[:, off[l]:off[l + 1], :]
        Kx = np.einsum('ab,ubk->uak', 0.5 * (K + K.T), xl)
        xb[:, off[l]:off[l + 1], :] = (gam[l][None, None, :] * gl / s[:, None, None]
                                        - (B / (s ** 3 * (l_max + 1) * C))[:, None, None] * Kx)
    return xb, gbar
