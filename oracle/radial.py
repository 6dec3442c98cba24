"""Oracle for the pages' radial network and the convolution it weights.

TEST INFRASTRUCTURE ONLY.  Plain fp64 numpy.  Follows the FlashCart paper,
App. E "Model architecture" (the radial weights w_{eta k}(r) of Eq. E1) and
App. F "Model architecture and training":

* features: eight Chebyshev functions of the cosine-transformed distance,
  T_n(cos(pi r / r_max)), n = 0..7, times a polynomial cutoff envelope with
  p = 6 whose value and first two derivatives vanish at r_max.  The pages
  name the envelope's property and source, not its formula; the reading is
  the polynomial with exactly that property,
      u(d) = 1 - (p+1)(p+2)/2 d^p + p(p+2) d^(p+1) - p(p+1)/2 d^(p+2),
  d = r / r_max < 1 (u = 0 beyond), i.e. u'(d) = -p(p+1)(p+2)/2 d^(p-1) (1-d)^2.
* a bias-free MLP with two hidden layers of width 64 and SiLU activations
  (sigma(0) = 0) and one output per coupling path and channel:
      w[e, :, :] = (SiLU(SiLU(phi_e W1) W2) W3).reshape(P, C),
  W1 [8, 64], W2 [64, 64], W3 [64, P C].
* the convolution of Eq. 1 / E1 with these weights (the explicit-weight
  oracle of conv.py), and its VJP carried through the MLP to the positions
  and to W1, W2, W3.

Parity pins (tests/test_oracle_radial.py): the Chebyshev features against
cos(n theta); the envelope's value and derivatives at 0 and r_max; the
pages' statement that w and its first two r-derivatives vanish at r_max;
the hand-written MLP VJP and the convolution VJP against complex-step
derivatives; the network on one edge with sparse weights against a closed
form in scalar code (layer order, both SiLUs, the path-major output column
order; tests/test_oracle_hand.py).
"""

from __future__ import annotations

import numpy as np
from numpy.polynomial import chebyshev as cheb

from . import conv

N_FEAT = 8
HIDDEN = 64
P_ENV = 6


def envelope(d, p: int = P_ENV):
    u = (1.0 - (p + 1) * (p + 2) / 2.0 * d ** p + p * (p + 2) * d ** (p + 1)
         - p * (p + 1) / 2.0 * d ** (p + 2))
    return np.where(np.real(d) < 1.0, u, 0.0)


def features(r, r_max: float):
    """phi [E, 8] = T_n(cos(pi r / r_max)) u(r / r_max)."""
    x = np.cos(np.pi * r / r_max)
    return cheb.chebvander(x, N_FEAT - 1) * envelope(r / r_max)[:, None]


def silu(a):
    return a / (1.0 + np.exp(-a))


def silu_grad(a):
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def radial_mlp(r, r_max: float, W1, W2, W3, P: int, C: int):
    """w [E, P, C]."""
    h1 = silu(features(r, r_max) @ W1)
    h2 = silu(h1 @ W2)
    return (h2 @ W3).reshape(len(r), P, C)


def radial_mlp_vjp(r, r_max: float, W1, W2, W3, w_bar):
    """(r_bar [E], W1_bar, W2_bar, W3_bar) of L = <w_bar, w>, by hand; the
    feature derivative d phi / d r by complex step (exact to rounding)."""
    E = len(r)
    phi = features(r, r_max)
    a1 = phi @ W1
    h1 = silu(a1)
    a2 = h1 @ W2
    h2 = silu(a2)
    wb = w_bar.reshape(E, W3.shape[1])
    W3b = h2.T @ wb
    a2b = (wb @ W3.T) * silu_grad(a2)
    W2b = h1.T @ a2b
    a1b = (a2b @ W2.T) * silu_grad(a1)
    W1b = phi.T @ a1b
    phib = a1b @ W1.T
    h = 1e-20
    dphi = features(r.astype(np.complex128) + 1j * h, r_max).imag / h
    return np.sum(phib * dphi, axis=1), W1b, W2b, W3b


def edge_lengths(pos, rowptr, sender, shift=None):
    """(r [E], r_vec [E, 3]) with r_vec = pos[v] - pos[u] + shift."""
    recv = conv.receivers(rowptr)
    rv = pos[sender] - pos[recv]
    if shift is not None:
        rv = rv + shift
    return np.sqrt(np.sum(rv * rv, axis=1)), rv


def edge_conv_fwd_mlp(spec, pos, rowptr, sender, x, W1, W2, W3, shift=None, r_max=None):
    """Eq. 1 with w = radial_mlp(r_e)."""
    r_max = spec.r_cut if r_max is None else r_max
    r, _ = edge_lengths(pos, rowptr, sender, shift)
    w = radial_mlp(r, r_max, W1, W2, W3, spec.n_paths, x.shape[-1])
    return conv.edge_conv_fwd_w(spec, pos, rowptr, sender, x, w, shift)


def edge_conv_vjp_mlp(spec, pos, rowptr, sender, x, W1, W2, W3, g, shift=None, r_max=None):
    """(x_bar, pos_bar, W1_bar, W2_bar, W3_bar) of L = <g, z>: the
    explicit-weight VJP (w held fixed) plus the chain rule through w(r_e)."""
    r_max = spec.r_cut if r_max is None else r_max
    N = pos.shape[0]
    r, rv = edge_lengths(pos, rowptr, sender, shift)
    w = radial_mlp(r, r_max, W1, W2, W3, spec.n_paths, x.shape[-1])
    xb, pb, wb = conv.edge_conv_vjp_w(spec, pos, rowptr, sender, x, w, g, shift)
    rb, W1b, W2b, W3b = radial_mlp_vjp(r, r_max, W1, W2, W3, wb)
    keep = np.real(r) > 0
    q = (rb / np.where(keep, r, 1.0) * keep)[:, None] * rv        # dL/dr_vec
    recv = conv.receivers(rowptr)
    pb = pb + conv.segment_sum(q, sender, N) - conv.segment_sum(q, recv, N)
    return xb, pb, W1b, W2b, W3b
