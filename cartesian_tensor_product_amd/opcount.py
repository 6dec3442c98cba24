"""Algorithmic operation counts of the edge convolution, per edge and channel.

Counted from the exact coupling tables of the generator (the nonzero terms
c x_b1 y_b2 of each path's bilinear polynomial, FlashCart paper App. B
Eq. B1), one fused multiply-add per term and per weight, for the leanest
formulation of Eq. 1 (forward) and Eq. C1 carried to the positions (VJP)
that this library evaluates.  For a path p = (l1, l2) -> L with T_p terms,
n1 = 2 l1 + 1 inputs, n2 = 2 l2 + 1 direction components and nL = 2L+1
outputs:

forward:
    w_p = sum_b R_b W[b, p]                 n_basis
    z  += w_p f_p(x, y)                     T_p + min(n1, nL)  (the radial
                                            weight scales the smaller side)
VJP:
    w_p and dw_p/dr                         2 n_basis
    x_bar += w_p VJP1_p(g, y)               T_p + min(n1, nL)
    v = VJP2_p(g, x)                        T_p
    y_bar += w_p v;  <g, f_p> = <v, y>      2 n2  (the radial derivative
                                            takes <g, f_p> from v)

With the radial network's output layer fused into the convolution the
basis is its 64 second-layer units (n_basis = 64): w_p = sum_h h2_h W3[h, p]
and dw_p/dr from dh2/dr, per edge and channel.

The products c y_b2 are formed once per edge and shared by all channels;
such per-edge work (geometry, direction tensors, the chain rule of y_bar to
the position) and the sums over lanes are not counted.  A flop is half an
FMA; on gfx950 one wave64 VALU instruction does 64 lane-operations.
"""

from __future__ import annotations

from functools import lru_cache

from cartesian_tensor_product_amd.gen import generate


@lru_cache(maxsize=None)
def _terms(l1: int, l2: int, L: int) -> int:
    return len(generate.coupling_terms(l1, l2, L))


def conv_paths(l_in: int, l_edge: int, l_out: int):
    return [(l1, l2, L) for L in range(l_out + 1) for l1 in range(l_in + 1) for l2 in range(l_edge + 1)
            if generate.admissible(l1, l2, L)]


def conv_fma_per_edge_channel(l_in: int, l_edge: int, l_out: int, n_basis: int = 8) -> dict:
    """{"fwd": FMAs, "vjp": FMAs, "terms": sum of T_p, "paths": P}."""
    paths = conv_paths(l_in, l_edge, l_out)
    T = sum(_terms(*p) for p in paths)
    side = sum(min(2 * l1 + 1, 2 * L + 1) for l1, _, L in paths)
    n2 = sum(2 * l2 + 1 for _, l2, _ in paths)
    fwd = n_basis * len(paths) + T + side
    vjp = 2 * n_basis * len(paths) + 2 * T + side + 2 * n2
    return {"fwd": fwd, "vjp": vjp, "terms": T, "paths": len(paths)}
