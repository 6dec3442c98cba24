"""Algorithmic operation counts of the edge convolution, per edge and channel.

Counted from the exact coupling tables of the generator (the nonzero terms
c x_b1 y_b2 of each path's bilinear polynomial, FlashCart paper App. B
Eq. B1), for the plain formulation of Eq. 1 (forward) and Eq. C1 carried to
the positions (VJP), one fused multiply-add per term and per weight:

forward, per path p = (l1, l2) -> L with T_p terms and 2L+1 outputs:
    w_p = sum_b R_b W[b, p]              n_basis FMAs
    f_p = sum of the T_p terms           T_p FMAs (the products c y_b2 are
                                         formed once per edge, shared by all
                                         channels, and not counted)
    z  += w_p f_p                        2L+1 FMAs
VJP, per path:
    w_p and dw_p/dr                      2 n_basis FMAs
    g_w = w_p g                          2L+1
    x_bar += VJP1(g_w, y)                T_p
    y_bar += VJP2(g_w, x)                T_p
    <g, f_p(x, y)> (radial derivative)   T_p + 2L+1

Per-edge work that is shared by the channels (geometry, direction tensors,
the chain rule of y_bar to the position) is not counted.  A flop is half an
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
    nL = sum(2 * p[2] + 1 for p in paths)
    fwd = n_basis * len(paths) + T + nL
    vjp = 2 * n_basis * len(paths) + nL + 3 * T + nL
    return {"fwd": fwd, "vjp": vjp, "terms": T, "paths": len(paths)}
