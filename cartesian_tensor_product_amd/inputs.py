"""Seeded synthetic inputs shared by the GPU path's tests/bench and the oracle.

This module holds no arithmetic of the method: it only draws positions,
neighbour graphs, features, weights and cotangents, in a fixed order from
``numpy.random.default_rng(seed)``, in float64, and rounds them to float32.
Shapes that depend on the coupling paths (number of paths, output rows) are
passed in by the caller.

Workloads (the FlashCart paper, §6 "Kernel microbenchmarks" and App. F
"Runtime and memory measurements"; synthetic, as the pages' own are):

* ``tiny``      32 nodes, 6 A cube, 8 neighbours, 8 channels, ranks <= 1, rc 6.
* ``micro``     1024 nodes, 20 A cube, 128 neighbours (E = 131072),
                128 channels, ranks <= 2, rc 5.
* ``micro_hi``  the same generator at ranks <= 3 and <= 4, plus a position
                cotangent for the VJP-of-VJP.
* ``ladder``    4096 nodes, 128 channels, ranks <= 3, order 4.
* ``diamond``   1000-atom diamond cell (5x5x5 conventional cells,
                a = 3.567 A, periodic), rc 5 A radius neighbour list.

Draw order within a workload: positions, graph, features, weights,
cotangents.  Neighbours of a node are drawn uniformly without replacement from
the other nodes and stored in increasing sender order; edges are sorted by
receiver (receiver-sorted CSR).
"""

from __future__ import annotations

import numpy as np

SEEDS = {"tiny": 0, "micro": 1, "micro_hi": 2, "ladder": 3, "diamond": 4,
         "diamond_rattle": 5}


def f32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))


def normal(rng, shape, std=1.0) -> np.ndarray:
    return f32(rng.standard_normal(shape) * std)


def random_graph(rng, n_nodes: int, k: int):
    """Receiver-sorted CSR with k distinct senders j != i per receiver i."""
    rowptr = np.arange(n_nodes + 1, dtype=np.int64) * k
    sender = np.empty(n_nodes * k, dtype=np.int64)
    for i in range(n_nodes):
        pick = rng.choice(n_nodes - 1, size=k, replace=False)
        pick = pick + (pick >= i)           # skip the receiver itself
        sender[i * k:(i + 1) * k] = np.sort(pick)
    return rowptr.astype(np.int32), sender.astype(np.int32)


def random_cloud(seed: int, n_nodes: int, k: int, box: float):
    """Positions uniform in [0, box)^3 (non-periodic) and a random graph."""
    rng = np.random.default_rng(seed)
    pos = f32(rng.uniform(0.0, box, size=(n_nodes, 3)))
    rowptr, sender = random_graph(rng, n_nodes, k)
    return rng, pos, rowptr, sender


def edge_conv_inputs(seed: int, n_nodes: int, k: int, box: float, channels: int,
                     n_in_rows: int, n_paths: int, n_out_rows: int,
                     n_basis: int = 8, with_vpos: bool = False, with_edge_w: bool = False):
    """Everything one edge-convolution call needs, drawn in the fixed order.

    Returns a dict with pos [N,3], rowptr [N+1], sender [E], shift None,
    x [N, n_in_rows, C] ~ N(0,1), W [n_basis, P, C] ~ N(0, 1/n_basis)
    (variance), g [N, n_out_rows, C] ~ N(0,1), optionally v_pos [N,3] and,
    last, explicit per-edge weights w [E, P, C] ~ N(0,1) for the interface
    that takes them given (drawing them does not change the earlier draws).
    """
    rng, pos, rowptr, sender = random_cloud(seed, n_nodes, k, box)
    x = normal(rng, (n_nodes, n_in_rows, channels))
    W = normal(rng, (n_basis, n_paths, channels), std=1.0 / np.sqrt(n_basis))
    g = normal(rng, (n_nodes, n_out_rows, channels))
    out = dict(pos=pos, rowptr=rowptr, sender=sender, shift=None, x=x, W=W, g=g)
    if with_vpos:
        out["v_pos"] = normal(rng, (n_nodes, 3))
    if with_edge_w:
        out["w"] = edge_weights(rng, len(sender), n_paths, channels)
    return out


def edge_weights(rng, n_edges: int, n_paths: int, channels: int) -> np.ndarray:
    """Per-edge weights w [E, P, C] ~ N(0,1), drawn in edge-row blocks so that
    large arrays never pass through a float64 copy of their full size."""
    w = np.empty((n_edges, n_paths, channels), dtype=np.float32)
    step = max(1, (1 << 22) // max(1, n_paths * channels))
    for e0 in range(0, n_edges, step):
        e1 = min(n_edges, e0 + step)
        w[e0:e1] = rng.standard_normal((e1 - e0, n_paths, channels)).astype(np.float32)
    return w


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------

WORKLOADS = {
    # name: (seed, nodes, neighbours, box [A], channels, l_max, r_cut [A])
    "tiny": (0, 32, 8, 6.0, 8, 1, 6.0),
    "micro": (1, 1024, 128, 20.0, 128, 2, 5.0),
    "micro_hi3": (2, 1024, 128, 20.0, 128, 3, 5.0),
    "micro_hi4": (2, 1024, 128, 20.0, 128, 4, 5.0),
}


def ladder_inputs(seed: int, n_nodes: int, channels: int, n_a_rows: int,
                  weight_shapes: list):
    """Node-local ladder inputs.

    ``weight_shapes`` lists (shape, kind, fan_in) in the flat weight order:
    kind 'normal' draws N(0, 1/fan_in), kind 'one_plus' draws 1 + 0.1 N(0,1)
    (a path weight a = 1 + delta with a nonzero delta so that swapped path
    weights are caught).  A ~ N(0,1) [N, n_a_rows, C]; then the weights;
    then the output cotangent g_z (shape given by the caller via
    ``gz_rows``) is drawn by ``ladder_cotangent``.
    """
    rng = np.random.default_rng(seed)
    A = normal(rng, (n_nodes, n_a_rows, channels))
    ws = []
    for shape, kind, fan_in in weight_shapes:
        if kind == "normal":
            ws.append(normal(rng, shape, std=1.0 / np.sqrt(fan_in)))
        elif kind == "one_plus":
            ws.append(f32(1.0 + 0.1 * rng.standard_normal(shape)))
        else:
            raise ValueError(kind)
    return rng, A, ws


def ladder_cotangent(rng, n_nodes: int, n_rows: int, channels: int):
    return normal(rng, (n_nodes, n_rows, channels))


# ----------------------------------------------------------------------------
# diamond cell
# ----------------------------------------------------------------------------

DIAMOND_A = 3.567


def diamond_positions(ncell: int = 5, a: float = DIAMOND_A):
    """Conventional diamond cells: fcc lattice plus the (1/4,1/4,1/4) basis."""
    fcc = np.array([[0, 0, 0], [0, .5, .5], [.5, 0, .5], [.5, .5, 0]])
    basis = np.concatenate([fcc, fcc + 0.25])
    cells = np.array([[i, j, k] for i in range(ncell) for j in range(ncell)
                      for k in range(ncell)], dtype=np.float64)
    pos = (cells[:, None, :] + basis[None, :, :]).reshape(-1, 3) * a
    return pos, ncell * a


def periodic_neighbours(pos64: np.ndarray, box: float, r_cut: float):
    """Receiver-sorted neighbour list under the minimum-image convention.

    Valid when r_cut < box/2 (each pair then has at most one image inside).
    Returns rowptr, sender, shift with r_e = pos[sender] - pos[receiver] + shift.
    """
    assert r_cut < box / 2
    n = pos64.shape[0]
    rowptr = [0]
    senders, shifts = [], []
    for i in range(n):
        d = pos64 - pos64[i]
        img = -box * np.round(d / box)
        dd = d + img
        r = np.sqrt(np.sum(dd * dd, axis=1))
        js = np.nonzero((r < r_cut) & (np.arange(n) != i))[0]
        senders.append(js)
        shifts.append(img[js])
        rowptr.append(rowptr[-1] + len(js))
    return (np.asarray(rowptr, dtype=np.int32),
            np.concatenate(senders).astype(np.int32),
            f32(np.concatenate(shifts)))


def diamond_inputs(channels: int = 128, r_cut: float = 5.0, rattle: float = 0.0,
                   ncell: int = 5, n_basis: int = 8, n_paths: int = 4,
                   ladder_weight_shapes: list = ()):
    """1000-atom diamond cell with one shared scalar embedding per atom.

    Draw order (seed 4): embedding e ~ N(0,1) [C], radial weights
    W [n_basis, n_paths, C] ~ N(0, 1/n_basis), then the ladder weights.  With
    ``rattle`` > 0 the positions get N(0, rattle^2) displacements drawn from
    seed 5 before the neighbour list is built.
    """
    pos64, box = diamond_positions(ncell)
    if rattle > 0:
        rr = np.random.default_rng(SEEDS["diamond_rattle"])
        pos64 = pos64 + rattle * rr.standard_normal(pos64.shape)
        pos64 = np.mod(pos64, box)
    pos = f32(pos64)
    rowptr, sender, shift = periodic_neighbours(pos.astype(np.float64), box, r_cut)
    rng = np.random.default_rng(SEEDS["diamond"])
    emb = normal(rng, (channels,))
    W = normal(rng, (n_basis, n_paths, channels), std=1.0 / np.sqrt(n_basis))
    ws = []
    for shape, kind, fan_in in ladder_weight_shapes:
        if kind == "normal":
            ws.append(normal(rng, shape, std=1.0 / np.sqrt(fan_in)))
        else:
            ws.append(f32(1.0 + 0.1 * rng.standard_normal(shape)))
    x = np.ascontiguousarray(np.broadcast_to(emb, (pos.shape[0], 1, channels)))
    return dict(pos=pos, box=box, rowptr=rowptr, sender=sender, shift=shift,
                x=x, W=W, ladder_weights=ws)


def radial_mlp_weights(rng, n_paths: int, channels: int) -> np.ndarray:
    """Flat weights of the radial network, W1 [8, 64] ~ N(0, 1/8), then
    W2 [64, 64] and W3 [64, P C] ~ N(0, 1/64) (variance 1/fan_in)."""
    W1 = normal(rng, (8, 64), std=1.0 / np.sqrt(8))
    W2 = normal(rng, (64, 64), std=1.0 / 8.0)
    W3 = normal(rng, (64, n_paths * channels), std=1.0 / 8.0)
    return np.concatenate([W1.ravel(), W2.ravel(), W3.ravel()])


def block_weights(seed: int, entries: list) -> dict:
    """Random weights of a message-passing block, drawn in the listed order
    from one generator: ``entries`` holds (name, shape, kind, fan_in) with
    kind 'normal' (N(0, 1/fan_in)), 'one_plus' (1 + 0.1 N(0,1)) or 'mlp' (the
    radial network's flat weights; shape = (n_paths, channels))."""
    rng = np.random.default_rng(seed)
    out = {}
    for name, shape, kind, fan_in in entries:
        if kind == "normal":
            out[name] = normal(rng, shape, std=1.0 / np.sqrt(fan_in))
        elif kind == "one_plus":
            out[name] = f32(1.0 + 0.1 * rng.standard_normal(shape))
        elif kind == "mlp":
            out[name] = radial_mlp_weights(rng, shape[0], shape[1])
        else:
            raise ValueError(kind)
    return out
