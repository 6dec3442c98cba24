"""Hand-expanded pins of the oracle's composite parts: the ladder with path
weights a != 1, the radial network on one edge, and the full message-passing
block on two atoms.

Each expected value is written out here in explicit 3 x 3 (and 3 x 3 x 3)
tensor algebra or scalar ``math`` code, step by step in the order the
FlashCart paper gives, without the oracle's probed coupling tensors,
projectors or reconstruction matrices.  A dropped term, a swapped path
weight, a transposed layer or a misplaced gate changes the numbers.

Coupling constants are the path normalisation used throughout (each path is
scaled so that the coupling of direction tensors T_l1(n), T_l2(n) gives
T_L(n)); at ranks <= 2 they are: (0,l)->l: 1, (1,1)->0: 1 (the dot product),
(1,1)->2: 3/2 (the paper's printed (1,1)->2 example), (1,2)->1: 1,
(2,2)->0: 2/3, (2,2)->2: 2; (3,3)->0: 2/5.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import ladder, model, radial

I3 = np.eye(3)


# --- stored components <-> full tensors, written out per rank ---------------
# stored order (the independent components of §3 "Symbolic construction"):
#   rank 1: x y z;  rank 2: xx xy yy xz yz;  rank 3: xxx xxy xyy yyy xxz xyz yyz

def full2(c):
    xx, xy, yy, xz, yz = c
    return np.array([[xx, xy, xz], [xy, yy, yz], [xz, yz, -xx - yy]])


def sel2(M):
    return np.array([M[0, 0], M[0, 1], M[1, 1], M[0, 2], M[1, 2]])


def full3(c):
    xxx, xxy, xyy, yyy, xxz, xyz, yyz = c
    val = {(3, 0, 0): xxx, (2, 1, 0): xxy, (1, 2, 0): xyy, (0, 3, 0): yyy,
           (2, 0, 1): xxz, (1, 1, 1): xyz, (0, 2, 1): yyz,
           (1, 0, 2): -xxx - xyy, (0, 1, 2): -xxy - yyy, (0, 0, 3): -xxz - yyz}
    T = np.zeros((3, 3, 3))
    for i in range(3):
        for j in range(3):
            for k in range(3):
                n = [0, 0, 0]
                for a in (i, j, k):
                    n[a] += 1
                T[i, j, k] = val[tuple(n)]
    return T


def stf2(X):
    S = 0.5 * (X + X.T)
    return S - np.trace(S) / 3.0 * I3


def to_full(l, c):
    return {0: lambda c: c[0], 1: lambda c: np.array(c), 2: full2, 3: full3}[l](c)


def to_stored(l, t):
    return {0: lambda t: np.array([t]), 1: lambda t: np.array(t), 2: sel2}[l](t)


def couple(l1, l2, L, X, Y):
    """Coupling of full tensors X (rank l1), Y (rank l2) into rank L."""
    if l1 == 0:
        return X * Y
    if l2 == 0:
        return X * Y
    if (l1, l2, L) == (1, 1, 0):
        return float(X @ Y)
    if (l1, l2, L) == (1, 1, 2):
        return 1.5 * stf2(np.outer(X, Y))
    if (l1, l2, L) == (1, 2, 1):
        return Y @ X
    if (l1, l2, L) == (2, 1, 1):
        return X @ Y
    if (l1, l2, L) == (2, 2, 0):
        return 2.0 / 3.0 * float(np.sum(X * Y))
    if (l1, l2, L) == (2, 2, 2):
        return 2.0 * stf2(X @ Y)
    raise KeyError((l1, l2, L))


# paths of one ladder step (L first, then (l1, l2) lexicographic), ranks <= 2
STEP_PATHS = {2: [(0, 0, 0), (1, 1, 0), (2, 2, 0), (0, 1, 1), (1, 0, 1), (1, 2, 1), (2, 1, 1),
                  (0, 2, 2), (1, 1, 2), (2, 0, 2), (2, 2, 2)],
              1: [(0, 0, 0), (1, 1, 0), (2, 2, 0), (0, 1, 1), (1, 0, 1), (1, 2, 1), (2, 1, 1)]}
OFF = [0, 1, 4, 9]


def split(A_node, C):
    """A[rows, C] -> {l: [C full tensors]} for ranks <= 2."""
    return {l: [to_full(l, A_node[OFF[l]:OFF[l + 1], k]) for k in range(C)] for l in range(3)}


def _zero(L):
    return 0.0 if L == 0 else (np.zeros(3) if L == 1 else np.zeros((3, 3)))


@pytest.mark.parametrize("variant", ["reduced", "full"])
def test_ladder_order_three_hand_expansion(variant):
    """§5 Eq. 2 (full) and App. E "Path-reduced products" at ranks <= 2,
    order 3, l_out = 1, width 2, with path weights a = 1 + 0.3 N(0,1):

      reduced: phi1_l = a1[l] A_l;
               phi^q_L = P_{q,L}^{-1/2} sum_{eta -> L} a^q[eta] (phi^{q-1}_l1 (x) A_l2)_L;
               z_L = W_L (phi1_L + phi2_L + phi3_L),  L <= 1
      full:    phi1_l = W1_l A_l;
               phi^q_L[k] = sum_{eta, k'} W^q_L[k, eta C + k'] (phi^{q-1}_l1[k'] (x) A_l2[k'])_L;
               z_L = phi1_L + phi2_L + phi3_L
    """
    C, order = 2, 3
    spec = ladder.LadderSpec(2, 2, 1, order, variant, C)
    assert spec.paths[2] == STEP_PATHS[2] and spec.paths[3] == STEP_PATHS[1]
    rng = np.random.default_rng(11)
    A = rng.normal(size=(2, 9, C))
    ws = []
    for name, shape, kind, fan in spec.weight_shapes():
        ws.append(1.0 + 0.3 * rng.normal(size=shape) if kind == "one_plus" else rng.normal(size=shape))
    w = dict(zip([s[0] for s in spec.weight_shapes()], ws))
    z = ladder.ladder_fwd(spec, A, ws)
    assert z.shape == (2, 4, C)

    for u in range(2):
        Af = split(A[u], C)
        # step 1
        if variant == "reduced":
            phi = {l: [w["a1"][l, k] * Af[l][k] for k in range(C)] for l in range(3)}
        else:
            phi = {l: [sum(w[f"W1_{l}"][k, j] * Af[l][j] for j in range(C)) for k in range(C)]
                   for l in range(3)}
        acc = {L: list(phi[L]) for L in range(2)}
        for q in (2, 3):
            paths = STEP_PATHS[2 if q == 2 else 1]
            Ls = sorted({p[2] for p in paths})
            new = {}
            for L in Ls:
                members = [(i, p) for i, p in enumerate(paths) if p[2] == L]
                if variant == "reduced":
                    s = 1.0 / math.sqrt(len(members))
                    new[L] = [s * sum(w[f"a{q}"][i, k] * couple(l1, l2, L, phi[l1][k], Af[l2][k])
                                      for i, (l1, l2, _) in members) for k in range(C)]
                else:
                    Wq = w[f"W{q}_{L}"]
                    new[L] = []
                    for k in range(C):
                        tot = _zero(L)
                        for eta, (_, (l1, l2, _)) in enumerate(members):
                            for kp in range(C):
                                tot = tot + Wq[k, eta * C + kp] * couple(l1, l2, L, phi[l1][kp], Af[l2][kp])
                        new[L].append(tot)
            for L in range(2):
                acc[L] = [acc[L][k] + new[L][k] for k in range(C)]
            phi = new
        for L in range(2):
            for k in range(C):
                if variant == "reduced":
                    want = sum(w[f"W_{L}"][k, j] * acc[L][j] for j in range(C))
                else:
                    want = acc[L][k]
                got = z[u, OFF[L]:OFF[L + 1], k]
                assert np.allclose(got, np.atleast_1d(want), rtol=1e-12, atol=1e-12), (u, L, k)


# --- radial network on one edge ---------------------------------------------

def silu(a):
    return a / (1.0 + math.exp(-a))


def test_radial_mlp_one_edge_closed_form():
    """App. E/F radial network on one edge at r = 5/3 A, r_max = 5 A.

    Features: T_n(cos(pi r / r_max)) = cos(n pi / 3) times the p = 6 envelope
    at d = 1/3, u(d) = 1 - 28 d^6 + 48 d^7 - 21 d^8 (exact rational here).
    With sparse weights the network reduces to
      h1_0 = SiLU(0.7 u),  h1_1 = SiLU((-1.3 cos(pi) + 0.4 cos(5 pi / 3)) u)
      h2_0 = SiLU(0.9 h1_1),  h2_2 = SiLU(1.1 h1_0 - 0.5 h1_1)
      w[eta, k] = c0[eta C + k] h2_0 + c2[eta C + k] h2_2
    so the layer order, each SiLU and the output column order (path-major,
    then channel) are all visible.
    """
    P, C = 2, 3
    d = Fraction(1, 3)
    u = float(1 - 28 * d ** 6 + 48 * d ** 7 - 21 * d ** 8)
    W1 = np.zeros((8, 64))
    W1[0, 0], W1[3, 1], W1[5, 1] = 0.7, -1.3, 0.4
    W2 = np.zeros((64, 64))
    W2[0, 2], W2[1, 0], W2[1, 2] = 1.1, 0.9, -0.5
    W3 = np.zeros((64, P * C))
    c0 = np.array([0.3, -0.2, 0.5, 1.7, -0.9, 0.25])
    c2 = np.array([-1.1, 0.6, 0.05, -0.4, 0.8, 2.0])
    W3[0], W3[2] = c0, c2
    r = np.array([5.0 / 3.0])
    w = radial.radial_mlp(r, 5.0, W1, W2, W3, P, C)
    h1_0 = silu(0.7 * u)
    h1_1 = silu((-1.3 * math.cos(math.pi) + 0.4 * math.cos(5 * math.pi / 3)) * u)
    h2_0 = silu(0.9 * h1_1)
    h2_2 = silu(1.1 * h1_0 - 0.5 * h1_1)
    for eta in range(P):
        for k in range(C):
            want = c0[eta * C + k] * h2_0 + c2[eta * C + k] * h2_2
            assert w[0, eta, k] == pytest.approx(want, rel=1e-13, abs=1e-15)
    # the envelope at d = 1/3 as an exact rational: 1 - 28/729 + 48/2187 - 21/6561
    assert u == pytest.approx(float(Fraction(6561 - 252 + 144 - 21, 6561)), rel=1e-15)


# --- the message-passing block on two atoms, C = 1 --------------------------

def t_dir(l, n):
    """T_l(n) for a unit vector n, stored components (closed forms,
    (2l-1)!!/l! STF(n^l))."""
    x, y, z = n
    if l == 0:
        return np.array([1.0])
    if l == 1:
        return np.array([x, y, z])
    if l == 2:
        return 1.5 * np.array([x * x - 1 / 3, x * y, y * y - 1 / 3, x * z, y * z])
    return 2.5 * np.array([x ** 3 - 0.6 * x, x * x * y - 0.2 * y, x * y * y - 0.2 * x, y ** 3 - 0.6 * y,
                           x * x * z - 0.2 * z, x * y * z, y * y * z - 0.2 * z])


def self_invariant(l, c):
    """(l,l)->0 coupling of a tensor with itself: the constant times the
    full contraction of the reconstructed tensor."""
    if l == 0:
        return c[0] * c[0]
    if l == 1:
        return float(np.dot(c, c))
    if l == 2:
        M = full2(c)
        return 2.0 / 3.0 * float(np.sum(M * M))
    T = full3(c)
    return 0.4 * float(np.sum(T * T))


def pair_invariant(l, a, b):
    if l == 0:
        return a[0] * b[0]
    if l == 1:
        return float(np.dot(a, b))
    if l == 2:
        return 2.0 / 3.0 * float(np.sum(full2(a) * full2(b)))
    return 0.4 * float(np.sum(full3(a) * full3(b)))


def hand_block_energy(pos, h0, w, r_cut, eps):
    """E of one message-passing block on two atoms that neighbour each other
    (C = 1, ranks <= 3, path-reduced ladder of order 2, l_out = 0), each step
    written out in the order of App. E "Model architecture":

      hb_v   = Mpre h0_v                                     (channel map before the convolution)
      a_u    = sum_{v} w_l(r_uv) hb_v T_l(r_hat_uv)         (Eq. E1, N_bar = 1)
      m_l    = M_l a_l,  m_0 += R0 h0_u                      (rank-wise map, residual)
      n      = gamma1 m / s,  s = sqrt(sum_l q_l / 4 + eps)  (RMS norm, q = (l,l)->0)
      y_0    = SiLU(n_0),  y_l = SiLU(n_0) n_l               (gates)
      A_l    = n_l + O_l y_l                                 (output map + input)
      phi1_l = a1_l A_l;  phi2 = 1/2 sum_l a2_l (phi1_l (x) A_l)_0
      z      = W_0 (phi1_0 + phi2)                           (ladder)
      o      = z + R2 A_0;  f = gamma2 o / sqrt(o^2 + eps)
      E_u    = sum_j wr3_j SiLU(sum_i Wr2_ij SiLU(Wr1_i f))
    """
    mlp = w["mlp"]
    W1, W2, W3 = mlp[:512].reshape(8, 64), mlp[512:4608].reshape(64, 64), mlp[4608:].reshape(64, 4)
    E = 0.0
    for u, v in ((0, 1), (1, 0)):
        rv = pos[v] - pos[u]
        r = math.sqrt(float(rv @ rv))
        n_hat = rv / r
        dd = r / r_cut
        env = 1 - 28 * dd ** 6 + 48 * dd ** 7 - 21 * dd ** 8
        theta = math.pi * r / r_cut
        feat = [math.cos(k * theta) * env for k in range(8)]
        h1 = [silu(sum(feat[i] * W1[i, j] for i in range(8))) for j in range(64)]
        h2 = [silu(sum(h1[i] * W2[i, j] for i in range(64))) for j in range(64)]
        wl = [sum(h2[i] * W3[i, l] for i in range(64)) for l in range(4)]
        a = {l: wl[l] * (w["Mpre"][0, 0] * h0[v]) * t_dir(l, n_hat) for l in range(4)}
        m = {l: w["M"][l, 0, 0] * a[l] for l in range(4)}
        m[0] = m[0] + w["R0"][0, 0] * h0[u]
        s = math.sqrt(sum(self_invariant(l, m[l]) for l in range(4)) / 4.0 + eps)
        n = {l: w["gamma1"][l, 0] * m[l] / s for l in range(4)}
        sg = silu(n[0][0])
        y = {0: np.array([sg])}
        for l in range(1, 4):
            y[l] = sg * n[l]
        A = {l: n[l] + w["O"][l, 0, 0] * y[l] for l in range(4)}
        a1, a2, W0 = w["ladder0"][:, 0], w["ladder1"][:, 0], w["ladder2"][0, 0]
        phi1 = {l: a1[l] * A[l] for l in range(4)}
        phi2 = 0.5 * sum(a2[l] * pair_invariant(l, phi1[l], A[l]) for l in range(4))
        zz = W0 * (phi1[0][0] + phi2)
        o = zz + w["R2"][0, 0] * A[0][0]
        f = w["gamma2"][0, 0] * o / math.sqrt(o * o + eps)
        g1 = [silu(w["Wr1"][0, j] * f) for j in range(64)]
        g2 = [silu(sum(g1[i] * w["Wr2"][i, j] for i in range(64))) for j in range(64)]
        E += sum(w["wr3"][j] * g2[j] for j in range(64))
    return E


def _two_atom_block(seed=35):
    from oracle import conv
    C, r_cut, eps = 1, 5.0, 1e-5
    cspec = conv.ConvSpec(0, 3, 3, r_cut)
    lspec = ladder.LadderSpec(3, 3, 0, 2, "reduced", C)
    rng = np.random.default_rng(seed)
    w = {}
    for name, shape in model.block_weight_shapes(C, 3, cspec.n_paths, lspec):
        if name.startswith("gamma"):
            w[name] = 1.0 + 0.2 * rng.normal(size=shape)
        elif name.startswith("ladder"):
            kind = lspec.weight_shapes()[int(name[6:])][2]
            shape = lspec.weight_shapes()[int(name[6:])][1]
            w[name] = (1.0 + 0.3 * rng.normal(size=shape)) if kind == "one_plus" else rng.normal(size=shape)
        elif name == "mlp":
            w[name] = np.concatenate([rng.normal(size=512) / math.sqrt(8), rng.normal(size=4096) / 8.0,
                                      rng.normal(size=256) / 8.0])
        else:
            w[name] = rng.normal(size=shape)
    pos = np.array([[0.1, -0.2, 0.3], [1.4, 0.9, -1.2]])
    h0 = np.array([0.8, -1.3])
    rowptr = np.array([0, 1, 2], dtype=np.int32)
    sender = np.array([1, 0], dtype=np.int32)
    return cspec, lspec, w, pos, rowptr, sender, h0, r_cut, eps


def test_block_two_atoms_hand_walkthrough():
    """The oracle's block energy equals the step-by-step scalar evaluation,
    and its forces equal fourth-order central differences of that scalar
    energy."""
    cspec, lspec, w, pos, rowptr, sender, h0, r_cut, eps = _two_atom_block()
    x = h0.reshape(2, 1, 1)
    E, e_atom = model.block_energy(cspec, lspec, w, pos, rowptr, sender, None, x, 1.0, eps)
    want = hand_block_energy(pos, h0, w, r_cut, eps)
    assert abs(want) > 1e-2
    assert E == pytest.approx(want, rel=1e-12)
    E2, _, F = model.block_energy_forces(cspec, lspec, w, pos, rowptr, sender, None, x, 1.0, eps)
    assert E2 == pytest.approx(want, rel=1e-12)
    # fourth-order central differences (truncation O(h^4))
    h = 5e-4
    for i in range(2):
        for j in range(3):
            e = {}
            for k in (-2, -1, 1, 2):
                pk = pos.copy()
                pk[i, j] += k * h
                e[k] = hand_block_energy(pk, h0, w, r_cut, eps)
            fd = -(-e[2] + 8 * e[1] - 8 * e[-1] + e[-2]) / (12 * h)
            assert F[i, j] == pytest.approx(fd, rel=1e-7, abs=1e-8 * np.abs(F).max())
    assert np.abs(F).max() > 1e-2
