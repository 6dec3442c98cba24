"""Pins of the oracle's tensor machinery against the FlashCart paper.

Every check compares the oracle with something other than itself: values the
paper prints (tests/golden), closed forms derived in the comments, textbook
routines, or invariants that the paper states.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import tensors as T

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def rand_rotation(rng, reflect=False):
    q, r = np.linalg.qr(rng.standard_normal((3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] *= -1
    return -q if reflect else q


def rotate_full(l, t, R):
    """Apply R to every index of full tensors t (..., 3^l)."""
    sh = t.shape[:-1]
    tt = t.reshape(sh + (3,) * l)
    for ax in range(l):
        tt = np.moveaxis(np.tensordot(tt, R, axes=([len(sh) + ax], [1])), -1, len(sh) + ax)
    return tt.reshape(sh + (3 ** l,))


def full_of(l, rng):
    return T.recon(l, rng.standard_normal(2 * l + 1))


# -------------------------------------------------------------- components --

@pytest.mark.parametrize("l", range(0, 6))
def test_independent_components(l):
    # 2l+1 stored components (paper §2: (l+1)(l+2)/2 - l(l-1)/2)
    assert len(T.comps(l)) == 2 * l + 1 == T.n_comp(l)
    v = RNG.standard_normal(2 * l + 1)
    t = T.recon(l, v)
    # reconstructed tensors are symmetric ...
    tt = t.reshape((3,) * l)
    for perm in itertools.permutations(range(l)):
        assert np.allclose(np.transpose(tt, perm), tt, atol=1e-13)
    # ... and trace free (trace relation of §3)
    if l >= 2:
        assert np.abs(np.einsum('ii...->...', tt)).max() < 1e-12
    # select o recon = identity
    assert np.allclose(T.select(l, t), v, atol=1e-14)
    # stored components carry at most one z index
    assert all(p[2] <= 1 and sum(p) == l for p in T.comps(l))


def test_component_order_low_ranks():
    assert T.comps(1) == ((1, 0, 0), (0, 1, 0), (0, 0, 1))
    assert T.comps(2) == ((2, 0, 0), (1, 1, 0), (0, 2, 0), (1, 0, 1), (0, 1, 1))


# ----------------------------------------------------------- STF projector --

@pytest.mark.parametrize("l", range(0, 6))
def test_stf_projector_vs_closed_form_detracer(l):
    P = T.stf_projector(l)
    assert np.allclose(P @ P, P, atol=1e-12) and np.allclose(P, P.T, atol=1e-13)
    assert round(np.trace(P)) == 2 * l + 1
    s = T.sym_matrix(l) @ RNG.standard_normal(3 ** l)      # random symmetric tensor
    a = T.stf(l, s)
    b = T.detrace_closed_form(l, s[None])[0]
    assert np.allclose(a, b, atol=1e-12)


def test_placement_counts():
    for l in range(7):
        for m in range(l // 2 + 1):
            want = math.factorial(l) // (math.factorial(l - 2 * m) * 2 ** m * math.factorial(m))
            assert len(T.placements(l, m)) == want


# ------------------------------------------------------- direction tensors --

def test_direction_tensor_low_ranks_closed_form():
    n = RNG.standard_normal(3)
    n /= np.linalg.norm(n)
    assert np.allclose(T.direction_tensor_full(0, n), [1.0])
    assert np.allclose(T.direction_tensor_full(1, n), n)
    # T_2 = (3!!/2!) (n n - I/3) = 3/2 (n n - I/3)
    assert np.allclose(T.direction_tensor_full(2, n), 1.5 * (np.outer(n, n) - np.eye(3) / 3).ravel())
    # {r (x) I}_ijk = r_i d_jk + r_j d_ik + r_k d_ij ; T_3 = 5/2 (n n n - {n I}/5)
    I = np.eye(3)
    rI = (np.einsum('i,jk->ijk', n, I) + np.einsum('j,ik->ijk', n, I) + np.einsum('k,ij->ijk', n, I))
    t3 = 2.5 * (np.einsum('i,j,k->ijk', n, n, n) - rI / 5)
    assert np.allclose(T.direction_tensor_full(3, n), t3.ravel())


@pytest.mark.parametrize("l", range(0, 6))
def test_direction_tensor_properties(l):
    n = RNG.standard_normal((7, 3))
    n /= np.linalg.norm(n, axis=1, keepdims=True)
    t = T.direction_tensor_full(l, n)
    nl = np.ones((7, 1))
    for _ in range(l):
        nl = (nl[:, :, None] * n[:, None, :]).reshape(7, -1)
    # full contraction with n^l is one (App. B)
    assert np.allclose(np.sum(t * nl, axis=1), 1.0, atol=1e-13)
    # STF
    assert np.allclose(T.stf(l, t), t, atol=1e-13)
    # equals (2l-1)!!/l! STF(n^l) built with the numerical projector
    assert np.allclose(t, T.dfact(2 * l - 1) / math.factorial(l) * T.stf(l, nl), atol=1e-12)
    # parity (-1)^l
    assert np.allclose(T.direction_tensor_full(l, -n), (-1) ** l * t, atol=1e-13)


@pytest.mark.parametrize("l", range(0, 5))
def test_direction_tensor_jacobian(l):
    r = RNG.standard_normal((5, 3)) * 2.0
    jac = T.direction_tensor_jac(l, r)
    h = 1e-6
    for j in range(3):
        rp, rm = r.copy(), r.copy()
        rp[:, j] += h
        rm[:, j] -= h
        fd = (T.direction_tensor(l, rp / np.linalg.norm(rp, axis=1, keepdims=True))
              - T.direction_tensor(l, rm / np.linalg.norm(rm, axis=1, keepdims=True))) / (2 * h)
        assert np.allclose(jac[:, :, j], fd, atol=1e-8)
        # complex step (exact to rounding)
        rc = r.astype(complex)
        rc[:, j] += 1e-20j
        rn = np.sqrt(np.sum(rc * rc, axis=1))[:, None]
        cs = T.direction_tensor(l, rc / rn).imag / 1e-20
        assert np.allclose(jac[:, :, j], cs, atol=1e-12)


# ---------------------------------------------------------------- couplings --

def test_worked_example_11_2():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_11_2.json")))
    K = T.coupling_tensor(*ex["path"])
    want = np.zeros((3, 3))
    axis = {"x": 0, "y": 1, "z": 2}
    for t in ex["terms"]:
        want[axis[t["x"]], axis[t["y"]]] += t["coef"]
    comp = T.comps(2).index((2, 0, 0))
    assert np.allclose(K[comp], want, atol=1e-14)


def test_rank1_rank1_products():
    x, y = RNG.standard_normal((2, 3))
    # (1,1)->0 is the dot product
    assert np.allclose(T.coupling(1, 1, 0, x, y), [x @ y], atol=1e-14)
    # (1,1)->2 is 3/2 times the symmetric trace-free outer product (§3 example)
    stf_outer = 0.5 * (np.outer(x, y) + np.outer(y, x)) - np.eye(3) * (x @ y) / 3
    assert np.allclose(T.coupling_full(1, 1, 2, x, y), 1.5 * stf_outer.ravel(), atol=1e-14)
    # (1,1)->1 has odd J: not a natural-parity path; the cross product is the
    # Levi-Civita extension
    assert not T.admissible(1, 1, 1)
    assert np.allclose(T.levi_civita_11_1(x, y), np.cross(x, y), atol=1e-14)


@pytest.mark.parametrize("l", range(0, 5))
def test_scalar_paths(l):
    v = RNG.standard_normal(2 * l + 1)
    s = RNG.standard_normal(1)
    assert np.allclose(T.coupling(0, l, l, s, v), s * v, atol=1e-13)
    assert np.allclose(T.coupling(l, 0, l, v, s), s * v, atol=1e-13)


def _a(l):
    return T.dfact(2 * l - 1) / math.factorial(l)


@pytest.mark.parametrize("l1,l2", [(1, 1), (1, 2), (2, 2), (1, 3), (2, 3), (3, 3), (1, 4)])
def test_stretched_path_normalisation(l1, l2):
    # T_l = a_l STF(n^l); Sym(T_a (x) T_b) = a_a a_b n^(a+b) + terms holding a
    # Kronecker delta, which STF removes, so the normalised coupling with
    # (T (x) T) = T requires N = a_{a+b} / (a_a a_b).
    assert T.path_norm(l1, l2, l1 + l2) == pytest.approx(_a(l1 + l2) / (_a(l1) * _a(l2)), rel=1e-12)


@pytest.mark.parametrize("l", range(1, 5))
def test_full_contraction_normalisation(l):
    # T_l : T_l = a_l (T_l : n^l) = a_l, so N_(l,l)->0 = 1 / a_l.
    assert T.path_norm(l, l, 0) == pytest.approx(1.0 / _a(l), rel=1e-12)


def test_hand_derived_contracted_paths():
    # (2,1)->1: T_2 . n = 3/2 (n - n/3) = n  ->  N = 1
    assert T.path_norm(2, 1, 1) == pytest.approx(1.0, rel=1e-12)
    # (1,2)->3: STF(n (x) T_2) = 3/2 STF(n^3) and T_3 = 5/2 STF(n^3)  ->  5/3
    assert T.path_norm(1, 2, 3) == pytest.approx(5.0 / 3.0, rel=1e-12)


ALL_PATHS = [(l1, l2, L) for l1 in range(5) for l2 in range(5) for L in range(5)
             if T.admissible(l1, l2, L)]


@pytest.mark.parametrize("path", ALL_PATHS)
def test_coupling_invariants(path):
    l1, l2, L = path
    rng = np.random.default_rng(hash(path) % 2 ** 32)
    x, y = full_of(l1, rng), full_of(l2, rng)
    f = T.coupling_full(l1, l2, L, x, y)
    # STF output
    assert np.allclose(T.stf(L, f), f, atol=1e-12)
    # O(3) equivariance (rotation and rotation-reflection), natural parity
    for reflect in (False, True):
        R = rand_rotation(rng, reflect)
        lhs = T.coupling_full(l1, l2, L, rotate_full(l1, x, R), rotate_full(l2, y, R))
        assert np.allclose(lhs, rotate_full(L, f, R), atol=1e-10)
    # exchange symmetry (§3)
    assert np.allclose(T.coupling_full(l2, l1, L, y, x), f, atol=1e-12)
    # Rule B at random directions: (T_l1(n) (x) T_l2(n))_L = T_L(n)
    n = rng.standard_normal(3)
    n /= np.linalg.norm(n)
    assert np.allclose(T.coupling_full(l1, l2, L, T.direction_tensor_full(l1, n),
                                       T.direction_tensor_full(l2, n)),
                       T.direction_tensor_full(L, n), atol=1e-11)
    # probed bilinear tensor reproduces the explicit evaluation
    xi, yi = T.select(l1, x), T.select(l2, y)
    K = T.coupling_tensor(l1, l2, L)
    assert np.allclose(np.einsum('abc,b,c->a', K, xi, yi), T.select(L, f), atol=1e-12)


# ------------------------------------------------------------- path counts --

def test_printed_counts():
    c = json.load(open(os.path.join(GOLDEN, "counts.json")))
    for lmax, want in c["distinct_couplings"]["by_max_rank"].items():
        lmax = int(lmax)
        got = {tuple(sorted(p[:2])) + (p[2],) for p in T.conv_paths(lmax, lmax, lmax)}
        assert len(got) == want
    for case in c["conv_paths"]["cases"]:
        assert len(T.conv_paths(case["l_in"], case["l_edge"], case["l_out"])) == case["paths"]
    lp = c["ladder_product_components"]
    paths = T.conv_paths(lp["l_max"], lp["l_max"], lp["l_max"])
    assert sum(2 * L + 1 for (_, _, L) in paths) == lp["B_components_per_channel"]
    assert sum(2 * l + 1 for l in range(lp["l_max"] + 1)) == lp["mixed_components_per_channel"]


# ------------------------------------------------- odd parity (reading) --

ODD_PATHS = [(l1, l2, L) for l1 in range(4) for l2 in range(4) for L in range(4)
             if T.triangle(l1, l2, L) and (l1 + l2 + L) % 2 == 1]


def test_odd_11_1_is_the_cross_product():
    rng = np.random.default_rng(31)
    x, y = rng.standard_normal((5, 3)), rng.standard_normal((5, 3))
    f = T.coupling(1, 1, 1, x, y)
    # stored rank-1 components are (x, y, z)
    assert np.allclose(f, np.cross(x, y), atol=1e-13)


def test_odd_22_1_is_the_axial_vector_of_the_matrix_product():
    """(2,2)->1: one pair contracted and one through eps: the axial vector of
    X Y for symmetric traceless X, Y."""
    rng = np.random.default_rng(32)
    x, y = rng.standard_normal(5), rng.standard_normal(5)
    X, Y = T.recon(2, x).reshape(3, 3), T.recon(2, y).reshape(3, 3)
    M = X @ Y
    want = np.array([M[1, 2] - M[2, 1], M[2, 0] - M[0, 2], M[0, 1] - M[1, 0]])
    assert np.allclose(T.coupling(2, 2, 1, x, y), want, atol=1e-13)


def test_odd_12_2_is_the_symmetric_part_of_columnwise_cross_products():
    """(1,2)->2: E[b, i] = (x cross Y[:, b])_i; the coupling is its symmetric
    part (already traceless for symmetric Y)."""
    rng = np.random.default_rng(33)
    x, y = rng.standard_normal(3), rng.standard_normal(5)
    Y = T.recon(2, y).reshape(3, 3)
    E = np.stack([np.cross(x, Y[:, b]) for b in range(3)])
    want = 0.5 * (E + E.T)
    assert abs(np.trace(want)) < 1e-13
    assert np.allclose(T.coupling(1, 2, 2, x, y), T.select(2, want.reshape(9)), atol=1e-13)


@pytest.mark.parametrize("path", ODD_PATHS)
def test_odd_coupling_invariants(path):
    """Traceless symmetric output; pseudo-tensor equivariance (a reflection
    flips the sign); antisymmetry under exchange of the operands."""
    l1, l2, L = path
    rng = np.random.default_rng(hash(path) % 2 ** 32)
    x, y = full_of(l1, rng), full_of(l2, rng)
    f = T.coupling_full(l1, l2, L, x, y)
    assert np.abs(f).max() > 1e-3
    assert np.allclose(T.stf(L, f), f, atol=1e-12)
    for reflect in (False, True):
        R = rand_rotation(rng, reflect)
        lhs = T.coupling_full(l1, l2, L, rotate_full(l1, x, R), rotate_full(l2, y, R))
        assert np.allclose(lhs, np.linalg.det(R) * rotate_full(L, f, R), atol=1e-10)
    assert np.allclose(T.coupling_full(l2, l1, L, y, x), -f, atol=1e-12)


def test_all_parity_path_counts():
    """With every triangle-allowed path: ranks <= 1 give the dot and cross
    products of two vectors plus the scalar products (five paths); ranks <= 2
    add to the 11 natural paths the odd (1,1)->1, (2,2)->1, (1,2)->2, (2,1)->2."""
    assert T.conv_paths(1, 1, 1, all_parities=True) == [(0, 0, 0), (1, 1, 0), (0, 1, 1), (1, 0, 1), (1, 1, 1)]
    odd = [p for p in T.conv_paths(2, 2, 2, all_parities=True) if not T.admissible(*p)]
    assert odd == [(1, 1, 1), (2, 2, 1), (1, 2, 2), (2, 1, 2)]
    assert len(T.conv_paths(2, 2, 2)) == 11
