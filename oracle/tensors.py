"""Symmetric trace-free (STF) Cartesian tensors, direction tensors and couplings.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Plain fp64 numpy on
full 3^l tensors; every function follows a passage of the FlashCart paper
("FlashCart: Fast Cartesian Tensor Products for Equivariant Interatomic
Potentials"):

* ``comps``/``recon_matrix``/``select_matrix``: independent components with at
  most one z index and the trace relation that rebuilds the other entries
  (§3 "Symbolic construction"; Fig. C1(a) for the picture of the stored entries).
* ``sym_matrix``/``stf_projector``: symmetrisation by averaging over all index
  permutations and trace removal as the orthogonal projection onto
  symmetric trace-free tensors (§2 "Irreducible Cartesian tensors", App. C).
* ``detrace_closed_form``: the classical closed-form detracer with the
  (-1)^m (2l-2m-1)!!/(2l-1)!! coefficients (the same coefficients as the
  direction-tensor formula of App. B); used only to cross-check the projector.
* ``direction_tensor_full``: T_l(n) exactly as the App. B formula, with the
  braces evaluated as an explicit sum over distinct index placements.
* ``coupling_full``: (x (x) y)_L = N_path * STF_L(Sym_L(x .n. y)),
  n = (l1+l2-L)/2 contracted pairs (§2, App. B Eq. B1, App. C).
* ``coupling_odd_full``: odd J = l1+l2+L, the Levi-Civita extension the pages
  name without defining it (§7 "Limitations"): reading below.

Reading of the pages (path normalisation).  The constant C_{l1 l2 l3} of
Eq. B1 is defined only by reference to other work and is not printed.  The
oracle fixes the normalisation N_path of every admissible path by the rule
    (T_l1(n) (x) T_l2(n))_L = T_L(n)   for every unit vector n,
which uses only objects defined on the pages (the T_l normalisation of App. B)
and reproduces the one printed worked example, the (1,1)->2 xx component of
§3.  Pins: the §3 worked example; dot product for (1,1)->0; scalar product for
(0,l)->l; closed forms for stretched paths (L = l1+l2) and for (l,l)->0;
equivariance, symmetry, tracelessness and exchange symmetry; path counts
printed in App. C Table C1 and App. E.  Beyond the worked example the
normalisation is a reading of the pages, not a value they print.

Reading of the pages (odd parity).  The pages restrict the method to natural
parity and only name Levi-Civita contractions as the way to odd J.  The
oracle's odd-J coupling takes the plainest construction: contract
n = (l1+l2-L-1)/2 index pairs between x and y, one more index of each through
the Levi-Civita symbol (its third index free), symmetrise and remove traces;
constant 1, so that (1,1)->1 is the cross product x × y.  Pins: the cross
product; pseudo-tensor equivariance (a reflection flips the sign);
antisymmetry under exchange of equal-rank operands; tracelessness; and the
generator's exact-rational construction.  Beyond the cross product the
normalisation is parity unpinned against the pages.
"""

from __future__ import annotations

import functools
import itertools
import math

import numpy as np


# ----------------------------------------------------------------------------
# small combinatorics
# ----------------------------------------------------------------------------

def dfact(n: int) -> int:
    """Double factorial with (-1)!! = 1 (App. B, direction-tensor formula)."""
    if n <= 0:
        return 1
    out = 1
    while n > 1:
        out *= n
        n -= 2
    return out


def n_comp(l: int) -> int:
    """dim V_l = (l+1)(l+2)/2 - l(l-1)/2 = 2l+1 (§2)."""
    return (l + 1) * (l + 2) // 2 - l * (l - 1) // 2


# ----------------------------------------------------------------------------
# independent components (§3 "Symbolic construction")
# ----------------------------------------------------------------------------

@functools.lru_cache(maxsize=None)
def comps(l: int) -> tuple:
    """The 2l+1 stored components (p_x, p_y, p_z) with p_z <= 1.

    Order: p_z = 0 block with p_x descending, then the p_z = 1 block with p_x
    descending.  l=1: x, y, z.  l=2: xx, xy, yy, xz, yz.
    """
    a = [(px, l - px, 0) for px in range(l, -1, -1)]
    b = [(px, l - 1 - px, 1) for px in range(l - 1, -1, -1)]
    return tuple(a + b)


def counts(idx) -> tuple:
    return (sum(1 for i in idx if i == 0), sum(1 for i in idx if i == 1),
            sum(1 for i in idx if i == 2))


def representative(p) -> tuple:
    return (0,) * p[0] + (1,) * p[1] + (2,) * p[2]


@functools.lru_cache(maxsize=None)
def recon_matrix(l: int) -> np.ndarray:
    """R_l of shape (3^l, 2l+1): full tensor (flattened) from stored components.

    Entries with p_z >= 2 follow the trace relation
    (x)_{px,py,pz} = -(x)_{px+2,py,pz-2} - (x)_{px,py+2,pz-2}.
    """
    cl = comps(l)
    pos = {p: i for i, p in enumerate(cl)}

    @functools.lru_cache(maxsize=None)
    def row(p):
        v = np.zeros(len(cl))
        if p[2] <= 1:
            v[pos[p]] = 1.0
            return v
        return -row((p[0] + 2, p[1], p[2] - 2)) - row((p[0], p[1] + 2, p[2] - 2))

    out = np.zeros((3 ** l, len(cl)))
    for flat, idx in enumerate(itertools.product(range(3), repeat=l)):
        out[flat] = row(counts(idx))
    return out


@functools.lru_cache(maxsize=None)
def select_matrix(l: int) -> np.ndarray:
    """S_l of shape (2l+1, 3^l): reads the stored components of a full tensor."""
    out = np.zeros((n_comp(l), 3 ** l))
    for i, p in enumerate(comps(l)):
        flat = int(np.ravel_multi_index(representative(p), (3,) * l)) if l else 0
        out[i, flat] = 1.0
    return out


def recon(l: int, v):
    """Full tensor(s) (..., 3^l) from stored components (..., 2l+1)."""
    return np.einsum('fi,...i->...f', recon_matrix(l), v)


def select(l: int, t):
    """Stored components (..., 2l+1) of full tensor(s) (..., 3^l)."""
    return np.einsum('if,...f->...i', select_matrix(l), t)


# ----------------------------------------------------------------------------
# symmetrisation and trace removal
# ----------------------------------------------------------------------------

@functools.lru_cache(maxsize=None)
def sym_matrix(l: int) -> np.ndarray:
    """Average over all l! permutations of the indices (App. C)."""
    d = 3 ** l
    out = np.zeros((d, d))
    perms = list(itertools.permutations(range(l)))
    for flat, idx in enumerate(itertools.product(range(3), repeat=l)):
        for p in perms:
            pidx = tuple(idx[k] for k in p)
            j = int(np.ravel_multi_index(pidx, (3,) * l)) if l else 0
            out[flat, j] += 1.0 / len(perms)
    return out


@functools.lru_cache(maxsize=None)
def trace_matrix(l: int) -> np.ndarray:
    """Map full rank-l tensor -> its trace over the first two indices (rank l-2)."""
    if l < 2:
        return np.zeros((0, 3 ** l))
    out = np.zeros((3 ** (l - 2), 3 ** l))
    for flat, idx in enumerate(itertools.product(range(3), repeat=l)):
        if idx[0] == idx[1]:
            j = int(np.ravel_multi_index(idx[2:], (3,) * (l - 2))) if l > 2 else 0
            out[j, flat] += 1.0
    return out


@functools.lru_cache(maxsize=None)
def stf_projector(l: int) -> np.ndarray:
    """Orthogonal projector onto symmetric trace-free rank-l tensors.

    Built numerically: an orthonormal basis of range(Sym) is restricted to the
    null space of the trace map.  Its rank must be 2l+1 (§2).
    """
    d = 3 ** l
    if l == 0:
        return np.ones((1, 1))
    u, s, _ = np.linalg.svd(sym_matrix(l))
    qs = u[:, s > 1e-10]                       # basis of symmetric tensors
    tr = trace_matrix(l) @ qs if l >= 2 else np.zeros((0, qs.shape[1]))
    if tr.shape[0]:
        _, s2, vt = np.linalg.svd(tr)
        rank = int(np.sum(s2 > 1e-10))
        ns = vt[rank:].T
    else:
        ns = np.eye(qs.shape[1])
    q = qs @ ns
    assert q.shape == (d, n_comp(l)), (l, q.shape)
    return q @ q.T


def stf(l: int, t):
    """STF projection of full tensor(s) (..., 3^l)."""
    return np.einsum('fg,...g->...f', stf_projector(l), t)


@functools.lru_cache(maxsize=None)
def placements(l: int, m: int) -> tuple:
    """All ways to put m identity factors on l index slots.

    Returns tuples (pairs, rest): ``pairs`` are m disjoint slot pairs, ``rest``
    the remaining slots in increasing order.  Choosing the 2m paired slots and
    then a perfect matching of them gives l!/((l-2m)! 2^m m!) placements
    (App. B).
    """
    def matchings(slots):
        if not slots:
            yield ()
            return
        first, others = slots[0], slots[1:]
        for i, partner in enumerate(others):
            remaining = others[:i] + others[i + 1:]
            for rest in matchings(remaining):
                yield ((first, partner),) + rest

    out = []
    for chosen in itertools.combinations(range(l), 2 * m):
        rest = tuple(s for s in range(l) if s not in chosen)
        for pairs in matchings(chosen):
            out.append((pairs, rest))
    return tuple(out)


def _placement_sum(l: int, m: int, core, batch_shape):
    """{core (x) I^m}: sum over distinct placements of m identity factors.

    ``core(rest_slots)`` returns the full tensor of rank l-2m that sits on
    the unpaired slots, shape batch + (3,)*(l-2m).  Result: batch + (3,)*l.
    """
    eye = np.eye(3)
    out = None
    letters = 'abcdefghijklmnop'
    for pairs, rest in placements(l, m):
        ops, subs = [], []
        for (i, j) in pairs:
            ops.append(eye)
            subs.append(letters[i] + letters[j])
        c = core(rest)
        ops.append(c)
        subs.append('Z' + ''.join(letters[k] for k in rest))
        expr = ','.join(subs) + '->Z' + letters[:l]
        term = np.einsum(expr, *ops)
        out = term if out is None else out + term
    return out.reshape(batch_shape + (3,) * l)


def detrace_closed_form(l: int, s):
    """Closed-form detracer of symmetric tensor(s) s (..., 3^l).

    STF(S) = sum_m (-1)^m (2l-2m-1)!!/(2l-1)!! {I^m (x) Tr^m S}.
    """
    batch = s.shape[:-1]
    sf = s.reshape((-1,) + (3,) * l)
    out = np.zeros_like(sf)
    for m in range(l // 2 + 1):
        tr = sf
        for _ in range(m):
            tr = np.einsum('zii...->z...', tr)
        coef = (-1) ** m * dfact(2 * l - 2 * m - 1) / dfact(2 * l - 1)
        out = out + coef * _placement_sum(l, m, lambda rest, tr=tr: tr, (sf.shape[0],))
    return out.reshape(batch + (3 ** l,))


# ----------------------------------------------------------------------------
# direction tensors (App. B)
# ----------------------------------------------------------------------------

def direction_tensor_full(l: int, n):
    """T_l(n) of App. B as full tensors, n of shape (..., 3) -> (..., 3^l).

    T_l = (2l-1)!!/l! sum_m (-1)^m (2l-2m-1)!!/(2l-1)!! {n^(l-2m) (x) I^m},
    the braces summing over distinct placements.  Works for complex n.
    """
    n = np.asarray(n)
    batch = n.shape[:-1]
    nf = n.reshape(-1, 3)
    if l == 0:
        return np.ones(batch + (1,), dtype=nf.dtype)
    pref = dfact(2 * l - 1) / math.factorial(l)
    out = 0
    for m in range(l // 2 + 1):
        k = l - 2 * m

        def core(rest, k=k):
            t = np.ones((nf.shape[0],), dtype=nf.dtype)
            for _ in range(k):
                t = t[..., None] * nf.reshape((nf.shape[0],) + (1,) * (t.ndim - 1) + (3,))
            return t

        coef = (-1) ** m * dfact(2 * l - 2 * m - 1) / dfact(2 * l - 1)
        out = out + coef * _placement_sum(l, m, core, (nf.shape[0],))
    return (pref * out).reshape(batch + (3 ** l,))


def direction_tensor(l: int, n):
    """Stored components of T_l(n): (..., 3) -> (..., 2l+1)."""
    return select(l, direction_tensor_full(l, n))


def direction_tensor_jac(l: int, r):
    """d T_l(r/|r|) / d r in stored components: (..., 3) -> (..., 2l+1, 3).

    For unit n = r/|r|, T_l = a_l STF(n^(x)l) with a_l = (2l-1)!!/l!, and
    d n / d r_j = (e_j - n_j n)/|r|, so
    d T_l / d r_j = a_l l / |r| [STF(n^(x)(l-1) (x) e_j) - n_j STF(n^(x)l)].
    Complex-safe (no conjugation), so it can be complex-stepped.
    """
    r = np.asarray(r)
    batch = r.shape[:-1]
    rf = r.reshape(-1, 3)
    E = rf.shape[0]
    rn = np.sqrt(np.sum(rf * rf, axis=-1))
    nf = rf / rn[:, None]
    if l == 0:
        return np.zeros(batch + (1, 3), dtype=rf.dtype)
    a = dfact(2 * l - 1) / math.factorial(l)
    # n^(l-1) as flattened full tensor
    t = np.ones((E, 1), dtype=rf.dtype)
    for _ in range(l - 1):
        t = (t[:, :, None] * nf[:, None, :]).reshape(E, -1)
    nl = (t[:, :, None] * nf[:, None, :]).reshape(E, -1)
    stf_nl = stf(l, nl)
    jac = np.zeros((E, n_comp(l), 3), dtype=np.result_type(rf.dtype, float))
    for j in range(3):
        ej = np.zeros(3)
        ej[j] = 1.0
        te = (t[:, :, None] * ej[None, None, :]).reshape(E, -1)
        d = stf(l, te) - nf[:, j:j + 1] * stf_nl
        jac[:, :, j] = (a * l / rn)[:, None] * select(l, d)
    return jac.reshape(batch + (n_comp(l), 3))


# ----------------------------------------------------------------------------
# couplings (§2, App. B Eq. B1, App. C)
# ----------------------------------------------------------------------------

def admissible(l1: int, l2: int, L: int) -> bool:
    """Triangle condition and even J = l1+l2+L (natural parity, §2)."""
    return abs(l1 - l2) <= L <= l1 + l2 and (l1 + l2 + L) % 2 == 0


def triangle(l1: int, l2: int, L: int) -> bool:
    """Triangle condition only: every path of either parity (the odd-J ones
    are the Levi-Civita extension the pages name in §7)."""
    return abs(l1 - l2) <= L <= l1 + l2


def levi_civita() -> np.ndarray:
    eps = np.zeros((3, 3, 3))
    eps[0, 1, 2] = eps[1, 2, 0] = eps[2, 0, 1] = 1.0
    eps[0, 2, 1] = eps[2, 1, 0] = eps[1, 0, 2] = -1.0
    return eps


def coupling_odd_full(l1: int, l2: int, L: int, xf, yf):
    """Odd-J coupling of full tensors (reading, see the module notes):
    STF_L(Sym_L(E)), E_{a.., b.., i} = eps_{i k j} x_{a.. c.. k} y_{c.. j b..}
    with n = (l1+l2-L-1)/2 pairs c contracted between x and y and one more
    index of each operand contracted through the Levi-Civita symbol, whose
    third index stays free.  Constant 1: (1,1)->1 is the cross product."""
    assert triangle(l1, l2, L) and (l1 + l2 + L) % 2 == 1
    n = (l1 + l2 - L - 1) // 2
    batch = np.broadcast_shapes(xf.shape[:-1], yf.shape[:-1])
    xb = np.broadcast_to(xf, batch + (3 ** l1,)).reshape((-1,) + (3,) * l1)
    yb = np.broadcast_to(yf, batch + (3 ** l2,)).reshape((-1,) + (3,) * l2)
    letters = 'abcdefghijklmnopqrs'
    fa = letters[:l1 - n - 1]                   # free indices of x
    cc = letters[l1 - n - 1:l1 - 1]             # contracted pairs
    k, j, i = 'x', 'y', 'w'
    fb = letters[l1 - 1:l1 - 1 + l2 - n - 1]    # free indices of y
    q = np.einsum(f'Z{fa}{cc}{k},Z{cc}{j}{fb},{i}{k}{j}->Z{fa}{fb}{i}', xb, yb, levi_civita())
    q = q.reshape(q.shape[0], 3 ** L)
    q = np.einsum('fg,zg->zf', sym_matrix(L), q)
    q = stf(L, q)
    return q.reshape(batch + (3 ** L,))


def coupling_unnormalised(l1: int, l2: int, L: int, xf, yf):
    """STF_L(Sym_L(x .n. y)) for full tensors xf (..., 3^l1), yf (..., 3^l2)."""
    assert admissible(l1, l2, L)
    n = (l1 + l2 - L) // 2
    batch = np.broadcast_shapes(xf.shape[:-1], yf.shape[:-1])
    xb = np.broadcast_to(xf, batch + (3 ** l1,)).reshape((-1,) + (3,) * l1)
    yb = np.broadcast_to(yf, batch + (3 ** l2,)).reshape((-1,) + (3,) * l2)
    letters = 'abcdefghijklmnop'
    xs = letters[:l1]
    # contract the last n slots of x with the first n slots of y
    ys = xs[l1 - n:] + letters[l1:l1 + l2 - n]
    out = xs[:l1 - n] + letters[l1:l1 + l2 - n]
    q = np.einsum('Z' + xs + ',Z' + ys + '->Z' + out, xb, yb)
    q = q.reshape(q.shape[0], 3 ** L)
    q = np.einsum('fg,zg->zf', sym_matrix(L), q)
    q = stf(L, q)
    return q.reshape(batch + (3 ** L,))


_N0 = np.array([1.0, 2.0, 2.0]) / 3.0   # a fixed unit vector


@functools.lru_cache(maxsize=None)
def path_norm(l1: int, l2: int, L: int) -> float:
    """N_path with (T_l1(n) (x) T_l2(n))_L = T_L(n)  (reading of Eq. B1's C)."""
    u = coupling_unnormalised(l1, l2, L, direction_tensor_full(l1, _N0),
                              direction_tensor_full(l2, _N0))
    t = direction_tensor_full(L, _N0)
    lam = float(np.dot(u, t) / np.dot(t, t))
    resid = np.linalg.norm(u - lam * t)
    assert resid < 1e-12 * max(1.0, np.linalg.norm(u)), (l1, l2, L, resid)
    return 1.0 / lam


def coupling_full(l1: int, l2: int, L: int, xf, yf):
    """Normalised Cartesian coupling of full tensors (odd J: the Levi-Civita
    reading of ``coupling_odd_full``)."""
    if (l1 + l2 + L) % 2 == 1:
        return coupling_odd_full(l1, l2, L, xf, yf)
    return path_norm(l1, l2, L) * coupling_unnormalised(l1, l2, L, xf, yf)


def coupling(l1: int, l2: int, L: int, x, y):
    """Explicit mode on stored components: select(coupling(recon x, recon y))."""
    return select(L, coupling_full(l1, l2, L, recon(l1, x), recon(l2, y)))


@functools.lru_cache(maxsize=None)
def coupling_tensor(l1: int, l2: int, L: int) -> np.ndarray:
    """Probed bilinear form K[a, b1, b2] with f_a(x, y) = sum K x_b1 y_b2.

    Obtained by evaluating ``coupling`` on basis vectors (it is bilinear).
    """
    n1, n2 = n_comp(l1), n_comp(l2)
    e1, e2 = np.eye(n1), np.eye(n2)
    xs = np.repeat(e1, n2, axis=0)          # (n1*n2, n1)
    ys = np.tile(e2, (n1, 1))               # (n1*n2, n2)
    f = coupling(l1, l2, L, xs, ys)         # (n1*n2, nL)
    return np.ascontiguousarray(f.reshape(n1, n2, -1).transpose(2, 0, 1))


# ----------------------------------------------------------------------------
# path lists and layouts
# ----------------------------------------------------------------------------

def conv_paths(l_in: int, l_edge: int, l_out: int, all_parities: bool = False) -> list:
    """Admissible (l1, l2, L), l1 <= l_in, l2 <= l_edge, L <= l_out (with
    ``all_parities``: every triangle-allowed path, odd J included).

    Ordered by L, then (l1, l2) lexicographically (the pages leave the order
    within an output rank open).
    """
    ok = triangle if all_parities else admissible
    out = []
    for L in range(l_out + 1):
        for l1 in range(l_in + 1):
            for l2 in range(l_edge + 1):
                if ok(l1, l2, L):
                    out.append((l1, l2, L))
    return out


def rank_offsets(lmax: int) -> list:
    """Row offsets of the rank blocks of a node-feature array (P_l = 1)."""
    off, acc = [], 0
    for l in range(lmax + 1):
        off.append(acc)
        acc += n_comp(l)
    off.append(acc)
    return off


def out_layout(paths: list, l_out: int):
    """Rows of the path-separated output for every (path index, component).

    Row of (path p = (l1, l2, L), component c) = off(L) + c * P_L + eta_L,
    where eta_L is p's position among the paths with output rank L (App. D
    "Data layout", Fig. D1).  Returns (rows, n_rows) with rows[p] an int array
    of length 2L+1.
    """
    per_L = {L: [p for p in paths if p[2] == L] for L in range(l_out + 1)}
    off, acc = {}, 0
    for L in range(l_out + 1):
        off[L] = acc
        acc += n_comp(L) * len(per_L[L])
    rows = []
    for p in paths:
        L = p[2]
        eta = per_L[L].index(p)
        P_L = len(per_L[L])
        rows.append(np.array([off[L] + c * P_L + eta for c in range(n_comp(L))]))
    return rows, acc


def summed_out_layout(paths: list, l_out: int):
    """Rows of the path-summed output (the pages' kernel option of summing
    the outputs of the coupling paths instead of keeping them separate, App.
    D "Executing Cartesian tensor products"): every path with output rank L adds into the
    single (2L+1)-row block of L; ranks without a path take no rows.
    Returns (rows, n_rows) like out_layout.
    """
    off, acc = {}, 0
    for L in range(l_out + 1):
        if any(p[2] == L for p in paths):
            off[L] = acc
            acc += n_comp(L)
    rows = [np.array([off[p[2]] + c for c in range(n_comp(p[2]))]) for p in paths]
    return rows, acc


def levi_civita_11_1(x, y):  # noqa: D401
    """eps_ijk x_j y_k: the odd-J (1,1)->1 coupling (cross product).

    The pages restrict the method to natural-parity (even J) paths and name
    Levi-Civita contractions as the extension for odd J (§7 "Limitations",
    App. B).  This standalone helper is not used by any path of the hot path;
    it exists so that the rank-1 x rank-1 products (dot, cross, symmetric
    trace-free outer product) can all be checked.
    """
    eps = np.zeros((3, 3, 3))
    eps[0, 1, 2] = eps[1, 2, 0] = eps[2, 0, 1] = 1.0
    eps[0, 2, 1] = eps[2, 1, 0] = eps[1, 0, 2] = -1.0
    return np.einsum('ijk,...j,...k->...i', eps, x, y)
