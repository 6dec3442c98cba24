"""Coupling-table generator for the HIP kernels.

Expands every natural-parity Cartesian coupling path (l1, l2) -> L with
l1, l2, L <= MAX_RANK (and every odd-J path up to ODD_MAX_RANK, through the
Levi-Civita reading below) into an exact bilinear polynomial over the 2l+1 stored
components of each operand, and every direction tensor T_l(n) into a
polynomial in (n_x, n_y, n_z), using exact rational arithmetic (stdlib
``fractions``).  The result is emitted as constexpr C++ tables in
``csrc/generated/fc_tables.h``, which the hand-written kernels iterate over
with fully unrolled loops.

Mathematics (FlashCart paper, arXiv 2610.06409):

* stored components: the 2l+1 entries with at most one z index, labelled by
  their index counts (p_x, p_y, p_z); every other entry follows from the
  trace relation (x)_{px,py,pz} = -(x)_{px+2,py,pz-2} - (x)_{px,py+2,pz-2}
  (§3 "Symbolic construction").
* coupling: App. B Eq. B1 evaluated literally, i.e.
      sum_{m=0}^{min(l1,l2)-n} (-2)^m (2L-2m-1)!!/(2L-1)!!
          {(x .(n+m). y) (x) I^m},
  the braces summing over distinct placements of the free indices (those
  left from x, those left from y, and the m identity factors), times a path
  constant.
* path constant: the pages leave C_{l1 l2 L} to another reference.  It is
  fixed here by requiring (T_l1(n) (x) T_l2(n))_L = T_L(n); at n = e_x the
  x...x entry of T_L(e_x) is T_L : e_x^L = 1, which fixes the constant exactly.
* direction tensors: App. B, T_l = (2l-1)!!/l! sum_m (-1)^m
  (2l-2m-1)!!/(2l-1)!! {n^(l-2m) (x) I^m}.
* odd J (the Levi-Civita extension the pages name in §7, a reading): contract
  (l1+l2-L-1)/2 index pairs and one more index of each operand through the
  Levi-Civita symbol, symmetrise over the L free slots and remove traces with
  the closed-form detracer; constant 1, so that (1,1)->1 is x × y.

Run as a script to (re)write the header; ``build()`` in the package does so.
"""

from __future__ import annotations

import itertools
import math
import os
import sys
from fractions import Fraction

MAX_RANK = 5
ODD_MAX_RANK = 4     # odd-J (Levi-Civita) paths are tabulated up to this rank


# ----------------------------------------------------------------------------
# index bookkeeping
# ----------------------------------------------------------------------------

def dfact(n: int) -> int:
    out = 1
    while n > 1:
        out *= n
        n -= 2
    return out


def stored(l: int):
    """(p_x, p_y, p_z) of the stored components, in storage order."""
    return ([(px, l - px, 0) for px in range(l, -1, -1)]
            + [(px, l - 1 - px, 1) for px in range(l - 1, -1, -1)])


def rep_index(p):
    return (0,) * p[0] + (1,) * p[1] + (2,) * p[2]


def index_counts(idx):
    c = [0, 0, 0]
    for i in idx:
        c[i] += 1
    return tuple(c)


def entry_in_stored(l: int):
    """Map counts (p_x,p_y,p_z) -> {stored comp: Fraction} via the trace relation."""
    pos = {p: i for i, p in enumerate(stored(l))}
    memo = {}

    def rec(p):
        if p in memo:
            return memo[p]
        if p[2] <= 1:
            out = {pos[p]: Fraction(1)}
        else:
            out = {}
            for q in ((p[0] + 2, p[1], p[2] - 2), (p[0], p[1] + 2, p[2] - 2)):
                for k, v in rec(q).items():
                    out[k] = out.get(k, Fraction(0)) - v
            out = {k: v for k, v in out.items() if v != 0}
        memo[p] = out
        return out

    return rec


def full_tensor(l: int, vec):
    """Dict index tuple -> Fraction of the STF tensor with stored comps ``vec``."""
    rec = entry_in_stored(l)
    out = {}
    for idx in itertools.product(range(3), repeat=l):
        val = Fraction(0)
        for k, c in rec(index_counts(idx)).items():
            val += c * vec[k]
        out[idx] = val
    return out


def matchings(slots):
    if not slots:
        yield ()
        return
    first, others = slots[0], slots[1:]
    for i, partner in enumerate(others):
        for rest in matchings(others[:i] + others[i + 1:]):
            yield ((first, partner),) + rest


# ----------------------------------------------------------------------------
# Eq. B1
# ----------------------------------------------------------------------------

def admissible(l1, l2, L):
    return abs(l1 - l2) <= L <= l1 + l2 and (l1 + l2 + L) % 2 == 0


def odd_path(l1, l2, L):
    return abs(l1 - l2) <= L <= l1 + l2 and (l1 + l2 + L) % 2 == 1


# ----------------------------------------------------------------------------
# odd J: the Levi-Civita extension named in the pages' §7 (reading)
# ----------------------------------------------------------------------------

def levi(i, k, j):
    return {(0, 1, 2): 1, (1, 2, 0): 1, (2, 0, 1): 1, (0, 2, 1): -1, (2, 1, 0): -1, (1, 0, 2): -1}.get((i, k, j), 0)


def stf_entry(L, S, out_idx):
    """Entry of the trace-free part of the symmetric rank-L tensor S (dict),
    by the closed-form detracer: sum_m (-1)^m (2L-2m-1)!!/(2L-1)!! over the
    placements of m Kronecker deltas among the L slots, times the m-fold
    trace of S on the remaining slots."""
    total = Fraction(0)
    for m in range(L // 2 + 1):
        coef = Fraction((-1) ** m * dfact(2 * L - 2 * m - 1), dfact(2 * L - 1))
        for chosen in itertools.combinations(range(L), 2 * m):
            rest = tuple(out_idx[s] for s in range(L) if s not in chosen)
            for pairs in matchings(chosen):
                if any(out_idx[a] != out_idx[b] for a, b in pairs):
                    continue
                tr = Fraction(0)
                for c in itertools.product(range(3), repeat=m):
                    tr += S[rest + tuple(v for cc in c for v in (cc, cc))]
                total += coef * tr
    return total


def odd_entry(l1, l2, L, X, Y, out_idx):
    """Entry ``out_idx`` of STF_L(Sym_L(E)) with
    E_{a.., b.., i} = sum eps_{i k j} X_{a.. c.. k} Y_{c.. j b..},
    n = (l1+l2-L-1)/2 contracted pairs c (constant 1)."""
    n = (l1 + l2 - L - 1) // 2
    fa, fb = l1 - n - 1, l2 - n - 1
    E = {}
    for idx in itertools.product(range(3), repeat=L):
        a, b, i = idx[:fa], idx[fa:fa + fb], idx[L - 1]
        v = Fraction(0)
        for c in itertools.product(range(3), repeat=n):
            for k in range(3):
                for j in range(3):
                    e = levi(i, k, j)
                    if e:
                        v += e * X[a + c + (k,)] * Y[c + (j,) + b]
        E[idx] = v
    perms = list(itertools.permutations(range(L)))
    S = {}
    for idx in itertools.product(range(3), repeat=L):
        S[idx] = sum((E[tuple(idx[p] for p in perm)] for perm in perms), Fraction(0)) / len(perms)
    return stf_entry(L, S, out_idx)


def odd_coupling_terms(l1, l2, L):
    """[(a, b1, b2, Fraction)] of the odd-J coupling (reading: constant 1)."""
    n1, n2 = 2 * l1 + 1, 2 * l2 + 1
    basis = lambda n, i: [Fraction(int(j == i)) for j in range(n)]
    fullx = [full_tensor(l1, basis(n1, i)) for i in range(n1)]
    fully = [full_tensor(l2, basis(n2, i)) for i in range(n2)]
    terms = []
    for a, p in enumerate(stored(L)):
        oi = rep_index(p)
        for b1 in range(n1):
            for b2 in range(n2):
                v = odd_entry(l1, l2, L, fullx[b1], fully[b2], oi)
                if v != 0:
                    terms.append((a, b1, b2, v))
    return terms


def b1_entry(l1, l2, L, X, Y, out_idx):
    """Entry ``out_idx`` of Eq. B1 without its path constant."""
    n = (l1 + l2 - L) // 2
    total = Fraction(0)
    for m in range(0, min(l1, l2) - n + 1):
        k = n + m
        fx, fy = l1 - k, l2 - k                # free indices left on x and y
        coef = Fraction((-2) ** m * dfact(2 * L - 2 * m - 1), dfact(2 * L - 1))
        acc = Fraction(0)
        slots = tuple(range(L))
        for sx in itertools.combinations(slots, fx):
            rest = tuple(s for s in slots if s not in sx)
            for sy in itertools.combinations(rest, fy):
                pair_slots = tuple(s for s in rest if s not in sy)
                for pairs in matchings(pair_slots):
                    if any(out_idx[a] != out_idx[b] for a, b in pairs):
                        continue
                    xi = tuple(out_idx[s] for s in sx)
                    yi = tuple(out_idx[s] for s in sy)
                    q = Fraction(0)
                    for c in itertools.product(range(3), repeat=k):
                        q += X[xi + c] * Y[c + yi]
                    acc += q
        total += coef * acc
    return total


# ----------------------------------------------------------------------------
# direction tensors as polynomials in n
# ----------------------------------------------------------------------------

def direction_poly(l: int, p):
    """T_l(n) stored comp with counts p as {(ex,ey,ez): Fraction}."""
    idx = rep_index(p)
    out = {}
    pref = Fraction(dfact(2 * l - 1), math.factorial(l))
    for m in range(l // 2 + 1):
        coef = pref * Fraction((-1) ** m * dfact(2 * l - 2 * m - 1), dfact(2 * l - 1))
        for chosen in itertools.combinations(range(l), 2 * m):
            rest = [s for s in range(l) if s not in chosen]
            for pairs in matchings(chosen):
                if any(idx[a] != idx[b] for a, b in pairs):
                    continue
                e = [0, 0, 0]
                for s in rest:
                    e[idx[s]] += 1
                key = tuple(e)
                out[key] = out.get(key, Fraction(0)) + coef
    return {k: v for k, v in out.items() if v != 0}


def direction_full_at_ex(l: int):
    """T_l(e_x) as a full tensor of Fractions (n = (1, 0, 0))."""
    out = {}
    for idx in itertools.product(range(3), repeat=l):
        poly = direction_poly_idx(l, idx)
        out[idx] = sum((c for (ex, ey, ez), c in poly.items() if ey == 0 and ez == 0),
                       Fraction(0))
    return out


def direction_poly_idx(l, idx):
    out = {}
    pref = Fraction(dfact(2 * l - 1), math.factorial(l))
    for m in range(l // 2 + 1):
        coef = pref * Fraction((-1) ** m * dfact(2 * l - 2 * m - 1), dfact(2 * l - 1))
        for chosen in itertools.combinations(range(l), 2 * m):
            rest = [s for s in range(l) if s not in chosen]
            for pairs in matchings(chosen):
                if any(idx[a] != idx[b] for a, b in pairs):
                    continue
                e = [0, 0, 0]
                for s in rest:
                    e[idx[s]] += 1
                out[tuple(e)] = out.get(tuple(e), Fraction(0)) + coef
    return out


# ----------------------------------------------------------------------------
# tables
# ----------------------------------------------------------------------------

def path_constant(l1, l2, L):
    X, Y = direction_full_at_ex(l1), direction_full_at_ex(l2)
    v = b1_entry(l1, l2, L, X, Y, (0,) * L)
    assert v != 0
    return 1 / v


def coupling_terms(l1, l2, L):
    """[(a, b1, b2, Fraction)] with f_a(x, y) = sum c x_b1 y_b2."""
    c = path_constant(l1, l2, L)
    n1, n2 = 2 * l1 + 1, 2 * l2 + 1
    basis = lambda n, i: [Fraction(int(j == i)) for j in range(n)]
    fullx = [full_tensor(l1, basis(n1, i)) for i in range(n1)]
    fully = [full_tensor(l2, basis(n2, i)) for i in range(n2)]
    terms = []
    for a, p in enumerate(stored(L)):
        oi = rep_index(p)
        for b1 in range(n1):
            for b2 in range(n2):
                v = c * b1_entry(l1, l2, L, fullx[b1], fully[b2], oi)
                if v != 0:
                    terms.append((a, b1, b2, v))
    return terms


def all_paths(max_rank=MAX_RANK, odd_max_rank=ODD_MAX_RANK):
    """Natural-parity path types (lexicographic), then the odd-J ones."""
    nat = [(l1, l2, L) for l1 in range(max_rank + 1) for l2 in range(max_rank + 1)
           for L in range(max_rank + 1) if admissible(l1, l2, L)]
    odd = [(l1, l2, L) for l1 in range(odd_max_rank + 1) for l2 in range(odd_max_rank + 1)
           for L in range(odd_max_rank + 1) if odd_path(l1, l2, L)]
    return nat + odd


def build_tables(max_rank=MAX_RANK, odd_max_rank=ODD_MAX_RANK):
    paths = all_paths(max_rank, odd_max_rank)
    cache = {}
    tables = {}
    for (l1, l2, L) in paths:
        if odd_path(l1, l2, L):
            tables[(l1, l2, L)] = odd_coupling_terms(l1, l2, L)
        elif (l2, l1, L) in cache:         # exchange symmetry: swap operands
            tables[(l1, l2, L)] = [(a, b2, b1, c) for (a, b1, b2, c) in cache[(l2, l1, L)]]
        else:
            cache[(l1, l2, L)] = coupling_terms(l1, l2, L)
            tables[(l1, l2, L)] = cache[(l1, l2, L)]
    tpoly = {l: [direction_poly(l, p) for p in stored(l)] for l in range(max_rank + 1)}
    return paths, tables, tpoly


# ----------------------------------------------------------------------------
# emission
# ----------------------------------------------------------------------------

def cfloat(fr: Fraction) -> str:
    if fr.denominator == 1:
        return f"{fr.numerator}.0f"
    return f"float({fr.numerator}.0 / {fr.denominator}.0)"


def first_flags(terms):
    """Per term: is it the first term of its path writing output a, VJP-1 slot
    b1, VJP-2 slot b2?  Lets the kernels start each sum with a product."""
    seen_a, seen_1, seen_2, out = set(), set(), set(), []
    for (a, b1, b2, c) in terms:
        out.append((a not in seen_a, b1 not in seen_1, b2 not in seen_2))
        seen_a.add(a)
        seen_1.add(b1)
        seen_2.add(b2)
    return out


def product_table(paths, tables, cfg, operand):
    """Distinct products |c| * v[g] used by the paths of one configuration.

    ``operand`` 2: v = edge tensor y, g = l2^2 + b2; the list starts with
    (g, 1) for every edge-tensor row, so y itself is its first entries.
    ``operand`` 1: v = node features x, g = l1^2 + b1; only |c| != 1 entries.
    Returns the list of (g, |c|) and, for every term of every path type, its
    index in the list (-1 when the path type is not part of the
    configuration, or for operand 1 when |c| = 1).
    """
    l_in, l_edge, l_out, allp = cfg_ranks(cfg)
    used = {p for p in paths if p[0] <= l_in and p[1] <= l_edge and p[2] <= l_out
            and (allp or admissible(*p))}
    keys, index = [], {}
    if operand == 2:
        for g in range((l_edge + 1) ** 2):
            index[(g, Fraction(1))] = len(keys)
            keys.append((g, Fraction(1)))
    term_idx = []
    for p in paths:
        for (a, b1, b2, c) in tables[p]:
            if p not in used or (operand == 1 and abs(c) == 1):
                term_idx.append(-1)
                continue
            key = (p[1] * p[1] + b2, abs(c)) if operand == 2 else (p[0] * p[0] + b1, abs(c))
            if key not in index:
                index[key] = len(keys)
                keys.append(key)
            term_idx.append(index[key])
    return keys, term_idx


def emit(path: str, max_rank=MAX_RANK) -> None:
    paths, tables, tpoly = build_tables(max_rank)
    lines = []
    w = lines.append
    w("// Generated by cartesian_tensor_product_amd/gen/generate.py -- do not edit.")
    w("// Exact rational coupling and direction-tensor tables (FlashCart paper,")
    w("// §3 'Symbolic construction', App. B Eq. B1 and the direction-tensor formula).")
    w("#pragma once")
    w("")
    w("namespace fc {")
    w("namespace tab {")
    w("")
    w(f"inline constexpr int kMaxRank = {max_rank};")
    w("")
    w("// f_a(x, y) = sum over terms c * x[b1] * y[b2]; fa/f1/f2 mark the first term of")
    w("// the path that writes output a / VJP-1 slot b1 / VJP-2 slot b2")
    w("struct Term { int a, b1, b2; float c; bool fa, f1, f2; };")
    w("struct Mono { int ex, ey, ez; float c; };")
    w("")
    w("// coupling path types (l1, l2 -> L): natural parity, lexicographic, then odd J")
    w(f"inline constexpr int kNumPathTypes = {len(paths)};")
    w("inline constexpr int kPathL1[] = {" + ", ".join(str(p[0]) for p in paths) + "};")
    w("inline constexpr int kPathL2[] = {" + ", ".join(str(p[1]) for p in paths) + "};")
    w("inline constexpr int kPathL[] = {" + ", ".join(str(p[2]) for p in paths) + "};")
    begins, allterms = [], []
    for p in paths:
        begins.append(len(allterms))
        for t, f in zip(tables[p], first_flags(tables[p])):
            allterms.append(t + f)
    begins.append(len(allterms))
    w("inline constexpr int kTermBegin[] = {" + ", ".join(map(str, begins)) + "};")
    w(f"inline constexpr int kNumTerms = {len(allterms)};")
    w("inline constexpr Term kTerms[] = {")
    k = 0
    for p in paths:
        w(f"  // ({p[0]},{p[1]})->{p[2]}: {len(tables[p])} terms")
        for _ in tables[p]:
            (a, b1, b2, c, fa, f1, f2) = allterms[k]
            k += 1
            bl = lambda v: "true" if v else "false"
            w(f"  {{{a}, {b1}, {b2}, {cfloat(c)}, {bl(fa)}, {bl(f1)}, {bl(f2)}}},")
    w("};")
    w("")
    w("// direction tensors T_l(n): stored component c of rank l is")
    w("// sum over monomials c * n_x^ex n_y^ey n_z^ez")
    mb, allmono = [], []
    for l in range(max_rank + 1):
        for poly in tpoly[l]:
            mb.append(len(allmono))
            for (ex, ey, ez), c in sorted(poly.items(), reverse=True):
                allmono.append((ex, ey, ez, c))
    mb.append(len(allmono))
    w("inline constexpr int kMonoBegin[] = {" + ", ".join(map(str, mb)) + "};")
    w("inline constexpr Mono kMono[] = {")
    for (ex, ey, ez, c) in allmono:
        w(f"  {{{ex}, {ey}, {ez}, {cfloat(c)}}},")
    w("};")
    w("")
    w("// per configuration (l_in, l_edge, l_out): the distinct products |c| * y[g]")
    w("// (CY, g = l2^2 + b2; y itself first) and |c| * x[g] with |c| != 1")
    w("// (CX, g = l1^2 + b1) its paths use, and for every term the product's index")
    w("// (a configuration with summed outputs uses the tables of its paths)")
    w("template <int LIN, int LEDGE, int LOUT> struct CY;")
    w("template <int LIN, int LEDGE, int LOUT> struct CX;")
    for cfg in conv_configs():
        if cfg_summed(cfg):
            continue
        for name, op in (("CY", 2), ("CX", 1)):
            keys, tidx = product_table(paths, tables, cfg, op)
            w(f"template <> struct {name}<{cfg[0]}, {cfg[1]}, {cfg[2]}> {{")
            w(f"  static constexpr int n = {len(keys)};")
            w("  static constexpr int g[] = {" + ", ".join(str(g) for g, _ in keys or [(0, 0)]) + "};")
            w("  static constexpr float c[] = {" + ", ".join(cfloat(c) for _, c in keys or [(0, Fraction(0))]) + "};")
            w("  static constexpr int term[] = {" + ", ".join(map(str, tidx)) + "};")
            w("};")
    w("")
    w("}  // namespace tab")
    w("}  // namespace fc")
    _write(path, "\n".join(lines) + "\n")


# (l_in, l_edge, l_out key) instantiated in the library: equal ranks 0..5
# (the microbenchmark grid of the pages), (l_prop, l_e, l_e) with
# l_prop <= min(l_e, 3), l_e <= 4 (model blocks; the first convolution has
# scalar senders, later ones propagate rank l_prop), and equal ranks 1..4 with
# every triangle-allowed path (odd J included), keyed by l_out + ALL_PARITIES,
# and equal ranks 1..4 with path-summed outputs, keyed by l_out + SUM_PATHS.
# The VJP-of-VJP is instantiated up to rank 4 (natural parity) and 3 (every
# path, or summed outputs); beyond, its path groups would need about 20
# sweeps per sender.
ALL_PARITIES = 8
SUM_PATHS = 16
VV_MAX_RANK = 5
VV_MAX_RANK_ALL = 4
VV_MAX_RANK_SUM = 4
VV_W_MAX_RANK = 4        # explicit-weight VJP-of-VJP, natural parity and paths separate
VV_W_MAX_RANK_OTHER = 3  # ... with every parity or summed paths
# from these ranks each VJP-of-VJP pass is compiled in a unit of its own
VV_SPLIT_RANK = 5
VV_SPLIT_RANK_OTHER = 4
SUM_MAX_RANK = 4
MLP_MAX_RANK = 3         # convolution with the radial network fused into its lanes


def cfg_ranks(cfg):
    """(l_in, l_edge, l_out, all parities) of a configuration key."""
    return cfg[0], cfg[1], cfg[2] % ALL_PARITIES, (cfg[2] // ALL_PARITIES) % 2 == 1


def cfg_summed(cfg) -> bool:
    return cfg[2] >= SUM_PATHS


def conv_configs():
    out = [(L, L, L) for L in range(MAX_RANK + 1)]
    for le in range(1, 5):
        for lp in range(0, 4):
            if lp <= le and (lp, le, le) not in out:
                out.append((lp, le, le))
    out += [(L, L, L + ALL_PARITIES) for L in range(1, ODD_MAX_RANK + 1)]
    out += [(L, L, L + SUM_PATHS) for L in range(1, SUM_MAX_RANK + 1)]
    return out


def has_vv(cfg) -> bool:
    li, le, lo, allp = cfg_ranks(cfg)
    if cfg_summed(cfg):
        return max(li, le, lo) <= VV_MAX_RANK_SUM
    return max(li, le, lo) <= (VV_MAX_RANK_ALL if allp else VV_MAX_RANK)


def has_vv_w(cfg) -> bool:
    li, le, lo, allp = cfg_ranks(cfg)
    other = allp or cfg_summed(cfg)
    return has_vv(cfg) and max(li, le, lo) <= (VV_W_MAX_RANK_OTHER if other else VV_W_MAX_RANK)


def vv_split(cfg) -> bool:
    li, le, lo, allp = cfg_ranks(cfg)
    other = allp or cfg_summed(cfg)
    return has_vv(cfg) and max(li, le, lo) >= (VV_SPLIT_RANK_OTHER if other else VV_SPLIT_RANK)


def has_mlp(cfg) -> bool:
    """Whether the convolution with the radial network's output layer fused
    into its lanes is instantiated (natural parity, paths kept apart)."""
    li, le, lo, allp = cfg_ranks(cfg)
    return not allp and not cfg_summed(cfg) and max(li, le, lo) <= MLP_MAX_RANK


def mlp_fwd_fused(cfg) -> bool:
    """Whether the forward weighted by the radial network runs fused by
    default: measured faster than the materialised forward (an MFMA GEMM
    writing w, then the explicit-weight kernel) for l_in <= 1 or ranks <= 2
    at 1024 nodes x 128 neighbours x 128 channels (e.g. 0.54 vs 0.56 ms at
    rank 2, 0.24 vs 0.28 ms at (0, 3, 3)), slower at (2, 3, 3) and (3, 3, 3)
    (1.04 vs 0.89, 1.35 vs 1.17 ms).  The VJP is materialised by default:
    with the output-layer GEMMs in their narrow and N-loop layouts it was as
    fast or faster at every rank set measured except (1, 1, 1) and (1, 2, 2)
    (within 4 %)."""
    li, le, lo, _ = cfg_ranks(cfg)
    return li <= 1 or max(li, le, lo) <= 2


# the passes of a split VJP-of-VJP: unit suffix, function, body
VV_PARTS = [("vr", "recv", "vv_part_recv<{r}>(a, st);"),
            ("vg", "wgrad", "vv_part_wgrad<{r}>(a, st);"),
            ("vs", "send", "vv_part_sender<{r}, false>(a, st);"),
            ("vx", "sendvx", "vv_part_sender<{r}, true>(a, st);")]


def emit_instances(gen_dir: str) -> list:
    """One translation unit per convolution configuration, plus the list."""
    cfgs = conv_configs()
    lines = ["// Generated by cartesian_tensor_product_amd/gen/generate.py -- do not edit.",
             "// (l_in, l_edge, l_out) instantiated in the library.", "#pragma once", "",
             "#define FC_CONV_CONFIGS(X) \\"]
    lines += [f"  X({a}, {b}, {c}) \\" for a, b, c in cfgs]
    lines += ["", "", "// ... of which the VJP-of-VJP is instantiated for", "#define FC_CONV_VV_CONFIGS(X) \\"]
    lines += [f"  X({a}, {b}, {c}) \\" for a, b, c in cfgs if has_vv((a, b, c))]
    lines += ["", "", "// ... and the VJP-of-VJP with explicit per-edge weights for", "#define FC_CONV_VV_W_CONFIGS(X) \\"]
    lines += [f"  X({a}, {b}, {c}) \\" for a, b, c in cfgs if has_vv_w((a, b, c))]
    lines += ["", "", "// ... and the convolution with the radial network's output layer fused for",
              "#define FC_CONV_MLP_CONFIGS(X) \\"]
    lines += [f"  X({a}, {b}, {c}) \\" for a, b, c in cfgs if has_mlp((a, b, c))]
    lines += ["", "", "// ... of which the forward runs fused by default for", "#define FC_CONV_MLP_FWD_FUSED_CONFIGS(X) \\"]
    lines += [f"  X({a}, {b}, {c}) \\" for a, b, c in cfgs if has_mlp((a, b, c)) and mlp_fwd_fused((a, b, c))]
    lines += ["", ""]
    _write(os.path.join(gen_dir, "fc_conv_configs.h"), "\n".join(lines))
    files = []
    head = "// Generated by cartesian_tensor_product_amd/gen/generate.py -- do not edit.\n"
    for a, b, c in cfgs:
        vv, split = has_vv((a, b, c)), vv_split((a, b, c))
        key, r = f"{a}{b}{c}", f"{a}, {b}, {c}"
        if split:
            # the VJP-of-VJP passes are compiled in units of their own (in
            # parallel) and composed here
            decl = "".join(f"void conv_vv{key}_{fn}(const ConvArgs& a, hipStream_t st);\n" for _, fn, _ in VV_PARTS)
            vv_line = (f"  else run_vjp_vjp(VVParts{{{', '.join(f'conv_vv{key}_{fn}' for _, fn, _ in VV_PARTS)}}},"
                       f" nrank({a}), ConvCfg<{r}>::P, args, stream);\n")
            for suf, fn, body in VV_PARTS:
                f = os.path.join(gen_dir, f"conv_inst_{key}{suf}.hip")
                _write(f, head + "#include \"../fc_conv_vv.h\"\n\nnamespace fc {\n\n"
                       f"void conv_vv{key}_{fn}(const ConvArgs& a, hipStream_t st) {{ {body.format(r=r)} }}\n\n"
                       "}  // namespace fc\n")
                files.append(f)
        else:
            decl = ""
            vv_line = f"  else launch_vjp_vjp<{r}>(args, stream);\n" if vv else "  else return false;\n"
        src = (head + f"#include \"../{'fc_conv_vv.h' if vv and not split else 'fc_conv_kernels.h'}\"\n\n"
               f"namespace fc {{\n\n" + decl + ("\n" if decl else "") +
               f"bool conv_run_{key}(int op, const ConvArgs& args, hipStream_t stream) {{\n"
               f"  if (op == 0) launch_fwd<{r}>(args, stream);\n"
               f"  else if (op == 1) launch_vjp<{r}>(args, stream);\n"
               + vv_line
               + f"  return true;\n}}\n\n}}  // namespace fc\n")
        f = os.path.join(gen_dir, f"conv_inst_{a}{b}{c}.hip")
        _write(f, src)
        files.append(f)
        if has_vv_w((a, b, c)):
            # the explicit-weight VJP-of-VJP in a unit of its own (compiles in parallel)
            src = (f"// Generated by cartesian_tensor_product_amd/gen/generate.py -- do not edit.\n"
                   f"#include \"../fc_conv_vv.h\"\n\n"
                   f"namespace fc {{\n\n"
                   f"void conv_run_w_{a}{b}{c}(const ConvArgs& args, hipStream_t stream) {{\n"
                   f"  launch_vjp_vjp_w<{a}, {b}, {c}>(args, stream);\n"
                   f"}}\n\n}}  // namespace fc\n")
            f = os.path.join(gen_dir, f"conv_inst_{a}{b}{c}w.hip")
            _write(f, src)
            files.append(f)
        if has_mlp((a, b, c)):
            src = (f"// Generated by cartesian_tensor_product_amd/gen/generate.py -- do not edit.\n"
                   f"#include \"../fc_conv_kernels.h\"\n\n"
                   f"namespace fc {{\n\n"
                   f"void conv_run_mlp_{a}{b}{c}(int op, const ConvArgs& args, hipStream_t stream) {{\n"
                   f"  if (op == 0) launch_fwd_mlp<{a}, {b}, {c}>(args, stream);\n"
                   f"  else launch_vjp_mlp<{a}, {b}, {c}>(args, stream);\n"
                   f"}}\n\n}}  // namespace fc\n")
            f = os.path.join(gen_dir, f"conv_inst_{a}{b}{c}m.hip")
            _write(f, src)
            files.append(f)
    return files


def _write(path: str, text: str) -> None:
    os.makedirs(os.path.dirname(path), exist_ok=True)
    if os.path.exists(path) and open(path).read() == text:
        return
    tmp = path + ".tmp"
    with open(tmp, "w") as f:
        f.write(text)
    os.replace(tmp, path)


HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "csrc", "generated", "fc_tables.h")


def emit_all() -> None:
    emit(HEADER)
    emit_instances(os.path.dirname(HEADER))


if __name__ == "__main__":
    emit_all()
