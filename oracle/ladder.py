"""Oracle for the node-local correlation ladder and its VJP.

TEST INFRASTRUCTURE ONLY.  Plain fp64 numpy, chunked over nodes (the ladder
acts on every node independently).  Follows the FlashCart paper:

* full ladder, §5 Eq. 2: phi1[l] = W1[l] A[l] (channel mixing per rank);
  for q = 2..nu, B[eta] = (phi^{q-1}[l1] (x) A[l2])_L channel-diagonal, and
  phi^q[L] = sum_{eta -> L, k'} W^q_L[k, eta*C + k'] B[eta][k'], L <= l_q;
  z = sum_q Pi_{<= l_out} phi^q.  l_q = l_prod for q < nu and l_out for q = nu.
* path-reduced products, App. E "Path-reduced products":
  phi1[l] = a1[l, k] A[l];
  phi^q[L] = P_{q,L}^{-1/2} sum_{eta -> L} a^q[eta, k] (phi^{q-1}[l1] (x) A[l2])_L;
  z[L] = W_L (sum_q phi^q[L]) for L <= l_out.
* VJP: the reverse of both recurrences by hand (transposed matmuls and the
  transposed bilinear forms of Eq. C1), giving dA and every weight gradient.
* VJP-of-VJP: the complex-step derivative of the forward and of the VJP
  along the cotangents (v_A, v_W) of (dA, weight gradients).

Paths of step q: admissible (l1, l2, L) with l1 <= l_{q-1}, l2 <= l_a and
L <= l_q, ordered by L and then (l1, l2) lexicographically; phi^1 keeps ranks
<= l_1 (l_prod, or l_out when nu = 1).

Weight list (the order of the flat weight buffer):
  full:    W1[l] (C x C) for l <= l_1; then for q = 2..nu and L <= l_q,
           W^q_L (C x P_{q,L} C), element [k_out, eta*C + k_in].
  reduced: a1 (l_1+1 x C); a^q (P_q x C) for q = 2..nu; W_L (C x C), L <= l_out.

Parity pins (tests/test_oracle_ladder.py): with nu = 1 the ladder is W1 A;
the recurrence equals the explicit tensor-train contraction of App. E
Eqs. E2-E4 on a tiny width; path-reduced with a = 1, nu = 2 is a sum of
couplings over sqrt(P); O(3) equivariance; finite differences of the VJP;
the product count "99 d components mixed down to 16 d" of App. E; order 3
at ranks <= 2 with path weights a != 1 (and the full variant's W^q column
order) against a hand expansion in explicit 3 x 3 tensor algebra
(tests/test_oracle_hand.py).
"""

from __future__ import annotations

import numpy as np

from . import tensors as T


class LadderSpec:
    def __init__(self, l_a: int, l_prod: int, l_out: int, order: int,
                 variant: str, channels: int):
        assert variant in ("full", "reduced")
        self.l_a, self.l_prod, self.l_out, self.order = l_a, l_prod, l_out, order
        self.variant, self.C = variant, channels
        self.lq = {}
        for q in range(1, order + 1):
            self.lq[q] = l_out if q == order else l_prod
        self.lq[1] = min(self.lq[1], l_a)
        self.paths = {}
        for q in range(2, order + 1):
            ps = []
            for L in range(self.lq[q] + 1):
                for l1 in range(self.lq[q - 1] + 1):
                    for l2 in range(l_a + 1):
                        if T.admissible(l1, l2, L):
                            ps.append((l1, l2, L))
            self.paths[q] = ps
        self.a_off = T.rank_offsets(l_a)
        self.out_off = T.rank_offsets(l_out)

    def P(self, q: int, L: int) -> int:
        return sum(1 for p in self.paths[q] if p[2] == L)

    def weight_shapes(self):
        """[(name, shape, kind, fan_in)] in flat-buffer order."""
        C, out = self.C, []
        if self.variant == "full":
            for l in range(self.lq[1] + 1):
                out.append((f"W1_{l}", (C, C), "normal", C))
            for q in range(2, self.order + 1):
                for L in range(self.lq[q] + 1):
                    P = self.P(q, L)
                    if P:
                        out.append((f"W{q}_{L}", (C, P * C), "normal", P * C))
        else:
            out.append(("a1", (self.lq[1] + 1, C), "one_plus", 1))
            for q in range(2, self.order + 1):
                out.append((f"a{q}", (len(self.paths[q]), C), "one_plus", 1))
            for L in range(self.l_out + 1):
                out.append((f"W_{L}", (C, C), "normal", C))
        return out

    def n_out_rows(self) -> int:
        return self.out_off[-1]


def _f64(a):
    """Promote to float64, keeping complex values (complex-step checks)."""
    return np.asarray(a, dtype=np.result_type(a.dtype, np.float64))


def _blk(arr, off, l):
    return arr[:, off[l]:off[l + 1], :]


def _prod(l1, l2, L, a, b):
    """Channel-diagonal coupling f[u, c, k] of a[u, b1, k] and b[u, b2, k]."""
    K = T.coupling_tensor(l1, l2, L)
    return np.einsum('abc,ubk,uck->uak', K, a, b, optimize=True)


def _weights(spec, ws):
    names = [s[0] for s in spec.weight_shapes()]
    assert len(names) == len(ws)
    return dict(zip(names, ws))


def _forward_chunk(spec, A, w, keep=False):
    """Returns z chunk and (if keep) the per-step states phi^q."""
    C = spec.C
    phis = {}
    phi = {}
    for l in range(spec.lq[1] + 1):
        Al = _blk(A, spec.a_off, l)
        if spec.variant == "full":
            phi[l] = np.einsum('ucj,kj->uck', Al, w[f"W1_{l}"])
        else:
            phi[l] = w["a1"][l][None, None, :] * Al
    phis[1] = phi
    acc = {L: (phi[L].copy() if L in phi else 0.0) for L in range(spec.l_out + 1)}
    for q in range(2, spec.order + 1):
        new = {}
        for L in range(spec.lq[q] + 1):
            plist = [(i, p) for i, p in enumerate(spec.paths[q]) if p[2] == L]
            if not plist:
                continue
            if spec.variant == "full":
                Bs = [_prod(l1, l2, L, phi[l1], _blk(A, spec.a_off, l2))
                      for _, (l1, l2, _L) in plist]
                B = np.stack(Bs, axis=2)                      # (u, c, P, k)
                Wq = w[f"W{q}_{L}"].reshape(C, len(plist), C)
                new[L] = np.einsum('ucpj,kpj->uck', B, Wq)
            else:
                s = 1.0 / np.sqrt(len(plist))
                tot = 0.0
                for i, (l1, l2, _L) in plist:
                    tot = tot + w[f"a{q}"][i][None, None, :] * _prod(
                        l1, l2, L, phi[l1], _blk(A, spec.a_off, l2))
                new[L] = s * tot
        for L in range(spec.l_out + 1):
            if L in new:
                acc[L] = acc[L] + new[L]
        phi = new
        phis[q] = phi
    outs = []
    for L in range(spec.l_out + 1):
        a = acc[L]
        if spec.variant == "reduced":
            a = np.einsum('ucj,kj->uck', a, w[f"W_{L}"])
        outs.append(a)
    z = np.concatenate(outs, axis=1)
    return (z, phis, acc) if keep else z


def ladder_fwd(spec: LadderSpec, A, ws, nodes=None, chunk: int = 256):
    """z [N or len(nodes), sum_{L<=l_out}(2L+1), C]."""
    w = _weights(spec, ws)
    idx = np.arange(A.shape[0]) if nodes is None else np.asarray(nodes)
    out = []
    for i in range(0, len(idx), chunk):
        out.append(_forward_chunk(spec, _f64(A[idx[i:i + chunk]]), w))
    return np.concatenate(out, axis=0)


def ladder_vjp(spec: LadderSpec, A, ws, gz, nodes=None, chunk: int = 256):
    """(A_bar, [weight grads in flat order]) of L = <g_z, z>."""
    w = _weights(spec, ws)
    names = [s[0] for s in spec.weight_shapes()]
    dt = np.result_type(A.dtype, gz.dtype, np.float64, *[np.asarray(v).dtype for v in ws])
    wb = {k: np.zeros(np.shape(v), dtype=dt) for k, v in w.items()}
    idx = np.arange(A.shape[0]) if nodes is None else np.asarray(nodes)
    A_bar = np.zeros((len(idx),) + A.shape[1:], dtype=dt)
    C = spec.C
    for i0 in range(0, len(idx), chunk):
        sel = idx[i0:i0 + chunk]
        Ac = _f64(A[sel])
        gc = _f64(gz[sel])
        z, phis, acc = _forward_chunk(spec, Ac, w, keep=True)
        Ab = np.zeros(Ac.shape, dtype=dt)
        # gradient of the output sum
        S_bar = {}
        for L in range(spec.l_out + 1):
            gL = _blk(gc, spec.out_off, L)
            if spec.variant == "reduced":
                S_bar[L] = np.einsum('uck,kj->ucj', gL, w[f"W_{L}"])
                wb[f"W_{L}"] += np.einsum('uck,ucj->kj', gL, acc[L])
            else:
                S_bar[L] = gL
        phib = {q: {} for q in range(1, spec.order + 1)}
        for q in range(1, spec.order + 1):
            for L in range(spec.lq[q] + 1):
                if L in phis[q] and L <= spec.l_out:
                    phib[q][L] = S_bar[L].copy()
        for q in range(spec.order, 1, -1):
            phi_prev = phis[q - 1]
            for L in range(spec.lq[q] + 1):
                if L not in phib[q]:
                    continue
                plist = [(i, p) for i, p in enumerate(spec.paths[q]) if p[2] == L]
                G = phib[q][L]
                if spec.variant == "full":
                    Wq = w[f"W{q}_{L}"].reshape(C, len(plist), C)
                    Bs = [_prod(l1, l2, L, phi_prev[l1], _blk(Ac, spec.a_off, l2))
                          for _, (l1, l2, _L) in plist]
                    B = np.stack(Bs, axis=2)
                    wb[f"W{q}_{L}"] += np.einsum('uck,ucpj->kpj', G, B).reshape(C, -1)
                    Bbar = np.einsum('uck,kpj->ucpj', G, Wq)
                    cot = [Bbar[:, :, j, :] for j in range(len(plist))]
                else:
                    s = 1.0 / np.sqrt(len(plist))
                    cot = []
                    for i, (l1, l2, _L) in plist:
                        F = _prod(l1, l2, L, phi_prev[l1], _blk(Ac, spec.a_off, l2))
                        wb[f"a{q}"][i] += s * np.einsum('uck,uck->k', G, F)
                        cot.append(s * w[f"a{q}"][i][None, None, :] * G)
                for (i, (l1, l2, _L)), cb in zip(plist, cot):
                    K = T.coupling_tensor(l1, l2, L)
                    A2 = _blk(Ac, spec.a_off, l2)
                    d1 = np.einsum('abc,uak,uck->ubk', K, cb, A2, optimize=True)
                    d2 = np.einsum('abc,uak,ubk->uck', K, cb, phi_prev[l1], optimize=True)
                    phib[q - 1][l1] = phib[q - 1].get(l1, 0.0) + d1
                    Ab[:, spec.a_off[l2]:spec.a_off[l2 + 1], :] += d2
        for l, G in phib[1].items():
            Al = _blk(Ac, spec.a_off, l)
            if spec.variant == "full":
                Ab[:, spec.a_off[l]:spec.a_off[l + 1], :] += np.einsum('uck,kj->ucj', G, w[f"W1_{l}"])
                wb[f"W1_{l}"] += np.einsum('uck,ucj->kj', G, Al)
            else:
                Ab[:, spec.a_off[l]:spec.a_off[l + 1], :] += w["a1"][l][None, None, :] * G
                wb["a1"][l] += np.einsum('uck,uck->k', G, Al)
        A_bar[i0:i0 + len(sel)] = Ab
    return A_bar, [wb[k] for k in names]


CSTEP = 1e-20


def ladder_vjp_vjp(spec: LadderSpec, A, ws, gz, v_A=None, v_ws=None, nodes=None, chunk: int = 256):
    """(g_hat, A_hat, [W_hat in flat order]) for the second-order term of
    App. C Eq. C2 applied to the ladder: s = <v_A, A_bar> + sum <v_W, W_bar>.

    s is the derivative of <g_z, z> along (v_A, v_W), so g_hat = dz/d eps
    and (A_hat, W_hat) = d (A_bar, W_bar) / d eps at (A + eps v_A,
    W + eps v_W), by complex step (exact to rounding for h = 1e-20).  A
    missing cotangent is zero.
    """
    h = CSTEP
    Ac = A.astype(np.complex128) + (0 if v_A is None else 1j * h * v_A)
    wc = [np.asarray(w, dtype=np.complex128) + (0 if v_ws is None else 1j * h * v)
          for w, v in zip(ws, v_ws if v_ws is not None else [None] * len(ws))]
    g_hat = ladder_fwd(spec, Ac, wc, nodes=nodes, chunk=chunk).imag / h
    Ab, Wb = ladder_vjp(spec, Ac, wc, gz, nodes=nodes, chunk=chunk)
    return g_hat, Ab.imag / h, [b.imag / h for b in Wb]
