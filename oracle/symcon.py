"""Symmetric contraction, degrees 1..3 (oracle side).

What is computed (e3nn-course Lesson 12a, section 21.4.1, and the
cuequivariance-torch skill document, "Other operations and layers"): the
descriptor ``symmetric_contraction(irreps_in, irreps_out, [1, 2, 3])`` has one
row per degree nu, ``[]*a[u]*b[u]...*b[u] -> C[u]`` with nu copies of b: every
channel u is contracted with itself only, the weights ``a`` carry the channel
index, and the weights are chosen per atom by an element (species) index.
Multiplicities must be uniform.  The degrees are summed into one output.

For one channel u let v in R^n be the components of all input blocks of that
channel, block after block (n = sum 2l+1; 16 for 0e+1o+2e+3o).  For degree nu
and output irrep L (each output block), a basis {U^{nu,L,k}} of the
symmetric equivariant maps Sym^nu(R^n) -> R^{2L+1} is built by this
procedure (the pages fix no basis; this is the reading used on both sides):

1. candidates, in this order: ordered block tuples (b1..bnu) in
   lexicographic order; for nu = 3 also the intermediate L12 ascending;
   kept when the parities multiply to the parity of L and the triangle
   rules hold.  The candidate tensor is the real coupling embedded at the
   blocks' component offsets: nu=1 the identity on a block of type L,
   nu=2 C(l1,l2,L), nu=3 sum_a C(l1,l2,L12)[i,j,a] C(L12,l3,L)[a,k,M]
   (C from :func:`oracle.cg.real_cg`);
2. symmetrise over all nu! permutations of the nu input slots;
3. accept it when its Gram-Schmidt residual against the tensors accepted so
   far exceeds 1e-8 of its norm; the accepted tensor is the symmetrised
   candidate itself (not the residual);
4. scale it so that its output components are orthonormal:
   sum_{m1..mnu} U[m.., M] U[m.., M'] = delta_MM'.

Then  out[a, L block, M, u] = sum_nu sum_k w[species_a, woff(nu, L, k) + u]
            * sum_{m1..mnu} U^{nu,L,k}[m1..mnu, M] * prod_i v_a,u[m_i],
weight segments ordered by nu ascending, then output block, then k, each
``mul`` channels wide.
"""

import itertools
import math

import numpy as np

from . import irreps as ir
from .cg import real_cg
from .layout import split_blocks, join_blocks

ACCEPT_TOL = 1e-8


def _embed_candidates(blocks, nu, L, pL):
    """Yield candidate tensors of shape (n,)*nu + (2L+1,) in the canonical order."""
    offs = np.cumsum([0] + [2 * l + 1 for _, l, _ in blocks])
    n = offs[-1]
    nb = len(blocks)
    for tup in itertools.product(range(nb), repeat=nu):
        ls = [blocks[b][1] for b in tup]
        par = 1
        for b in tup:
            par *= blocks[b][2]
        if par != pL:
            continue
        if nu == 1:
            if ls[0] != L:
                continue
            t = np.zeros((n, 2 * L + 1))
            t[offs[tup[0]]:offs[tup[0]] + 2 * L + 1, :] = np.eye(2 * L + 1)
            yield t
        elif nu == 2:
            if not abs(ls[0] - ls[1]) <= L <= ls[0] + ls[1]:
                continue
            t = np.zeros((n, n, 2 * L + 1))
            t[offs[tup[0]]:offs[tup[0]] + 2 * ls[0] + 1,
              offs[tup[1]]:offs[tup[1]] + 2 * ls[1] + 1, :] = real_cg(ls[0], ls[1], L)
            yield t
        elif nu == 3:
            for l12 in range(abs(ls[0] - ls[1]), ls[0] + ls[1] + 1):
                if not abs(l12 - ls[2]) <= L <= l12 + ls[2]:
                    continue
                c = np.einsum("ija,akM->ijkM", real_cg(ls[0], ls[1], l12), real_cg(l12, ls[2], L))
                t = np.zeros((n, n, n, 2 * L + 1))
                t[offs[tup[0]]:offs[tup[0]] + 2 * ls[0] + 1,
                  offs[tup[1]]:offs[tup[1]] + 2 * ls[1] + 1,
                  offs[tup[2]]:offs[tup[2]] + 2 * ls[2] + 1, :] = c
                yield t
        else:
            raise ValueError("degrees 1..3 only")


def _symmetrize(t, nu):
    perms = list(itertools.permutations(range(nu)))
    s = np.zeros_like(t)
    for p in perms:
        s += np.transpose(t, p + (nu,))
    return s / len(perms)


def coupling_basis(blocks, nu, L, pL):
    """The accepted, scaled basis tensors for degree nu and output type (L, pL)."""
    accepted = []     # as returned
    ortho = []        # orthonormal (Frobenius) copy of their span, for the test
    for t in _embed_candidates(blocks, nu, L, pL):
        s = _symmetrize(t, nu)
        ns = np.linalg.norm(s)
        if ns < 1e-12:
            continue
        r = s.copy()
        for q in ortho:
            r -= np.vdot(q, r) * q
        nr = np.linalg.norm(r)
        if nr <= ACCEPT_TOL * ns:
            continue
        ortho.append(r / nr)
        accepted.append(s * (math.sqrt(2 * L + 1) / ns))
    return accepted


class SymmetricContraction:
    def __init__(self, irreps_in, irreps_out, degrees=(1, 2, 3)):
        self.inp = ir.parse(irreps_in)
        self.out = ir.parse(irreps_out)
        muls = {m for m, _, _ in self.inp} | {m for m, _, _ in self.out}
        if len(muls) != 1:
            raise ValueError("symmetric contraction needs one multiplicity for all blocks")
        self.mul = muls.pop()
        self.degrees = tuple(degrees)
        self.n = sum(2 * l + 1 for _, l, _ in self.inp)
        # basis[(nu, out block)] = list of U tensors
        self.basis = {}
        self.segments = []    # (nu, out block, k) in weight order
        for nu in self.degrees:
            for ob, (_, L, pL) in enumerate(self.out):
                us = coupling_basis(self.inp, nu, L, pL)
                self.basis[(nu, ob)] = us
                self.segments.extend((nu, ob, k) for k in range(len(us)))
        self.weight_numel = self.mul * len(self.segments)
        self.dim_in = ir.dim(self.inp)
        self.dim_out = ir.dim(self.out)

    def counts(self):
        """{(nu, out block): K} numbers of couplings."""
        return {key: len(v) for key, v in self.basis.items()}

    def num_paths(self, nu):
        """Non-zero entries of the coupling tensors of degree nu, summed over
        output blocks and couplings (each (k, m1..mnu, M) is one path)."""
        return int(sum(np.count_nonzero(np.abs(u) > 1e-12)
                       for (d, _), us in self.basis.items() if d == nu for u in us))

    def weight_fan_in(self):
        """Per weight column: K of its (nu, output block)."""
        k = self.counts()
        return np.concatenate([np.full(self.mul, k[(nu, ob)]) for nu, ob, _ in self.segments]) \
            if self.segments else np.zeros(0)

    def _entries(self, nu, ob, k, absolute):
        """Non-zero entries of a coupling tensor: (slot component indices
        [nu][nnz], output component M [nnz], value c [nnz])."""
        u = self.basis[(nu, ob)][k]
        if absolute:
            u = np.abs(u)
        nz = np.nonzero(u)
        return [nz[i] for i in range(nu)], nz[nu], u[nz]

    def _per_atom(self, x, species, w, layout, absolute, g=None, chunk=128):
        """Forward (g None) or forward plus vector-Jacobian product, as the
        sum over the non-zero entries (m1..mnu, M, c) of every coupling
        tensor.  Every (atom, channel) pair is one row b of a batch (atoms
        in chunks); gathering the entries' components and scattering to
        output (or input) components are products with 0/1 matrices."""
        x = np.asarray(x, dtype=np.float64)
        w = np.asarray(w, dtype=np.float64)
        species = np.asarray(species, dtype=np.int64)
        if absolute:
            x, w = np.abs(x), np.abs(w)
        n_el, mul, A = w.shape[0], self.mul, x.shape[0]
        valid = (species >= 0) & (species < n_el)
        sp = np.where(valid, species, 0)
        # [A, n, mul] -> rows b = (atom, channel): [A * mul, n]
        v_all = np.concatenate(split_blocks(x, self.inp, layout), axis=1).transpose(0, 2, 1).reshape(A * mul, -1)
        out = [np.zeros((A * mul, 2 * L + 1)) for _, L, _ in self.out]
        if g is not None:
            g = np.asarray(g, dtype=np.float64)
            if absolute:
                g = np.abs(g)
            g_all = [b.transpose(0, 2, 1).reshape(A * mul, -1) for b in split_blocks(g, self.out, layout)]
            dv_all = np.zeros_like(v_all)
            dw = np.zeros_like(w)
        n = v_all.shape[1]
        entries = []
        for nu, ob, k in self.segments:
            slots, M, c = self._entries(nu, ob, k, absolute)
            to_M = np.zeros((len(c), out[ob].shape[1]))
            to_M[np.arange(len(c)), M] = 1.0
            to_m = []
            for i in range(nu):
                t = np.zeros((len(c), n))
                t[np.arange(len(c)), slots[i]] = 1.0
                to_m.append(t)
            entries.append((slots, M, c, to_M, to_m))
        for a0 in range(0, A, chunk):
            a1 = min(A, a0 + chunk)
            rows = slice(a0 * mul, a1 * mul)
            v = v_all[rows]
            # per row: the weights of its atom's species and channel
            wa = (w[sp[a0:a1]] * valid[a0:a1, None]).reshape(a1 - a0, -1, mul)   # [a, seg, mul]
            for s_idx, ((nu, ob, _), (slots, M, c, to_M, to_m)) in enumerate(zip(self.segments, entries)):
                ws = wa[:, s_idx, :].reshape(-1)                                  # [b]
                factors = [v[:, m] for m in slots]                               # each [b, nnz]
                prod = c[None, :] * factors[0]
                for f in factors[1:]:
                    prod = prod * f
                p = prod @ to_M                                                  # [b, 2L+1]
                out[ob][rows] += p * ws[:, None]
                if g is None:
                    continue
                gb = g_all[ob][rows]
                contrib = np.sum(gb * p, axis=1).reshape(a1 - a0, mul) * valid[a0:a1, None]
                np.add.at(dw[:, s_idx * mul:(s_idx + 1) * mul], sp[a0:a1], contrib)
                gw = (gb * ws[:, None])[:, M] * c[None, :]                         # [b, nnz]
                for i in range(nu):                                              # product rule, slot i free
                    rest = gw
                    for j in range(nu):
                        if j != i:
                            rest = rest * factors[j]
                    dv_all[rows] += rest @ to_m[i]
        back = lambda t, irreps: join_blocks(
            [b.reshape(A, mul, -1).transpose(0, 2, 1)
             for b in np.split(t, np.cumsum([2 * l + 1 for _, l, _ in irreps])[:-1], axis=1)], layout)
        res = join_blocks([o.reshape(A, mul, -1).transpose(0, 2, 1) for o in out], layout)
        if g is None:
            return res
        return back(dv_all, self.inp), dw

    def eval_plain(self, x, species, w, layout="ir_mul"):
        """The definition written out, for small cases: per atom a and
        channel u, with v the components of x[a, :, u] (all input blocks in
        order), out[a, L:M, u] = sum over the weight segments (nu, L, k) of
        w[species_a, seg, u] * (U^k contracted with v in each of its nu input
        slots)[M], each contraction one dense np.einsum.  Loops over atoms
        and channels; no batching, gathering or scattering.  Same result as
        :meth:`eval` up to rounding."""
        x = np.asarray(x, dtype=np.float64)
        w = np.asarray(w, dtype=np.float64)
        comps = np.concatenate(split_blocks(x, self.inp, layout), axis=1)     # [A, n, mul]
        outs = [np.zeros((x.shape[0], 2 * L + 1, self.mul)) for _, L, _ in self.out]
        for a in range(x.shape[0]):
            s = int(species[a])
            if not 0 <= s < w.shape[0]:
                continue
            for u in range(self.mul):
                v = comps[a, :, u]
                for s_idx, (nu, ob, k) in enumerate(self.segments):
                    U = self.basis[(nu, ob)][k]
                    if nu == 1:
                        t = np.einsum("iM,i->M", U, v)
                    elif nu == 2:
                        t = np.einsum("ijM,i,j->M", U, v, v)
                    else:
                        t = np.einsum("ijkM,i,j,k->M", U, v, v, v)
                    outs[ob][a, :, u] += w[s, s_idx * self.mul + u] * t
        return join_blocks(outs, layout)

    def eval_vjp_plain(self, x, species, w, g, layout="ir_mul"):
        """:meth:`eval_vjp` written out the same way: per atom and channel,
        dw gets g . (U contracted with v) and dv gets, for each input slot,
        w g . (U contracted with v in the other slots), one dense np.einsum
        each (the product rule with no use of U being symmetric)."""
        x = np.asarray(x, dtype=np.float64)
        w = np.asarray(w, dtype=np.float64)
        comps = np.concatenate(split_blocks(x, self.inp, layout), axis=1)
        gs = split_blocks(np.asarray(g, dtype=np.float64), self.out, layout)   # each [A, 2L+1, mul]
        dv = np.zeros_like(comps)
        dw = np.zeros_like(w)
        for a in range(x.shape[0]):
            s = int(species[a])
            if not 0 <= s < w.shape[0]:
                continue
            for u in range(self.mul):
                v = comps[a, :, u]
                for s_idx, (nu, ob, k) in enumerate(self.segments):
                    U = self.basis[(nu, ob)][k]
                    gm = gs[ob][a, :, u]
                    col = s_idx * self.mul + u
                    if nu == 1:
                        dw[s, col] += np.einsum("iM,i,M->", U, v, gm)
                        dv[a, :, u] += w[s, col] * np.einsum("iM,M->i", U, gm)
                    elif nu == 2:
                        dw[s, col] += np.einsum("ijM,i,j,M->", U, v, v, gm)
                        dv[a, :, u] += w[s, col] * (np.einsum("ijM,j,M->i", U, v, gm)
                                                    + np.einsum("ijM,i,M->j", U, v, gm))
                    else:
                        dw[s, col] += np.einsum("ijkM,i,j,k,M->", U, v, v, v, gm)
                        dv[a, :, u] += w[s, col] * (np.einsum("ijkM,j,k,M->i", U, v, v, gm)
                                                    + np.einsum("ijkM,i,k,M->j", U, v, v, gm)
                                                    + np.einsum("ijkM,i,j,M->k", U, v, v, gm))
        blocks = np.split(dv, np.cumsum([2 * l + 1 for _, l, _ in self.inp])[:-1], axis=1)
        return join_blocks(blocks, layout), dw

    def eval(self, x, species, w, layout="ir_mul", absolute=False):
        """x [n_atoms, dim_in] in ``layout``; species [n_atoms] integers;
        w [num_elements, weight_numel].  Returns float64 [n_atoms, dim_out].
        An atom whose species is outside [0, num_elements) gets a zero row.
        ``absolute`` evaluates the same sums over |x|, |w| and |U|."""
        return self._per_atom(x, species, w, layout, absolute)

    def eval_vjp(self, x, species, w, g, layout="ir_mul", absolute=False):
        """Vector-Jacobian product of :meth:`eval`: given g = dL/d(out)
        [n_atoms, dim_out] in ``layout``, return (dL/dx [n_atoms, dim_in] in
        ``layout``, dL/dw [num_elements, weight_numel]), num_elements =
        w.shape[0].

        From the definition, with p_k[a, M, u] = sum U^k[m1..mnu, M] prod_i
        v[a, m_i, u] (U^k the coupling of weight segment k):
            dw[s, k, u]  = sum over atoms a of species s of sum_M g[a, M, u] p_k[a, M, u]
            dv[a, m, u] += w[s_a, k, u] sum_M g[a, M, u] dp_k[a, M, u] / dv[a, m, u],
        the derivative of the degree-nu product by the product rule: one
        term per input slot, that slot left free and the others contracted
        with v (no use is made of the basis being symmetric).  Species
        outside [0, num_elements) select no weights: zero dx, nothing
        added to dw.  ``absolute`` evaluates the same sums over |x|, |w|,
        |g| and |U|."""
        return self._per_atom(x, species, w, layout, absolute, g=g)
