"""Equivariant linear layer (oracle side).  Test infrastructure only.

What is computed (cuequivariance-torch skill document, "Linear: layout
conversion and rotations", and e3nn-course Lesson 12a, the closing example
with ``cuet.Linear``): a map from irreps_in to irreps_out that commutes with
rotations.  By Schur's lemma it can only mix blocks of the same irrep type
(l, p), channel by channel with the same matrix for every component m:

    out[n, block o, m, v] = alpha_t * sum over input blocks i of type t of
                            sum_u W_io[u, v] * x[n, block i, m, u]

for every output block o of type t (zero if no input block has type t).

Weights.  One segment W_io of mul_i * mul_o values per (input block i,
output block o) pair of equal type, pairs in the order i ascending, then o
ascending; inside a segment u (input channel) major, v fastest.  The page's
example ``3x0 + 2x1 -> 2x0 + 4x1`` then has 3*2 + 2*4 = 14 weights.  Shared
weights are one row ``[1, weight_numel]``; class-indexed weights (the
species-indexed Linear of "Other operations and layers") are rows
``[num_classes, weight_numel]`` picked per sample by an index.

Normalisation (the pages state only that descriptor coefficients include
normalisation factors): alpha_t = 1 / sqrt(fan_in_t), fan_in_t = the sum of
the multiplicities of the input blocks of type t, so that unit-variance
inputs and weights give unit-variance outputs.  This is a reading.
"""

import numpy as np

from . import irreps as ir
from .layout import split_blocks, join_blocks


class Linear:
    def __init__(self, irreps_in, irreps_out):
        self.inp = ir.parse(irreps_in)
        self.out = ir.parse(irreps_out)
        self.dim_in = ir.dim(self.inp)
        self.dim_out = ir.dim(self.out)
        # (input block, output block, weight offset) per pair of equal type
        self.pairs = []
        off = 0
        for i, (mi, li, pi) in enumerate(self.inp):
            for o, (mo, lo, po) in enumerate(self.out):
                if (li, pi) == (lo, po):
                    self.pairs.append((i, o, off))
                    off += mi * mo
        self.weight_numel = off
        self.fan_in = {}
        for mi, li, pi in self.inp:
            self.fan_in[(li, pi)] = self.fan_in.get((li, pi), 0) + mi

    def alpha(self, o):
        _, l, p = self.out[o]
        return 1.0 / np.sqrt(self.fan_in[(l, p)])

    def fwd(self, x, w, layout="ir_mul", indices=None, absolute=False):
        """x [n, dim_in] in ``layout``; w [1, weight_numel] (shared) or
        [num_classes, weight_numel] with ``indices`` [n] picking a row per
        sample (an index outside [0, num_classes) gives a zero row).
        Returns float64 [n, dim_out].  ``absolute`` takes |x|, |w|."""
        x = np.asarray(x, dtype=np.float64)
        w = np.asarray(w, dtype=np.float64)
        if absolute:
            x, w = np.abs(x), np.abs(w)
        n = x.shape[0]
        wr, valid = self._rows(w, n, indices)
        xb = split_blocks(x, self.inp, layout)                     # [n, 2l+1, mul]
        ob = [np.zeros((n, 2 * l + 1, m)) for m, l, _ in self.out]
        for i, o, off in self.pairs:
            mi, mo = self.inp[i][0], self.out[o][0]
            W = wr[:, off:off + mi * mo].reshape(-1, mi, mo)       # [n or 1, u, v]
            ob[o] += self.alpha(o) * np.einsum("nuv,nku->nkv", np.broadcast_to(W, (n, mi, mo)), xb[i])
        for o in range(len(self.out)):
            ob[o] *= valid[:, None, None]
        return join_blocks(ob, layout)

    def vjp(self, x, w, g, layout="ir_mul", indices=None, absolute=False):
        """Vector-Jacobian product of :meth:`fwd` for g = dL/d(out): returns
        (dx [n, dim_in] in ``layout``, dw shaped like w).  From the
        definition (the output is linear in x and in w):
            dx[n, i, m, u] = sum over pairs (i, o) of alpha_o sum_v W_io[u, v] g[n, o, m, v]
            dW_io[u, v]   = alpha_o sum over the samples n using the row and m of x[n, i, m, u] g[n, o, m, v]."""
        x = np.asarray(x, dtype=np.float64)
        w = np.asarray(w, dtype=np.float64)
        g = np.asarray(g, dtype=np.float64)
        if absolute:
            x, w, g = np.abs(x), np.abs(w), np.abs(g)
        n = x.shape[0]
        wr, valid = self._rows(w, n, indices)
        xb = split_blocks(x, self.inp, layout)
        gb = split_blocks(g, self.out, layout)
        dxb = [np.zeros_like(b) for b in xb]
        dw = np.zeros_like(w)
        rows = np.zeros(n, dtype=np.int64) if indices is None else np.where(valid, np.asarray(indices), 0)
        for i, o, off in self.pairs:
            mi, mo = self.inp[i][0], self.out[o][0]
            W = wr[:, off:off + mi * mo].reshape(-1, mi, mo)
            a = self.alpha(o)
            gv = gb[o] * valid[:, None, None]
            dxb[i] += a * np.einsum("nuv,nkv->nku", np.broadcast_to(W, (n, mi, mo)), gv)
            per = a * np.einsum("nku,nkv->nuv", xb[i], gv).reshape(n, mi * mo)
            np.add.at(dw[:, off:off + mi * mo], rows, per)
        return join_blocks(dxb, layout), dw

    @staticmethod
    def _rows(w, n, indices):
        if indices is None:
            if w.shape[0] != 1:
                raise ValueError("shared weights are one row")
            return w, np.ones(n, dtype=bool)
        idx = np.asarray(indices, dtype=np.int64)
        valid = (idx >= 0) & (idx < w.shape[0])
        return w[np.where(valid, idx, 0)] * valid[:, None], valid
