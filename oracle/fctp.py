"""Fully connected ("uvw") tensor product (oracle side).  Test infrastructure
only.

What is computed (cuequivariance-torch skill document, "CPU tensor product
and backward": ``FullyConnectedTensorProduct(irreps, irreps, irreps)`` with
trainable weights, gradients of both inputs and of the weights; "Channelwise
product with external per-example weights": it "accepts desired output
irreps"): every channel of input 1 couples with every channel of input 2
into every channel of each output block.

Paths.  For every input-1 block i (mul1 x l1 p1), input-2 block j
(mul2 x l2 p2) and output block o (mul3 x l3 p3) with
|l1 - l2| <= l3 <= l1 + l2 and p3 = p1 p2, in the order i, then j, then o.
The output irreps are taken as given, multiplicities included.  SO(3)
irreps strings (terms without a parity letter, as in the pages' "0 + 1"
example) drop the parity condition.

Weights.  One segment per path of mul1 * mul2 * mul3 values, u (input 1)
slowest, then v (input 2), w (output) fastest; shared by all samples
([1, weight_numel]).

    out[n, o, k, w] = alpha_o sum over paths (i, j, o) of
                      sum_uv W_p[u, v, w] sum_ab C[a, b, k] x1[n, i, a, u] x2[n, j, b, v]

with C = :func:`oracle.cg.real_cg` (the coupling of the channelwise product)
and alpha_o = 1 / sqrt(sum over the paths into o of mul1 * mul2), so that
unit-variance inputs and weights give unit-variance outputs (the pages only
say that normalisation factors are included: a reading).
"""

import re

import numpy as np

from . import irreps as ir
from .cg import real_cg
from .layout import split_blocks, join_blocks


_SO3_TERM = re.compile(r"^(?:(\d+)\s*x\s*)?(\d+)$")


def parse_any(s):
    """O(3) irreps via :func:`oracle.irreps.parse`; an SO(3) string (no
    parity letters) gives blocks with parity 0, which satisfies p3 = p1 p2
    for every triple."""
    terms = [t.strip() for t in s.split("+") if t.strip()]
    if terms and all(_SO3_TERM.match(t) for t in terms):
        out = []
        for t in terms:
            m = _SO3_TERM.match(t)
            out.append((int(m.group(1)) if m.group(1) else 1, int(m.group(2)), 0))
        return out
    return ir.parse(s)


class FullyConnectedTP:
    def __init__(self, irreps_in1, irreps_in2, irreps_out):
        self.in1 = parse_any(irreps_in1)
        self.in2 = parse_any(irreps_in2)
        self.out = parse_any(irreps_out)
        if len({p == 0 for _, _, p in self.in1 + self.in2 + self.out}) > 1:
            raise ValueError("mixing SO(3) and O(3) irreps")
        self.dim_in1, self.dim_in2, self.dim_out = ir.dim(self.in1), ir.dim(self.in2), ir.dim(self.out)
        self.paths = []   # (i, j, o, weight offset)
        off = 0
        for i, (m1, l1, p1) in enumerate(self.in1):
            for j, (m2, l2, p2) in enumerate(self.in2):
                for o, (m3, l3, p3) in enumerate(self.out):
                    if abs(l1 - l2) <= l3 <= l1 + l2 and p3 == p1 * p2:
                        self.paths.append((i, j, o, off))
                        off += m1 * m2 * m3
        self.weight_numel = off
        fan = [0] * len(self.out)
        for i, j, o, _ in self.paths:
            fan[o] += self.in1[i][0] * self.in2[j][0]
        self.alpha = [1.0 / np.sqrt(f) if f else 0.0 for f in fan]

    def _segment(self, w, p):
        i, j, o, off = self.paths[p]
        m1, m2, m3 = self.in1[i][0], self.in2[j][0], self.out[o][0]
        return w[0, off:off + m1 * m2 * m3].reshape(m1, m2, m3)

    def fwd(self, x1, x2, w, layout="mul_ir", absolute=False):
        """x1 [n, dim_in1], x2 [n, dim_in2] in ``layout``; w [1, weight_numel]
        (shared), or [n, weight_numel] with n > 1: one row per sample (the
        skill document's external weights with shared_weights=False,
        "distinct weights per item", "Layouts and weights").  Returns float64
        [n, dim_out].  ``absolute`` takes |x1|, |x2|, |w|, |C|."""
        x1, x2, w = (np.asarray(a, dtype=np.float64) for a in (x1, x2, w))
        if absolute:
            x1, x2, w = np.abs(x1), np.abs(x2), np.abs(w)
        a = split_blocks(x1, self.in1, layout)
        b = split_blocks(x2, self.in2, layout)
        n = x1.shape[0]
        per = n > 1 and w.shape[0] == n
        ob = [np.zeros((n, 2 * l + 1, m)) for m, l, _ in self.out]
        for p, (i, j, o, off) in enumerate(self.paths):
            c = real_cg(self.in1[i][1], self.in2[j][1], self.out[o][1])
            if absolute:
                c = np.abs(c)
            if per:
                m1, m2, m3 = self.in1[i][0], self.in2[j][0], self.out[o][0]
                W = w[:, off:off + m1 * m2 * m3].reshape(n, m1, m2, m3)
                ob[o] += self.alpha[o] * np.einsum("abk,nau,nbv,nuvw->nkw", c, a[i], b[j], W, optimize=True)
                continue
            W = self._segment(w, p)
            ob[o] += self.alpha[o] * np.einsum("abk,nau,nbv,uvw->nkw", c, a[i], b[j], W, optimize=True)
        return join_blocks(ob, layout)

    def vjp(self, x1, x2, w, g, layout="mul_ir", absolute=False, edge_weights=None):
        """Vector-Jacobian product of :meth:`fwd` for g = dL/d(out): returns
        (dx1, dx2, dw); the output is linear in each of x1, x2 and w.  With
        ``edge_weights`` [n, weight_numel] (one row per sample, w unused) dw
        is per sample, [n, weight_numel]."""
        per = edge_weights is not None
        if per:
            w = edge_weights
        x1, x2, w, g = (np.asarray(a, dtype=np.float64) for a in (x1, x2, w, g))
        if absolute:
            x1, x2, w, g = np.abs(x1), np.abs(x2), np.abs(w), np.abs(g)
        a = split_blocks(x1, self.in1, layout)
        b = split_blocks(x2, self.in2, layout)
        gb = split_blocks(g, self.out, layout)
        da = [np.zeros_like(t) for t in a]
        db = [np.zeros_like(t) for t in b]
        dw = np.zeros_like(w)
        for p, (i, j, o, off) in enumerate(self.paths):
            c = real_cg(self.in1[i][1], self.in2[j][1], self.out[o][1])
            if absolute:
                c = np.abs(c)
            al = self.alpha[o]
            m1, m2, m3 = self.in1[i][0], self.in2[j][0], self.out[o][0]
            if per:
                W = w[:, off:off + m1 * m2 * m3].reshape(-1, m1, m2, m3)
                da[i] += al * np.einsum("abk,nbv,nuvw,nkw->nau", c, b[j], W, gb[o], optimize=True)
                db[j] += al * np.einsum("abk,nau,nuvw,nkw->nbv", c, a[i], W, gb[o], optimize=True)
                dW = al * np.einsum("abk,nau,nbv,nkw->nuvw", c, a[i], b[j], gb[o], optimize=True)
                dw[:, off:off + m1 * m2 * m3] = dW.reshape(dW.shape[0], -1)
                continue
            W = self._segment(w, p)
            da[i] += al * np.einsum("abk,nbv,uvw,nkw->nau", c, b[j], W, gb[o], optimize=True)
            db[j] += al * np.einsum("abk,nau,uvw,nkw->nbv", c, a[i], W, gb[o], optimize=True)
            dW = al * np.einsum("abk,nau,nbv,nkw->uvw", c, a[i], b[j], gb[o], optimize=True)
            dw[0, off:off + dW.size] = dW.reshape(-1)
        return join_blocks(da, layout), join_blocks(db, layout), dw

    def dw_entries(self, x1, x2, g, flat, layout="mul_ir", absolute=False):
        """Selected entries of the weight gradient (the ``dw`` of
        :meth:`vjp`) at flat weight indices ``flat``, each from its
        definition alpha_o sum_n sum_(a, b, k) C[a, b, k] x1[n, i, a, u]
        x2[n, j, b, v] g[n, o, k, w]: the whole batch, one entry at a time."""
        x1, x2, g = (np.asarray(a, dtype=np.float64) for a in (x1, x2, g))
        if absolute:
            x1, x2, g = np.abs(x1), np.abs(x2), np.abs(g)
        a = split_blocks(x1, self.in1, layout)
        b = split_blocks(x2, self.in2, layout)
        gb = split_blocks(g, self.out, layout)
        out = np.zeros(len(flat))
        for r, e in enumerate(flat):
            p = max(q for q in range(len(self.paths)) if self.paths[q][3] <= e)
            i, j, o, off = self.paths[p]
            m2, m3 = self.in2[j][0], self.out[o][0]
            u, rem = divmod(e - off, m2 * m3)
            v, w = divmod(rem, m3)
            c = real_cg(self.in1[i][1], self.in2[j][1], self.out[o][1])
            if absolute:
                c = np.abs(c)
            out[r] = self.alpha[o] * np.einsum("abk,na,nb,nk->", c, a[i][:, :, u], b[j][:, :, v], gb[o][:, :, w])
        return out

    def conv(self, x1, x2, w, src, dst, n_nodes, layout="mul_ir", reduce="sum", absolute=False):
        """The fully connected product as a graph convolution (the
        convolution layer of the cuequivariance-torch skill document, "Other
        operations and layers": source features, edge harmonics and one
        weight row per edge from the edge MLP, summed or averaged into the
        destinations):

            out[n] = s_n sum over edges e with dst[e] = n of fwd(x1[src[e]], x2[e]; w[e]),

        s_n = 1, or 1 / (number of such edges) with reduce="mean" (rows
        without edges are zero).  x1 [n_src, dim_in1]; x2 [n_edges, dim_in2];
        w [n_edges, weight_numel] or [1, weight_numel] (shared).  Returns
        float64 [n_nodes, dim_out]."""
        x1, x2, w = (np.asarray(a, dtype=np.float64) for a in (x1, x2, w))
        if absolute:
            x1, x2, w = np.abs(x1), np.abs(x2), np.abs(w)
        src = np.asarray(src, dtype=np.int64)
        dst = np.asarray(dst, dtype=np.int64)
        a = split_blocks(x1, self.in1, layout)
        b = split_blocks(x2, self.in2, layout)
        ob = [np.zeros((n_nodes, 2 * l + 1, m)) for m, l, _ in self.out]
        for p, (i, j, o, off) in enumerate(self.paths):
            m1, m2, m3 = self.in1[i][0], self.in2[j][0], self.out[o][0]
            c = real_cg(self.in1[i][1], self.in2[j][1], self.out[o][1])
            if absolute:
                c = np.abs(c)
            We = w[:, off:off + m1 * m2 * m3].reshape(-1, m1, m2, m3)
            msg = self.alpha[o] * np.einsum("abk,eau,ebv,euvw->ekw", c, a[i][src], b[j], We, optimize=True)
            np.add.at(ob[o], dst, msg)
        if reduce == "mean":
            deg = np.bincount(dst, minlength=n_nodes)[:n_nodes].astype(np.float64)
            inv = np.where(deg > 0, 1.0 / np.maximum(deg, 1.0), 0.0)
            ob = [t * inv[:, None, None] for t in ob]
        elif reduce != "sum":
            raise ValueError("reduce is 'sum' or 'mean'")
        return join_blocks(ob, layout)

    def conv_vjp(self, x1, x2, w, src, dst, n_nodes, g, layout="mul_ir", reduce="sum", absolute=False):
        """Vector-Jacobian product of :meth:`conv` for g = dL/d(out)
        [n_nodes, dim_out]: returns (dx1 [n_src, dim_in1], dx2 [n_edges,
        dim_in2], dw shaped like w).  Per edge e (source s, destination n,
        G = g[n] scaled by 1/deg(n) with reduce="mean") it is the batch VJP of
        the edge's product; dx1 sums the edges that read each source.  One
        shared weight row [1, weight_numel] enters every edge, so its
        gradient is the sum of the per-edge gradients (chain rule through
        the broadcast)."""
        x1, x2, w, g = (np.asarray(a, dtype=np.float64) for a in (x1, x2, w, g))
        src = np.asarray(src, dtype=np.int64)
        dst = np.asarray(dst, dtype=np.int64)
        if reduce == "mean":
            deg = np.bincount(dst, minlength=n_nodes)[:n_nodes].astype(np.float64)
            g = g * np.where(deg > 0, 1.0 / np.maximum(deg, 1.0), 0.0)[:, None]
        elif reduce != "sum":
            raise ValueError("reduce is 'sum' or 'mean'")
        shared = w.shape[0] == 1 and x2.shape[0] != 1
        we = np.broadcast_to(w, (x2.shape[0], w.shape[1])) if shared else w
        d1, d2, dw = self.vjp(x1[src], x2, None, g[dst], layout=layout, absolute=absolute, edge_weights=we)
        dx1 = np.zeros_like(x1)
        np.add.at(dx1, src, d1)
        if shared:
            dw = dw.sum(axis=0, keepdims=True)
        return dx1, d2, dw
