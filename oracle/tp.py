"""Channelwise (uvu) tensor product with gather and sum-scatter (oracle side).

What is computed (e3nn-course Lesson 12a, section 21.4, the descriptor
``[ijk]*a[uv]*b[iu]*c[jv] -> D[kuv]`` with a = weights, b = input 1,
c = input 2, u the channel of input 1, v = 1 for input 2; cuequivariance-torch
skill document, "Channelwise product with external per-example weights",
"SegmentedPolynomial: gather and scatter" and "Layouts and weights"):

Paths.  For every block i of input 1 (mul_i x l1 p1), every block j of
input 2 (1 x l2 p2) and every lo = |l1-l2| .. l1+l2 (the selection rule of
section 21.4), the path (i, j, lo) with output parity p1*p2 is kept when the
type (lo, p1*p2) is one the output argument lists.  The output argument
selects irrep *types*, not multiplicities: each kept path gets its own
output block of multiplicity mul_i.  Enumeration order is i, then j, then
lo ascending; paths are then stably sorted by the output type (l, natural
parity first), which is the order of the output blocks and of the weight
segments.  (The page's example: ``32x0e+32x1o`` x ``0e+1o`` with output
``32x0e+32x1o`` has 4 paths, 128 weights and output
``32x0e+32x0e+32x1o+32x1o``.)

Weights.  One segment of mul_i values per path (channel u fastest); a row
per edge ``[n_edges, weight_numel]``, or one shared row ``[1, weight_numel]``.

Per edge e and path p:
    m_e[p][k, u] = w[e, woff_p + u] * sum_ij C_p[i, j, k] * X1[src_e, blk1_p, i, u] * X2[e, blk2_p, j]
    out[n] = sum over edges with dst_e = n of m_e       (zero if none)

C_p is :func:`oracle.cg.real_cg`.  Without indices (batch mode) src and dst
are the identity.

Merged output (``merge=True``; the e3nn instruction list the pages print has
one output block per instruction, and several instructions may write one
irrep): a reading of the pages, not a printed example.  The paths of one
output type sum into a single block of that type, in the same type order;
all paths of a type must then have the same multiplicity.  Weights and path
order are unchanged.
"""

import numpy as np

from . import irreps as ir
from .cg import real_cg
from .layout import split_blocks, join_blocks


class ChannelwiseTP:
    """Descriptor of one channelwise tensor product."""

    def __init__(self, irreps_in1, irreps_in2, irreps_out, merge=False):
        self.in1 = ir.parse(irreps_in1)
        self.in2 = ir.parse(irreps_in2)
        for mul, _, _ in self.in2:
            if mul != 1:
                raise ValueError("input 2 must have multiplicity 1 per block (v = 1)")
        keep = {(l, p) for _, l, p in ir.parse(irreps_out)}
        paths = []
        for i, (mul1, l1, p1) in enumerate(self.in1):
            for j, (_, l2, p2) in enumerate(self.in2):
                for lo in range(abs(l1 - l2), l1 + l2 + 1):
                    po = p1 * p2
                    if (lo, po) in keep:
                        paths.append((i, j, lo, po))
        # stable sort by output type: output block order = weight order
        paths.sort(key=lambda t: ir.type_key(t[2], t[3]))
        self.paths = paths
        self.out = [(self.in1[i][0], lo, po) for i, _, lo, po in paths]
        self.weight_numel = sum(self.in1[i][0] for i, _, _, _ in paths)
        self.dim_in1 = ir.dim(self.in1)
        self.dim_in2 = ir.dim(self.in2)
        self.merge = merge
        self.path_out = list(range(len(paths)))   # output block of each path
        self.out_blocks = list(self.out)          # the output row's blocks
        if merge:
            types, self.out_blocks = [], []
            for p, (mul, lo, po) in enumerate(self.out):
                if (lo, po) not in types:
                    types.append((lo, po))
                    self.out_blocks.append((mul, lo, po))
                t = types.index((lo, po))
                if self.out_blocks[t][0] != mul:
                    raise ValueError("merged paths of one type need one multiplicity")
                self.path_out[p] = t
        self.dim_out = ir.dim(self.out_blocks)

    @property
    def irreps_out(self):
        return ir.to_str(self.out_blocks)

    def _merge_parts(self, parts):
        """Per-path output blocks -> the row's blocks (sums per type when
        merged)."""
        if not self.merge:
            return parts
        out = [None] * len(self.out_blocks)
        for p, part in enumerate(parts):
            t = self.path_out[p]
            out[t] = part if out[t] is None else out[t] + part
        return out

    @property
    def num_paths(self):
        return len(self.paths)

    def path_table(self):
        """[(l1, l2, lo, nnz of C)] in path order."""
        rows = []
        for i, j, lo, _ in self.paths:
            l1, l2 = self.in1[i][1], self.in2[j][1]
            rows.append((l1, l2, lo, int(np.count_nonzero(real_cg(l1, l2, lo)))))
        return rows

    def weight_fan_in(self):
        """Per weight column: the number of paths whose output block has the
        same irrep type (the fan-in reading of N(0,1)/sqrt(fan-in))."""
        cnt = {}
        for _, lo, po in self.out:
            cnt[(lo, po)] = cnt.get((lo, po), 0) + 1
        return np.concatenate([np.full(mul, cnt[(lo, po)]) for mul, lo, po in self.out])

    def conv(self, x, sh, w, src=None, dst=None, n_nodes=None, layout="mul_ir",
             absolute=False, nodes=None, reduce="sum"):
        """Gather, couple and sum-scatter.

        x   [n_src, dim_in1] in ``layout``;  sh [n_edges, dim_in2];
        w   [n_edges, weight_numel] or [1, weight_numel] (shared);
        src, dst [n_edges] integer indices (None, None: batch mode);
        n_nodes  number of destination rows;
        absolute use |x|, |sh|, |w| and |C| (the forward-error scale);
        nodes    optional sorted array of destination rows to compute: only
                 edges whose dst is listed contribute and the result has
                 len(nodes) rows in that order;
        reduce   "sum", or "mean": each destination row divided by the number
                 of edges whose dst it is (rows without edges stay zero) --
                 the ``reduce="mean"`` option of the pages' convolution layer
                 (cuequivariance-torch skill document, "Other operations and
                 layers").
        Returns float64 [n_nodes or len(nodes), dim_out] in ``layout``."""
        x = np.asarray(x, dtype=np.float64)
        sh = np.asarray(sh, dtype=np.float64)
        w = np.asarray(w, dtype=np.float64)
        if absolute:
            x, sh, w = np.abs(x), np.abs(sh), np.abs(w)
        n_edges = sh.shape[0]
        if src is None:
            src = np.arange(n_edges)
            dst = np.arange(n_edges)
            n_nodes = n_edges if n_nodes is None else n_nodes
        src = np.asarray(src, dtype=np.int64)
        dst = np.asarray(dst, dtype=np.int64)
        if nodes is not None:
            nodes = np.asarray(nodes, dtype=np.int64)
            sel = np.isin(dst, nodes)
            src, dst, sh = src[sel], dst[sel], sh[sel]
            if w.shape[0] != 1:
                w = w[sel]
            dst = np.searchsorted(nodes, dst)   # destination row within `nodes`
            n_rows = len(nodes)
        else:
            n_rows = n_nodes
        x1 = split_blocks(x, self.in1, layout)          # per block [n_src, 2l+1, mul]
        x2 = split_blocks(sh, self.in2, "ir_mul")       # per block [n_edges, 2l+1, 1]
        out_parts = []
        woff = 0
        for i, j, lo, _ in self.paths:
            mul, l1, _ = self.in1[i]
            l2 = self.in2[j][1]
            c = real_cg(l1, l2, lo)
            if absolute:
                c = np.abs(c)
            a = x1[i][src]                               # gather: [E, 2l1+1, mul]
            b = x2[j][:, :, 0]                           # [E, 2l2+1]
            ww = w[:, woff:woff + mul]                   # [E or 1, mul]
            m = np.einsum("ijk,eiu,ej->eku", c, a, b) * ww[:, None, :]
            blk = np.zeros((n_rows, 2 * lo + 1, mul))
            np.add.at(blk, dst, m)                       # sum-scatter (index_add)
            out_parts.append(blk)
            woff += mul
        if reduce == "mean":
            deg = np.bincount(dst, minlength=n_rows)[:n_rows].astype(np.float64)
            inv = np.where(deg > 0, 1.0 / np.maximum(deg, 1.0), 0.0)
            out_parts = [b * inv[:, None, None] for b in out_parts]
        elif reduce != "sum":
            raise ValueError("reduce is 'sum' or 'mean'")
        return join_blocks(self._merge_parts(out_parts), layout)

    def conv_vjp(self, x, sh, w, src, dst, n_nodes, g, layout="mul_ir", shared_weights=False,
                 absolute=False, reduce="sum"):
        """Vector-Jacobian product of :meth:`conv` (per-edge weights, or one
        shared row with ``shared_weights``): given g = dL/d(out) [n_nodes,
        dim_out] in ``layout``, return (dL/dx [n_src, dim_in1] in ``layout``,
        dL/dsh [n_edges, dim_in2], dL/dw [n_edges or 1, weight_numel]).

        From the definition, per path p and channel u (the forward is linear
        in each operand):
            dw[e, p, u]     = sum_k g[dst_e, p, k, u] sum_ij C[i,j,k] x[src_e, i, u] sh[e, j]
            dsh[e, blk2_p, j] += sum_u w[e, p, u] sum_ik C[i,j,k] x[src_e, i, u] g[dst_e, p, k, u]
            dx[src_e, blk1_p, i, u] += w[e, p, u] sum_jk C[i,j,k] sh[e, j] g[dst_e, p, k, u]

        ``absolute`` evaluates the same sums over |x|, |sh|, |w|, |g| and |C|:
        the scale of the rounding error of any summation order.  With
        reduce="mean" the output row n is the sum over its edges divided by
        their number, so g[n] enters divided by it."""
        x = np.asarray(x, dtype=np.float64)
        sh = np.asarray(sh, dtype=np.float64)
        w = np.asarray(w, dtype=np.float64)
        g = np.asarray(g, dtype=np.float64)
        if absolute:
            x, sh, w, g = np.abs(x), np.abs(sh), np.abs(w), np.abs(g)
        n_edges = sh.shape[0]
        if src is None:
            src = np.arange(n_edges)
            dst = np.arange(n_edges)
        src = np.asarray(src, dtype=np.int64)
        dst = np.asarray(dst, dtype=np.int64)
        if reduce == "mean":
            deg = np.bincount(dst, minlength=g.shape[0])[:g.shape[0]].astype(np.float64)
            g = g * np.where(deg > 0, 1.0 / np.maximum(deg, 1.0), 0.0)[:, None]
        elif reduce != "sum":
            raise ValueError("reduce is 'sum' or 'mean'")
        x1 = split_blocks(x, self.in1, layout)          # per block [n_src, 2l+1, mul]
        x2 = split_blocks(sh, self.in2, "ir_mul")       # per block [n_edges, 2l+1, 1]
        gb = split_blocks(g, self.out_blocks, layout)   # per output block [n_nodes, 2lo+1, mul]
        gb = [gb[self.path_out[p]] for p in range(len(self.paths))]   # per path
        dx1 = [np.zeros_like(b) for b in x1]
        dsh = np.zeros_like(sh)
        dw = np.zeros((n_edges, self.weight_numel))
        off2 = np.cumsum([0] + [2 * l + 1 for _, l, _ in self.in2])
        woff = 0
        for p, (i, j, lo, _) in enumerate(self.paths):
            mul, l1, _ = self.in1[i]
            l2 = self.in2[j][1]
            c = real_cg(l1, l2, lo)
            if absolute:
                c = np.abs(c)
            a = x1[i][src]                               # [E, 2l1+1, mul]
            b = x2[j][:, :, 0]                           # [E, 2l2+1]
            ge = gb[p][dst]                              # [E, 2lo+1, mul]
            ww = np.broadcast_to(w[:, woff:woff + mul], (n_edges, mul))
            dw[:, woff:woff + mul] = np.einsum("ijk,eiu,ej,eku->eu", c, a, b, ge, optimize=True)
            dsh[:, off2[j]:off2[j + 1]] += np.einsum("ijk,eiu,eku,eu->ej", c, a, ge, ww, optimize=True)
            np.add.at(dx1[i], src, np.einsum("ijk,ej,eku,eu->eiu", c, b, ge, ww, optimize=True))
            woff += mul
        if shared_weights:
            dw = dw.sum(axis=0, keepdims=True)
        return join_blocks(dx1, layout), dsh, dw
