"""Edge embedding assembly of the fully connected convolution layer (oracle
side).  Test infrastructure only.

cuequivariance-torch skill document, "Other operations and layers": the
convolution layer takes an edge embedding and, optionally, per-node
src_scalars and dst_scalars; they go with the edge embedding into the edge
MLP that makes the per-edge weights.  The reading here (the pages give no
formula): the MLP input of edge e is the concatenation

    [edge_emb[e], src_scalars[src[e]], dst_scalars[dst[e]]]

(either scalar part may be absent), and its backward returns the slice for
the edge embedding and the sums of the slices over the edges that read
each source row and each destination row.
"""

import numpy as np


def concat(edge_emb, src_scalars, dst_scalars, src, dst):
    """[n_edges, d_emb + d_src + d_dst] float64."""
    parts = [np.asarray(edge_emb, dtype=np.float64)]
    if src_scalars is not None:
        parts.append(np.asarray(src_scalars, dtype=np.float64)[np.asarray(src)])
    if dst_scalars is not None:
        parts.append(np.asarray(dst_scalars, dtype=np.float64)[np.asarray(dst)])
    return np.concatenate(parts, axis=1)


def concat_vjp(g, d_emb, d_src, d_dst, src, dst, n_src, n_dst):
    """(d edge_emb [n_edges, d_emb], d src_scalars [n_src, d_src] or None,
    d dst_scalars [n_dst, d_dst] or None) for g = dL/d(concat)."""
    g = np.asarray(g, dtype=np.float64)
    de = g[:, :d_emb].copy()
    ds = dd = None
    if d_src:
        ds = np.zeros((n_src, d_src))
        np.add.at(ds, np.asarray(src), g[:, d_emb:d_emb + d_src])
    if d_dst:
        dd = np.zeros((n_dst, d_dst))
        np.add.at(dd, np.asarray(dst), g[:, d_emb + d_src:d_emb + d_src + d_dst])
    return de, ds, dd
