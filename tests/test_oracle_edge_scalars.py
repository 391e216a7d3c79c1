"""Pins of the edge-embedding assembly oracle: rows written out by hand and
the adjoint identity of its VJP.  CPU only."""

import numpy as np

from oracle import edge_scalars as es


def test_rows_by_hand_and_absent_parts():
    emb = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    ssc = np.array([[10.0], [20.0]])
    dsc = np.array([[0.5, 0.25], [1.5, 1.25], [2.5, 2.25]])
    src, dst = np.array([1, 0, 1]), np.array([0, 2, 2])
    out = es.concat(emb, ssc, dsc, src, dst)
    assert out.tolist() == [[1, 2, 20, 0.5, 0.25], [3, 4, 10, 2.5, 2.25], [5, 6, 20, 2.5, 2.25]]
    assert es.concat(emb, None, None, src, dst).tolist() == emb.tolist()
    assert es.concat(emb, None, dsc, src, dst).shape == (3, 4)


def test_vjp_adjoint_identity():
    rng = np.random.default_rng(0)
    E, ns, nd = 11, 4, 5
    src, dst = rng.integers(0, ns, E), np.sort(rng.integers(0, nd, E))
    emb, ssc, dsc = rng.normal(size=(E, 3)), rng.normal(size=(ns, 2)), rng.normal(size=(nd, 4))
    g = rng.normal(size=(E, 9))
    de, ds, dd = es.concat_vjp(g, 3, 2, 4, src, dst, ns, nd)
    ve, vs, vd = rng.normal(size=emb.shape), rng.normal(size=ssc.shape), rng.normal(size=dsc.shape)
    lhs = np.sum(g * es.concat(ve, vs, vd, src, dst))
    assert np.isclose(lhs, np.sum(de * ve) + np.sum(ds * vs) + np.sum(dd * vd), rtol=1e-12)
    unread = np.setdiff1d(np.arange(ns), src)
    assert np.count_nonzero(ds[unread]) == 0
