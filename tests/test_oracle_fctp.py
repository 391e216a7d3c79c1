"""Pins of the fully connected (uvw) tensor-product oracle: the pages'
"0 + 1" example and m^3 weight count, a reduction to the channelwise product
(itself pinned by a brute force and the pages' descriptor counts), a dense
brute force with hand-written offsets, O(3) equivariance, the layout round
trip, the variance the normalisation is chosen for, and the adjoint
identities of the vector-Jacobian product.  CPU only."""

import numpy as np
import pytest

from oracle import fctp, irreps as ir, layout as ol, sh, tp, wigner
from oracle.cg import real_cg


def test_page_example_so3():
    """cuequivariance-torch skill document, "CPU tensor product and
    backward": FullyConnectedTensorProduct(irreps, irreps, irreps) for the
    SO(3) irreps "0 + 1", fed features and the l = 0, 1 harmonics of two
    vectors, returns shape (2, irreps.dim) and non-zero gradients for the
    features, the vectors and the weights."""
    f = fctp.FullyConnectedTP("0 + 1", "0 + 1", "0 + 1")
    # SO(3) keeps 1 x 1 -> 1, which O(3) parity would remove for 1o x 1o -> 1o
    assert [(i, j, o) for i, j, o, _ in f.paths] == [(0, 0, 0), (0, 1, 1), (1, 0, 1), (1, 1, 0), (1, 1, 1)]
    assert f.weight_numel == 5 and f.dim_out == 4
    rng = np.random.default_rng(0)
    feats = rng.normal(size=(2, 4))
    vecs = np.array([[0.3, -0.7, 1.1], [1.2, 0.4, -0.2]])
    y2 = sh.real_sh([0, 1], vecs, normalize=False)
    w = rng.normal(size=(1, 5))
    out = f.fwd(feats, y2, w)
    assert out.shape == (2, 4)
    dx1, dx2, dw = f.vjp(feats, y2, w, 2 * out)       # d(sum out^2)
    dvec = sh.real_sh_vjp([0, 1], vecs, dx2, normalize=False)
    for g in (dx1, dvec, dw):
        assert np.all(np.isfinite(g)) and np.abs(g).sum() > 0


def test_weight_count_scales_as_cube():
    """e3nn-course Lesson 12a, exercise 1: the fully connected product's
    weights carry three channel indices (u, v, w), so they grow as m^3 where
    the channelwise product's grow as m."""
    for m in (8, 16, 32):
        a = f"{m}x0e+{m}x1o"
        f = fctp.FullyConnectedTP(a, a, a)
        # 0e0e->0e, 0e1o->1o, 1o0e->1o, 1o1o->0e (1o1o->1e has no output block)
        assert len(f.paths) == 4 and f.weight_numel == 4 * m ** 3
        c = tp.ChannelwiseTP(a, "0e+1o", a)
        assert c.weight_numel % m == 0 and c.weight_numel // m == c.num_paths


@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
def test_reduces_to_channelwise(lay):
    """With one channel in input 2 and W_p[u, 0, w] = delta_uw c_p[u] on the
    paths that pair input block i with its own output block (zero elsewhere),
    the fully connected product is alpha_o times the channelwise product with
    per-sample-shared weights c."""
    in1, in2 = "3x0e+2x1o+2x2e", "1x0e+1x1o+1x2e"
    c = tp.ChannelwiseTP(in1, in2, "3x0e+2x1o+2x1e+2x2e")
    f = fctp.FullyConnectedTP(in1, in2, c.irreps_out)
    rng = np.random.default_rng(1)
    n = 5
    x1 = rng.normal(size=(n, c.dim_in1))
    x2 = rng.normal(size=(n, c.dim_in2))
    cw = rng.normal(size=(1, c.weight_numel))
    W = np.zeros((1, f.weight_numel))
    cw_off = np.cumsum([0] + [c.in1[i][0] for i, _, _, _ in c.paths])
    for q, (i, j, lo, po) in enumerate(c.paths):
        # channelwise path q writes output block q; find the FC path (i, j, q)
        hits = [p for p in f.paths if (p[0], p[1], p[2]) == (i, j, q)]
        assert len(hits) == 1
        m = c.in1[i][0]
        seg = np.zeros((m, 1, m))
        seg[np.arange(m), 0, np.arange(m)] = cw[0, cw_off[q]:cw_off[q] + m]
        W[0, hits[0][3]:hits[0][3] + m * m] = seg.reshape(-1)
    got = f.fwd(x1, x2, W, layout=lay)
    want = c.conv(x1, x2, cw, layout=lay)
    scale = np.concatenate([np.full(m * (2 * l + 1), f.alpha[o]) for o, (m, l, _) in enumerate(f.out)])
    assert np.allclose(got, want * scale, atol=1e-12)


def test_dense_brute_force():
    """Loops over every (path, u, v, w, a, b, k) with mul_ir offsets written
    out by hand: out[n, off_o + w (2l3+1) + k] += alpha_o W C x1 x2."""
    in1, in2, out = "2x0e+2x1o", "1x0e+2x1o", "2x0e+1x1o+2x1e"
    f = fctp.FullyConnectedTP(in1, in2, out)
    rng = np.random.default_rng(2)
    x1 = rng.normal(size=(3, f.dim_in1))
    x2 = rng.normal(size=(3, f.dim_in2))
    w = rng.normal(size=(1, f.weight_numel))
    b1, b2, bo = ir.parse(in1), ir.parse(in2), ir.parse(out)
    o1 = np.cumsum([0] + [m * (2 * l + 1) for m, l, _ in b1])
    o2 = np.cumsum([0] + [m * (2 * l + 1) for m, l, _ in b2])
    oo = np.cumsum([0] + [m * (2 * l + 1) for m, l, _ in bo])
    fan = np.zeros(len(bo))
    want = np.zeros((3, f.dim_out))
    woff = 0
    for i, (m1, l1, p1) in enumerate(b1):
        for j, (m2, l2, p2) in enumerate(b2):
            for o, (m3, l3, p3) in enumerate(bo):
                if not (abs(l1 - l2) <= l3 <= l1 + l2 and p3 == p1 * p2):
                    continue
                fan[o] += m1 * m2
                C = real_cg(l1, l2, l3)
                for u in range(m1):
                    for v in range(m2):
                        for ww in range(m3):
                            wt = w[0, woff + (u * m2 + v) * m3 + ww]
                            for a in range(2 * l1 + 1):
                                for b in range(2 * l2 + 1):
                                    for k in range(2 * l3 + 1):
                                        want[:, oo[o] + ww * (2 * l3 + 1) + k] += (
                                            wt * C[a, b, k] * x1[:, o1[i] + u * (2 * l1 + 1) + a]
                                            * x2[:, o2[j] + v * (2 * l2 + 1) + b])
                woff += m1 * m2 * m3
    assert woff == f.weight_numel
    for o, (m3, l3, _) in enumerate(bo):
        want[:, oo[o]:oo[o + 1]] /= np.sqrt(fan[o])
    assert np.allclose(f.fwd(x1, x2, w), want, atol=1e-12)


@pytest.mark.parametrize("parity", [1, -1])
def test_equivariance(parity):
    in1, in2, out = "3x0e+2x1o+1x2e", "2x0e+1x1o+2x1e", "2x0e+3x1o+2x1e+1x2e+1x2o"
    f = fctp.FullyConnectedTP(in1, in2, out)
    rng = np.random.default_rng(3)
    x1 = rng.normal(size=(4, f.dim_in1))
    x2 = rng.normal(size=(4, f.dim_in2))
    w = rng.normal(size=(1, f.weight_numel))
    aa = np.array([0.4, -0.2, 0.7])
    D1 = wigner.wigner_d_irreps(f.in1, aa, parity=parity)
    D2 = wigner.wigner_d_irreps(f.in2, aa, parity=parity)
    Do = wigner.wigner_d_irreps(f.out, aa, parity=parity)
    assert np.allclose(f.fwd(x1 @ D1.T, x2 @ D2.T, w), f.fwd(x1, x2, w) @ Do.T, atol=1e-11)


def test_layout_round_trip():
    in1, in2, out = "3x0e+2x1o", "2x0e+2x1o", "2x0e+3x1o+1x1e"
    f = fctp.FullyConnectedTP(in1, in2, out)
    rng = np.random.default_rng(4)
    x1 = rng.normal(size=(3, f.dim_in1))
    x2 = rng.normal(size=(3, f.dim_in2))
    w = rng.normal(size=(1, f.weight_numel))
    y = f.fwd(x1, x2, w, layout="mul_ir")
    y_ir = f.fwd(ol.transpose(x1, f.in1, "mul_ir", "ir_mul"), ol.transpose(x2, f.in2, "mul_ir", "ir_mul"), w,
                 layout="ir_mul")
    assert np.allclose(ol.transpose(y_ir, f.out, "ir_mul", "mul_ir"), y, atol=1e-13)


def test_normalisation_gives_unit_variance():
    """alpha_o = 1 / sqrt(sum over paths into o of mul1 mul2): with N(0, 1)
    inputs and weights each output component has variance 1 (the coupling
    has sum_ab C[a, b, k]^2 = 1 for every k)."""
    f = fctp.FullyConnectedTP("8x0e+6x1o", "4x0e+3x1o", "5x0e+4x1o+3x1e")
    rng = np.random.default_rng(5)
    x1 = rng.normal(size=(4000, f.dim_in1))
    x2 = rng.normal(size=(4000, f.dim_in2))
    var = []
    for _ in range(8):
        w = rng.normal(size=(1, f.weight_numel))
        var.append(f.fwd(x1, x2, w, layout="ir_mul").var(axis=0).mean())
    assert abs(np.mean(var) - 1.0) < 0.1


@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
def test_vjp_adjoint_identities(lay):
    f = fctp.FullyConnectedTP("3x0e+2x1o+1x2e", "2x0e+1x1o", "2x0e+2x1o+1x1e+2x2e")
    rng = np.random.default_rng(6)
    x1 = rng.normal(size=(5, f.dim_in1))
    x2 = rng.normal(size=(5, f.dim_in2))
    w = rng.normal(size=(1, f.weight_numel))
    g = rng.normal(size=(5, f.dim_out))
    dx1, dx2, dw = f.vjp(x1, x2, w, g, layout=lay)
    v1, v2, vw = rng.normal(size=x1.shape), rng.normal(size=x2.shape), rng.normal(size=w.shape)
    assert np.isclose(np.sum(g * f.fwd(v1, x2, w, layout=lay)), np.sum(dx1 * v1), rtol=1e-12)
    assert np.isclose(np.sum(g * f.fwd(x1, v2, w, layout=lay)), np.sum(dx2 * v2), rtol=1e-12)
    assert np.isclose(np.sum(g * f.fwd(x1, x2, vw, layout=lay)), np.sum(dw * vw), rtol=1e-12)


def test_output_without_paths_is_zero_and_absolute_bounds():
    f = fctp.FullyConnectedTP("2x0e+1x1o", "1x0e", "2x0e+1x1o+2x2e")
    rng = np.random.default_rng(7)
    x1 = rng.normal(size=(3, f.dim_in1))
    x2 = rng.normal(size=(3, f.dim_in2))
    w = rng.normal(size=(1, f.weight_numel))
    y = f.fwd(x1, x2, w)
    assert f.alpha[2] == 0.0 and np.count_nonzero(y[:, 5:]) == 0
    assert np.all(np.abs(y) <= f.fwd(x1, x2, w, absolute=True) + 1e-15)


def test_dw_entries_match_vjp():
    f = fctp.FullyConnectedTP("3x0e+2x1o", "2x0e+1x1o", "2x0e+2x1o+1x1e")
    rng = np.random.default_rng(8)
    x1 = rng.normal(size=(6, f.dim_in1))
    x2 = rng.normal(size=(6, f.dim_in2))
    w = rng.normal(size=(1, f.weight_numel))
    g = rng.normal(size=(6, f.dim_out))
    for lay in ("mul_ir", "ir_mul"):
        _, _, dw = f.vjp(x1, x2, w, g, layout=lay)
        flat = np.arange(f.weight_numel)
        assert np.allclose(f.dw_entries(x1, x2, g, flat, layout=lay), dw[0], atol=1e-12)
        assert np.allclose(f.dw_entries(x1, x2, g, flat, layout=lay, absolute=True),
                           f.vjp(x1, x2, w, g, layout=lay, absolute=True)[2][0], atol=1e-12)


def _graph(rng, n_src, n_nodes, n_edges):
    dst = np.sort(rng.integers(0, n_nodes, n_edges))
    src = rng.integers(0, n_src, n_edges)
    return src, dst


@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
def test_conv_edge_by_edge(lay):
    """The convolution form against a loop over edges that evaluates the
    batch product of one edge with that edge's weight row and adds it into
    its destination; rows without edges stay zero."""
    f = fctp.FullyConnectedTP("3x0e+2x1o", "0e+1o+2e", "2x0e+3x1o+1x2e")
    rng = np.random.default_rng(9)
    src, dst = _graph(rng, 7, 6, 15)
    dst[dst == 4] = 5                     # node 4 has no edges
    x1 = rng.normal(size=(7, f.dim_in1))
    x2 = rng.normal(size=(15, f.dim_in2))
    w = rng.normal(size=(15, f.weight_numel))
    want = np.zeros((6, f.dim_out))
    for e in range(15):
        want[dst[e]] += f.fwd(x1[src[e]:src[e] + 1], x2[e:e + 1], w[e:e + 1], layout=lay)[0]
    got = f.conv(x1, x2, w, src, dst, 6, layout=lay)
    assert np.allclose(got, want, atol=1e-12)
    assert np.count_nonzero(got[4]) == 0
    # one shared row = the same row on every edge
    assert np.allclose(f.conv(x1, x2, w[:1], src, dst, 6, layout=lay),
                       f.conv(x1, x2, np.repeat(w[:1], 15, axis=0), src, dst, 6, layout=lay), atol=1e-12)


def test_conv_identity_graph_is_batch_product():
    f = fctp.FullyConnectedTP("2x0e+2x1o", "1x0e+1x1o", "2x0e+2x1o")
    rng = np.random.default_rng(10)
    x1 = rng.normal(size=(8, f.dim_in1))
    x2 = rng.normal(size=(8, f.dim_in2))
    w = rng.normal(size=(1, f.weight_numel))
    idx = np.arange(8)
    assert np.allclose(f.conv(x1, x2, w, idx, idx, 8), f.fwd(x1, x2, w), atol=1e-13)


def test_conv_mean_and_equivariance():
    f = fctp.FullyConnectedTP("3x0e+2x1o", "0e+1o", "2x0e+2x1o+1x1e")
    rng = np.random.default_rng(11)
    src, dst = _graph(rng, 5, 4, 12)
    x1 = rng.normal(size=(5, f.dim_in1))
    x2 = rng.normal(size=(12, f.dim_in2))
    w = rng.normal(size=(12, f.weight_numel))
    s = f.conv(x1, x2, w, src, dst, 4)
    m = f.conv(x1, x2, w, src, dst, 4, reduce="mean")
    deg = np.bincount(dst, minlength=4)
    for n in range(4):
        assert np.allclose(m[n], s[n] / max(deg[n], 1), atol=1e-13)
    aa = np.array([0.3, 0.5, -0.4])
    D1 = wigner.wigner_d_irreps(f.in1, aa, parity=-1)
    D2 = wigner.wigner_d_irreps(f.in2, aa, parity=-1)
    Do = wigner.wigner_d_irreps(f.out, aa, parity=-1)
    assert np.allclose(f.conv(x1 @ D1.T, x2 @ D2.T, w, src, dst, 4), s @ Do.T, atol=1e-11)


@pytest.mark.parametrize("reduce", ["sum", "mean"])
def test_conv_vjp_adjoint_identities(reduce):
    f = fctp.FullyConnectedTP("3x0e+2x1o", "0e+1o+2e", "2x0e+3x1o+1x2e")
    rng = np.random.default_rng(12)
    src, dst = _graph(rng, 6, 5, 14)
    dst[dst == 2] = 3                       # node 2 without edges
    x1 = rng.normal(size=(6, f.dim_in1))
    x2 = rng.normal(size=(14, f.dim_in2))
    w = rng.normal(size=(14, f.weight_numel))
    g = rng.normal(size=(5, f.dim_out))
    for lay in ("mul_ir", "ir_mul"):
        dx1, dx2, dw = f.conv_vjp(x1, x2, w, src, dst, 5, g, layout=lay, reduce=reduce)
        v1, v2, vw = rng.normal(size=x1.shape), rng.normal(size=x2.shape), rng.normal(size=w.shape)
        F = lambda a, b, c: f.conv(a, b, c, src, dst, 5, layout=lay, reduce=reduce)
        assert np.isclose(np.sum(g * F(v1, x2, w)), np.sum(dx1 * v1), rtol=1e-11)
        assert np.isclose(np.sum(g * F(x1, v2, w)), np.sum(dx2 * v2), rtol=1e-11)
        assert np.isclose(np.sum(g * F(x1, x2, vw)), np.sum(dw * vw), rtol=1e-11)
        # one shared weight row: the forward is still linear in it
        ws = rng.normal(size=(1, f.weight_numel))
        _, s2, sw = f.conv_vjp(x1, x2, ws, src, dst, 5, g, layout=lay, reduce=reduce)
        vs = rng.normal(size=ws.shape)
        assert sw.shape == ws.shape
        assert np.isclose(np.sum(g * F(x1, x2, vs)), np.sum(sw * vs), rtol=1e-11)
        assert np.isclose(np.sum(g * F(x1, v2, ws)), np.sum(s2 * v2), rtol=1e-11)
    # sources no edge reads get zero; absolute mode bounds every gradient
    unread = np.setdiff1d(np.arange(6), src)
    assert np.count_nonzero(dx1[unread]) == 0
    a1, a2, aw = f.conv_vjp(x1, x2, w, src, dst, 5, g, reduce=reduce, absolute=True)
    r1, r2, rw = f.conv_vjp(x1, x2, w, src, dst, 5, g, reduce=reduce)
    for r, a in ((r1, a1), (r2, a2), (rw, aw)):
        assert np.all(np.abs(r) <= a + 1e-12)


@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
def test_per_sample_weights(lay):
    """One weight row per sample: each sample is the shared-row product with
    its own row (sample by sample), the same as the convolution form on the
    identity graph; a per-sample weight matrix with equal rows is the shared
    product; the product is linear in the rows, and the VJP's per-sample dw
    (vjp with edge_weights) is its adjoint."""
    f = fctp.FullyConnectedTP("3x0e+2x1o", "2x0e+1x1o", "2x0e+3x1o+1x1e")
    rng = np.random.default_rng(21)
    n = 6
    x1 = rng.normal(size=(n, f.dim_in1))
    x2 = rng.normal(size=(n, f.dim_in2))
    w = rng.normal(size=(n, f.weight_numel))
    got = f.fwd(x1, x2, w, layout=lay)
    for s in range(n):
        assert np.allclose(got[s], f.fwd(x1[s:s + 1], x2[s:s + 1], w[s:s + 1], layout=lay)[0], atol=1e-12)
    idx = np.arange(n)
    assert np.allclose(got, f.conv(x1, x2, w, idx, idx, n, layout=lay), atol=1e-12)
    assert np.allclose(f.fwd(x1, x2, np.repeat(w[:1], n, axis=0), layout=lay), f.fwd(x1, x2, w[:1], layout=lay),
                       atol=1e-12)
    g = rng.normal(size=(n, f.dim_out))
    dx1, dx2, dw = f.vjp(x1, x2, None, g, layout=lay, edge_weights=w)
    assert dw.shape == w.shape
    v = rng.normal(size=w.shape)
    assert np.isclose(np.sum(g * f.fwd(x1, x2, v, layout=lay)), np.sum(dw * v), rtol=1e-11)
    v1 = rng.normal(size=x1.shape)
    assert np.isclose(np.sum(g * f.fwd(v1, x2, w, layout=lay)), np.sum(dx1 * v1), rtol=1e-11)
    v2 = rng.normal(size=x2.shape)
    assert np.isclose(np.sum(g * f.fwd(x1, v2, w, layout=lay)), np.sum(dx2 * v2), rtol=1e-11)
    assert np.all(np.abs(got) <= f.fwd(x1, x2, w, layout=lay, absolute=True) + 1e-12)

