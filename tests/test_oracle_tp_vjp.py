"""Pins of the oracle's vector-Jacobian product of the convolution: the
adjoint identity for each operand (the forward is linear in each), and a
dense brute force.  CPU only."""

import numpy as np
import pytest

from oracle import layout, tp
from oracle.cg import real_cg


def _case(seed, shared=False, lay="mul_ir"):
    d = tp.ChannelwiseTP("3x0e+2x1o+2x2e", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o")
    rng = np.random.default_rng(seed)
    n_src, n_dst, n_e = 6, 5, 23
    x = rng.normal(size=(n_src, d.dim_in1))
    sh = rng.normal(size=(n_e, d.dim_in2))
    w = rng.normal(size=(1 if shared else n_e, d.weight_numel))
    src = rng.integers(0, n_src, n_e)
    dst = np.sort(rng.integers(0, n_dst, n_e))
    g = rng.normal(size=(n_dst, d.dim_out))
    return d, x, sh, w, src, dst, n_dst, g, rng


@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
@pytest.mark.parametrize("shared", [False, True])
def test_adjoint_identity_each_operand(lay, shared):
    d, x, sh, w, src, dst, n, g, rng = _case(1, shared, lay)
    dx, dsh, dw = d.conv_vjp(x, sh, w, src, dst, n, g, layout=lay, shared_weights=shared)
    vx, vs, vw = rng.normal(size=x.shape), rng.normal(size=sh.shape), rng.normal(size=w.shape)
    # linear in x, in sh and in w separately: <g, F(v)> = <VJP(g), v>
    assert np.isclose(np.sum(g * d.conv(vx, sh, w, src, dst, n, layout=lay)), np.sum(dx * vx), rtol=1e-12)
    assert np.isclose(np.sum(g * d.conv(x, vs, w, src, dst, n, layout=lay)), np.sum(dsh * vs), rtol=1e-12)
    assert np.isclose(np.sum(g * d.conv(x, sh, vw, src, dst, n, layout=lay)), np.sum(dw * vw), rtol=1e-12)


def test_dense_brute_force():
    d, x, sh, w, src, dst, n, g, _ = _case(2)
    off1 = np.cumsum([0] + [m * (2 * l + 1) for m, l, _ in d.in1])
    off2 = np.cumsum([0] + [m * (2 * l + 1) for m, l, _ in d.in2])
    offo = np.cumsum([0] + [m * (2 * l + 1) for m, l, _ in d.out])
    T = np.zeros((d.dim_in1, d.dim_in2, d.dim_out, d.weight_numel))
    woff = 0
    for p, (i, j, lo, _) in enumerate(d.paths):
        mul, l1, _ = d.in1[i]
        c = real_cg(l1, d.in2[j][1], lo)
        for u in range(mul):
            for a in range(2 * l1 + 1):
                for b in range(c.shape[1]):
                    for k in range(2 * lo + 1):
                        T[off1[i] + u * (2 * l1 + 1) + a, off2[j] + b, offo[p] + u * (2 * lo + 1) + k, woff + u] = c[a, b, k]
        woff += mul
    dx_ref = np.zeros_like(x)
    dsh_ref = np.zeros_like(sh)
    dw_ref = np.zeros_like(w)
    for e in range(len(src)):
        ge = g[dst[e]]
        dx_ref[src[e]] += np.einsum("abkc,b,k,c->a", T, sh[e], ge, w[e])
        dsh_ref[e] = np.einsum("abkc,a,k,c->b", T, x[src[e]], ge, w[e])
        dw_ref[e] = np.einsum("abkc,a,b,k->c", T, x[src[e]], sh[e], ge)
    dx, dsh, dw = d.conv_vjp(x, sh, w, src, dst, n, g)
    assert np.allclose(dx, dx_ref, atol=1e-12)
    assert np.allclose(dsh, dsh_ref, atol=1e-12)
    assert np.allclose(dw, dw_ref, atol=1e-12)


def test_isolated_sources_get_zero_gradient():
    d, x, sh, w, src, dst, n, g, _ = _case(3)
    dx, _, _ = d.conv_vjp(x, sh, w, src, dst, n, g)
    unused = np.setdiff1d(np.arange(x.shape[0]), src)
    assert np.all(dx[unused] == 0)


def test_absolute_mode_bounds_and_adjoint():
    """The error scale: elementwise at least |VJP| (triangle inequality),
    and the adjoint of the forward's absolute mode (both take |operands| and
    |C|), operand by operand."""
    d, x, sh, w, src, dst, n, g, rng = _case(4)
    dx, dsh, dw = d.conv_vjp(x, sh, w, src, dst, n, g)
    ax, ash, aw = d.conv_vjp(x, sh, w, src, dst, n, g, absolute=True)
    for a, b in ((ax, dx), (ash, dsh), (aw, dw)):
        assert np.all(a >= np.abs(b) - 1e-12)
    vx, vs, vw = np.abs(rng.normal(size=x.shape)), np.abs(rng.normal(size=sh.shape)), np.abs(rng.normal(size=w.shape))
    ag = np.abs(g)
    assert np.isclose(np.sum(ag * d.conv(vx, sh, w, src, dst, n, absolute=True)), np.sum(ax * vx), rtol=1e-12)
    assert np.isclose(np.sum(ag * d.conv(x, vs, w, src, dst, n, absolute=True)), np.sum(ash * vs), rtol=1e-12)
    assert np.isclose(np.sum(ag * d.conv(x, sh, vw, src, dst, n, absolute=True)), np.sum(aw * vw), rtol=1e-12)
