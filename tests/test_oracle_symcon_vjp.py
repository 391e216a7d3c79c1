"""Pins of the oracle's vector-Jacobian product of the symmetric
contraction: the adjoint identity for the weights (the output is linear in
them), the exact directional derivative in x (the output is a polynomial of
degree <= 3 in x, so the five-point difference quotient is exact), an
independent brute force over ordered component tuples with the product rule
written out, and the species bookkeeping.  CPU only."""

import itertools

import numpy as np
import pytest

from oracle import layout as ol
from oracle import symcon


def _case(seed, ins="2x0e+2x1o+2x2e", outs="2x0e+2x1o", lay="ir_mul", n_el=3, A=9):
    s = symcon.SymmetricContraction(ins, outs)
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(A, s.dim_in))
    w = rng.normal(size=(n_el, s.weight_numel))
    sp = rng.integers(0, n_el, A)
    g = rng.normal(size=(A, s.dim_out))
    return s, x, sp, w, g, rng


@pytest.mark.parametrize("lay", ["ir_mul", "mul_ir"])
def test_weight_adjoint_identity(lay):
    s, x, sp, w, g, rng = _case(1, lay=lay)
    _, dw = s.eval_vjp(x, sp, w, g, layout=lay)
    vw = rng.normal(size=w.shape)
    assert np.isclose(np.sum(g * s.eval(x, sp, vw, layout=lay)), np.sum(dw * vw), rtol=1e-12)


@pytest.mark.parametrize("lay", ["ir_mul", "mul_ir"])
def test_exact_directional_derivative_in_x(lay):
    """F(x + t d) is a cubic in t, so (8 (F(1) - F(-1)) - (F(2) - F(-2))) / 12
    is its exact t-derivative at 0 (up to rounding)."""
    s, x, sp, w, g, rng = _case(2, lay=lay)
    dx, _ = s.eval_vjp(x, sp, w, g, layout=lay)
    d = rng.normal(size=x.shape)
    F = lambda t: np.sum(g * s.eval(x + t * d, sp, w, layout=lay))
    deriv = (8 * (F(1.0) - F(-1.0)) - (F(2.0) - F(-2.0))) / 12
    assert np.isclose(deriv, np.sum(dx * d), rtol=1e-10)


def test_brute_force_product_rule():
    """Per atom and channel, loops over every ordered component tuple of
    every coupling tensor: d/dv_m prod_i v[m_i] = sum over slots i with
    m_i = m of the product of the other slots."""
    s, x, sp, w, g, _ = _case(3, ins="1x0e+1x1o", outs="1x0e+1x1o", A=4)
    dx, dw = s.eval_vjp(x, sp, w, g, layout="mul_ir")
    n = s.n
    mul = s.mul   # 1
    out_off = np.cumsum([0] + [2 * L + 1 for _, L, _ in s.out])
    dx_ref = np.zeros_like(x)
    dw_ref = np.zeros_like(w)
    for a in range(x.shape[0]):
        v = x[a]          # mul = 1: the row is the component vector in both layouts
        for k, (nu, ob, kk) in enumerate(s.segments):
            U = s.basis[(nu, ob)][kk]
            wk = w[sp[a], k * mul]
            for idx in itertools.product(range(n), repeat=nu):
                for M in range(U.shape[-1]):
                    c = U[idx + (M,)]
                    if c == 0.0:
                        continue
                    gm = g[a, out_off[ob] + M]
                    dw_ref[sp[a], k * mul] += gm * c * np.prod([v[m] for m in idx])
                    for i in range(nu):
                        rest = np.prod([v[idx[j]] for j in range(nu) if j != i])
                        dx_ref[a, idx[i]] += wk * gm * c * rest
    assert np.allclose(dx, dx_ref, rtol=1e-12, atol=1e-12)
    assert np.allclose(dw, dw_ref, rtol=1e-12, atol=1e-12)


def test_species_bookkeeping():
    """dw[s] sums the atoms of species s (one call = the sum of per-atom
    calls); an atom whose species is out of range gets dx = 0 and adds
    nothing to dw."""
    s, x, sp, w, g, _ = _case(4)
    dx, dw = s.eval_vjp(x, sp, w, g)
    acc = np.zeros_like(dw)
    for a in range(x.shape[0]):
        dxa, dwa = s.eval_vjp(x[a:a + 1], sp[a:a + 1], w, g[a:a + 1])
        assert np.allclose(dxa, dx[a:a + 1], rtol=1e-13, atol=1e-13)
        acc += dwa
    assert np.allclose(acc, dw, rtol=1e-12, atol=1e-12)
    bad = sp.copy()
    bad[[0, 3]] = [w.shape[0], -1]
    dxb, dwb = s.eval_vjp(x, bad, w, g)
    assert np.count_nonzero(dxb[[0, 3]]) == 0
    keep = np.ones(len(sp), bool)
    keep[[0, 3]] = False
    dxk, dwk = s.eval_vjp(x[keep], sp[keep], w, g[keep])
    assert np.allclose(dwb, dwk, rtol=1e-12, atol=1e-12)
    assert np.allclose(dxb[keep], dxk, rtol=1e-12, atol=1e-12)


def test_layouts_agree():
    s, x, sp, w, g, _ = _case(5)
    dx, dw = s.eval_vjp(x, sp, w, g, layout="ir_mul")
    xm = ol.transpose(x, s.inp, "ir_mul", "mul_ir")
    gm = ol.transpose(g, s.out, "ir_mul", "mul_ir")
    dxm, dwm = s.eval_vjp(xm, sp, w, gm, layout="mul_ir")
    assert np.allclose(ol.transpose(dxm, s.inp, "mul_ir", "ir_mul"), dx, rtol=1e-13, atol=1e-13)
    assert np.allclose(dwm, dw, rtol=1e-13, atol=1e-13)


def test_absolute_mode_bounds():
    s, x, sp, w, g, _ = _case(6)
    dx, dw = s.eval_vjp(x, sp, w, g)
    ax, aw = s.eval_vjp(x, sp, w, g, absolute=True)
    assert np.all(ax >= np.abs(dx) - 1e-12)
    assert np.all(aw >= np.abs(dw) - 1e-12)
    # the weight part is the adjoint of the forward's absolute mode
    vw = np.abs(np.random.default_rng(7).normal(size=w.shape))
    assert np.isclose(np.sum(np.abs(g) * s.eval(x, sp, vw, absolute=True)), np.sum(aw * vw), rtol=1e-12)


@pytest.mark.parametrize("lay", ["ir_mul", "mul_ir"])
def test_batched_oracle_equals_plain_definition(lay):
    """The batched evaluation (sums over the coupling tensors' non-zero
    entries with 0/1 gather/scatter matrices) against the definition written
    out with dense einsums per atom and channel, forward and VJP, at the
    irreps of the 50,000-atom workload (4 channels instead of 128), with an
    out-of-range species."""
    sc = symcon.SymmetricContraction("4x0e+4x1o+4x2e+4x3o", "4x0e+4x1o")
    rng = np.random.default_rng(17)
    n_atoms, n_el = 5, 3
    x = rng.normal(size=(n_atoms, sc.dim_in))
    sp = np.array([2, 0, 3, 1, 2])          # 3 is outside [0, 3)
    w = rng.normal(size=(n_el, sc.weight_numel))
    g = rng.normal(size=(n_atoms, sc.dim_out))
    assert np.allclose(sc.eval(x, sp, w, layout=lay), sc.eval_plain(x, sp, w, layout=lay), rtol=1e-12, atol=1e-12)
    dx, dw = sc.eval_vjp(x, sp, w, g, layout=lay)
    px, pw = sc.eval_vjp_plain(x, sp, w, g, layout=lay)
    assert np.allclose(dx, px, rtol=1e-12, atol=1e-12)
    assert np.allclose(dw, pw, rtol=1e-12, atol=1e-12)
    assert np.count_nonzero(px[2]) == 0
