"""Pins of the oracle's equivariant linear layer and its vector-Jacobian
product: the pages' printed sizes, the layout round trip and the rotation
check of the skill document's Linear example, a dense brute force, the
variance the normalisation is chosen for, the identity map, and the adjoint
identities.  CPU only."""

import numpy as np
import pytest

from oracle import irreps as ir
from oracle import layout as ol
from oracle import linear, wigner


def test_page_sizes():
    # "3x0 + 2x1 -> 2x0 + 4x1": 3*2 + 2*4 weights (the skill document's Linear
    # example, SO3 irreps written here with the parity of a vector)
    assert linear.Linear("3x0e+2x1o", "2x0e+4x1o").weight_numel == 14
    # Lesson 12a's closing example: (4, 128) -> (4, 64)
    lin = linear.Linear("32x0e+32x1o", "16x0e+16x1o")
    assert (lin.dim_in, lin.dim_out) == (128, 64)
    x = np.random.default_rng(0).normal(size=(4, 128))
    w = np.random.default_rng(1).normal(size=(1, lin.weight_numel))
    assert lin.fwd(x, w).shape == (4, 64)


@pytest.mark.parametrize("ins,outs", [("3x0e+2x1o", "2x0e+4x1o"),
                                      ("4x0e+3x1o+2x1e+5x2e", "2x0e+3x1o+1x2e+2x3o"),
                                      ("2x0e+3x0e+2x1o+1x1o", "3x0e+2x1o+2x1o")])
def test_layout_round_trip_and_rotation(ins, outs):
    """The skill document's checks: mul_ir and ir_mul agree after
    transposition, and rotating the input rotates the output (x @ D.T)."""
    lin = linear.Linear(ins, outs)
    rng = np.random.default_rng(2)
    x = rng.normal(size=(5, lin.dim_in))
    w = rng.normal(size=(1, lin.weight_numel))
    y = lin.fwd(x, w, layout="mul_ir")
    y_ir = lin.fwd(ol.transpose(x, lin.inp, "mul_ir", "ir_mul"), w, layout="ir_mul")
    assert np.allclose(ol.transpose(y_ir, lin.out, "ir_mul", "mul_ir"), y, atol=1e-13)
    aa = np.array([0.2, -0.3, 0.1])
    for parity in (1, -1):
        din = wigner.wigner_d_irreps(lin.inp, aa, parity=parity)
        dout = wigner.wigner_d_irreps(lin.out, aa, parity=parity)
        assert np.allclose(lin.fwd(x @ din.T, w, layout="mul_ir"), y @ dout.T, atol=1e-12)


def test_dense_brute_force():
    lin = linear.Linear("2x0e+3x1o+2x0e", "3x0e+2x1o+1x2e")
    rng = np.random.default_rng(3)
    w = rng.normal(size=(1, lin.weight_numel))
    M = np.zeros((lin.dim_in, lin.dim_out))
    ioff = np.cumsum([0] + [m * (2 * l + 1) for m, l, _ in lin.inp])
    ooff = np.cumsum([0] + [m * (2 * l + 1) for m, l, _ in lin.out])
    fan = {}
    for m, l, p in lin.inp:
        fan[(l, p)] = fan.get((l, p), 0) + m
    woff = 0
    for i, (mi, li, pi) in enumerate(lin.inp):
        for o, (mo, lo, po) in enumerate(lin.out):
            if (li, pi) != (lo, po):
                continue
            for u in range(mi):
                for v in range(mo):
                    for k in range(2 * li + 1):    # mul_ir: block index u * (2l+1) + k
                        M[ioff[i] + u * (2 * li + 1) + k, ooff[o] + v * (2 * lo + 1) + k] += \
                            w[0, woff + u * mo + v] / np.sqrt(fan[(li, pi)])
            woff += mi * mo
    x = rng.normal(size=(6, lin.dim_in))
    assert np.allclose(lin.fwd(x, w, layout="mul_ir"), x @ M, atol=1e-12)
    # the 2e output block has no input of its type: zero
    assert np.count_nonzero((x @ M)[:, ooff[2]:ooff[3]]) == 0


def test_normalisation_gives_unit_variance():
    lin = linear.Linear("40x0e+24x0e+16x1o", "32x0e+8x1o")
    rng = np.random.default_rng(4)
    x = rng.normal(size=(20000, lin.dim_in))
    w = rng.normal(size=(1, lin.weight_numel))
    y = lin.fwd(x, w, layout="ir_mul")
    # per output channel the variance over samples is the squared weight
    # column norm / fan-in: averaged over channels, 1 within sampling error
    assert abs(y.var(axis=0).mean() - 1.0) < 0.08


def test_identity_map():
    lin = linear.Linear("3x0e+2x1o+1x2e", "3x0e+2x1o+1x2e")
    w = np.concatenate([np.eye(m).reshape(-1) * np.sqrt(m) for m, _, _ in lin.inp])[None, :]
    x = np.random.default_rng(5).normal(size=(4, lin.dim_in))
    for lay in ("mul_ir", "ir_mul"):
        assert np.allclose(lin.fwd(x, w, layout=lay), x, atol=1e-13)


@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
def test_vjp_adjoint_identities(lay):
    lin = linear.Linear("4x0e+3x1o+2x1o", "2x0e+5x1o")
    rng = np.random.default_rng(6)
    x = rng.normal(size=(7, lin.dim_in))
    w = rng.normal(size=(1, lin.weight_numel))
    g = rng.normal(size=(7, lin.dim_out))
    dx, dw = lin.vjp(x, w, g, layout=lay)
    vx, vw = rng.normal(size=x.shape), rng.normal(size=w.shape)
    assert np.isclose(np.sum(g * lin.fwd(vx, w, layout=lay)), np.sum(dx * vx), rtol=1e-12)
    assert np.isclose(np.sum(g * lin.fwd(x, vw, layout=lay)), np.sum(dw * vw), rtol=1e-12)


def test_class_indexed_weights():
    """Per-sample rows: each sample uses its class's row; dw of a class sums
    its samples; an index out of range gives a zero output row, zero dx and
    no dw contribution."""
    lin = linear.Linear("3x0e+2x1o", "2x0e+2x1o")
    rng = np.random.default_rng(7)
    x = rng.normal(size=(9, lin.dim_in))
    w = rng.normal(size=(3, lin.weight_numel))
    idx = np.array([0, 2, 1, 1, 5, 0, 2, -1, 1])
    g = rng.normal(size=(9, lin.dim_out))
    y = lin.fwd(x, w, indices=idx)
    dx, dw = lin.vjp(x, w, g, indices=idx)
    for n in range(9):
        if 0 <= idx[n] < 3:
            assert np.allclose(y[n], lin.fwd(x[n:n + 1], w[idx[n]:idx[n] + 1])[0])
        else:
            assert np.count_nonzero(y[n]) == 0 and np.count_nonzero(dx[n]) == 0
    acc = np.zeros_like(w)
    for n in range(9):
        if 0 <= idx[n] < 3:
            _, d1 = lin.vjp(x[n:n + 1], w[idx[n]:idx[n] + 1], g[n:n + 1])
            acc[idx[n]] += d1[0]
    assert np.allclose(dw, acc, atol=1e-13)
