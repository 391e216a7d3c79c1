"""Pins of the oracle's vector-Jacobian product of the real spherical
harmonics: closed forms for l = 1 and l = 2 written out by hand, Euler's
identity for homogeneous polynomials, the tangency and a central difference
of the normalised harmonics, and rotation covariance.  CPU only."""

import numpy as np
import pytest

from oracle import sh, wigner


def test_l1_closed_form():
    # Y_1 = sqrt(3) (y, z, x) without normalisation
    rng = np.random.default_rng(0)
    v = rng.normal(size=(6, 3))
    g = rng.normal(size=(6, 3))
    d = sh.real_sh_vjp([1], v, g, normalize=False)
    ref = np.sqrt(3) * np.stack([g[:, 2], g[:, 0], g[:, 1]], axis=1)
    assert np.allclose(d, ref, atol=1e-13)


def test_l2_closed_form():
    # without normalisation: Y_2 = (sqrt15 xy, sqrt15 yz, sqrt5/2 (3z^2 - r^2),
    # sqrt15 xz, sqrt15/2 (x^2 - y^2)); gradients by hand
    rng = np.random.default_rng(1)
    v = rng.normal(size=(6, 3))
    g = rng.normal(size=(6, 5))
    x, y, z = v.T
    s15, s5 = np.sqrt(15), np.sqrt(5)
    J = np.zeros((6, 5, 3))
    J[:, 0] = np.stack([s15 * y, s15 * x, 0 * x], 1)
    J[:, 1] = np.stack([0 * x, s15 * z, s15 * y], 1)
    J[:, 2] = np.stack([-s5 * x, -s5 * y, 2 * s5 * z], 1)
    J[:, 3] = np.stack([s15 * z, 0 * x, s15 * x], 1)
    J[:, 4] = np.stack([s15 * x, -s15 * y, 0 * x], 1)
    ref = np.einsum("nj,nja->na", g, J)
    assert np.allclose(sh.real_sh_vjp([2], v, g, normalize=False), ref, atol=1e-12)


@pytest.mark.parametrize("l", [1, 2, 3, 4, 5, 6])
def test_euler_homogeneity(l):
    rng = np.random.default_rng(2 + l)
    v = rng.normal(size=(8, 3))
    g = rng.normal(size=(8, 2 * l + 1))
    d = sh.real_sh_vjp([l], v, g, normalize=False)
    y = sh.real_sh([l], v, normalize=False)
    assert np.allclose(np.sum(d * v, axis=1), l * np.sum(g * y, axis=1), rtol=1e-11, atol=1e-11)


def test_normalised_tangent_and_central_difference():
    rng = np.random.default_rng(7)
    v = rng.normal(size=(5, 3))
    ls = [0, 1, 2, 3, 4, 5, 6]
    g = rng.normal(size=(5, 49))
    d = sh.real_sh_vjp(ls, v, g, normalize=True)
    assert np.allclose(np.sum(d * v, axis=1), 0, atol=1e-12)
    eps = 1e-6
    fd = np.zeros_like(v)
    for a in range(3):
        e = np.zeros(3)
        e[a] = eps
        fd[:, a] = (np.sum(g * sh.real_sh(ls, v + e), 1) - np.sum(g * sh.real_sh(ls, v - e), 1)) / (2 * eps)
    assert np.allclose(d, fd, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("normalize", [False, True])
def test_rotation_covariance(normalize):
    """Y(R v) = D(R) Y(v), so the VJP at R v with D g is R times the VJP at v."""
    rng = np.random.default_rng(9)
    ls = [0, 1, 2, 3, 4, 5, 6]
    v = rng.normal(size=(4, 3))
    g = rng.normal(size=(4, 49))
    aa = np.array([0.3, -0.8, 0.5])
    R = wigner.rotation_matrix(aa)
    blocks = [(1, l, (-1) ** l) for l in ls]
    D = wigner.wigner_d_irreps(blocks, aa)
    lhs = sh.real_sh_vjp(ls, v @ R.T, g @ D.T, normalize=normalize)
    rhs = sh.real_sh_vjp(ls, v, g, normalize=normalize) @ R.T
    assert np.allclose(lhs, rhs, atol=1e-11)


@pytest.mark.parametrize("l", [3, 4, 5, 6])
def test_sectoral_closed_form(l):
    """m = +-l without normalisation: Y = sqrt2 N (2l-1)!! Re / Im (x + i y)^l
    with N = sqrt((2l+1) / (2l)!), so the gradient is sqrt2 N (2l-1)!! l times
    (Re, -Im, 0) (x + i y)^(l-1) for m = l and (Im, Re, 0) (x + i y)^(l-1) for
    m = -l; written out here from the definition, not from the oracle's
    difference quotient."""
    import math
    rng = np.random.default_rng(40 + l)
    v = rng.normal(size=(7, 3))
    c = (v[:, 0] + 1j * v[:, 1]) ** (l - 1)
    k = math.sqrt(2.0) * math.sqrt((2 * l + 1) / math.factorial(2 * l)) * math.prod(range(1, 2 * l, 2)) * l
    for m, ref in ((l, np.stack([c.real, -c.imag, 0 * c.real], 1)), (-l, np.stack([c.imag, c.real, 0 * c.real], 1))):
        g = np.zeros((7, 2 * l + 1))
        g[:, l + m] = 1.0
        assert np.allclose(sh.real_sh_vjp([l], v, g, normalize=False), k * ref, rtol=1e-12, atol=1e-12)


def test_seven_point_rejects_degree_seven():
    with pytest.raises(ValueError):
        sh.real_sh_vjp([7], np.ones((1, 3)), np.ones((1, 15)))


# ------------------------------------------------ absolute-sum scale of Y

def test_abs_scale_closed_forms_l1_l2():
    """l = 1: sqrt3 (|y|, |z|, |x|).  l = 2 on the sphere, from the monomials
    sqrt15 xy, sqrt15 yz, (sqrt5 / 2)(3 z^2 - 1), sqrt15 xz, (sqrt15 / 2)(x^2 - y^2):
    the middle one becomes (sqrt5 / 2)(3 z^2 + 1) and the last (sqrt15 / 2)(x^2 + y^2)."""
    rng = np.random.default_rng(11)
    v = rng.normal(size=(9, 3))
    u = v / np.linalg.norm(v, axis=1, keepdims=True)
    x, y, z = np.abs(u).T
    assert np.allclose(sh.real_sh_l_abs(1, v), np.sqrt(3) * np.stack([y, z, x], 1), rtol=1e-14)
    s15, s5 = np.sqrt(15), np.sqrt(5)
    ref = np.stack([s15 * x * y, s15 * y * z, s5 / 2 * (3 * z * z + 1), s15 * x * z, s15 / 2 * (x * x + y * y)], 1)
    assert np.allclose(sh.real_sh_l_abs(2, v), ref, rtol=1e-14)
    # without normalisation the constant term of the middle one carries r^2
    r2 = np.sum(v * v, 1)
    xa, ya, za = np.abs(v).T
    assert np.allclose(sh.real_sh_l_abs(2, v, normalize=False)[:, 2], s5 / 2 * (3 * za * za + r2), rtol=1e-14)


@pytest.mark.parametrize("l", range(7))
def test_abs_scale_bounds_and_equality(l):
    """|Y| <= A everywhere; at the pole only the powers of z survive, so the
    m = 0 scale is sqrt(2l+1) times the sum of the absolute power-series
    coefficients of P_l, while Y itself is sqrt(2l+1) P_l(1) = sqrt(2l+1)."""
    rng = np.random.default_rng(60 + l)
    v = rng.normal(size=(50, 3))
    for nz in (True, False):
        y = sh.real_sh_l(l, v, nz)
        a = sh.real_sh_l_abs(l, v, nz)
        assert np.all(a >= np.abs(y) * (1 - 1e-13))
    pole = np.array([[0.0, 0.0, 2.0]])
    assert np.allclose(sh.real_sh_l_abs(l, pole)[0, l], np.sqrt(2 * l + 1) * sum(
        abs(c) for c in np.polynomial.legendre.leg2poly(np.eye(l + 1)[l])), rtol=1e-13)
    assert np.isclose(abs(sh.real_sh_l(l, pole)[0, l]), np.sqrt(2 * l + 1), rtol=1e-13)


def test_vjp_abs_scale_l1_closed_form_and_bound():
    """l = 1 without normalisation: Y = sqrt3 (y, z, x), so the scale of the
    gradient is sqrt3 (|g_2|, |g_0|, |g_1|) whatever v; with normalisation
    and all degrees up to 6 the scale bounds the gradient."""
    rng = np.random.default_rng(12)
    v = rng.normal(size=(6, 3))
    g = rng.normal(size=(6, 3))
    ref = np.sqrt(3) * np.abs(np.stack([g[:, 2], g[:, 0], g[:, 1]], 1))
    assert np.allclose(sh.real_sh_vjp_abs([1], v, g, normalize=False), ref, rtol=1e-12)
    ls = list(range(7))
    g = rng.normal(size=(6, 49))
    for nz in (True, False):
        assert np.all(sh.real_sh_vjp_abs(ls, v, g, nz) >= np.abs(sh.real_sh_vjp(ls, v, g, nz)))
