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


@pytest.mark.parametrize("l", [1, 2, 3, 4])
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
    ls = [0, 1, 2, 3]
    g = rng.normal(size=(5, 16))
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
    ls = [0, 1, 2, 3]
    v = rng.normal(size=(4, 3))
    g = rng.normal(size=(4, 16))
    aa = np.array([0.3, -0.8, 0.5])
    R = wigner.rotation_matrix(aa)
    blocks = [(1, l, (-1) ** l) for l in ls]
    D = wigner.wigner_d_irreps(blocks, aa)
    lhs = sh.real_sh_vjp(ls, v @ R.T, g @ D.T, normalize=normalize)
    rhs = sh.real_sh_vjp(ls, v, g, normalize=normalize) @ R.T
    assert np.allclose(lhs, rhs, atol=1e-11)
