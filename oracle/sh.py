"""Real spherical harmonics, "component" normalisation (oracle side).

The pages use spherical harmonics as the second operand of the convolution
(cuequivariance-torch skill document, "Spherical harmonics and a NumPy
reference" and "Trainable message passing"; e3nn-course Lesson 12a,
section 21.5) with ``normalization="component"`` and say that
``normalize=True`` normalises the vectors first while ``normalize=False``
evaluates the raw polynomial.  The pages do not print the basis, so this is
the textbook real basis, index m = -l..l:

    m < 0 :  sqrt(2) N_l|m| P_l^|m|(cos t) sin(|m| phi)
    m = 0 :          N_l0   P_l(cos t)
    m > 0 :  sqrt(2) N_lm   P_l^m(cos t)  cos(m phi)

with P_l^m the associated Legendre function *without* the Condon-Shortley
phase and N_lm = sqrt((2l+1) (l-m)!/(l+m)!), i.e. the orthonormal harmonics
times sqrt(4 pi), so that sum_m Y_lm(r)^2 = 2l+1 on the unit sphere.  Then
l=1 is sqrt(3) (y, z, x).

For a unit vector (x, y, z), P_l^m(z) e^{i m phi} = (d^m P_l / dz^m)(z) (x + i y)^m,
which is how it is evaluated here (no angles, no pole singularity).
"""

import math

import numpy as np
from numpy.polynomial import legendre as npleg


def _legendre_deriv(l, m, z):
    """d^m P_l / dz^m evaluated at z (numpy Legendre series as a step)."""
    coef = np.zeros(l + 1)
    coef[l] = 1.0
    return npleg.legval(z, npleg.legder(coef, m)) if m > 0 else npleg.legval(z, coef)


def real_sh_l(l, vecs, normalize=True):
    """Real harmonics of degree l for vectors [..., 3] -> [..., 2l+1].

    normalize=True evaluates on the normalised vector; normalize=False
    evaluates the homogeneous polynomial |r|^l Y_l(r/|r|)."""
    v = np.asarray(vecs, dtype=np.float64)
    r = np.linalg.norm(v, axis=-1)
    u = v / r[..., None]
    x, y, z = u[..., 0], u[..., 1], u[..., 2]
    out = np.empty(v.shape[:-1] + (2 * l + 1,))
    for m in range(-l, l + 1):
        a = abs(m)
        n = math.sqrt((2 * l + 1) * math.factorial(l - a) / math.factorial(l + a))
        p = _legendre_deriv(l, a, z)
        if m == 0:
            out[..., l] = n * p
        else:
            cplx = (x + 1j * y) ** a
            trig = cplx.real if m > 0 else cplx.imag
            out[..., l + m] = math.sqrt(2.0) * n * p * trig
    if not normalize:
        out = out * (r ** l)[..., None]
    return out


def real_sh(ls, vecs, normalize=True):
    """Concatenation of :func:`real_sh_l` for each l in ``ls`` (the layout
    of an ``0e + 1o + 2e + ...`` operand with multiplicity one)."""
    return np.concatenate([real_sh_l(l, vecs, normalize) for l in ls], axis=-1)


def real_sh_vjp(ls, vecs, g, normalize=True):
    """Vector-Jacobian product of :func:`real_sh`: given g = dL/d(Y) with
    the columns of ``real_sh(ls, vecs)``, return dL/d(vecs) [..., 3].

    Without normalisation every column is a homogeneous polynomial of degree
    l in (x, y, z), so its derivative along an axis at t = 0 of
    Y(v + t e_a) is the derivative of a polynomial in t of degree l, which
    the five-point quotient (8 (f(h) - f(-h)) - (f(2h) - f(-2h))) / (12 h)
    gives exactly for l <= 4 (up to rounding).  With normalisation Y depends
    on u = v / |v| only, and the chain rule gives
    dY/dv = (I - u u^T) / |v| * grad P(u), P the polynomial of the
    unnormalised harmonics (its radial part drops out)."""
    if max(ls) > 4:
        raise ValueError("the exact difference quotient covers l <= 4")
    v = np.asarray(vecs, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    r = np.linalg.norm(v, axis=-1, keepdims=True)
    base = v / r if normalize else v
    h = 0.5 * np.maximum(np.abs(base).max(axis=-1, keepdims=True), 1e-3)
    grad = np.zeros(v.shape[:-1] + (3,))          # grad of sum_j g_j P_j at base
    for a in range(3):
        e = np.zeros(3)
        e[a] = 1.0
        f = lambda t: np.sum(g * real_sh(ls, base + t * e, normalize=False), axis=-1)
        grad[..., a] = (8 * (f(h[..., 0:1] * 1) - f(-h[..., 0:1] * 1)) - (f(2 * h[..., 0:1]) - f(-2 * h[..., 0:1]))) \
            / (12 * h[..., 0])
    if not normalize:
        return grad
    u = base
    radial = np.sum(u * grad, axis=-1, keepdims=True)
    return (grad - u * radial) / r
