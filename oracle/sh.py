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
