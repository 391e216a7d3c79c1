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


def _abs_terms_poly(l, x, y, z, r2):
    """The polynomial of :func:`real_sh_l_abs` at (x, y, z) with r2 standing
    for x^2 + y^2 + z^2 (or 1 on the sphere): every coefficient replaced by
    its absolute value, evaluated without taking absolute values of the
    variables (so it can be differentiated)."""
    out = np.empty(np.shape(x) + (2 * l + 1,))
    for m in range(-l, l + 1):
        a = abs(m)
        n = math.sqrt((2 * l + 1) * math.factorial(l - a) / math.factorial(l + a))
        coef = np.zeros(l + 1)
        coef[l] = 1.0
        pw = npleg.leg2poly(npleg.legder(coef, a) if a > 0 else coef)   # power series of P_l^(a)
        # l - a - k is even wherever c_k != 0 (P_l^(a) has the parity of l - a)
        zpart = sum(abs(c) * z ** k * r2 ** ((l - a - k) // 2) for k, c in enumerate(pw) if c != 0)
        parity = 0 if m >= 0 else 1                                       # Re: even j, Im: odd j
        xy = sum(math.comb(a, j) * x ** (a - j) * y ** j for j in range(parity, a + 1, 2)) if a else 1.0
        out[..., l + m] = (math.sqrt(2.0) if m != 0 else 1.0) * n * zpart * xy
    return out


def real_sh_l_abs(l, vecs, normalize=True):
    """Sum of the absolute values of the terms of :func:`real_sh_l`, the
    forward-error scale of the parity gate.

    Each harmonic is written as N P_l^(m)(z) times Re or Im of (x + i y)^m;
    expanding P_l^(m) as a power series in z and (x + i y)^m by the binomial
    theorem gives one monomial x^(m-j) y^j z^k per pair (j, k), so the sum of
    the absolute terms is N (sum_k |c_k| |z|^k) (sum_j binom(m, j) |x|^(m-j) |y|^j)
    over the j of the real (even) or imaginary (odd) part.  Without
    normalisation the homogeneous form carries r^(l-m-k) beside each z^k."""
    v = np.asarray(vecs, dtype=np.float64)
    r = np.linalg.norm(v, axis=-1)
    u = np.abs(v if not normalize else v / r[..., None])
    r2 = r * r if not normalize else np.ones_like(r)
    return _abs_terms_poly(l, u[..., 0], u[..., 1], u[..., 2], r2)


def real_sh_abs(ls, vecs, normalize=True):
    """Concatenation of :func:`real_sh_l_abs` for each l in ``ls``."""
    return np.concatenate([real_sh_l_abs(l, vecs, normalize) for l in ls], axis=-1)


def real_sh(ls, vecs, normalize=True):
    """Concatenation of :func:`real_sh_l` for each l in ``ls`` (the layout
    of an ``0e + 1o + 2e + ...`` operand with multiplicity one)."""
    return np.concatenate([real_sh_l(l, vecs, normalize) for l in ls], axis=-1)


def real_sh_vjp(ls, vecs, g, normalize=True):
    """Vector-Jacobian product of :func:`real_sh`: given g = dL/d(Y) with
    the columns of ``real_sh(ls, vecs)``, return dL/d(vecs) [..., 3].

    Without normalisation every column is a homogeneous polynomial of degree
    l in (x, y, z), so along an axis t -> Y(v + t e_a) is a polynomial in t of
    degree l, whose derivative at t = 0 the seven-point central quotient
    (45 (f(h) - f(-h)) - 9 (f(2h) - f(-2h)) + (f(3h) - f(-3h))) / (60 h)
    gives exactly for degree <= 6 (its error term is the seventh derivative),
    up to rounding.  With normalisation Y depends on u = v / |v| only, and the
    chain rule gives dY/dv = (I - u u^T) / |v| * grad P(u), P the polynomial
    of the unnormalised harmonics (its radial part drops out)."""
    if max(ls) > 6:
        raise ValueError("the exact seven-point quotient covers l <= 6")
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
        d1, d2, d3 = (f(k * h) - f(-k * h) for k in (1, 2, 3))
        grad[..., a] = (45 * d1 - 9 * d2 + d3) / (60 * h[..., 0])
    if not normalize:
        return grad
    u = base
    radial = np.sum(u * grad, axis=-1, keepdims=True)
    return (grad - u * radial) / r


def real_sh_vjp_abs(ls, vecs, g, normalize=True):
    """Forward-error scale of :func:`real_sh_vjp`: the same product with |g|
    and the gradient of the absolute-term polynomial of
    :func:`real_sh_l_abs` at (|x|, |y|, |z|) (each monomial of dY/dv_a
    enters with its absolute value), then, with normalisation, the sums of
    absolute terms of the tangential projection (|grad| + |u| (|u| . |grad|)) / |v|.
    Same seven-point quotient as :func:`real_sh_vjp` (exact, degree <= 6)."""
    if max(ls) > 6:
        raise ValueError("the exact seven-point quotient covers l <= 6")
    v = np.asarray(vecs, dtype=np.float64)
    g = np.abs(np.asarray(g, dtype=np.float64))
    r = np.linalg.norm(v, axis=-1, keepdims=True)
    base = np.abs(v / r if normalize else v)
    h = 0.5 * np.maximum(base.max(axis=-1, keepdims=True), 1e-3)
    grad = np.zeros(v.shape[:-1] + (3,))
    for a in range(3):
        e = np.zeros(3)
        e[a] = 1.0

        def f(t):
            p = base + t * e
            r2 = np.sum(p * p, axis=-1)
            return np.sum(g * np.concatenate([_abs_terms_poly(l, p[..., 0], p[..., 1], p[..., 2], r2)
                                               for l in ls], axis=-1), axis=-1)
        d1, d2, d3 = (f(k * h) - f(-k * h) for k in (1, 2, 3))
        grad[..., a] = (45 * d1 - 9 * d2 + d3) / (60 * h[..., 0])
    if not normalize:
        return grad
    radial = np.sum(base * grad, axis=-1, keepdims=True)
    return (grad + base * radial) / r
