"""Clebsch-Gordan coupling tensors in the real basis (oracle side).

The pages give the role of the coefficients but not their values: the
``[ijk]`` factor of ``[ijk]*a[uv]*b[iu]*c[jv] -> D[kuv]`` is the
Clebsch-Gordan tensor, "known at compile time and mostly zero"
(e3nn-course Lesson 12a, sections 21.1 and 21.4), and "descriptor
coefficients include normalization factors" (cuequivariance-torch skill
document, "SegmentedPolynomial: gather and scatter").  This module is the
textbook construction, with the readings below.

1. Complex Condon-Shortley coefficients <l1 m1 l2 m2 | l3 m3> by Racah's
   closed formula, in exact rational arithmetic (one square root at the end).
2. Change of basis to the real harmonics of :mod:`oracle.sh`:
   real Y_m = sum_mu Q[m, mu] complex Y^mu with
       m < 0 : (i/sqrt2) (Y^m - (-1)^m Y^-m)
       m = 0 : Y^0
       m > 0 : (1/sqrt2) (Y^-m + (-1)^m Y^m)
   C_R[m1,m2,m3] = sum conj(Q1[m1,mu1]) conj(Q2[m2,mu2]) Q3[m3,mu3] CG[mu1,mu2,mu3];
   the result is real or purely imaginary; take that part.  This step runs
   in 40-digit arithmetic (mpmath) and rounds each entry once.
3. Scaling ("component" reading): sum_ij C_ijk C_ijk' = delta_kk', i.e.
   sqrt(2 l3 + 1) times the unit-Frobenius tensor, which is what the unitary
   change of basis of step 2 already gives.  The paths 0 x l -> l and
   l x 0 -> l are then exactly the identity.
4. Sign (the pages fix none): if l1+l2+l3 is even, coupling the harmonics
   of one unit vector with themselves gives a positive multiple of the
   harmonics of degree l3; if odd, the first non-zero entry in index order
   (m1, m2, m3 each from -l) is positive.
"""

import math
from fractions import Fraction
from functools import lru_cache

import mpmath
import numpy as np

from .sh import real_sh_l


def _f(n):
    return math.factorial(n)


def cg_complex_exact(l1, m1, l2, m2, l3, m3):
    """<l1 m1 l2 m2 | l3 m3> (Condon-Shortley) by Racah's formula, returned
    exactly as (sign, square) with the square a Fraction (0 if it vanishes)."""
    if m1 + m2 != m3 or not (abs(l1 - l2) <= l3 <= l1 + l2):
        return 0, Fraction(0)
    if abs(m1) > l1 or abs(m2) > l2 or abs(m3) > l3:
        return 0, Fraction(0)
    pre = Fraction((2 * l3 + 1) * _f(l3 + l1 - l2) * _f(l3 - l1 + l2) * _f(l1 + l2 - l3),
                   _f(l1 + l2 + l3 + 1))
    pre *= _f(l3 + m3) * _f(l3 - m3) * _f(l1 - m1) * _f(l1 + m1) * _f(l2 - m2) * _f(l2 + m2)
    s = Fraction(0)
    for k in range(0, l1 + l2 - l3 + 1):
        dens = (k, l1 + l2 - l3 - k, l1 - m1 - k, l2 + m2 - k, l3 - l2 + m1 + k, l3 - l1 - m2 + k)
        if min(dens) < 0:
            continue
        d = 1
        for t in dens:
            d *= _f(t)
        s += Fraction((-1) ** k, d)
    if s == 0:
        return 0, Fraction(0)
    return (1 if s > 0 else -1), s * s * pre


def cg_complex_entry(l1, m1, l2, m2, l3, m3):
    """<l1 m1 l2 m2 | l3 m3> as a float64."""
    sg, sq = cg_complex_exact(l1, m1, l2, m2, l3, m3)
    return sg * math.sqrt(float(sq)) if sg else 0.0


def cg_complex(l1, l2, l3):
    """Complex CG tensor [2l1+1, 2l2+1, 2l3+1], index m + l, float64."""
    c = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
    for m1 in range(-l1, l1 + 1):
        for m2 in range(-l2, l2 + 1):
            m3 = m1 + m2
            if abs(m3) <= l3:
                c[m1 + l1, m2 + l2, m3 + l3] = cg_complex_entry(l1, m1, l2, m2, l3, m3)
    return c


def _q_entry(m, mu):
    """Q_l[m, mu] of the complex-to-real change of basis (independent of l),
    as an mpmath complex; zero unless |mu| = |m|."""
    s = 1 / mpmath.sqrt(2)
    if m == 0:
        return mpmath.mpc(1) if mu == 0 else mpmath.mpc(0)
    if m < 0:
        if mu == m:
            return mpmath.mpc(0, s)
        if mu == -m:
            return mpmath.mpc(0, -s * (-1) ** m)
        return mpmath.mpc(0)
    if mu == -m:
        return mpmath.mpc(s)
    if mu == m:
        return mpmath.mpc(s * (-1) ** m)
    return mpmath.mpc(0)


def complex_to_real(l):
    """Q_l with real Y_m = sum_mu Q[m, mu] complex Y^mu (rows m, columns mu,
    both indexed m + l), complex128."""
    with mpmath.workdps(_DPS):
        q = np.zeros((2 * l + 1, 2 * l + 1), dtype=np.complex128)
        for m in range(-l, l + 1):
            for mu in (m, -m):
                q[m + l, mu + l] = complex(_q_entry(m, mu))
    return q


# working precision of the change of basis; every entry is rounded to
# float64 once, so exact values (the identity paths) come out exact
_DPS = 40

# a fixed generic unit vector for the even-parity sign rule
_SIGN_VEC = np.array([0.3, -0.5, 0.81])
_SIGN_VEC = _SIGN_VEC / np.linalg.norm(_SIGN_VEC)


@lru_cache(maxsize=None)
def _real_cg_cached(l1, l2, l3):
    shape = (2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1)
    if not (abs(l1 - l2) <= l3 <= l1 + l2):
        return np.zeros(shape)
    with mpmath.workdps(_DPS):
        re = np.zeros(shape, dtype=object)
        im = np.zeros(shape, dtype=object)
        for m1 in range(-l1, l1 + 1):
            for m2 in range(-l2, l2 + 1):
                for m3 in range(-l3, l3 + 1):
                    acc = mpmath.mpc(0)
                    # Q is non-zero only at mu = +-m, and CG needs mu3 = mu1 + mu2
                    for mu1 in sorted({m1, -m1}):
                        for mu2 in sorted({m2, -m2}):
                            mu3 = mu1 + mu2
                            if abs(mu3) != abs(m3):
                                continue
                            sg, sq = cg_complex_exact(l1, mu1, l2, mu2, l3, mu3)
                            if not sg:
                                continue
                            c = sg * mpmath.sqrt(mpmath.mpf(sq.numerator) / sq.denominator)
                            acc += (mpmath.conj(_q_entry(m1, mu1)) * mpmath.conj(_q_entry(m2, mu2))
                                    * _q_entry(m3, mu3) * c)
                    re[m1 + l1, m2 + l2, m3 + l3] = acc.real
                    im[m1 + l1, m2 + l2, m3 + l3] = acc.imag
        nre = max(abs(v) for v in re.ravel())
        nim = max(abs(v) for v in im.ravel())
        # the unitary change of basis keeps sum_ij C_ijk C_ijk' = delta_kk'
        # ("component" scaling) and leaves a real or purely imaginary tensor
        part = re if nre >= nim else im
        # entries below 1e-30 are cancellations of the 40-digit sums: exactly zero
        r = np.array([0.0 if abs(v) < 1e-30 else float(v) for v in part.ravel()]).reshape(shape)
    # sign rule
    if (l1 + l2 + l3) % 2 == 0:
        y1, y2, y3 = (real_sh_l(l, _SIGN_VEC) for l in (l1, l2, l3))
        s = np.einsum("ijk,i,j,k->", r, y1, y2, y3)
    else:
        flat = r.ravel()
        s = flat[np.nonzero(np.abs(flat) > 1e-9 * np.abs(flat).max())[0][0]]
    if s < 0:
        r = -r
    r.setflags(write=False)
    return r


def real_cg(l1, l2, l3):
    """Real coupling tensor C[i, j, k] (i, j, k = m + l) with the scaling and
    sign rule in the module docstring; zero if the triangle rule fails.
    This is the coefficient of one channelwise path l1 x l2 -> l3."""
    return _real_cg_cached(l1, l2, l3).copy()


def wigner_3j_m0(l1, l2, l3):
    """(l1 l2 l3; 0 0 0) by its textbook closed form (zero if l1+l2+l3 odd):
    (-1)^g sqrt((2g-2l1)!(2g-2l2)!(2g-2l3)!/(2g+1)!) g!/((g-l1)!(g-l2)!(g-l3)!),
    2g = l1+l2+l3.  Used only to pin the SH-coupling identity."""
    J = l1 + l2 + l3
    if J % 2 or not (abs(l1 - l2) <= l3 <= l1 + l2):
        return 0.0
    g = J // 2
    v = math.sqrt(Fraction(_f(2 * g - 2 * l1) * _f(2 * g - 2 * l2) * _f(2 * g - 2 * l3), _f(2 * g + 1)))
    v *= _f(g) / (_f(g - l1) * _f(g - l2) * _f(g - l3))
    return (-1) ** g * v
