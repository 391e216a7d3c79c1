"""Real Wigner-D matrices, two independent ways (oracle side, test utility).

The pages check equivariance by rotating row-vector features as ``x @ D.T``
with the representation matrix of a rotation (cuequivariance-torch skill
document, "Linear: layout conversion and rotations").  Convention here:
D_l(R) is the matrix with  Y_l(R r) = D_l(R) Y_l(r)  for the real harmonics of
:mod:`oracle.sh`; then D_1(R) = P R P^T with P the row permutation
(x, y, z) -> (y, z, x).

* :func:`wigner_d_lstsq` solves that defining relation by least squares over
  many vectors (uses the harmonics);
* :func:`wigner_d_expm` exponentiates the real-basis angular-momentum
  generators built from the complex ladder operators (uses neither the
  harmonics nor the CG code);
the tests check the two against each other and the l = 1 closed form.
"""

import math

import numpy as np
from scipy.linalg import expm

from .cg import complex_to_real
from .sh import real_sh_l


def rotation_matrix(axis_angle):
    """3x3 rotation for an axis-angle vector (axis * angle), by Rodrigues'
    formula."""
    v = np.asarray(axis_angle, dtype=np.float64)
    th = np.linalg.norm(v)
    if th == 0:
        return np.eye(3)
    k = v / th
    K = np.array([[0, -k[2], k[1]], [k[2], 0, -k[0]], [-k[1], k[0], 0]])
    return np.eye(3) + math.sin(th) * K + (1 - math.cos(th)) * (K @ K)


def wigner_d_lstsq(l, R, n=64, seed=0):
    """Solve Y_l(R r) = D Y_l(r) for D over ``n`` random unit vectors."""
    rng = np.random.default_rng(seed)
    r = rng.normal(size=(n, 3))
    r /= np.linalg.norm(r, axis=1, keepdims=True)
    a = real_sh_l(l, r)             # rows Y(r)^T
    b = real_sh_l(l, r @ R.T)       # rows Y(R r)^T = Y(r)^T D^T
    dt, *_ = np.linalg.lstsq(a, b, rcond=None)
    return dt.T


def _generators_complex(l):
    """Complex |l m> matrices of J_x, J_y, J_z (m = -l..l, index m + l)."""
    d = 2 * l + 1
    jz = np.diag(np.arange(-l, l + 1)).astype(np.complex128)
    jp = np.zeros((d, d), dtype=np.complex128)
    for m in range(-l, l):
        jp[m + 1 + l, m + l] = math.sqrt(l * (l + 1) - m * (m + 1))
    jm = jp.conj().T
    return (jp + jm) / 2, (jp - jm) / (2j), jz


def real_generators(l):
    """Real antisymmetric generators G_a with D_l(exp(t [e_a]_x)) = expm(t G_a).

    With the rotation operator U(R) = exp(-i t n.J) acting on functions as
    (U f)(r) = f(R^-1 r), the harmonics obey Y(R r) = conj(U(R)) Y(r) in the
    |l m> basis, so the generator of D in the complex basis is i conj(J_a);
    in the real basis G_a = Q (i conj(J_a)) Q^dagger, which is real."""
    q = complex_to_real(l)
    out = []
    for j in _generators_complex(l):
        g = q @ (1j * j.conj()) @ q.conj().T
        assert np.abs(g.imag).max() < 1e-12
        out.append(g.real)
    return out


def wigner_d_expm(l, axis_angle):
    """D_l for the rotation by ``axis_angle`` (axis * angle) as
    expm(sum_a theta n_a G_a)."""
    g = real_generators(l)
    v = np.asarray(axis_angle, dtype=np.float64)
    return expm(v[0] * g[0] + v[1] * g[1] + v[2] * g[2])


def wigner_d_irreps(blocks, axis_angle, parity=1):
    """Block-diagonal representation matrix of an irreps list in ``mul_ir``
    order for the rotation ``axis_angle`` composed with inversion when
    ``parity == -1`` (block of parity p picks up p)."""
    mats = []
    for mul, l, p in blocks:
        d = wigner_d_expm(l, axis_angle) * (p if parity == -1 else 1)
        mats.extend([d] * mul)
    n = sum(m.shape[0] for m in mats)
    out = np.zeros((n, n))
    o = 0
    for m in mats:
        k = m.shape[0]
        out[o:o + k, o:o + k] = m
        o += k
    return out
