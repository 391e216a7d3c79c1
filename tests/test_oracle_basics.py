"""Pins of the oracle's irreps, layouts, harmonics, CG and Wigner-D against
values the pages print, textbook closed forms, a library routine (sympy) and
mathematical identities.  CPU only."""

import json
import math
import os

import numpy as np
import pytest

from oracle import cg, irreps, layout, sh, wigner
import workloads


def _rot(seed):
    rng = np.random.default_rng(seed)
    aa = rng.normal(size=3)
    return aa, wigner.rotation_matrix(aa)


# ---------------------------------------------------------------- irreps, layout

def test_irreps_dim_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "irreps_dims.json")))
    for c in g["cases"]:
        b = irreps.parse(c["irreps"])
        assert irreps.dim(b) == c["dim"]
        assert irreps.to_str(b) == c["str"]


def test_irreps_parse_forms():
    assert irreps.parse("0e + 1o") == [(1, 0, 1), (1, 1, -1)]
    assert irreps.parse("3x2e+1x3o") == [(3, 2, 1), (1, 3, -1)]
    assert irreps.parse("") == []
    with pytest.raises(ValueError):
        irreps.parse("32x1q")


def test_layout_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "layout_2x1o.json")))
    blocks = irreps.parse(g["irreps"])
    x = np.array(g["flat"], dtype=np.float64)
    assert np.array_equal(x.reshape(g["mul_ir_shape"]), np.array(g["mul_ir"]))
    conv = layout.transpose(x, blocks, "mul_ir", "ir_mul")
    assert np.array_equal(conv.reshape(g["ir_mul_shape"]), np.array(g["ir_mul"]))
    # split_blocks gives the (2l+1, mul) view whatever the layout
    (b_mul,) = layout.split_blocks(x, blocks, "mul_ir")
    (b_ir,) = layout.split_blocks(conv, blocks, "ir_mul")
    assert np.array_equal(b_mul, np.array(g["ir_mul"]))
    assert np.array_equal(b_ir, np.array(g["ir_mul"]))


def test_layout_roundtrip_blockwise():
    blocks = irreps.parse("3x0e+2x1o+4x2e")
    x = np.arange(irreps.dim(blocks), dtype=np.float64)
    y = layout.transpose(x, blocks, "mul_ir", "ir_mul")
    assert np.array_equal(layout.transpose(y, blocks, "ir_mul", "mul_ir"), x)
    # per block, not a whole-vector reshape: the 0e block is unchanged
    assert np.array_equal(y[:3], x[:3])


# ---------------------------------------------------------------- harmonics

def test_sh_closed_forms():
    rng = np.random.default_rng(0)
    v = rng.normal(size=(50, 3))
    u = v / np.linalg.norm(v, axis=1, keepdims=True)
    x, y, z = u.T
    assert np.allclose(sh.real_sh_l(0, v), 1.0, atol=0, rtol=1e-15)
    assert np.allclose(sh.real_sh_l(1, v), math.sqrt(3) * np.stack([y, z, x], -1), atol=1e-14)
    s15 = math.sqrt(15)
    y2 = np.stack([s15 * x * y, s15 * y * z, math.sqrt(5) / 2 * (3 * z ** 2 - 1),
                   s15 * x * z, s15 / 2 * (x ** 2 - y ** 2)], -1)
    assert np.allclose(sh.real_sh_l(2, v), y2, atol=1e-14)


@pytest.mark.parametrize("l", range(7))
def test_sh_component_norm(l):
    rng = np.random.default_rng(l)
    y = sh.real_sh_l(l, rng.normal(size=(100, 3)))
    assert np.allclose((y ** 2).sum(-1), 2 * l + 1, rtol=1e-12)


@pytest.mark.parametrize("l", range(6))
def test_sh_orthogonality_quadrature(l):
    # component normalisation: the mean over the sphere of Y_lm Y_lm' is
    # delta_mm' (Gauss-Legendre in z times a uniform grid in phi is exact here)
    from numpy.polynomial.legendre import leggauss
    zs, wz = leggauss(20)
    phis = np.linspace(0, 2 * np.pi, 40, endpoint=False)
    Z, P = np.meshgrid(zs, phis, indexing="ij")
    s = np.sqrt(1 - Z ** 2)
    v = np.stack([s * np.cos(P), s * np.sin(P), Z], -1).reshape(-1, 3)
    wts = (wz[:, None] * np.ones_like(P)).ravel() * (2 * np.pi / 40) / (4 * np.pi)
    y = sh.real_sh_l(l, v)
    g = (y * wts[:, None]).T @ y
    assert np.allclose(g, np.eye(2 * l + 1), atol=1e-12)


def test_sh_unnormalized_is_homogeneous():
    rng = np.random.default_rng(1)
    v = rng.normal(size=(10, 3))
    for l in range(4):
        a = sh.real_sh_l(l, 2.5 * v, normalize=False)
        b = sh.real_sh_l(l, v, normalize=False) * 2.5 ** l
        assert np.allclose(a, b, rtol=1e-12)


def test_workload_harmonics_match_oracle():
    rng = np.random.default_rng(3)
    v = rng.normal(size=(200, 3))
    a = workloads.edge_harmonics(v, (0, 1, 2, 3))
    b = sh.real_sh([0, 1, 2, 3], v)
    assert np.allclose(a, b, atol=1e-13)


# ---------------------------------------------------------------- Wigner-D

@pytest.mark.parametrize("l", range(7))
def test_wigner_two_constructions_agree(l):
    aa, R = _rot(10 + l)
    a = wigner.wigner_d_lstsq(l, R)
    b = wigner.wigner_d_expm(l, aa)
    assert np.allclose(a, b, atol=1e-11)
    assert np.allclose(b @ b.T, np.eye(2 * l + 1), atol=1e-12)


def test_wigner_l1_closed_form():
    aa, R = _rot(3)
    P = np.array([[0, 1, 0], [0, 0, 1], [1, 0, 0]], dtype=np.float64)
    assert np.allclose(wigner.wigner_d_expm(1, aa), P @ R @ P.T, atol=1e-13)


def test_wigner_homomorphism():
    a1, R1 = _rot(4)
    a2, R2 = _rot(5)
    for l in range(4):
        d12 = wigner.wigner_d_lstsq(l, R1 @ R2)
        assert np.allclose(d12, wigner.wigner_d_expm(l, a1) @ wigner.wigner_d_expm(l, a2), atol=1e-11)


@pytest.mark.parametrize("l", range(5))
def test_sh_equivariance(l):
    aa, R = _rot(20 + l)
    rng = np.random.default_rng(l)
    v = rng.normal(size=(30, 3))
    d = wigner.wigner_d_expm(l, aa)
    assert np.allclose(sh.real_sh_l(l, v @ R.T), sh.real_sh_l(l, v) @ d.T, atol=1e-12)


# ---------------------------------------------------------------- CG

def test_complex_cg_matches_sympy():
    from sympy import S
    from sympy.physics.wigner import clebsch_gordan
    worst = 0.0
    for l1 in range(5):
        for l2 in range(5):
            for l3 in range(abs(l1 - l2), l1 + l2 + 1):
                c = cg.cg_complex(l1, l2, l3)
                for m1 in range(-l1, l1 + 1):
                    for m2 in range(-l2, l2 + 1):
                        m3 = m1 + m2
                        if abs(m3) > l3:
                            continue
                        ref = float(clebsch_gordan(S(l1), S(l2), S(l3), S(m1), S(m2), S(m3)))
                        worst = max(worst, abs(ref - c[m1 + l1, m2 + l2, m3 + l3]))
    assert worst < 1e-15


def _triples(lmax):
    """Every coupling (l1, l2, l3) with all three at most lmax: at lmax = 6,
    every one the library's descriptors can hold."""
    for l1 in range(lmax + 1):
        for l2 in range(lmax + 1):
            for l3 in range(abs(l1 - l2), min(l1 + l2, lmax) + 1):
                yield l1, l2, l3


@pytest.mark.parametrize("l1,l2,l3", list(_triples(6)))
def test_real_cg_orthonormal_and_equivariant(l1, l2, l3):
    c = cg.real_cg(l1, l2, l3)
    assert np.allclose(np.einsum("ijk,ijl->kl", c, c), np.eye(2 * l3 + 1), atol=1e-14)
    aa, R = _rot(100 + 16 * l1 + 4 * l2 + l3)
    d1, d2, d3 = (wigner.wigner_d_expm(l, aa) for l in (l1, l2, l3))
    rng = np.random.default_rng(l1 + 7 * l2 + 49 * l3)
    a, b = rng.normal(size=2 * l1 + 1), rng.normal(size=2 * l2 + 1)
    lhs = np.einsum("ijk,i,j->k", c, d1 @ a, d2 @ b)
    rhs = d3 @ np.einsum("ijk,i,j->k", c, a, b)
    assert np.allclose(lhs, rhs, atol=1e-13)


def test_real_cg_identity_paths_exact():
    for l in range(7):
        e = np.eye(2 * l + 1)
        assert np.array_equal(cg.real_cg(0, l, l)[0], e)
        assert np.array_equal(cg.real_cg(l, 0, l)[:, 0, :], e)


def test_real_cg_closed_forms_l1():
    # 1 x 1 -> 0: delta / sqrt(3);  1 x 1 -> 1: Levi-Civita in the (y, z, x)
    # component order, / sqrt(2) (first non-zero entry positive)
    assert np.allclose(cg.real_cg(1, 1, 0)[:, :, 0], np.eye(3) / math.sqrt(3), atol=1e-16)
    eps = np.zeros((3, 3, 3))
    for (i, j, k), s in {(0, 1, 2): 1, (1, 2, 0): 1, (2, 0, 1): 1,
                         (0, 2, 1): -1, (2, 1, 0): -1, (1, 0, 2): -1}.items():
        eps[i, j, k] = s
    assert np.allclose(cg.real_cg(1, 1, 1), eps / math.sqrt(2), atol=1e-16)


@pytest.mark.parametrize("l1,l2,l3", [t for t in _triples(6) if sum(t) % 2 == 0])
def test_sh_coupling_identity(l1, l2, l3):
    # Gaunt: with orthonormal harmonics, sum CG Y1 Y2 = sqrt((2l1+1)(2l2+1)/(4 pi (2l3+1)))
    # <l1 0 l2 0|l3 0> Y3, and <l1 0 l2 0|l3 0> = +-sqrt(2l3+1) (l1 l2 l3; 0 0 0).  With
    # component-normalised harmonics (sqrt(4 pi) larger) and the unitary
    # change to the real basis this is sqrt((2l1+1)(2l2+1)) |3j| Y3, positive
    # by the sign rule.
    rng = np.random.default_rng(sum((l1, 3 * l2, 9 * l3)))
    v = rng.normal(size=(20, 3))
    c = cg.real_cg(l1, l2, l3)
    y1, y2, y3 = (sh.real_sh_l(l, v) for l in (l1, l2, l3))
    lhs = np.einsum("ijk,ei,ej->ek", c, y1, y2)
    const = math.sqrt((2 * l1 + 1) * (2 * l2 + 1)) * abs(cg.wigner_3j_m0(l1, l2, l3))
    assert const > 0
    assert np.allclose(lhs, const * y3, atol=1e-12)


def test_real_cg_nonzero_counts():
    # non-zero counts of the real coupling tensors (cross-check of sparsity)
    expect = {(0, 0, 0): 1, (1, 1, 0): 3, (1, 1, 1): 6, (1, 1, 2): 11, (1, 2, 1): 11,
              (1, 2, 2): 16, (2, 1, 2): 16, (2, 2, 0): 5, (2, 2, 1): 16, (2, 2, 2): 25,
              (1, 3, 2): 21, (2, 3, 1): 21, (2, 3, 2): 28}
    for k, n in expect.items():
        assert np.count_nonzero(cg.real_cg(*k)) == n, k


def test_real_cg_sign_rule():
    for l1, l2, l3 in _triples(6):
        c = cg.real_cg(l1, l2, l3)
        if (l1 + l2 + l3) % 2 == 0:
            assert c[l1, l2, l3] > 0            # the m = 0 entry
        else:
            flat = c.ravel()
            assert flat[np.nonzero(flat)[0][0]] > 0
