"""Pins of the symmetric-contraction oracle: the page's descriptor counts,
coupling multiplicities by the character formula, symmetry and equivariance
of every basis tensor, closed forms at degrees 1 and 2, a per-channel brute
force, and equivariance of the output.  CPU only."""

import itertools
import json
import math
import os

import numpy as np
import pytest

from oracle import irreps, layout, symcon, wigner


def test_page_symcon_descriptor(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "symcon_descriptor.json")))
    sc = symcon.SymmetricContraction(g["irreps_in"], g["irreps_out"], g["degrees"])
    # weights 32x0e+64x0e+64x0e: K = 1, 2, 2 couplings of width 32
    wts = [int(t.split("x")[0]) for t in g["weights_irreps"].split("+")]
    assert [sc.counts()[(nu, 0)] * g["mul"] for nu in (1, 2, 3)] == wts
    assert sc.weight_numel == sum(wts)
    for nu, n in g["num_paths"].items():
        assert sc.num_paths(int(nu)) == n


def _chi(l, theta):
    """Character of the SO(3) irrep l at rotation angle theta."""
    return np.sum([np.cos(m * theta) for m in range(-l, l + 1)], axis=0)


def _multiplicity_by_characters(blocks, nu, L, pL):
    """Multiplicity of (L, pL) in Sym^nu of the per-channel representation,
    by integrating characters over O(3) = SO(3) x {1, inversion} (Weyl
    measure (1 - cos t)/pi on [0, pi]); exact for these trig polynomials on
    a fine Gauss-Legendre grid."""
    t, wt = np.polynomial.legendre.leggauss(200)
    th = (t + 1) * np.pi / 2
    wt = wt * np.pi / 2 * (1 - np.cos(th)) / np.pi

    def chi_v(k, improper):
        # character of the whole per-channel representation at g^k
        s = 0
        for _, l, p in blocks:
            s = s + _chi(l, k * th) * (p ** k if improper else 1)
        return s

    tot = 0.0
    for improper in (False, True):
        c1, c2, c3 = chi_v(1, improper), chi_v(2, improper), chi_v(3, improper)
        sym = {1: c1, 2: (c1 ** 2 + c2) / 2, 3: (c1 ** 3 + 3 * c2 * c1 + 2 * c3) / 6}[nu]
        chi_l = _chi(L, th) * (pL if improper else 1)
        tot += 0.5 * np.sum(wt * sym * chi_l)
    return int(round(tot))


@pytest.mark.parametrize("ins,outs", [
    ("0e+1o+2e+3o", "0e+1o"),
    ("0e+1o", "0e"),
    ("0e+1o+2e", "0e+1o+2e"),
    ("0e+1e+2e", "0e+1e"),
])
def test_counts_match_character_formula(ins, outs):
    mul = 4
    tag = lambda s: "+".join(f"{mul}x{t}" for t in s.split("+"))
    sc = symcon.SymmetricContraction(tag(ins), tag(outs))
    for (nu, ob), k in sc.counts().items():
        _, L, pL = sc.out[ob]
        assert k == _multiplicity_by_characters(sc.inp, nu, L, pL), (nu, L, pL)


def test_workload5_counts():
    sc = symcon.SymmetricContraction("128x0e+128x1o+128x2e+128x3o", "128x0e+128x1o")
    assert [sc.counts()[(nu, ob)] for nu in (1, 2, 3) for ob in (0, 1)] == [1, 1, 4, 3, 8, 12]
    assert sc.weight_numel == 29 * 128


def test_basis_symmetric_and_equivariant():
    blocks = irreps.parse("1x0e+1x1o+1x2e+1x3o")
    aa = np.array([0.4, -1.1, 0.3])
    dv = wigner.wigner_d_irreps(blocks, aa)
    di = wigner.wigner_d_irreps(blocks, np.zeros(3), parity=-1)
    for nu in (1, 2, 3):
        for L, pL in ((0, 1), (1, -1)):
            us = symcon.coupling_basis(blocks, nu, L, pL)
            dl = wigner.wigner_d_expm(L, aa)
            for u in us:
                for perm in itertools.permutations(range(nu)):
                    assert np.allclose(np.transpose(u, perm + (nu,)), u, atol=1e-14)
                # output components orthonormal
                flat = u.reshape(-1, 2 * L + 1)
                assert np.allclose(flat.T @ flat, np.eye(2 * L + 1), atol=1e-12)
                # equivariance: contract every input slot with D
                r = u
                for _ in range(nu):
                    r = np.tensordot(dv, r, axes=([0], [0]))
                    r = np.moveaxis(r, 0, nu - 1)
                assert np.allclose(r, u @ dl.T, atol=1e-11)
                ri = u
                for _ in range(nu):
                    ri = np.tensordot(di, ri, axes=([0], [0]))
                    ri = np.moveaxis(ri, 0, nu - 1)
                assert np.allclose(ri, u * pL, atol=1e-12)


def test_degree1_and_degree2_closed_forms():
    mul = 3
    sc = symcon.SymmetricContraction(f"{mul}x0e+{mul}x1o+{mul}x2e", f"{mul}x0e", degrees=(1, 2))
    rng = np.random.default_rng(4)
    x = rng.normal(size=(5, sc.dim_in))
    sp = rng.integers(0, 2, 5)
    w = rng.normal(size=(2, sc.weight_numel))
    got = sc.eval(x, sp, w, layout="ir_mul")
    comps = np.concatenate(layout.split_blocks(x, sc.inp, "ir_mul"), axis=1)   # [A, 9, mul]
    # degree 1: identity on the 0e block; degree 2: x0^2, |x1|^2/sqrt3, |x2|^2/sqrt5
    q = [comps[:, 0], comps[:, 0] ** 2, (comps[:, 1:4] ** 2).sum(1) / math.sqrt(3),
         (comps[:, 4:9] ** 2).sum(1) / math.sqrt(5)]
    assert [k for _, _, k in sc.segments] == [0, 0, 1, 2]
    ref = sum(w[sp][:, s * mul:(s + 1) * mul] * q[s] for s in range(4))
    assert np.allclose(got[:, :mul], ref, atol=1e-13)


@pytest.mark.parametrize("lay", ["ir_mul", "mul_ir"])
def test_brute_force_per_channel(lay):
    sc = symcon.SymmetricContraction("2x0e+2x1o+2x2e", "2x0e+2x1o")
    rng = np.random.default_rng(9)
    x = rng.normal(size=(3, sc.dim_in))
    sp = np.array([1, 0, 1])
    w = rng.normal(size=(2, sc.weight_numel))
    got = layout.transpose(sc.eval(x, sp, w, layout=lay), sc.out, lay, "ir_mul")
    comps = np.concatenate(layout.split_blocks(x, sc.inp, lay), axis=1)
    ref = np.zeros_like(got)
    ooff = np.cumsum([0] + [m * (2 * l + 1) for m, l, _ in sc.out])
    for a in range(3):
        for u in range(sc.mul):
            v = comps[a, :, u]
            for s_idx, (nu, ob, k) in enumerate(sc.segments):
                U = sc.basis[(nu, ob)][k]
                L = sc.out[ob][1]
                for M in range(2 * L + 1):
                    val = 0.0
                    for idx in itertools.product(range(sc.n), repeat=nu):
                        c = U[idx + (M,)]
                        if c != 0:
                            val += c * np.prod([v[i] for i in idx])
                    ref[a, ooff[ob] + M * sc.mul + u] += w[sp[a], s_idx * sc.mul + u] * val
    assert np.allclose(got, ref, atol=1e-12)


def test_output_equivariance():
    sc = symcon.SymmetricContraction("2x0e+2x1o+2x2e+2x3o", "2x0e+2x1o")
    rng = np.random.default_rng(12)
    x = rng.normal(size=(4, sc.dim_in))
    sp = rng.integers(0, 3, 4)
    w = rng.normal(size=(3, sc.weight_numel))
    aa = rng.normal(size=3)
    base = sc.eval(x, sp, w, layout="mul_ir")
    rot = sc.eval(x @ wigner.wigner_d_irreps(sc.inp, aa).T, sp, w, layout="mul_ir")
    assert np.allclose(rot, base @ wigner.wigner_d_irreps(sc.out, aa).T, atol=1e-11)
    inv = sc.eval(x @ wigner.wigner_d_irreps(sc.inp, np.zeros(3), -1).T, sp, w, layout="mul_ir")
    assert np.allclose(inv, base @ wigner.wigner_d_irreps(sc.out, np.zeros(3), -1).T, atol=1e-12)


def test_nonuniform_multiplicity_rejected():
    with pytest.raises(ValueError):
        symcon.SymmetricContraction("2x0e+3x1o", "2x0e")
