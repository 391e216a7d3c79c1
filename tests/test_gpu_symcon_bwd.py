"""GPU parity of the backward (vector-Jacobian product) of the symmetric
contraction: the HIP kernels, called through the C ABI, against the float64
oracle's eval_vjp on the same seeded inputs.  Tolerance: scaled error
(oracle.metrics, scale = the VJP over absolute operands) <= 1e-5 in float32,
<= 1e-12 in float64."""

import numpy as np
import pytest

import workloads
from oracle import symcon as osym
from tests._gpu import announce, check_scaled, dev, need_gpu

pytestmark = pytest.mark.gpu


def _sp():
    need_gpu()
    import segmented_polynomials_amd as sp
    return sp


def _bwd(sp, h, x, species, w, g, perm=None):
    import torch
    td = torch.float32 if h.dtype == "f32" else torch.float64
    if perm is None:
        perm = workloads.species_permutation(species)
    out = sp.symcon_bwd(h, dev(x, td), dev(species), dev(w, td), dev(g, td), dev(perm))
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _oracle(o, x, species, w, g, layout):
    ref = o.eval_vjp(x, species, w, g, layout=layout)
    scale = o.eval_vjp(x, species, w, g, layout=layout, absolute=True)
    return ref, scale


@pytest.mark.parametrize("layout", ["ir_mul", "mul_ir"])
def test_workload5_vjp_parity(layout):
    sp = _sp()
    wl = workloads.WORKLOADS[5]
    o = osym.SymmetricContraction(wl.irreps_in, wl.irreps_out)
    h = sp.symcon_create(wl.irreps_in, wl.irreps_out, 3, wl.num_elements, layout=layout)
    assert h.specialized
    inp = workloads.symcon_inputs(wl, o.weight_fan_in(), n_atoms=300)
    g = workloads.output_gradient(300, o.dim_out, "f32", seed=50)
    announce(f"symcon bwd workload 5 {layout} atoms=300")
    dx, dw = _bwd(sp, h, inp["x"], inp["species"], inp["w"], g)
    (rx, rw), (sx, sw) = _oracle(o, inp["x"], inp["species"], inp["w"], g, layout)
    check_scaled(dx, rx, sx, "f32", f"symcon bwd {layout} dx")
    check_scaled(dw, rw, sw, "f32", f"symcon bwd {layout} dw")


def test_workload5_full_size_sampled():
    """50,000 atoms in the launch configuration the benchmark times.  dx of
    sampled atoms against the oracle on those atoms; for dw a second call
    whose output gradient is zero except on the sampled atoms, so the
    oracle on those atoms alone gives all of dw, and every other atom's dx
    is exactly zero."""
    sp = _sp()
    wl = workloads.WORKLOADS[5]
    o = osym.SymmetricContraction(wl.irreps_in, wl.irreps_out)
    h = sp.symcon_create(wl.irreps_in, wl.irreps_out, 3, wl.num_elements, layout="ir_mul")
    inp = workloads.symcon_inputs(wl, o.weight_fan_in())
    g = workloads.output_gradient(wl.n_atoms, o.dim_out, "f32", seed=55)
    rng = np.random.default_rng(56)
    atoms = np.unique(np.concatenate([[0, wl.n_atoms - 1], rng.integers(0, wl.n_atoms, 200)]))
    announce("symcon bwd full-size workload 5")
    dx, dw = _bwd(sp, h, inp["x"], inp["species"], inp["w"], g)
    (rx, _), (sx, _) = _oracle(o, inp["x"][atoms], inp["species"][atoms], inp["w"], g[atoms], "ir_mul")
    check_scaled(dx[atoms], rx, sx, "f32", f"symcon bwd full size dx ({len(atoms)} atoms)")
    assert np.all(np.isfinite(dx)) and np.all(np.isfinite(dw))
    g_s = np.zeros_like(g)
    g_s[atoms] = g[atoms]
    announce("symcon bwd full-size workload 5, sampled gradient")
    dx2, dw2 = _bwd(sp, h, inp["x"], inp["species"], inp["w"], g_s)
    (_, rw), (_, sw) = _oracle(o, inp["x"][atoms], inp["species"][atoms], inp["w"], g[atoms], "ir_mul")
    check_scaled(dw2, rw, sw, "f32", "symcon bwd full size dw (sampled gradient)")
    others = np.ones(wl.n_atoms, bool)
    others[atoms] = False
    assert np.count_nonzero(dx2[others]) == 0
    assert np.array_equal(dx2[atoms], dx[atoms])


@pytest.mark.parametrize("mul,layout", [(32, "ir_mul"), (70, "mul_ir"), (200, "ir_mul")])
def test_page_descriptor_tiles(mul, layout):
    """The page's descriptor structure at multiplicities of one, two and
    four channel tiles (partial last tiles)."""
    sp = _sp()
    ins, outs = f"{mul}x0e+{mul}x1o", f"{mul}x0e"
    o = osym.SymmetricContraction(ins, outs)
    h = sp.symcon_create(ins, outs, 3, 4, layout=layout)
    assert h.specialized
    rng = np.random.default_rng(mul)
    n = 150
    x = rng.standard_normal((n, o.dim_in), dtype=np.float32)
    w = (rng.standard_normal((4, o.weight_numel)) / np.sqrt(o.weight_fan_in())).astype(np.float32)
    species = rng.integers(0, 4, n).astype(np.int32)
    g = rng.standard_normal((n, o.dim_out), dtype=np.float32)
    announce(f"symcon bwd page descriptor mul={mul} {layout}")
    dx, dw = _bwd(sp, h, x, species, w, g)
    (rx, rw), (sx, sw) = _oracle(o, x, species, w, g, layout)
    check_scaled(dx, rx, sx, "f32", f"symcon bwd mul={mul} dx")
    check_scaled(dw, rw, sw, "f32", f"symcon bwd mul={mul} dw")


def test_float64_int64_bad_species_and_absent_elements():
    """Out-of-range species get dx = 0 and add nothing to dw; an element
    without atoms gets dw = 0; float64 and int64 indices."""
    sp = _sp()
    ins, outs = "32x0e+32x1o", "32x0e"
    o = osym.SymmetricContraction(ins, outs)
    rng = np.random.default_rng(4)
    n = 60
    x = rng.standard_normal((n, o.dim_in))
    w = rng.standard_normal((5, o.weight_numel))
    species = rng.integers(0, 4, n).astype(np.int64)    # element 4 has no atoms
    species[[3, 17, 40]] = [5, -1, 9]                   # outside [0, 5)
    g = rng.standard_normal((n, o.dim_out))
    h = sp.symcon_create(ins, outs, 3, 5, layout="ir_mul", dtype="f64")
    announce("symcon bwd f64 int64 bad species")
    dx, dw = _bwd(sp, h, x, species, w, g)
    ok = np.ones(n, bool)
    ok[[3, 17, 40]] = False
    assert np.count_nonzero(dx[~ok]) == 0
    assert np.count_nonzero(dw[4]) == 0
    (rx, rw), (sx, sw) = _oracle(o, x[ok], species[ok], w, g[ok], "ir_mul")
    check_scaled(dx[ok], rx, sx, "f64", "symcon bwd f64 dx")
    check_scaled(dw, rw, sw, "f64", "symcon bwd f64 dw")


def test_deterministic_and_no_atoms():
    sp = _sp()
    import torch
    wl = workloads.WORKLOADS[5]
    o = osym.SymmetricContraction(wl.irreps_in, wl.irreps_out)
    h = sp.symcon_create(wl.irreps_in, wl.irreps_out, 3, wl.num_elements, layout="ir_mul")
    inp = workloads.symcon_inputs(wl, o.weight_fan_in(), n_atoms=2000)
    g = workloads.output_gradient(2000, o.dim_out, "f32", seed=57)
    announce("symcon bwd determinism")
    a = _bwd(sp, h, inp["x"], inp["species"], inp["w"], g)
    b = _bwd(sp, h, inp["x"], inp["species"], inp["w"], g)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    announce("symcon bwd no atoms")
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    w = torch.randn(wl.num_elements, h.weight_numel, device="cuda")
    dx, dw = sp.symcon_bwd(h, torch.empty(0, h.dim_in, device="cuda"), e, w,
                           torch.empty(0, h.dim_out, device="cuda"), e)
    torch.cuda.synchronize()
    assert dx.numel() == 0 and torch.count_nonzero(dw).item() == 0
