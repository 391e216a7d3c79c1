"""GPU parity of the symmetric contraction (degrees 1..3): HIP kernels via
the C ABI against the float64 oracle on the same seeded inputs."""

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


def _run(sp, h, x, species, w):
    import torch
    td = torch.float32 if h.dtype == "f32" else torch.float64
    out = sp.symcon_fwd(h, dev(x, td), dev(species), dev(w, td))
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle(o, x, species, w, layout, chunk=64):
    """Oracle in chunks of atoms (memory of its einsum intermediates)."""
    refs, scales = [], []
    for a in range(0, x.shape[0], chunk):
        sl = slice(a, a + chunk)
        refs.append(o.eval(x[sl], species[sl], w, layout=layout))
        scales.append(o.eval(x[sl], species[sl], w, layout=layout, absolute=True))
    return np.concatenate(refs), np.concatenate(scales)


@pytest.mark.parametrize("layout", ["ir_mul", "mul_ir"])
def test_workload5_parity(layout):
    sp = _sp()
    wl = workloads.WORKLOADS[5]
    o = osym.SymmetricContraction(wl.irreps_in, wl.irreps_out)
    h = sp.symcon_create(wl.irreps_in, wl.irreps_out, 3, wl.num_elements, layout=layout)
    assert h.specialized
    inp = workloads.symcon_inputs(wl, o.weight_fan_in(), n_atoms=300)
    announce(f"symcon workload 5 {layout} atoms=300")
    got = _run(sp, h, inp["x"], inp["species"], inp["w"])
    ref, scale = _oracle(o, inp["x"], inp["species"], inp["w"], layout)
    check_scaled(got, ref, scale, "f32", f"symcon workload 5 {layout}")


def test_workload5_full_size_sampled_atoms():
    sp = _sp()
    wl = workloads.WORKLOADS[5]
    o = osym.SymmetricContraction(wl.irreps_in, wl.irreps_out)
    h = sp.symcon_create(wl.irreps_in, wl.irreps_out, 3, wl.num_elements, layout="ir_mul")
    inp = workloads.symcon_inputs(wl, o.weight_fan_in())
    announce("symcon full-size workload 5")
    got = _run(sp, h, inp["x"], inp["species"], inp["w"])
    rng = np.random.default_rng(5)
    atoms = np.unique(np.concatenate([[0, wl.n_atoms - 1], rng.integers(0, wl.n_atoms, 126)]))
    ref, scale = _oracle(o, inp["x"][atoms], inp["species"][atoms], inp["w"], "ir_mul")
    check_scaled(got[atoms], ref, scale, "f32", f"symcon full size ({len(atoms)} atoms)")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("ins,outs,layout,fg", [
    ("32x0e+32x1o", "32x0e", "ir_mul", False),                 # the page's descriptor
    ("32x0e+32x1o", "32x0e", "mul_ir", True),
    ("128x0e+128x1o+128x2e+128x3o", "128x0e+128x1o", "ir_mul", True),   # registered, forced generic
    ("5x0e+5x1o+5x2e", "5x0e+5x1o+5x2e", "mul_ir", False),     # unregistered -> generic
    ("70x0e+70x1o", "70x0e+70x1o", "ir_mul", False),           # two channel tiles, ragged
])
def test_other_descriptors(ins, outs, layout, fg):
    sp = _sp()
    o = osym.SymmetricContraction(ins, outs)
    h = sp.symcon_create(ins, outs, 3, 4, layout=layout, force_generic=fg)
    rng = np.random.default_rng(17)
    n = 90
    x = rng.standard_normal((n, o.dim_in), dtype=np.float32)
    w = (rng.standard_normal((4, o.weight_numel)) / np.sqrt(o.weight_fan_in())).astype(np.float32)
    species = rng.integers(0, 4, n).astype(np.int32)
    announce(f"symcon {ins} -> {outs} {layout} {h.specialized}")
    got = _run(sp, h, x, species, w)
    ref, scale = _oracle(o, x, species, w, layout)
    check_scaled(got, ref, scale, "f32", f"symcon {ins}")


def test_float64_int64_and_bad_species():
    sp = _sp()
    ins, outs = "32x0e+32x1o", "32x0e"
    o = osym.SymmetricContraction(ins, outs)
    rng = np.random.default_rng(2)
    n = 40
    x = rng.standard_normal((n, o.dim_in))
    w = rng.standard_normal((3, o.weight_numel))
    species = rng.integers(0, 3, n).astype(np.int64)
    species[[5, 11]] = [3, -1]                         # outside [0, 3): zero rows
    for fg in (False, True):
        h = sp.symcon_create(ins, outs, 3, 3, layout="ir_mul", dtype="f64", force_generic=fg)
        announce(f"symcon f64 int64 generic={fg}")
        got = _run(sp, h, x, species, w)
        ok = np.ones(n, bool)
        ok[[5, 11]] = False
        ref, scale = _oracle(o, x[ok], species[ok], w, "ir_mul")
        check_scaled(got[ok], ref, scale, "f64", f"symcon f64 generic={fg}")
        assert np.count_nonzero(got[~ok]) == 0
