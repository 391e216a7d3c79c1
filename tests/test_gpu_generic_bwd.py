"""GPU parity of the table-driven backward (descriptors without a generated
kernel, or forced onto the table-driven path): the tensor-product
convolution's and the symmetric contraction's vector-Jacobian products,
called through the C ABI, against the float64 oracle's VJPs on the same
seeded inputs.  Tolerance: scaled error (oracle.metrics, scale = the VJP
over absolute operands) <= 1e-5 in float32, <= 1e-12 in float64."""

import numpy as np
import pytest

import workloads
from oracle import symcon as osym
from oracle import tp as otp
from tests._gpu import announce, check_scaled, dev, need_gpu

pytestmark = pytest.mark.gpu


def _sp():
    need_gpu()
    import segmented_polynomials_amd as sp
    return sp


def _tp_bwd(sp, h, inp, g, idx_dtype):
    import torch
    td = torch.float32 if h.dtype == "f32" else torch.float64
    x, s, w, gd = dev(inp["x"], td), dev(inp["sh"], td), dev(inp["w"], td), dev(g, td)
    src = dst = perm = None
    if inp["src"] is not None:
        src, dst = dev(inp["src"], idx_dtype), dev(inp["dst"], idx_dtype)
        perm = dev(workloads.src_permutation(inp["src"]), idx_dtype)
    out = sp.tp_conv_bwd(h, x, s, w, gd, src, dst, perm, n_nodes=inp["n_nodes"])
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _tp_check(o, inp, g, got, layout, dtype, what, **kw):
    args = (inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"], g)
    ref = o.conv_vjp(*args, layout=layout, **kw)
    scale = o.conv_vjp(*args, layout=layout, absolute=True, **kw)
    for name, a, b, c in zip(("dx", "dsh", "dw"), got, ref, scale):
        assert a.shape == b.shape, (name, a.shape, b.shape)
        check_scaled(a, b, c, dtype, f"{what} {name}")


def _graph(rng, o, n_src, n_dst, n_e, dtype, out_of_range=False):
    npd = np.float32 if dtype == "f32" else np.float64
    src = rng.integers(0, n_src, n_e)
    dst = np.sort(rng.integers(0, n_dst, n_e))
    if out_of_range:
        src[::9] = n_src + 2
    return dict(x=rng.standard_normal((n_src, o.dim_in1)).astype(npd).astype(np.float64),
                sh=rng.standard_normal((n_e, o.dim_in2)).astype(npd).astype(np.float64),
                w=rng.standard_normal((n_e, o.weight_numel)).astype(npd).astype(np.float64),
                src=src, dst=dst, n_nodes=n_dst)


@pytest.mark.parametrize("case", [
    ("3x0e+5x1o+2x2e+4x3o", "0e+1o+2e", "0e+1o+1e+2e+3o+3e", "mul_ir", "f32"),   # non-uniform muls
    ("64x0e+64x1o+64x2e", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o", "ir_mul", "f32"),   # registered, forced generic
    ("7x1e+7x2o", "0e+1o+2e", "0e+1o+2e+2o+3e", "ir_mul", "f32"),                 # unregistered
    ("70x0e+70x1o", "0e+1o", "0e+1o", "mul_ir", "f32"),                          # two channel tiles
    ("3x6e+2x5o", "6e+4e", "0e+2e+4e+6e+1o+3o+5o", "ir_mul", "f64"),             # l up to 6
])
@pytest.mark.parametrize("idx", ["int32", "int64"])
def test_tp_generic_backward(case, idx):
    """Ragged graph with destinations that have no edges, more sources than
    destinations and sources that no edge reads, some sources out of range."""
    sp = _sp()
    import torch
    in1, in2, filt, layout, dtype = case
    o = otp.ChannelwiseTP(in1, in2, filt)
    h = sp.tp_create(in1, in2, filt, layout=layout, dtype=dtype, force_generic=True)
    assert not h.specialized
    rng = np.random.default_rng(61)
    inp = _graph(rng, o, 31, 23, 170, dtype, out_of_range=True)
    g = rng.standard_normal((23, o.dim_out)).astype(np.float32 if dtype == "f32" else np.float64).astype(np.float64)
    announce(f"tp generic bwd {in1} {layout} {dtype} {idx}")
    got = _tp_bwd(sp, h, inp, g, getattr(torch, idx))
    ok = inp["src"] < 31
    assert np.count_nonzero(got[1][~ok]) == 0 and np.count_nonzero(got[2][~ok]) == 0
    sub = dict(inp, sh=inp["sh"][ok], w=inp["w"][ok], src=inp["src"][ok], dst=inp["dst"][ok])
    args = (sub["x"], sub["sh"], sub["w"], sub["src"], sub["dst"], sub["n_nodes"], g)
    ref = o.conv_vjp(*args, layout=layout)
    scale = o.conv_vjp(*args, layout=layout, absolute=True)
    check_scaled(got[0], ref[0], scale[0], dtype, "generic dx")
    check_scaled(got[1][ok], ref[1], scale[1], dtype, "generic dsh")
    check_scaled(got[2][ok], ref[2], scale[2], dtype, "generic dw")


@pytest.mark.parametrize("layout", ["mul_ir", "ir_mul"])
def test_tp_generic_backward_mean_shared_batch(layout):
    """reduce="mean", one shared weight row (2,300 edges: three partial sums),
    and batch mode (edge e feeds row e), on the table-driven path."""
    sp = _sp()
    import torch
    in1, in2, filt = "5x0e+3x1o+4x2e", "0e+1o+2e", "0e+1o+2e"
    o = otp.ChannelwiseTP(in1, in2, filt)
    rng = np.random.default_rng(62)
    # mean
    h = sp.tp_create(in1, in2, filt, layout=layout, reduce="mean")
    assert not h.specialized
    inp = _graph(rng, o, 40, 35, 300, "f32")
    g = rng.standard_normal((35, o.dim_out)).astype(np.float32).astype(np.float64)
    announce(f"tp generic bwd mean {layout}")
    _tp_check(o, inp, g, _tp_bwd(sp, h, inp, g, torch.int32), layout, "f32", "generic mean", reduce="mean")
    # shared weights
    hs = sp.tp_create(in1, in2, filt, layout=layout, shared_weights=True)
    inp = _graph(rng, o, 50, 60, 2300, "f32")
    inp["w"] = np.ascontiguousarray(inp["w"][:1])
    g = rng.standard_normal((60, o.dim_out)).astype(np.float32).astype(np.float64)
    announce(f"tp generic bwd shared {layout}")
    got = _tp_bwd(sp, hs, inp, g, torch.int32)
    assert got[2].shape == (1, o.weight_numel)
    _tp_check(o, inp, g, got, layout, "f32", "generic shared", shared_weights=True)
    # batch mode
    hb = sp.tp_create(in1, in2, filt, layout=layout)
    n = 33
    inp = dict(x=rng.standard_normal((n + 4, o.dim_in1)).astype(np.float32).astype(np.float64),
               sh=rng.standard_normal((n, o.dim_in2)).astype(np.float32).astype(np.float64),
               w=rng.standard_normal((n, o.weight_numel)).astype(np.float32).astype(np.float64),
               src=None, dst=None, n_nodes=n)
    g = rng.standard_normal((n, o.dim_out)).astype(np.float32).astype(np.float64)
    announce(f"tp generic bwd batch {layout}")
    _tp_check(o, inp, g, _tp_bwd(sp, hb, inp, g, torch.int32), layout, "f32", "generic batch")


def test_tp_generic_backward_deterministic_and_matches_specialised():
    """Two calls give the same bits; on a descriptor that also has a
    generated kernel both backward paths agree with the oracle."""
    sp = _sp()
    import torch
    wl = workloads.WORKLOADS[2]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    inp = workloads.tp_inputs(wl, o.weight_fan_in())
    g = workloads.output_gradient(inp["n_nodes"], o.dim_out, "f32", seed=63)
    hg = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, force_generic=True)
    announce("tp generic bwd determinism (molecules)")
    a = _tp_bwd(sp, hg, inp, g, torch.int32)
    b = _tp_bwd(sp, hg, inp, g, torch.int32)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    _tp_check(o, inp, g, a, "mul_ir", "f32", "generic molecules")


def _sym_bwd(sp, h, x, species, w, g, td):
    import torch
    perm = workloads.species_permutation(species)
    out = sp.symcon_bwd(h, dev(x, td), dev(species), dev(w, td), dev(g, td), dev(perm))
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


@pytest.mark.parametrize("case", [
    ("8x0e+8x1o+8x2e+8x3o", "8x0e+8x1o", 3, "ir_mul", "f32"),     # the 50k-atom structure, forced generic
    ("8x0e+8x1o+8x2e+8x3o", "8x0e+8x1o", 3, "mul_ir", "f32"),
    ("70x0e+70x1o+70x2e", "70x0e+70x2e", 3, "ir_mul", "f32"),     # unregistered, two channel tiles
    ("4x0e+4x1o", "4x0e+4x1o", 2, "mul_ir", "f64"),               # degrees 1..2
])
def test_symcon_generic_backward(case):
    """Species out of range (zero dx, nothing added to dw) and an element
    without atoms (zero dw row)."""
    sp = _sp()
    import torch
    ins, outs, deg, layout, dtype = case
    o = osym.SymmetricContraction(ins, outs, degrees=tuple(range(1, deg + 1)))
    n_el = 5
    h = sp.symcon_create(ins, outs, deg, n_el, layout=layout, dtype=dtype, force_generic=True)
    assert not h.specialized
    rng = np.random.default_rng(64)
    n = 137
    npd = np.float32 if dtype == "f32" else np.float64
    x = rng.standard_normal((n, o.dim_in)).astype(npd).astype(np.float64)
    species = rng.integers(0, 3, n)            # elements 3 and 4 get no atoms
    species[::11] = 7                          # out of range
    species = species.astype(np.int32)
    w = rng.standard_normal((n_el, o.weight_numel)).astype(npd).astype(np.float64)
    g = rng.standard_normal((n, o.dim_out)).astype(npd).astype(np.float64)
    td = torch.float32 if dtype == "f32" else torch.float64
    announce(f"symcon generic bwd {ins} -> {outs} {layout} {dtype}")
    dx, dw = _sym_bwd(sp, h, x, species, w, g, td)
    rx, rw = o.eval_vjp(x, species, w, g, layout=layout)
    sx, sw = o.eval_vjp(x, species, w, g, layout=layout, absolute=True)
    check_scaled(dx, rx, sx, dtype, "symcon generic dx")
    check_scaled(dw, rw, sw, dtype, "symcon generic dw")
    assert np.count_nonzero(dx[species == 7]) == 0
    assert np.count_nonzero(dw[3:]) == 0
    again = _sym_bwd(sp, h, x, species, w, g, td)
    assert np.array_equal(again[0], dx) and np.array_equal(again[1], dw)


def test_symcon_generic_backward_no_atoms():
    sp = _sp()
    import torch
    h = sp.symcon_create("4x0e+4x1o", "4x0e", 3, 3, force_generic=True)
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    x = torch.empty(0, h.dim_in, device="cuda")
    w = torch.randn(3, h.weight_numel, device="cuda")
    announce("symcon generic bwd no atoms")
    dx, dw = sp.symcon_bwd(h, x, e, w, torch.empty(0, h.dim_out, device="cuda"), e,
                           grad_w=torch.full((3, h.weight_numel), 5.0, device="cuda"))
    torch.cuda.synchronize()
    assert dx.numel() == 0 and torch.count_nonzero(dw).item() == 0
