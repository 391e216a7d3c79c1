"""GPU parity of the fully connected (uvw) tensor product on the matrix cores
(forward, both input gradients, the weight gradient), called through the C
ABI, against the float64 oracle on the same seeded inputs.  Tolerance:
scaled error (oracle.metrics) <= 1e-5 in float32, <= 1e-12 in float64."""

import numpy as np
import pytest

import workloads
from oracle import fctp as ofc
from oracle import layout as ol
from oracle import sh as osh
from tests._gpu import announce, check_scaled, dev, need_gpu

pytestmark = pytest.mark.gpu


def _sp():
    need_gpu()
    import segmented_polynomials_amd as sp
    return sp


def _td(dtype):
    import torch
    return torch.float32 if dtype == "f32" else torch.float64


def _inputs(f, n, dtype, seed):
    rng = np.random.default_rng(seed)
    dt = np.float32 if dtype == "f32" else np.float64
    x1 = rng.standard_normal((n, f.dim_in1)).astype(dt)
    x2 = rng.standard_normal((n, f.dim_in2)).astype(dt)
    w = rng.standard_normal((1, f.weight_numel)).astype(dt)
    g = rng.standard_normal((n, f.dim_out)).astype(dt)
    return x1, x2, w, g


def _run(sp, h, x1, x2, w, g, dtype):
    import torch
    td = _td(dtype)
    X1, X2, W, G = dev(x1, td), dev(x2, td), dev(w, td), dev(g, td)
    out = sp.fctp_fwd(h, X1, X2, W)
    g1, g2, gw = sp.fctp_bwd(h, X1, X2, W, G)
    torch.cuda.synchronize()
    return out.cpu().numpy(), g1.cpu().numpy(), g2.cpu().numpy(), gw.cpu().numpy()


def _check_all(f, lay, dtype, x1, x2, w, g, res, what):
    out, g1, g2, gw = res
    check_scaled(out, f.fwd(x1, x2, w, layout=lay), f.fwd(x1, x2, w, layout=lay, absolute=True), dtype,
                 f"{what} fwd")
    r1, r2, rw = f.vjp(x1, x2, w, g, layout=lay)
    a1, a2, aw = f.vjp(x1, x2, w, g, layout=lay, absolute=True)
    check_scaled(g1, r1, a1, dtype, f"{what} dx1")
    check_scaled(g2, r2, a2, dtype, f"{what} dx2")
    check_scaled(gw, rw, aw, dtype, f"{what} dw")


CASES = [
    # (in1, in2, out, n): ragged sample counts (tiles of 64 samples for
    # scalar outputs, 42 for vectors), odd multiplicities, one-channel input 2,
    # two column tiles (80 channels), an output block without paths
    ("32x0e+32x1o", "32x0e+32x1o", "32x0e+32x1o", 257),
    ("3x0e+2x1o+1x2e", "2x0e+1x1o+2x1e", "2x0e+3x1o+2x1e+1x2e+1x2o", 133),
    ("16x0e+16x1o+16x2e", "0e+1o+2e", "16x0e+16x1o+16x2e", 300),
    ("64x0e+48x1o", "8x0e+8x1o", "80x0e+40x1o", 70),
    ("2x0e+1x1o", "1x0e", "2x0e+1x1o+2x2e", 5),
    # every compiled coupling-count class (entries per component, rounded to
    # 1, 2, 3, 4, 6, 8): the launch runs the largest class among its terms
    ("4x0e+3x1o", "2x0e", "3x0e+2x1o", 91),          # forward 1, dx1 1, dx2 3
    ("3x1o", "2x1o", "2x1e", 77),                    # 1 x 1 -> 1: 2 everywhere
    ("3x1o", "2x2e", "2x1o", 65),                    # forward 4, dx1 4, dx2 3
    ("2x2e", "3x2e", "2x2e", 50),                    # 6 everywhere
    ("2x2e", "2x2e", "2x4e", 45),                    # forward 6, dx1 8, dx2 8
    ("2x3o", "1x3o", "2x1e+2x2e", 40),               # 3 x 3: up to 10 entries (class 16)
    ("1x4e", "2x4e", "1x3e+1x4e", 30),               # 4 x 4: up to 14 entries (class 16)
]


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_parity(case, lay, dtype):
    sp = _sp()
    in1, in2, out, n = CASES[case]
    f = ofc.FullyConnectedTP(in1, in2, out)
    h = sp.fctp_create(in1, in2, out, layout=lay, dtype=dtype)
    assert (h.dim_in1, h.dim_in2, h.dim_out, h.weight_numel, h.num_paths) == \
        (f.dim_in1, f.dim_in2, f.dim_out, f.weight_numel, len(f.paths))
    x1, x2, w, g = _inputs(f, n, dtype, 100 + case)
    announce(f"fctp case {case} {in1} x {in2} -> {out} n={n} {lay} {dtype}")
    res = _run(sp, h, x1, x2, w, g, dtype)
    _check_all(f, lay, dtype, x1, x2, w, g, res, f"case {case} {lay} {dtype}")


def test_page_example_so3_f64():
    """The skill document's CPU example: FullyConnectedTensorProduct of the
    SO(3) irreps "0 + 1" with itself, fed features and the l = 0, 1
    harmonics (normalize=False) of its two vectors, float64 mul_ir."""
    sp = _sp()
    f = ofc.FullyConnectedTP("0 + 1", "0 + 1", "0 + 1")
    h = sp.fctp_create("0 + 1", "0 + 1", "0 + 1", layout="mul_ir", dtype="f64")
    assert h.num_paths == 5 and h.weight_numel == 5
    rng = np.random.default_rng(0)
    x1 = rng.standard_normal((2, 4))
    vecs = np.array([[0.3, -0.7, 1.1], [1.2, 0.4, -0.2]])
    x2 = osh.real_sh([0, 1], vecs, normalize=False)
    w = rng.standard_normal((1, 5))
    out = f.fwd(x1, x2, w)
    g = 2 * out
    announce("fctp page example SO(3) 0 + 1 f64")
    res = _run(sp, h, x1, x2, w, g, "f64")
    _check_all(f, "mul_ir", "f64", x1, x2, w, g, res, "page example")


@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
def test_layouts_agree(lay):
    """mul_ir and ir_mul results agree after the blockwise transposition."""
    sp = _sp()
    in1, in2, out, n = CASES[1]
    f = ofc.FullyConnectedTP(in1, in2, out)
    x1, x2, w, g = _inputs(f, n, "f64", 7)
    announce(f"fctp layouts {lay}")
    h = sp.fctp_create(in1, in2, out, layout=lay, dtype="f64")
    r = _run(sp, h, ol.transpose(x1, f.in1, "mul_ir", lay), ol.transpose(x2, f.in2, "mul_ir", lay), w,
             ol.transpose(g, f.out, "mul_ir", lay), "f64")
    h0 = sp.fctp_create(in1, in2, out, layout="mul_ir", dtype="f64")
    r0 = _run(sp, h0, x1, x2, w, g, "f64")
    assert np.allclose(ol.transpose(r[0], f.out, lay, "mul_ir"), r0[0], atol=1e-12)
    assert np.allclose(ol.transpose(r[1], f.in1, lay, "mul_ir"), r0[1], atol=1e-12)
    assert np.allclose(r[3], r0[3], atol=1e-12)


def test_empty_and_single_sample():
    import torch
    sp = _sp()
    in1, in2, out, _ = CASES[0]
    f = ofc.FullyConnectedTP(in1, in2, out)
    h = sp.fctp_create(in1, in2, out, dtype="f32")
    x1, x2, w, g = _inputs(f, 1, "f32", 9)
    announce("fctp n=1")
    _check_all(f, "mul_ir", "f32", x1, x2, w, g, _run(sp, h, x1, x2, w, g, "f32"), "n=1")
    announce("fctp n=0")
    e1 = torch.empty((0, f.dim_in1), device="cuda")
    e2 = torch.empty((0, f.dim_in2), device="cuda")
    eg = torch.empty((0, f.dim_out), device="cuda")
    W = dev(w)
    assert sp.fctp_fwd(h, e1, e2, W).shape == (0, f.dim_out)
    g1, g2, gw = sp.fctp_bwd(h, e1, e2, W, eg)
    torch.cuda.synchronize()
    assert g1.shape == (0, f.dim_in1) and g2.shape == (0, f.dim_in2)
    assert np.count_nonzero(gw.cpu().numpy()) == 0


def test_weight_alignment_selects_the_staging():
    """Weights that are not 16-byte aligned take the register-staged path
    instead of the LDS-direct one (whose copies need aligned rows); both
    must give the oracle's result."""
    import torch
    sp = _sp()
    in1, in2, out, n = CASES[0]
    f = ofc.FullyConnectedTP(in1, in2, out)
    h = sp.fctp_create(in1, in2, out, dtype="f32")
    x1, x2, w, g = _inputs(f, n, "f32", 13)
    X1, X2 = dev(x1, torch.float32), dev(x2, torch.float32)
    announce("fctp weights aligned and misaligned")
    buf = torch.empty(f.weight_numel + 1, dtype=torch.float32, device="cuda")
    Wm = buf[1:].view(1, f.weight_numel)
    Wm.copy_(dev(w, torch.float32))
    assert Wm.data_ptr() % 16 != 0
    Wa = dev(w, torch.float32)
    assert Wa.data_ptr() % 16 == 0
    ref = f.fwd(x1, x2, w)
    scale = f.fwd(x1, x2, w, absolute=True)
    for W, what in ((Wa, "aligned"), (Wm, "misaligned")):
        got = sp.fctp_fwd(h, X1, X2, W)
        torch.cuda.synchronize()
        check_scaled(got.cpu().numpy(), ref, scale, "f32", f"weights {what}")


def test_deterministic():
    import torch
    sp = _sp()
    in1, in2, out, n = CASES[0]
    f = ofc.FullyConnectedTP(in1, in2, out)
    h = sp.fctp_create(in1, in2, out, dtype="f32")
    x1, x2, w, g = _inputs(f, 5000, "f32", 11)
    announce("fctp determinism n=5000")
    a = _run(sp, h, x1, x2, w, g, "f32")
    b = _run(sp, h, x1, x2, w, g, "f32")
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    del torch


@pytest.mark.slow
@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
def test_full_size_workload(lay):
    """The 100k-sample workload in the launch configuration the benchmark
    times: sampled rows of the forward and input gradients (rows are
    independent samples) and sampled weight-gradient entries, each against
    the oracle's definition over the whole batch."""
    import torch
    sp = _sp()
    wl = workloads.WORKLOADS[8]
    f = ofc.FullyConnectedTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    h = sp.fctp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=lay, dtype=wl.dtype)
    inp = workloads.fc_inputs(wl, f.weight_numel)
    g = workloads.output_gradient(wl.n, f.dim_out, wl.dtype, seed=2000 + wl.number)
    announce(f"fctp full size n={wl.n} {lay}")
    td = _td(wl.dtype)
    X1, X2, W, G = dev(inp["x1"], td), dev(inp["x2"], td), dev(inp["w"], td), dev(g, td)
    out = sp.fctp_fwd(h, X1, X2, W)
    g1, g2, gw = sp.fctp_bwd(h, X1, X2, W, G)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(8), wl.n - 1 - np.arange(8),
                                     np.random.default_rng(5).integers(0, wl.n, 48)]))
    x1, x2, w, gg = inp["x1"][rows], inp["x2"][rows], inp["w"], g[rows]
    check_scaled(out.cpu().numpy()[rows], f.fwd(x1, x2, w, layout=lay), f.fwd(x1, x2, w, layout=lay, absolute=True),
                 wl.dtype, "full fwd rows")
    r1, r2, _ = f.vjp(x1, x2, w, gg, layout=lay)
    a1, a2, _ = f.vjp(x1, x2, w, gg, layout=lay, absolute=True)
    check_scaled(g1.cpu().numpy()[rows], r1, a1, wl.dtype, "full dx1 rows")
    check_scaled(g2.cpu().numpy()[rows], r2, a2, wl.dtype, "full dx2 rows")
    flat = np.unique(np.random.default_rng(6).integers(0, f.weight_numel, 24))
    ref = f.dw_entries(inp["x1"], inp["x2"], g, flat, layout=lay)
    scale = f.dw_entries(inp["x1"], inp["x2"], g, flat, layout=lay, absolute=True)
    check_scaled(gw.cpu().numpy()[0, flat], ref, scale, wl.dtype, "full dw entries")
