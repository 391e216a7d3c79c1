"""GPU parity of the fully connected product as a graph convolution with
per-edge weights (fctp_conv_fwd, and its backward fctp_conv_bwd), called
through the C ABI, against the float64 oracle on the same seeded inputs.  Tolerance: scaled error
(oracle.metrics) <= 1e-5 in float32, <= 1e-12 in float64."""

import numpy as np
import pytest

import workloads
from oracle import fctp as ofc
from oracle import layout as ol
from tests._gpu import announce, check_scaled, dev, need_gpu

pytestmark = pytest.mark.gpu


def _sp():
    need_gpu()
    import segmented_polynomials_amd as sp
    return sp


def _td(dtype):
    import torch
    return torch.float32 if dtype == "f32" else torch.float64


def _graph(rng, n_nodes, max_degree, n_src):
    deg = rng.integers(0, max_degree + 1, size=n_nodes)
    deg[rng.random(n_nodes) < 0.2] = 0          # isolated destinations
    dst = np.repeat(np.arange(n_nodes), deg)
    src = rng.integers(0, n_src, size=dst.shape[0])
    return src, dst


def _case_inputs(f, n_nodes, max_degree, n_src, dtype, seed, shared=False):
    rng = np.random.default_rng(seed)
    dt = np.float32 if dtype == "f32" else np.float64
    src, dst = _graph(rng, n_nodes, max_degree, n_src)
    E = dst.shape[0]
    x = rng.standard_normal((n_src, f.dim_in1)).astype(dt)
    sh = rng.standard_normal((E, f.dim_in2)).astype(dt)
    w = rng.standard_normal((1 if shared else E, f.weight_numel)).astype(dt)
    return x, sh, w, src, dst


def _run(sp, h, x, sh, w, src, dst, n_nodes, dtype, idx="int32"):
    import torch
    td = _td(dtype)
    it = torch.int32 if idx == "int32" else torch.int64
    out = sp.fctp_conv_fwd(h, dev(x, td), dev(sh, td), dev(w, td), dev(src).to(it), dev(dst).to(it), n_nodes)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # (in1, sh, out, n_nodes, max in-degree, n_src): the workload's irreps
    # (4 edges per wave), odd multiplicities (8 edges per wave), 64 input
    # channels and an 80-channel output block (two tiles), l = 2 features
    ("16x0e+16x1o", "0e+1o+2e", "16x0e+16x1o", 150, 12, 170),
    ("5x0e+3x1o+2x2e", "0e+1o+2e", "4x0e+3x1o+2x1e+1x2e", 90, 9, 60),
    ("64x0e+40x1o", "0e+1o", "80x0e+24x1o", 40, 7, 45),
    ("8x0e+8x1o+8x2e", "0e+1o+2e", "8x0e+8x1o+8x2e+4x2o", 60, 10, 60),
    # more than 64 input channels (two u tiles of 64: full chunks in both,
    # and 100 / 70 channels: chunks then single channels in the second)
    ("128x0e+80x1o", "0e+1o", "24x0e+16x1o", 30, 6, 35),
    ("100x0e+70x1o+3x2e", "0e+1o+2e", "12x0e+8x1o+4x2e", 25, 5, 30),
]


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_parity(case, lay, dtype):
    sp = _sp()
    in1, in2, out, n_nodes, deg, n_src = CASES[case]
    f = ofc.FullyConnectedTP(in1, in2, out)
    h = sp.fctp_create(in1, in2, out, layout=lay, dtype=dtype)
    x, sh, w, src, dst = _case_inputs(f, n_nodes, deg, n_src, dtype, 300 + case)
    idx = "int32" if (case + (lay == "ir_mul")) % 2 == 0 else "int64"
    announce(f"fcconv case {case} {in1} x {in2} -> {out} E={dst.shape[0]} {lay} {dtype} {idx}")
    got = _run(sp, h, x, sh, w, src, dst, n_nodes, dtype, idx)
    check_scaled(got, f.conv(x, sh, w, src, dst, n_nodes, layout=lay),
                 f.conv(x, sh, w, src, dst, n_nodes, layout=lay, absolute=True), dtype, f"fcconv case {case}")
    deg_n = np.bincount(dst, minlength=n_nodes)
    assert np.count_nonzero(got[deg_n == 0]) == 0


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_shared_weights_and_mean(dtype):
    sp = _sp()
    in1, in2, out, n_nodes, deg, n_src = CASES[1]
    f = ofc.FullyConnectedTP(in1, in2, out)
    x, sh, w, src, dst = _case_inputs(f, n_nodes, deg, n_src, dtype, 310, shared=True)
    announce(f"fcconv shared weights {dtype}")
    h = sp.fctp_create(in1, in2, out, dtype=dtype)
    got = _run(sp, h, x, sh, w, src, dst, n_nodes, dtype)
    check_scaled(got, f.conv(x, sh, w, src, dst, n_nodes), f.conv(x, sh, w, src, dst, n_nodes, absolute=True),
                 dtype, "shared")
    announce(f"fcconv reduce=mean {dtype}")
    hm = sp.fctp_create(in1, in2, out, dtype=dtype, reduce="mean")
    x, sh, w, src, dst = _case_inputs(f, n_nodes, deg, n_src, dtype, 311)
    got = _run(sp, hm, x, sh, w, src, dst, n_nodes, dtype)
    check_scaled(got, f.conv(x, sh, w, src, dst, n_nodes, reduce="mean"),
                 f.conv(x, sh, w, src, dst, n_nodes, reduce="mean", absolute=True), dtype, "mean")


def test_layouts_agree_and_empty_graph():
    import torch
    sp = _sp()
    in1, in2, out, n_nodes, deg, n_src = CASES[3]
    f = ofc.FullyConnectedTP(in1, in2, out)
    x, sh, w, src, dst = _case_inputs(f, n_nodes, deg, n_src, "f64", 312)
    announce("fcconv layouts agree")
    a = _run(sp, sp.fctp_create(in1, in2, out, layout="mul_ir", dtype="f64"), x, sh, w, src, dst, n_nodes, "f64")
    b = _run(sp, sp.fctp_create(in1, in2, out, layout="ir_mul", dtype="f64"),
             ol.transpose(x, f.in1, "mul_ir", "ir_mul"), sh, w, src, dst, n_nodes, "f64")
    assert np.allclose(ol.transpose(b, f.out, "ir_mul", "mul_ir"), a, atol=1e-12)
    announce("fcconv empty graph")
    h = sp.fctp_create(in1, in2, out, dtype="f32")
    e = np.zeros(0, dtype=np.int32)
    got = _run(sp, h, x.astype(np.float32), sh[:0].astype(np.float32), w[:1].astype(np.float32), e, e, 7, "f32")
    assert got.shape == (7, f.dim_out) and np.count_nonzero(got) == 0
    del torch


def test_page_example_so3_two_edges():
    """The skill document's "0 + 1" product of two feature rows with the
    harmonics of its two vectors, both edges into one destination."""
    from oracle import sh as osh
    sp = _sp()
    f = ofc.FullyConnectedTP("0 + 1", "0 + 1", "0 + 1")
    h = sp.fctp_create("0 + 1", "0 + 1", "0 + 1", dtype="f64")
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 4))
    vecs = np.array([[0.3, -0.7, 1.1], [1.2, 0.4, -0.2]])
    sh = osh.real_sh([0, 1], vecs, normalize=False)
    w = rng.standard_normal((2, 5))
    src, dst = np.array([0, 1]), np.array([0, 0])
    announce("fcconv page example")
    got = _run(sp, h, x, sh, w, src, dst, 1, "f64")
    want = f.fwd(x[:1], sh[:1], w[:1]) + f.fwd(x[1:], sh[1:], w[1:])
    check_scaled(got, want, f.conv(x, sh, w, src, dst, 1, absolute=True), "f64", "page example")


@pytest.mark.slow
@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
def test_full_size_workload_sampled(lay):
    """The 600k-edge workload in the launch configuration the benchmark
    times; sampled destination rows against the oracle on their edges."""
    import torch
    sp = _sp()
    wl = workloads.WORKLOADS[9]
    f = ofc.FullyConnectedTP(wl.irreps_in1, wl.irreps_sh, wl.irreps_out)
    h = sp.fctp_create(wl.irreps_in1, wl.irreps_sh, wl.irreps_out, layout=lay, dtype=wl.dtype)
    inp = workloads.fcconv_inputs(wl, f.weight_numel)
    N = inp["n_nodes"]
    announce(f"fcconv full size E={inp['dst'].shape[0]} {lay}")
    got = _run(sp, h, inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], N, wl.dtype)
    nodes = np.unique(np.concatenate([np.arange(6), N - 1 - np.arange(6),
                                      np.random.default_rng(7).integers(0, N, 40)]))
    sel = np.isin(inp["dst"], nodes)
    dsel = np.searchsorted(nodes, inp["dst"][sel])
    args = (inp["x"], inp["sh"][sel], inp["w"][sel], inp["src"][sel], dsel, len(nodes))
    check_scaled(got[nodes], f.conv(*args, layout=lay), f.conv(*args, layout=lay, absolute=True), wl.dtype,
                 "full size rows")
    del torch


def _bwd(sp, h, x, sh, w, g, src, dst, n_nodes, dtype, idx="int32"):
    import torch
    td = _td(dtype)
    it = torch.int32 if idx == "int32" else torch.int64
    perm = np.argsort(src, kind="stable")
    out = sp.fctp_conv_bwd(h, dev(x, td), dev(sh, td), dev(w, td), dev(g, td), dev(src).to(it), dev(dst).to(it),
                           dev(perm).to(it), n_nodes=n_nodes)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_parity(case, lay, dtype):
    sp = _sp()
    in1, in2, out, n_nodes, deg, n_src = CASES[case]
    f = ofc.FullyConnectedTP(in1, in2, out)
    h = sp.fctp_create(in1, in2, out, layout=lay, dtype=dtype)
    x, sh, w, src, dst = _case_inputs(f, n_nodes, deg, n_src, dtype, 320 + case)
    g = np.random.default_rng(330 + case).standard_normal((n_nodes, f.dim_out)).astype(x.dtype)
    idx = "int64" if (case + (lay == "ir_mul")) % 2 == 0 else "int32"
    announce(f"fcconv backward case {case} E={dst.shape[0]} {lay} {dtype} {idx}")
    got = _bwd(sp, h, x, sh, w, g, src, dst, n_nodes, dtype, idx)
    ref = f.conv_vjp(x, sh, w, src, dst, n_nodes, g, layout=lay)
    scale = f.conv_vjp(x, sh, w, src, dst, n_nodes, g, layout=lay, absolute=True)
    for name, a, b, c in zip(("dx", "dsh", "dw"), got, ref, scale):
        check_scaled(a, b, c, dtype, f"fcconv backward case {case} {name}")


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_backward_shared_weights(dtype):
    """One weight row for every edge: grad_w [1, numel] is the sum of the
    per-edge gradients (summed in chunks of 1024 edges, then in order);
    dx and dsh as with that row repeated per edge."""
    sp = _sp()
    in1, in2, out = CASES[1][:3]
    f = ofc.FullyConnectedTP(in1, in2, out)
    h = sp.fctp_create(in1, in2, out, layout="ir_mul", dtype=dtype)
    n_nodes = 900
    x, sh, w, src, dst = _case_inputs(f, n_nodes, 8, 700, dtype, 360, shared=True)
    assert w.shape[0] == 1 and dst.shape[0] > 2048
    g = np.random.default_rng(361).standard_normal((n_nodes, f.dim_out)).astype(x.dtype)
    announce(f"fcconv backward shared weights E={dst.shape[0]} {dtype}")
    got = _bwd(sp, h, x, sh, w, g, src, dst, n_nodes, dtype)
    assert got[2].shape == w.shape
    ref = f.conv_vjp(x, sh, w, src, dst, n_nodes, g, layout="ir_mul")
    scale = f.conv_vjp(x, sh, w, src, dst, n_nodes, g, layout="ir_mul", absolute=True)
    for name, a, b, c in zip(("dx", "dsh", "dw"), got, ref, scale):
        check_scaled(a, b, c, dtype, f"fcconv backward shared weights {name}")


def test_backward_mean_and_outside_edges():
    """reduce="mean" scales the output gradient by 1/in-degree; edges whose
    destination is past the last row get zero gradients."""
    sp = _sp()
    in1, in2, out, n_nodes, deg, n_src = CASES[1]
    f = ofc.FullyConnectedTP(in1, in2, out)
    hm = sp.fctp_create(in1, in2, out, dtype="f64", reduce="mean")
    x, sh, w, src, dst = _case_inputs(f, n_nodes, deg, n_src, "f64", 340)
    g = np.random.default_rng(341).standard_normal((n_nodes, f.dim_out))
    announce("fcconv backward mean")
    got = _bwd(sp, hm, x, sh, w, g, src, dst, n_nodes, "f64")
    ref = f.conv_vjp(x, sh, w, src, dst, n_nodes, g, reduce="mean")
    scale = f.conv_vjp(x, sh, w, src, dst, n_nodes, g, reduce="mean", absolute=True)
    for name, a, b, c in zip(("dx", "dsh", "dw"), got, ref, scale):
        check_scaled(a, b, c, "f64", f"mean {name}")
    # the output holds only the first 30 destinations: later edges lie outside
    announce("fcconv backward edges outside the output")
    h = sp.fctp_create(in1, in2, out, dtype="f64")
    keep = 30
    got = _bwd(sp, h, x, sh, w, g[:keep], src, dst, keep, "f64")
    inside = dst < keep
    ref = f.conv_vjp(x, sh[inside], w[inside], src[inside], dst[inside], keep, g[:keep])
    assert np.allclose(got[0], ref[0], atol=1e-12)
    assert np.allclose(got[1][inside], ref[1], atol=1e-12) and np.count_nonzero(got[1][~inside]) == 0
    assert np.allclose(got[2][inside], ref[2], atol=1e-12) and np.count_nonzero(got[2][~inside]) == 0


def test_out_of_range_source_and_validate():
    """Without VALIDATE an edge whose source index is out of range
    contributes nothing (forward) and gets zero dW and dsh (backward), like
    the edge left out; with VALIDATE the forward and backward report
    unsorted destinations, out-of-range indices and a bad permutation."""
    import torch
    sp = _sp()
    in1, in2, out, n_nodes, deg, n_src = CASES[1]
    f = ofc.FullyConnectedTP(in1, in2, out)
    x, sh, w, src, dst = _case_inputs(f, n_nodes, deg, n_src, "f64", 350)
    bad = src.copy()
    bad[::7] = n_src + 3                       # every 7th edge reads past the table
    keep = bad < n_src
    h = sp.fctp_create(in1, in2, out, dtype="f64")
    announce("fcconv out-of-range sources")
    got = _run(sp, h, x, sh, w, bad, dst, n_nodes, "f64")
    want = f.conv(x, sh[keep], w[keep], src[keep], dst[keep], n_nodes)
    assert np.allclose(got, want, atol=1e-12)
    g = np.random.default_rng(351).standard_normal((n_nodes, f.dim_out))
    gx, gs, gw = _bwd(sp, h, x, sh, w, g, bad, dst, n_nodes, "f64")
    rx, rs, rw = f.conv_vjp(x, sh[keep], w[keep], src[keep], dst[keep], n_nodes, g)
    assert np.allclose(gx, rx, atol=1e-12)
    assert np.allclose(gs[keep], rs, atol=1e-12) and np.count_nonzero(gs[~keep]) == 0
    assert np.allclose(gw[keep], rw, atol=1e-12) and np.count_nonzero(gw[~keep]) == 0
    announce("fcconv VALIDATE")
    hv = sp.fctp_create(in1, in2, out, dtype="f64", validate=True)
    td = torch.float64
    X, S, W, G = dev(x, td), dev(sh, td), dev(w, td), dev(g, td)
    with pytest.raises(sp.SegpolyError) as ei:
        sp.fctp_conv_fwd(hv, X, S, W, dev(bad), dev(dst), n_nodes)
    assert ei.value.code == sp.E_RANGE
    with pytest.raises(sp.SegpolyError) as ei:
        sp.fctp_conv_fwd(hv, X, S, W, dev(src), dev(dst[::-1].copy()), n_nodes)
    assert ei.value.code == sp.E_UNSORTED
    perm = np.argsort(src, kind="stable")
    with pytest.raises(sp.SegpolyError) as ei:
        sp.fctp_conv_bwd(hv, X, S, W, G, dev(src), dev(dst), dev(perm[::-1].copy()), n_nodes)
    assert ei.value.code == sp.E_UNSORTED
    ok = sp.fctp_conv_bwd(hv, X, S, W, G, dev(src), dev(dst), dev(perm), n_nodes)
    torch.cuda.synchronize()
    assert np.allclose(ok[2].cpu().numpy(), f.conv_vjp(x, sh, w, src, dst, n_nodes, g)[2], atol=1e-12)
