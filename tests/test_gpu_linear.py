"""GPU parity of the equivariant linear layer on the matrix cores (forward
and backward), called through the C ABI, against the float64 oracle on the
same seeded inputs.  Tolerance: scaled error (oracle.metrics) <= 1e-5 in
float32, <= 1e-12 in float64."""

import numpy as np
import pytest

import workloads
from oracle import layout as ol
from oracle import linear as olin
from tests._gpu import announce, check_scaled, dev, need_gpu

pytestmark = pytest.mark.gpu


def _sp():
    need_gpu()
    import segmented_polynomials_amd as sp
    return sp


def _fwd(sp, h, x, w, classes=None):
    import torch
    td = torch.float32 if h.dtype == "f32" else torch.float64
    c = None if classes is None else dev(classes)
    out = sp.linear_fwd(h, dev(x, td), dev(w, td), classes=c, num_classes=None if classes is None else w.shape[0])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _bwd(sp, h, x, w, g, classes=None, need_dw=True):
    import torch
    td = torch.float32 if h.dtype == "f32" else torch.float64
    c = None if classes is None else dev(classes)
    gx, gw = sp.linear_bwd(h, dev(x, td), dev(w, td), dev(g, td), classes=c,
                           num_classes=None if classes is None else w.shape[0], need_dw=need_dw)
    torch.cuda.synchronize()
    return gx.cpu().numpy(), None if gw is None else gw.cpu().numpy()


def test_page_example_f64_both_layouts():
    """The skill document's Linear example: 3x0 + 2x1 -> 2x0 + 4x1, 14
    weights; mul_ir and ir_mul agree after transposition."""
    sp = _sp()
    ins, outs = "3x0e+2x1o", "2x0e+4x1o"
    o = olin.Linear(ins, outs)
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, o.dim_in))
    w = rng.standard_normal((1, o.weight_numel))
    res = {}
    for lay in ("mul_ir", "ir_mul"):
        h = sp.linear_create(ins, outs, layout=lay, dtype="f64")
        assert h.weight_numel == 14
        xl = ol.transpose(x, o.inp, "mul_ir", lay)
        announce(f"linear page example {lay}")
        got = _fwd(sp, h, xl, w)
        check_scaled(got, o.fwd(xl, w, layout=lay), o.fwd(xl, w, layout=lay, absolute=True), "f64", f"page {lay}")
        res[lay] = ol.transpose(got, o.out, lay, "mul_ir")
    assert np.allclose(res["mul_ir"], res["ir_mul"], atol=1e-14)


@pytest.mark.parametrize("layout", ["ir_mul", "mul_ir"])
def test_workload6_forward_and_backward(layout):
    sp = _sp()
    wl = workloads.WORKLOADS[6]
    o = olin.Linear(wl.irreps_in, wl.irreps_out)
    h = sp.linear_create(wl.irreps_in, wl.irreps_out, layout=layout)
    inp = workloads.linear_inputs(wl, o.weight_numel, n=300)
    g = workloads.output_gradient(300, o.dim_out, "f32", seed=61)
    announce(f"linear workload 6 {layout} n=300")
    got = _fwd(sp, h, inp["x"], inp["w"])
    check_scaled(got, o.fwd(inp["x"], inp["w"], layout=layout),
                 o.fwd(inp["x"], inp["w"], layout=layout, absolute=True), "f32", f"linear fwd {layout}")
    gx, gw = _bwd(sp, h, inp["x"], inp["w"], g)
    (rx, rw), (sx, sw) = (o.vjp(inp["x"], inp["w"], g, layout=layout),
                          o.vjp(inp["x"], inp["w"], g, layout=layout, absolute=True))
    check_scaled(gx, rx, sx, "f32", f"linear dx {layout}")
    check_scaled(gw, rw, sw, "f32", f"linear dw {layout}")


def test_workload6_full_size_sampled_rows():
    sp = _sp()
    wl = workloads.WORKLOADS[6]
    o = olin.Linear(wl.irreps_in, wl.irreps_out)
    h = sp.linear_create(wl.irreps_in, wl.irreps_out, layout="ir_mul")
    inp = workloads.linear_inputs(wl, o.weight_numel)
    announce("linear workload 6 full size")
    got = _fwd(sp, h, inp["x"], inp["w"])
    rows = np.unique(np.concatenate([[0, wl.n - 1], np.random.default_rng(6).integers(0, wl.n, 100)]))
    check_scaled(got[rows], o.fwd(inp["x"][rows], inp["w"]), o.fwd(inp["x"][rows], inp["w"], absolute=True),
                 "f32", f"linear full size ({len(rows)} rows)")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("layout", ["ir_mul", "mul_ir"])
def test_ragged_tiles(layout):
    """Multiplicities that leave partial row, column and K tiles, two column
    tiles, several input blocks of one type and an output type no input
    has (zero block)."""
    sp = _sp()
    ins, outs = "77x0e+33x1o+20x1o+5x2e", "50x0e+130x1o+3x3o"
    o = olin.Linear(ins, outs)
    h = sp.linear_create(ins, outs, layout=layout)
    rng = np.random.default_rng(9)
    x = rng.standard_normal((37, o.dim_in), dtype=np.float32)
    w = rng.standard_normal((1, o.weight_numel), dtype=np.float32)
    g = rng.standard_normal((37, o.dim_out), dtype=np.float32)
    announce(f"linear ragged {layout}")
    got = _fwd(sp, h, x, w)
    check_scaled(got, o.fwd(x, w, layout=layout), o.fwd(x, w, layout=layout, absolute=True), "f32", "ragged fwd")
    gx, gw = _bwd(sp, h, x, w, g)
    (rx, rw), (sx, sw) = o.vjp(x, w, g, layout=layout), o.vjp(x, w, g, layout=layout, absolute=True)
    check_scaled(gx, rx, sx, "f32", "ragged dx")
    check_scaled(gw, rw, sw, "f32", "ragged dw")


@pytest.mark.parametrize("n", [400, 3000])
@pytest.mark.parametrize("order", ["sorted", "sorted_out_of_range_ends", "unsorted"])
def test_class_indexed(order, n):
    """Species-indexed weights: sorted classes (the pages' contract) and an
    unsorted order (still exact), out-of-range classes (zero row, zero dx,
    no weight-gradient contribution), int64 indices for the unsorted case;
    3000 samples span several row chunks of the weight gradient.  "sorted"
    puts an out-of-range class inside the first chunk (which then takes the
    masked pass); "sorted_out_of_range_ends" keeps the order sorted with
    leading -1 and trailing num_classes, so every chunk takes the
    binary-searched pass over its classes' runs, including the end chunks."""
    sp = _sp()
    wl = workloads.WORKLOADS[7]
    o = olin.Linear(wl.irreps_in, wl.irreps_out)
    h = sp.linear_create(wl.irreps_in, wl.irreps_out, layout="ir_mul")
    inp = workloads.linear_inputs(wl, o.weight_numel, n=n)
    cls = inp["classes"].copy()
    if order == "unsorted":
        cls = np.random.default_rng(3).permutation(cls).astype(np.int64)
    if order == "sorted_out_of_range_ends":
        cls[:3] = -1
        cls[-4:] = wl.num_classes
        assert np.all(np.diff(cls) >= 0)
        oob = np.r_[0:3, n - 4:n]
    else:
        cls[5] = wl.num_classes      # out of range
        oob = np.array([5])
    g = workloads.output_gradient(n, o.dim_out, "f32", seed=71)
    announce(f"linear class-indexed {order} n={n}")
    got = _fwd(sp, h, inp["x"], inp["w"], cls)
    check_scaled(got, o.fwd(inp["x"], inp["w"], indices=cls), o.fwd(inp["x"], inp["w"], indices=cls, absolute=True),
                 "f32", f"class-indexed fwd {order}")
    assert np.count_nonzero(got[oob]) == 0
    gx, gw = _bwd(sp, h, inp["x"], inp["w"], g, cls, need_dw=False)
    assert gw is None
    rx, rw = o.vjp(inp["x"], inp["w"], g, indices=cls)
    sx, sw = o.vjp(inp["x"], inp["w"], g, indices=cls, absolute=True)
    check_scaled(gx, rx, sx, "f32", f"class-indexed dx {order}")
    assert np.count_nonzero(gx[oob]) == 0
    # weight gradient: one row per class, each summing its own samples
    gx2, gw = _bwd(sp, h, inp["x"], inp["w"], g, cls)
    assert gw.shape == inp["w"].shape
    assert np.array_equal(gx2, gx)
    check_scaled(gw, rw, sw, "f32", f"class-indexed dw {order}")


@pytest.mark.parametrize("layout", ["ir_mul", "mul_ir"])
def test_class_indexed_full_size(layout):
    """The species layer at the shape the benchmark times: 50,000 atoms,
    10 sorted classes (about 25 weight-gradient row chunks), in the same
    launch configuration.  Forward and dx on 256 sampled rows (the oracle on
    those rows); for the weight gradient a second call whose output gradient
    is zero except on 1,024 sampled rows spread over every chunk, so the
    oracle on those rows alone gives all of dw (the oracle over all 50,000
    rows takes minutes)."""
    sp = _sp()
    wl = workloads.WORKLOADS[7]
    o = olin.Linear(wl.irreps_in, wl.irreps_out)
    h = sp.linear_create(wl.irreps_in, wl.irreps_out, layout=layout)
    inp = workloads.linear_inputs(wl, o.weight_numel)
    n = wl.n
    cls = inp["classes"]
    assert n == 50000 and np.all(np.diff(cls) >= 0) and len(np.unique(cls)) == wl.num_classes
    g = workloads.output_gradient(n, o.dim_out, "f32", seed=72)
    announce(f"linear class-indexed full size {layout} n={n}")
    got = _fwd(sp, h, inp["x"], inp["w"], cls)
    gx, gw = _bwd(sp, h, inp["x"], inp["w"], g, cls)
    rows = np.sort(np.random.default_rng(73).choice(n, 256, replace=False))
    xs, cs, gs = inp["x"][rows], cls[rows], g[rows]
    check_scaled(got[rows], o.fwd(xs, inp["w"], layout=layout, indices=cs),
                 o.fwd(xs, inp["w"], layout=layout, indices=cs, absolute=True), "f32", f"full-size fwd {layout}")
    (rx, _), (sx, _) = (o.vjp(xs, inp["w"], gs, layout=layout, indices=cs),
                        o.vjp(xs, inp["w"], gs, layout=layout, indices=cs, absolute=True))
    check_scaled(gx[rows], rx, sx, "f32", f"full-size dx {layout}")
    assert gw.shape == inp["w"].shape and np.all(np.isfinite(gw))
    keep = np.sort(np.random.default_rng(74).choice(n, 1024, replace=False))
    gm = np.zeros_like(g)
    gm[keep] = g[keep]
    _, gw2 = _bwd(sp, h, inp["x"], inp["w"], gm, cls)
    xk, ck, gk = inp["x"][keep], cls[keep], g[keep]
    (_, rw), (_, sw) = (o.vjp(xk, inp["w"], gk, layout=layout, indices=ck),
                        o.vjp(xk, inp["w"], gk, layout=layout, indices=ck, absolute=True))
    check_scaled(gw2, rw, sw, "f32", f"full-size dw {layout}")


@pytest.mark.parametrize("layout", ["ir_mul", "mul_ir"])
@pytest.mark.parametrize("classes", [False, True])
def test_many_tiles_per_workgroup(layout, classes):
    """More tiles than the device holds workgroups at once (2,800 tiles
    of 128 rows), an output block no input type feeds (zero tiles), and
    with classes: a sorted half and an unsorted half, out-of-range classes,
    and a run of 400 samples with no valid class (tiles with no pass,
    stored as zeros)."""
    sp = _sp()
    import torch
    ins, outs = "32x0e+16x1o+8x1o", "40x0e+24x1o+8x2e"
    o = olin.Linear(ins, outs)
    h = sp.linear_create(ins, outs, layout=layout)
    n, nc = 40000, 7
    rng = np.random.default_rng(75)
    x = rng.standard_normal((n, o.dim_in), dtype=np.float32)
    w = rng.standard_normal((nc if classes else 1, o.weight_numel), dtype=np.float32)
    cls = None
    if classes:
        cls = rng.integers(-1, nc + 1, n).astype(np.int32)
        cls[:20000] = np.sort(cls[:20000])
        cls[25000:25400] = -1
    announce(f"linear many tiles {layout} classes={classes}")
    out = sp.linear_fwd(h, dev(x), dev(w), classes=None if cls is None else dev(cls),
                        num_classes=nc if classes else None)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    rows = np.sort(np.concatenate([rng.choice(n, 600, replace=False), np.arange(24990, 25010), [0, n - 1]]))
    kw = {} if cls is None else {"indices": cls[rows]}
    check_scaled(got[rows], o.fwd(x[rows], w, layout=layout, **kw), o.fwd(x[rows], w, layout=layout, absolute=True, **kw),
                 "f32", f"many tiles {layout} classes={classes}")
    if classes:
        bad = (cls < 0) | (cls >= nc)
        assert np.count_nonzero(got[bad]) == 0
    # the 2e block (the last 8 x 5 columns in either layout) has no input of its type
    assert np.count_nonzero(got[:, o.dim_out - 40:]) == 0


def test_float64_backward_and_determinism():
    sp = _sp()
    ins, outs = "16x0e+8x1o+8x1o", "12x0e+20x1o"
    o = olin.Linear(ins, outs)
    h = sp.linear_create(ins, outs, layout="mul_ir", dtype="f64")
    rng = np.random.default_rng(12)
    x = rng.standard_normal((3000, o.dim_in))
    w = rng.standard_normal((1, o.weight_numel))
    g = rng.standard_normal((3000, o.dim_out))
    announce("linear f64 backward")
    gx, gw = _bwd(sp, h, x, w, g)
    (rx, rw), (sx, sw) = o.vjp(x, w, g, layout="mul_ir"), o.vjp(x, w, g, layout="mul_ir", absolute=True)
    check_scaled(gx, rx, sx, "f64", "f64 dx")
    check_scaled(gw, rw, sw, "f64", "f64 dw (several row chunks)")
    gx2, gw2 = _bwd(sp, h, x, w, g)
    assert np.array_equal(gx, gx2) and np.array_equal(gw, gw2)


def test_empty_batch():
    sp = _sp()
    import torch
    h = sp.linear_create("4x0e+2x1o", "3x0e+2x1o")
    x = torch.empty(0, h.dim_in, device="cuda")
    w = torch.randn(1, h.weight_numel, device="cuda")
    announce("linear empty batch")
    out = sp.linear_fwd(h, x, w)
    gx, gw = sp.linear_bwd(h, x, w, torch.empty(0, h.dim_out, device="cuda"))
    torch.cuda.synchronize()
    assert out.shape == (0, h.dim_out) and gx.shape == (0, h.dim_in)
    assert torch.count_nonzero(gw).item() == 0
