"""GPU parity of the backward (vector-Jacobian product) of the fused
channelwise tensor-product convolution: the HIP kernels, called through the
C ABI, against the float64 oracle's conv_vjp on the same seeded inputs.
Tolerance: scaled error (oracle.metrics, scale = the VJP over absolute
operands) <= 1e-5 in float32, <= 1e-12 in float64."""

import numpy as np
import pytest

import workloads
from oracle import layout as ol
from oracle import tp as otp
from tests._gpu import announce, check_scaled, dev, need_gpu

pytestmark = pytest.mark.gpu


def _sp():
    need_gpu()
    import segmented_polynomials_amd as sp
    return sp


def _bwd(sp, h, inp, g, idx_dtype=None):
    import torch
    td = torch.float32 if h.dtype == "f32" else torch.float64
    x, s, w, gd = dev(inp["x"], td), dev(inp["sh"], td), dev(inp["w"], td), dev(g, td)
    src = dst = perm = None
    if inp["src"] is not None:
        it = idx_dtype or torch.int32
        src, dst = dev(inp["src"], it), dev(inp["dst"], it)
        perm = dev(workloads.src_permutation(inp["src"]), it)
    out = sp.tp_conv_bwd(h, x, s, w, gd, src, dst, perm, n_nodes=inp["n_nodes"])
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


def _oracle(o, inp, g, layout):
    args = (inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"], g)
    ref = o.conv_vjp(*args, layout=layout)
    scale = o.conv_vjp(*args, layout=layout, absolute=True)
    return ref, scale


def _check_all(got, ref, scale, dtype, what):
    for name, a, b, c in zip(("dx", "dsh", "dw"), got, ref, scale):
        assert a.shape == b.shape, (name, a.shape, b.shape)
        check_scaled(a, b, c, dtype, f"{what} {name}")


@pytest.mark.parametrize("n,layout,kw", [
    (1, "mul_ir", {}),
    (2, "mul_ir", {}),
    (3, "ir_mul", dict(n_nodes=800, degree=16)),
    (4, "mul_ir", dict(n_nodes=300, degree=30)),
    (4, "ir_mul", dict(n_nodes=300, degree=30)),
])
def test_workload_vjp_parity(n, layout, kw):
    sp = _sp()
    wl = workloads.WORKLOADS[n]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=layout, dtype=wl.dtype)
    inp = workloads.tp_inputs(wl, o.weight_fan_in(), **kw)
    g = workloads.output_gradient(inp["n_nodes"], o.dim_out, wl.dtype, seed=70 + n)
    announce(f"tp bwd workload {n} {layout} edges={inp['sh'].shape[0]}")
    got = _bwd(sp, h, inp, g)
    ref, scale = _oracle(o, inp, g, layout)
    _check_all(got, ref, scale, wl.dtype, f"workload {n} {layout}")


@pytest.mark.parametrize("layout", ["mul_ir", "ir_mul"])
def test_full_size_workload4_sampled(layout):
    """600k edges, 20k nodes, in the launch configuration the benchmark
    times; the oracle recomputes the gradients of a sample of sources from
    the edges that read them (all of them, so those dx rows are complete)."""
    sp = _sp()
    wl = workloads.WORKLOADS[4]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=layout)
    inp = workloads.tp_inputs(wl, o.weight_fan_in())
    g = workloads.output_gradient(wl.n_nodes, o.dim_out, "f32", seed=74)
    announce(f"tp bwd full-size workload 4 {layout}")
    dx, dsh, dw = _bwd(sp, h, inp, g)
    rng = np.random.default_rng(98)
    srcs = np.unique(np.concatenate([[0, wl.n_nodes - 1], rng.integers(0, wl.n_nodes, 40)]))
    sel = np.nonzero(np.isin(inp["src"], srcs))[0]
    sub = dict(inp, sh=inp["sh"][sel], w=inp["w"][sel], src=inp["src"][sel], dst=inp["dst"][sel])
    ref, scale = _oracle(o, sub, g, layout)
    check_scaled(dx[srcs], ref[0][srcs], scale[0][srcs], "f32", f"full workload 4 {layout} dx")
    check_scaled(dsh[sel], ref[1], scale[1], "f32", f"full workload 4 {layout} dsh")
    check_scaled(dw[sel], ref[2], scale[2], "f32", f"full workload 4 {layout} dw")
    for a in (dx, dsh, dw):
        assert np.all(np.isfinite(a))


@pytest.mark.parametrize("mul,layout", [(40, "mul_ir"), (64, "ir_mul"), (80, "ir_mul"), (128, "mul_ir"),
                                        (200, "ir_mul"), (77, "mul_ir")])
def test_ragged_graph_and_partial_tiles(mul, layout):
    """In-degrees 0..6 with isolated destinations, sources that no edge
    reads, partial channel tiles, several tiles (200 channels: two tiles of
    pairs; 77, odd: two tiles of single channels) with the harmonic
    gradient folded from per-tile partials; int64 indices for one case."""
    sp = _sp()
    import torch
    in1 = f"{mul}x0e+{mul}x1o+{mul}x2e"
    o = otp.ChannelwiseTP(in1, "0e+1o+2e+3o", "0e+1o+2e")
    h = sp.tp_create(in1, "0e+1o+2e+3o", "0e+1o+2e", layout=layout)
    wl = workloads.TPWorkload(**{**workloads.WORKLOADS[4].__dict__, "irreps_in1": in1})
    inp = workloads.tp_inputs(wl, o.weight_fan_in(), n_nodes=157, degree=6, graph="ragged", seed=mul)
    unread = np.bincount(inp["src"], minlength=157) == 0
    assert np.any(unread)
    g = workloads.output_gradient(157, o.dim_out, "f32", seed=mul + 1)
    announce(f"tp bwd ragged mul={mul} {layout}")
    got = _bwd(sp, h, inp, g, idx_dtype=torch.int64 if mul == 80 else torch.int32)
    ref, scale = _oracle(o, inp, g, layout)
    _check_all(got, ref, scale, "f32", f"ragged mul={mul} {layout}")
    assert np.count_nonzero(got[0][unread]) == 0


def test_float64():
    sp = _sp()
    wl = workloads.WORKLOADS[4]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    wl64 = workloads.TPWorkload(**{**wl.__dict__, "dtype": "f64"})
    inp = workloads.tp_inputs(wl64, o.weight_fan_in(), n_nodes=50, degree=9)
    g = workloads.output_gradient(50, o.dim_out, "f64", seed=5)
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout="mul_ir", dtype="f64")
    announce("tp bwd f64")
    got = _bwd(sp, h, inp, g)
    ref, scale = _oracle(o, inp, g, "mul_ir")
    _check_all(got, ref, scale, "f64", "f64")


def test_out_of_range_edges_get_zero_gradients():
    """Without VALIDATE, edges whose source or destination is outside its
    range contribute nothing: their gradients are zero and they add nothing
    to any source; the other edges match the oracle on the valid subset."""
    sp = _sp()
    in1, in2, filt = "32x0e+32x1o", "0e+1o+2e", "0e+1o+2e"
    o = otp.ChannelwiseTP(in1, in2, filt)
    h = sp.tp_create(in1, in2, filt)
    rng = np.random.default_rng(12)
    n_src, n_dst, n_e = 13, 9, 120
    src = rng.integers(0, n_src, n_e)
    src[::7] = n_src + 3                        # sources out of range
    dst = np.sort(rng.integers(-2, n_dst + 2, n_e))   # some destinations out of range
    inp = dict(x=rng.standard_normal((n_src, o.dim_in1), dtype=np.float32),
               sh=rng.standard_normal((n_e, o.dim_in2), dtype=np.float32),
               w=rng.standard_normal((n_e, o.weight_numel), dtype=np.float32),
               src=src.astype(np.int32), dst=dst.astype(np.int32), n_nodes=n_dst)
    g = workloads.output_gradient(n_dst, o.dim_out, "f32", seed=3)
    announce("tp bwd out-of-range edges")
    dx, dsh, dw = _bwd(sp, h, inp, g)
    ok = (src < n_src) & (dst >= 0) & (dst < n_dst)
    assert (~ok).sum() > 10 and ok.sum() > 50
    assert np.count_nonzero(dsh[~ok]) == 0 and np.count_nonzero(dw[~ok]) == 0
    sub = dict(inp, sh=inp["sh"][ok], w=inp["w"][ok], src=inp["src"][ok], dst=inp["dst"][ok])
    ref, scale = _oracle(o, sub, g, "mul_ir")
    check_scaled(dx, ref[0], scale[0], "f32", "out-of-range dx")
    check_scaled(dsh[ok], ref[1], scale[1], "f32", "out-of-range dsh")
    check_scaled(dw[ok], ref[2], scale[2], "f32", "out-of-range dw")


def test_no_edges_and_no_nodes():
    sp = _sp()
    import torch
    h = sp.tp_create("32x0e+32x1o", "0e+1o+2e", "0e+1o+2e")
    x = torch.randn(4, h.dim_in1, device="cuda")
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    announce("tp bwd no edges")
    dx, dsh, dw = sp.tp_conv_bwd(h, x, torch.empty(0, h.dim_in2, device="cuda"),
                                 torch.empty(0, h.weight_numel, device="cuda"),
                                 torch.randn(6, h.dim_out, device="cuda"), e, e, e, n_nodes=6)
    torch.cuda.synchronize()
    assert dx.shape == x.shape and torch.count_nonzero(dx).item() == 0
    assert dsh.numel() == 0 and dw.numel() == 0
    # edges but no destinations: every gradient is zero
    n_e = 10
    src = torch.randint(0, 4, (n_e,), dtype=torch.int32, device="cuda")
    dst = torch.zeros(n_e, dtype=torch.int32, device="cuda")
    perm = torch.argsort(src, stable=True).to(torch.int32)
    announce("tp bwd no destinations")
    dx, dsh, dw = sp.tp_conv_bwd(h, x, torch.randn(n_e, h.dim_in2, device="cuda"),
                                 torch.randn(n_e, h.weight_numel, device="cuda"),
                                 torch.empty(0, h.dim_out, device="cuda"), src, dst, perm, n_nodes=0)
    torch.cuda.synchronize()
    for a in (dx, dsh, dw):
        assert torch.count_nonzero(a).item() == 0


def test_deterministic_and_layouts_agree():
    sp = _sp()
    wl = workloads.WORKLOADS[4]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    inp = workloads.tp_inputs(wl, o.weight_fan_in(), n_nodes=200, degree=30)
    g = workloads.output_gradient(200, o.dim_out, "f32", seed=8)
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout="mul_ir")
    announce("tp bwd determinism")
    a = _bwd(sp, h, inp, g)
    b = _bwd(sp, h, inp, g)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    h_ir = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout="ir_mul")
    inp_ir = dict(inp, x=ol.transpose(inp["x"], o.in1, "mul_ir", "ir_mul").astype(np.float32))
    g_ir = ol.transpose(g, o.out, "mul_ir", "ir_mul").astype(np.float32)
    c = _bwd(sp, h_ir, inp_ir, g_ir)
    assert np.array_equal(ol.transpose(c[0], o.in1, "ir_mul", "mul_ir").astype(np.float32), a[0])
    assert np.array_equal(c[2], a[2])
    # dsh reduces over channels in the same order in both layouts
    assert np.array_equal(c[1], a[1])




def test_mean_reduction_backward():
    sp = _sp()
    wl = workloads.WORKLOADS[4]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout="ir_mul", reduce="mean")
    inp = workloads.tp_inputs(wl, o.weight_fan_in(), n_nodes=150, degree=12, graph="ragged", seed=78)
    g = workloads.output_gradient(150, o.dim_out, "f32", seed=79)
    announce("tp bwd mean reduction")
    got = _bwd(sp, h, inp, g)
    args = (inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"], g)
    ref = o.conv_vjp(*args, layout="ir_mul", reduce="mean")
    scale = o.conv_vjp(*args, layout="ir_mul", absolute=True, reduce="mean")
    _check_all(got, ref, scale, "f32", "mean reduction")


@pytest.mark.parametrize("layout,dtype", [("mul_ir", "f32"), ("ir_mul", "f32"), ("mul_ir", "f64")])
def test_shared_weights_backward(layout, dtype):
    """One weight row shared by every edge: grad_w [1, numel] sums the
    per-edge gradients (2,700 edges: three partial sums of 1,024 edges, the
    last ragged); no edges gives a zero row."""
    sp = _sp()
    import torch
    wl = workloads.WORKLOADS[4]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    wlt = workloads.TPWorkload(**{**wl.__dict__, "dtype": dtype})
    inp = workloads.tp_inputs(wlt, o.weight_fan_in(), n_nodes=300, degree=9, seed=91)
    inp = dict(inp, w=np.ascontiguousarray(inp["w"][:1]))
    g = workloads.output_gradient(300, o.dim_out, dtype, seed=92)
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=layout, dtype=dtype, shared_weights=True)
    announce(f"tp bwd shared weights {layout} {dtype} n_edges={len(inp['src'])}")
    got = _bwd(sp, h, inp, g)
    assert got[2].shape == (1, o.weight_numel)
    args = (inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"], g)
    ref = o.conv_vjp(*args, layout=layout, shared_weights=True)
    scale = o.conv_vjp(*args, layout=layout, absolute=True, shared_weights=True)
    _check_all(got, ref, scale, dtype, f"shared weights {layout} {dtype}")
    if dtype == "f32" and layout == "mul_ir":
        td = torch.float32
        x = torch.randn(4, h.dim_in1, device="cuda")
        e = torch.empty(0, dtype=torch.int32, device="cuda")
        announce("tp bwd shared weights, no edges")
        dx, dsh, dw = sp.tp_conv_bwd(h, x, torch.empty(0, h.dim_in2, device="cuda"),
                                     torch.randn(1, h.weight_numel, device="cuda", dtype=td),
                                     torch.randn(6, h.dim_out, device="cuda"), e, e, e, n_nodes=6,
                                     grad_w=torch.full((1, h.weight_numel), 7.0, device="cuda"))
        torch.cuda.synchronize()
        assert torch.count_nonzero(dx).item() == 0 and torch.count_nonzero(dw).item() == 0


@pytest.mark.parametrize("mul,layout,dtype,shared", [
    (1, "ir_mul", "f32", False), (7, "mul_ir", "f64", False), (32, "ir_mul", "f32", True),
    (19, "mul_ir", "f64", True), (32, "mul_ir", "f32", False),
])
def test_edge_parallel_small_multiplicities(mul, layout, dtype, shared):
    """Multiplicities up to 32 take one edge per half-wave: an odd number of
    edges (the last wave's second half idle), sources and destinations out
    of range, isolated nodes, per-edge or shared weights, both layouts and
    float64, against the oracle on the valid edges."""
    sp = _sp()
    in1, in2, filt = f"{mul}x0e+{mul}x1o+{mul}x2e", "0e+1o+2e+3o", "0e+1o+2e"
    o = otp.ChannelwiseTP(in1, in2, filt)
    h = sp.tp_create(in1, in2, filt, layout=layout, dtype=dtype, shared_weights=shared)
    rng = np.random.default_rng(200 + mul)
    n_src, n_dst, n_e = 23, 17, 301
    src = rng.integers(0, n_src - 2, n_e)
    src[::11] = n_src + 1                              # sources out of range
    dst = np.sort(rng.integers(-1, n_dst + 1, n_e))    # destinations out of range at both ends
    npd = np.float32 if dtype == "f32" else np.float64
    rows = 1 if shared else n_e
    inp = dict(x=rng.standard_normal((n_src, o.dim_in1)).astype(npd), sh=rng.standard_normal((n_e, o.dim_in2)).astype(npd),
               w=rng.standard_normal((rows, o.weight_numel)).astype(npd),
               src=src.astype(np.int32), dst=dst.astype(np.int32), n_nodes=n_dst)
    g = workloads.output_gradient(n_dst, o.dim_out, dtype, seed=201)
    announce(f"tp bwd edge-parallel mul={mul} {layout} {dtype} shared={shared}")
    dx, dsh, dw = _bwd(sp, h, inp, g)
    ok = (src < n_src) & (dst >= 0) & (dst < n_dst)
    assert np.count_nonzero(dsh[~ok]) == 0
    if not shared:
        assert np.count_nonzero(dw[~ok]) == 0
    sub = dict(inp, sh=inp["sh"][ok], src=inp["src"][ok], dst=inp["dst"][ok],
               w=inp["w"] if shared else inp["w"][ok])
    args = (sub["x"], sub["sh"], sub["w"], sub["src"], sub["dst"], n_dst, g)
    ref = o.conv_vjp(*args, layout=layout, shared_weights=shared)
    scale = o.conv_vjp(*args, layout=layout, shared_weights=shared, absolute=True)
    check_scaled(dx, ref[0], scale[0], dtype, "edge-parallel dx")
    check_scaled(dsh[ok], ref[1], scale[1], dtype, "edge-parallel dsh")
    check_scaled(dw if shared else dw[ok], ref[2], scale[2], dtype, "edge-parallel dw")


@pytest.mark.parametrize("dtype", ["f32", "f64"])
def test_batch_mode_shared_weights_small_multiplicity(dtype):
    """Batch mode (edge e is node e and source e, no indices) with one shared
    weight row at 8 channels: the edge-parallel kernel writes per-edge weight
    gradients that are summed in fixed chunks; 2,500 samples (three chunks,
    the last ragged) and more source rows than samples."""
    sp = _sp()
    in1, in2, filt = "8x0e+8x1o", "0e+1o+2e", "0e+1o+2e"
    o = otp.ChannelwiseTP(in1, in2, filt)
    h = sp.tp_create(in1, in2, filt, layout="mul_ir", dtype=dtype, shared_weights=True)
    rng = np.random.default_rng(210)
    npd = np.float32 if dtype == "f32" else np.float64
    n, n_src = 2500, 2600
    inp = dict(x=rng.standard_normal((n_src, o.dim_in1)).astype(npd), sh=rng.standard_normal((n, o.dim_in2)).astype(npd),
               w=rng.standard_normal((1, o.weight_numel)).astype(npd), src=None, dst=None, n_nodes=n)
    g = workloads.output_gradient(n, o.dim_out, dtype, seed=211)
    announce(f"tp bwd batch mode shared weights {dtype}")
    dx, dsh, dw = _bwd(sp, h, inp, g)
    assert np.count_nonzero(dx[n:]) == 0          # source rows past the batch receive nothing
    args = (inp["x"][:n], inp["sh"], inp["w"], None, None, n, g)
    ref = o.conv_vjp(*args, layout="mul_ir", shared_weights=True)
    scale = o.conv_vjp(*args, layout="mul_ir", shared_weights=True, absolute=True)
    check_scaled(dx[:n], ref[0], scale[0], dtype, "batch shared dx")
    check_scaled(dsh, ref[1], scale[1], dtype, "batch shared dsh")
    check_scaled(dw, ref[2], scale[2], dtype, "batch shared dw")
