"""GPU checks of the row-pointer form of the channelwise convolution: the
row pointers built on the device equal a host binary search of the sorted
destinations (and of the sources in src_perm order), tp_conv_fwd_rowptr
reproduces tp_conv_fwd and tp_conv_bwd_rowptr reproduces tp_conv_bwd bit
for bit (the same edges in the same order) on the specialised kernels
(molecular batch, medium graph), the destination-split kernel and the
table-driven kernel, with sum and mean, shared weights and both index
widths; forward and backward are also checked against the float64 oracle
(scaled error <= 1e-5); at the large workload's full size the row-pointer
forms match the searching ones bit for bit."""

import numpy as np
import pytest

import workloads
from oracle import tp as otp
from tests._gpu import announce, check_scaled, dev, need_gpu

pytestmark = pytest.mark.gpu


def _sp():
    need_gpu()
    import segmented_polynomials_amd as sp
    return sp


@pytest.mark.parametrize("idx", ["int32", "int64"])
def test_rowptr_build_matches_host_search(idx):
    sp = _sp()
    import torch
    rng = np.random.default_rng(81)
    n_nodes = 1000
    dst = np.sort(rng.integers(0, n_nodes + 5, 20000))   # some destinations past n_nodes
    dst[:7] = 0
    D = dev(dst, getattr(torch, idx))
    announce(f"rowptr build {idx}")
    rp = sp.tp_rowptr_build(D, n_nodes).cpu().numpy()
    ref = np.searchsorted(dst, np.arange(n_nodes + 1), side="left")
    assert rp.dtype == np.dtype(idx) and np.array_equal(rp, ref)
    # no edges: every pointer is zero
    E = torch.empty(0, dtype=getattr(torch, idx), device="cuda")
    assert int(sp.tp_rowptr_build(E, 5).abs().sum()) == 0


def _pair(sp, h, inp, it):
    import torch
    td = torch.float32 if h.dtype == "f32" else torch.float64
    x, s, w = dev(inp["x"], td), dev(inp["sh"], td), dev(inp["w"], td)
    src, dst = dev(inp["src"], it), dev(inp["dst"], it)
    n = inp["n_nodes"]
    a = sp.tp_conv_fwd(h, x, s, w, src, dst, n_nodes=n)
    rp = sp.tp_rowptr_build(dst, n)
    b = sp.tp_conv_fwd_rowptr(h, x, s, w, src, rp)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


@pytest.mark.parametrize("n", [2, 3])
@pytest.mark.parametrize("idx", ["int32", "int64"])
def test_workloads_rowptr_equals_search(n, idx):
    """The molecular batch (destination-split kernel) and the medium graph
    (one wave per destination)."""
    sp = _sp()
    import torch
    wl = workloads.WORKLOADS[n]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    inp = workloads.tp_inputs(wl, o.weight_fan_in())
    lay = wl.layouts[0]
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=lay)
    announce(f"rowptr forward {wl.name} {idx} ({h.kernel_name})")
    a, b = _pair(sp, h, inp, getattr(torch, idx))
    assert np.array_equal(a, b)
    args = (inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"])
    check_scaled(b, o.conv(*args, layout=lay), o.conv(*args, layout=lay, absolute=True), "f32", "rowptr fwd")


@pytest.mark.parametrize("case", [
    dict(force_generic=True),
    dict(reduce="mean"),
    dict(shared_weights=True),
])
def test_rowptr_variants(case):
    """Table-driven kernel, mean reduction and one shared weight row, on a
    ragged graph with isolated destinations."""
    sp = _sp()
    import torch
    in1, in2, filt = "16x0e+16x1o+16x2e", "0e+1o+2e", "0e+1o+2e"
    o = otp.ChannelwiseTP(in1, in2, filt)
    rng = np.random.default_rng(82)
    n_src, n_dst, n_e = 40, 37, 400
    src = rng.integers(0, n_src, n_e)
    dst = np.sort(rng.integers(0, n_dst, n_e))
    rows = 1 if case.get("shared_weights") else n_e
    inp = dict(x=rng.standard_normal((n_src, o.dim_in1)).astype(np.float32).astype(np.float64),
               sh=rng.standard_normal((n_e, o.dim_in2)).astype(np.float32).astype(np.float64),
               w=rng.standard_normal((rows, o.weight_numel)).astype(np.float32).astype(np.float64),
               src=src, dst=dst, n_nodes=n_dst)
    h = sp.tp_create(in1, in2, filt, layout="ir_mul", **case)
    announce(f"rowptr variant {case} ({h.kernel_name})")
    a, b = _pair(sp, h, inp, torch.int32)
    assert np.array_equal(a, b)
    args = (inp["x"], inp["sh"], inp["w"], src, dst, n_dst)
    red = case.get("reduce", "sum")
    ref = o.conv(*args, layout="ir_mul", reduce=red)
    scale = o.conv(*args, layout="ir_mul", reduce=red, absolute=True)
    check_scaled(b, ref, scale, "f32", "rowptr variant")


def test_rowptr_validate():
    """With VALIDATE the pointers are checked on the host: a decreasing
    entry is E_UNSORTED, a wrong end is E_RANGE."""
    sp = _sp()
    import torch
    h = sp.tp_create("8x0e+8x1o", "0e+1o", "0e+1o", validate=True)
    n_e, n = 30, 6
    x = torch.zeros((10, h.dim_in1), device="cuda")
    s = torch.zeros((n_e, h.dim_in2), device="cuda")
    w = torch.zeros((n_e, h.weight_numel), device="cuda")
    src = torch.zeros(n_e, dtype=torch.int32, device="cuda")
    good = torch.tensor([0, 5, 10, 15, 20, 25, 30], dtype=torch.int32, device="cuda")
    announce("rowptr validate")
    sp.tp_conv_fwd_rowptr(h, x, s, w, src, good)
    bad = torch.tensor([0, 5, 4, 15, 20, 25, 30], dtype=torch.int32, device="cuda")
    with pytest.raises(sp.SegpolyError, match="-4"):
        sp.tp_conv_fwd_rowptr(h, x, s, w, src, bad)
    end = torch.tensor([0, 5, 10, 15, 20, 25, 29], dtype=torch.int32, device="cuda")
    with pytest.raises(sp.SegpolyError, match="-7"):
        sp.tp_conv_fwd_rowptr(h, x, s, w, src, end)


@pytest.mark.parametrize("idx", ["int32", "int64"])
def test_src_rowptr_build_matches_host_search(idx):
    sp = _sp()
    import torch
    rng = np.random.default_rng(83)
    n_src, n_e = 700, 15000
    src = rng.integers(0, n_src, n_e)
    src[:9] = 3
    perm = np.argsort(src, kind="stable")
    S, P = dev(src, getattr(torch, idx)), dev(perm, getattr(torch, idx))
    announce(f"src rowptr build {idx}")
    rp = sp.tp_src_rowptr_build(S, P, n_src).cpu().numpy()
    ref = np.searchsorted(src[perm], np.arange(n_src + 1), side="left")
    assert rp.dtype == np.dtype(idx) and np.array_equal(rp, ref)


def _bwd_pair(sp, h, inp, it, g):
    import torch
    td = torch.float32 if h.dtype == "f32" else torch.float64
    x, s, w, G = dev(inp["x"], td), dev(inp["sh"], td), dev(inp["w"], td), dev(g, td)
    src, dst = dev(inp["src"], it), dev(inp["dst"], it)
    perm = dev(np.argsort(inp["src"], kind="stable"), it)
    n = inp["n_nodes"]
    a = sp.tp_conv_bwd(h, x, s, w, G, src, dst, perm, n_nodes=n)
    rp = sp.tp_rowptr_build(dst, n)
    srp = sp.tp_src_rowptr_build(src, perm, x.shape[0])
    b = sp.tp_conv_bwd_rowptr(h, x, s, w, G, src, dst, perm, rp, srp)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in a], [t.cpu().numpy() for t in b]


@pytest.mark.parametrize("n", [2, 3])
@pytest.mark.parametrize("idx", ["int32", "int64"])
def test_workloads_bwd_rowptr_equals_search(n, idx):
    sp = _sp()
    import torch
    wl = workloads.WORKLOADS[n]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    inp = workloads.tp_inputs(wl, o.weight_fan_in())
    lay = wl.layouts[0]
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=lay)
    g = workloads.output_gradient(inp["n_nodes"], h.dim_out, "f32", seed=85)
    announce(f"rowptr backward {wl.name} {idx} ({h.kernel_name})")
    a, b = _bwd_pair(sp, h, inp, getattr(torch, idx), g)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    args = (inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"], g)
    ref = o.conv_vjp(*args, layout=lay)
    scale = o.conv_vjp(*args, layout=lay, absolute=True)
    for got, r, sc, name in zip(b, ref, scale, ("dx", "dsh", "dw")):
        check_scaled(got, r, sc, "f32", f"rowptr bwd {name}")


@pytest.mark.parametrize("case", [
    dict(force_generic=True),
    dict(force_generic=True, reduce="mean"),
    dict(reduce="mean"),
    dict(shared_weights=True),
])
def test_bwd_rowptr_variants(case):
    """Table-driven kernels (sum and mean), mean reduction and one shared
    weight row, on a ragged graph with isolated destinations and sources."""
    sp = _sp()
    import torch
    in1, in2, filt = "16x0e+16x1o+16x2e", "0e+1o+2e", "0e+1o+2e"
    o = otp.ChannelwiseTP(in1, in2, filt)
    rng = np.random.default_rng(84)
    n_src, n_dst, n_e = 40, 37, 400
    src = rng.integers(0, n_src - 3, n_e)       # the last sources have no edges
    dst = np.sort(rng.integers(0, n_dst, n_e))
    rows = 1 if case.get("shared_weights") else n_e
    inp = dict(x=rng.standard_normal((n_src, o.dim_in1)).astype(np.float32).astype(np.float64),
               sh=rng.standard_normal((n_e, o.dim_in2)).astype(np.float32).astype(np.float64),
               w=rng.standard_normal((rows, o.weight_numel)).astype(np.float32).astype(np.float64),
               src=src, dst=dst, n_nodes=n_dst)
    g = rng.standard_normal((n_dst, o.dim_out)).astype(np.float32).astype(np.float64)
    h = sp.tp_create(in1, in2, filt, layout="ir_mul", **case)
    announce(f"rowptr backward variant {case} ({h.kernel_name})")
    a, b = _bwd_pair(sp, h, inp, torch.int32, g)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    kw = dict(layout="ir_mul", reduce=case.get("reduce", "sum"), shared_weights=case.get("shared_weights", False))
    ref = o.conv_vjp(inp["x"], inp["sh"], inp["w"], src, dst, n_dst, g, **kw)
    scale = o.conv_vjp(inp["x"], inp["sh"], inp["w"], src, dst, n_dst, g, absolute=True, **kw)
    for got, r, sc, name in zip(b, ref, scale, ("dx", "dsh", "dw")):
        check_scaled(got, r, sc, "f32", f"rowptr bwd variant {name}")


def test_bwd_rowptr_validate():
    """With VALIDATE each pointer array must equal what its builder gives:
    E_RANGE for a wrong entry of either."""
    sp = _sp()
    import torch
    h = sp.tp_create("8x0e+8x1o", "0e+1o", "0e+1o", validate=True)
    n_e, n, n_src = 30, 6, 10
    x = torch.zeros((n_src, h.dim_in1), device="cuda")
    s = torch.zeros((n_e, h.dim_in2), device="cuda")
    w = torch.zeros((n_e, h.weight_numel), device="cuda")
    g = torch.zeros((n, h.dim_out), device="cuda")
    src_h = np.arange(n_e) % n_src
    src = dev(src_h, torch.int32)
    dst = dev(np.repeat(np.arange(n), 5), torch.int32)
    perm = dev(np.argsort(src_h, kind="stable"), torch.int32)
    rp = sp.tp_rowptr_build(dst, n)
    srp = sp.tp_src_rowptr_build(src, perm, n_src)
    announce("rowptr backward validate")
    sp.tp_conv_bwd_rowptr(h, x, s, w, g, src, dst, perm, rp, srp)
    bad = rp.clone()
    bad[2] += 1
    with pytest.raises(sp.SegpolyError, match="-7"):
        sp.tp_conv_bwd_rowptr(h, x, s, w, g, src, dst, perm, bad, srp)
    bad = srp.clone()
    bad[4] -= 1
    with pytest.raises(sp.SegpolyError, match="-7"):
        sp.tp_conv_bwd_rowptr(h, x, s, w, g, src, dst, perm, rp, bad)


def test_full_size_rowptr_equals_search():
    """The large workload (600k edges, 20k nodes, ir_mul, two channels per
    lane) in the benchmark's launch configuration: the row-pointer forward
    and backward reproduce the searching ones bit for bit, and a sample of
    destination rows matches the oracle."""
    sp = _sp()
    import torch
    wl = workloads.WORKLOADS[4]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout="ir_mul")
    inp = workloads.tp_inputs(wl, o.weight_fan_in())
    announce(f"rowptr full-size workload 4 ({h.kernel_name})")
    a, b = _pair(sp, h, inp, torch.int32)
    assert np.array_equal(a, b)
    rng = np.random.default_rng(86)
    nodes = np.unique(np.concatenate([[0, wl.n_nodes - 1], rng.integers(0, wl.n_nodes, 30)]))
    sel = np.nonzero(np.isin(inp["dst"], nodes))[0]
    args = (inp["x"], inp["sh"][sel], inp["w"][sel], inp["src"][sel], inp["dst"][sel], wl.n_nodes)
    ref = o.conv(*args, layout="ir_mul")
    scale = o.conv(*args, layout="ir_mul", absolute=True)
    check_scaled(b[nodes], ref[nodes], scale[nodes], "f32", "rowptr full-size fwd")
    del a, b
    g = workloads.output_gradient(wl.n_nodes, h.dim_out, "f32", seed=87)
    ga, gb = _bwd_pair(sp, h, inp, torch.int32, g)
    for u, v in zip(ga, gb):
        assert np.array_equal(u, v)
