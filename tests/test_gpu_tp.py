"""GPU parity of the fused channelwise tensor-product convolution: the HIP
kernels, called through the C ABI, against the float64 oracle on the same
seeded inputs.  Tolerance: scaled error (oracle.metrics) <= 1e-5 in float32,
<= 1e-12 in float64; integer plumbing bit-exact."""

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


def _run(sp, h, inp, idx_dtype=None):
    import torch
    td = torch.float32 if h.dtype == "f32" else torch.float64
    x, s, w = dev(inp["x"], td), dev(inp["sh"], td), dev(inp["w"], td)
    src = dst = None
    if inp["src"] is not None:
        it = idx_dtype or torch.int32
        src, dst = dev(inp["src"], it), dev(inp["dst"], it)
    out = sp.tp_conv_fwd(h, x, s, w, src, dst, n_nodes=inp["n_nodes"])
    torch.cuda.synchronize()
    return out.cpu().numpy()


def _oracle(o, inp, layout, nodes=None):
    args = (inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"])
    ref = o.conv(*args, layout=layout, nodes=nodes)
    scale = o.conv(*args, layout=layout, absolute=True, nodes=nodes)
    return ref, scale


@pytest.mark.parametrize("n,layout,kw", [
    (1, "mul_ir", {}),
    (2, "mul_ir", {}),
    (3, "ir_mul", {}),
    (4, "mul_ir", dict(n_nodes=400, degree=30)),
    (4, "ir_mul", dict(n_nodes=400, degree=30)),
])
def test_workload_parity(n, layout, kw):
    sp = _sp()
    wl = workloads.WORKLOADS[n]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=layout, dtype=wl.dtype)
    assert h.specialized
    inp = workloads.tp_inputs(wl, o.weight_fan_in(), **kw)
    announce(f"tp workload {n} {layout} {h.kernel_name} edges={inp['sh'].shape[0]}")
    got = _run(sp, h, inp)
    ref, scale = _oracle(o, inp, layout)
    check_scaled(got, ref, scale, wl.dtype, f"workload {n} {layout}")


@pytest.mark.parametrize("layout", ["mul_ir", "ir_mul"])
def test_full_size_workload4_sampled_rows(layout):
    """600k edges, 20k nodes, in the launch configuration the benchmark
    times; the oracle checks a sample of destination rows one by one."""
    sp = _sp()
    wl = workloads.WORKLOADS[4]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=layout)
    inp = workloads.tp_inputs(wl, o.weight_fan_in())
    announce(f"tp full-size workload 4 {layout}")
    got = _run(sp, h, inp)
    rng = np.random.default_rng(99)
    nodes = np.unique(np.concatenate([[0, wl.n_nodes - 1], rng.integers(0, wl.n_nodes, 62)]))
    ref, scale = _oracle(o, inp, layout, nodes=nodes)
    check_scaled(got[nodes], ref, scale, "f32", f"full workload 4 {layout} ({len(nodes)} rows)")
    assert np.all(np.isfinite(got))


@pytest.mark.parametrize("mul", [80, 128, 200])
@pytest.mark.parametrize("layout", ["mul_ir", "ir_mul"])
def test_ragged_graph_and_ragged_channel_tiles(mul, layout):
    """In-degrees 0..40 with isolated destinations; multiplicities that leave
    a partial channel tile; int64 indices for one of the cases."""
    sp = _sp()
    import torch
    in1 = f"{mul}x0e+{mul}x1o+{mul}x2e"
    o = otp.ChannelwiseTP(in1, "0e+1o+2e+3o", "0e+1o+2e")
    h = sp.tp_create(in1, "0e+1o+2e+3o", "0e+1o+2e", layout=layout)
    assert h.specialized
    wl = workloads.WORKLOADS[4]
    wl = workloads.TPWorkload(**{**wl.__dict__, "irreps_in1": in1})
    inp = workloads.tp_inputs(wl, o.weight_fan_in(), n_nodes=157, degree=40, graph="ragged", seed=mul)
    assert np.any(np.bincount(inp["dst"], minlength=157) == 0)
    announce(f"tp ragged mul={mul} {layout}")
    got = _run(sp, h, inp, idx_dtype=torch.int64 if mul == 200 else torch.int32)
    ref, scale = _oracle(o, inp, layout)
    check_scaled(got, ref, scale, "f32", f"ragged mul={mul} {layout}")
    iso = np.bincount(inp["dst"], minlength=157) == 0
    assert np.count_nonzero(got[iso]) == 0


@pytest.mark.parametrize("mul", [32, 16, 12, 5])
@pytest.mark.parametrize("layout", ["mul_ir", "ir_mul"])
def test_small_multiplicities(mul, layout):
    """Multiplicities of at most 32 (most lanes of the wave idle): ragged
    in-degrees 0..40 with isolated destinations, channel counts that are not
    powers of two (12 and 5), int64 indices for one case, and bitwise
    repeatable results."""
    sp = _sp()
    import torch
    wl = workloads.WORKLOADS[2]
    in1 = f"{mul}x0e+{mul}x1o"
    o = otp.ChannelwiseTP(in1, wl.irreps_in2, wl.irreps_out)
    h = sp.tp_create(in1, wl.irreps_in2, wl.irreps_out, layout=layout)
    assert h.specialized
    wl4 = workloads.WORKLOADS[4]
    wl2 = workloads.TPWorkload(**{**wl4.__dict__, "irreps_in1": in1, "irreps_in2": wl.irreps_in2,
                                  "irreps_out": wl.irreps_out, "sh_ls": wl.sh_ls})
    inp = workloads.tp_inputs(wl2, o.weight_fan_in(), n_nodes=157, degree=40, graph="ragged", seed=300 + mul)
    announce(f"tp small multiplicity mul={mul} {layout}")
    it = torch.int64 if mul == 12 else torch.int32
    got = _run(sp, h, inp, idx_dtype=it)
    again = _run(sp, h, inp, idx_dtype=it)
    assert np.array_equal(got, again)
    ref, scale = _oracle(o, inp, layout)
    check_scaled(got, ref, scale, "f32", f"small multiplicity mul={mul} {layout}")
    iso = np.bincount(inp["dst"], minlength=157) == 0
    assert iso.any() and np.count_nonzero(got[iso]) == 0


@pytest.mark.parametrize("case", [
    ("3x0e+5x1o+2x2e+4x3o", "0e+1o+2e", "0e+1o+1e+2e+3o+3e", "mul_ir"),   # non-uniform muls
    ("64x0e+64x1o+64x2e", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o", "ir_mul"),   # registered, forced generic
    ("7x1e+7x2o", "0e+1o+2e", "0e+1o+2e+2o+3e", "ir_mul"),                  # unregistered
])
def test_generic_kernel(case):
    sp = _sp()
    in1, in2, filt, layout = case
    o = otp.ChannelwiseTP(in1, in2, filt)
    h = sp.tp_create(in1, in2, filt, layout=layout, force_generic=True)
    assert h.kernel_name == "tp_conv_generic"
    rng = np.random.default_rng(3)
    n_src, n_dst, n_e = 37, 29, 300
    src = rng.integers(0, n_src, n_e).astype(np.int32)
    dst = np.sort(rng.integers(0, n_dst, n_e)).astype(np.int32)
    ls = [int(t[0]) for t in in2.split("+")]
    inp = dict(x=rng.standard_normal((n_src, o.dim_in1), dtype=np.float32),
               sh=workloads.edge_harmonics(rng.standard_normal((n_e, 3)), ls).astype(np.float32),
               w=rng.standard_normal((n_e, o.weight_numel), dtype=np.float32),
               src=src, dst=dst, n_nodes=n_dst)
    announce(f"tp generic {in1} {layout}")
    got = _run(sp, h, inp)
    ref, scale = _oracle(o, inp, layout)
    check_scaled(got, ref, scale, "f32", f"generic {in1}")


@pytest.mark.parametrize("case", [
    ("5x5o+3x6e", "0e+1o+2e", "4e+4o+5e+5o+6e+6o", "mul_ir", "f32"),
    ("2x6o+3x4e", "6e+5o", "0e+1o+2e+3o+4e+5o+6e+0o+1e+2o+3e+4o+5e+6o", "ir_mul", "f32"),
    ("3x6e+2x5o", "6e+4e", "0e+2e+4e+6e+1o+3o+5o", "ir_mul", "f64"),
    ("3x6e+2x5o", "6e+4e", "0e+2e+4e+6e+1o+3o+5o", "mul_ir", "f64"),
])
def test_generic_kernel_high_l(case):
    """Inputs and outputs up to l = 6, the top of the descriptor envelope:
    every coupling with l1, l2 in 4..6 runs through the table-driven kernel
    (the second operand is any per-edge block, here N(0,1) values)."""
    sp = _sp()
    import torch
    in1, in2, filt, layout, dtype = case
    o = otp.ChannelwiseTP(in1, in2, filt)
    h = sp.tp_create(in1, in2, filt, layout=layout, dtype=dtype)
    assert h.kernel_name == "tp_conv_generic"
    rng = np.random.default_rng(31)
    n_src, n_dst, n_e = 23, 41, 260
    src = rng.integers(0, n_src, n_e).astype(np.int64)
    dst = np.sort(rng.integers(0, n_dst, n_e)).astype(np.int64)
    npd = np.float32 if dtype == "f32" else np.float64
    inp = dict(x=rng.standard_normal((n_src, o.dim_in1)).astype(npd).astype(np.float64),
               sh=rng.standard_normal((n_e, o.dim_in2)).astype(npd).astype(np.float64),
               w=rng.standard_normal((n_e, o.weight_numel)).astype(npd).astype(np.float64),
               src=src, dst=dst, n_nodes=n_dst)
    announce(f"tp generic high l {in1} x {in2} {layout} {dtype}")
    got = _run(sp, h, inp, idx_dtype=torch.int64)
    ref, scale = _oracle(o, inp, layout)
    check_scaled(got, ref, scale, dtype, f"generic high l {in1} {layout} {dtype}")


def test_float64_specialized_and_generic():
    sp = _sp()
    wl = workloads.WORKLOADS[3]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    wl64 = workloads.TPWorkload(**{**wl.__dict__, "dtype": "f64"})
    inp = workloads.tp_inputs(wl64, o.weight_fan_in(), n_nodes=60, degree=7)
    ref, scale = _oracle(o, inp, "ir_mul")
    for fg in (False, True):
        h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout="ir_mul", dtype="f64",
                         force_generic=fg)
        announce(f"tp f64 force_generic={fg}")
        check_scaled(_run(sp, h, inp), ref, scale, "f64", f"f64 generic={fg}")


def test_shared_weights_and_source_count():
    sp = _sp()
    in1, in2, filt = "32x0e+32x1o", "0e+1o+2e", "0e+1o+2e"
    o = otp.ChannelwiseTP(in1, in2, filt)
    h = sp.tp_create(in1, in2, filt, shared_weights=True)
    rng = np.random.default_rng(8)
    n_src, n_dst, n_e = 11, 50, 90          # more destinations than sources
    inp = dict(x=rng.standard_normal((n_src, o.dim_in1), dtype=np.float32),
               sh=rng.standard_normal((n_e, o.dim_in2), dtype=np.float32),
               w=rng.standard_normal((1, o.weight_numel), dtype=np.float32),
               src=rng.integers(0, n_src, n_e).astype(np.int32),
               dst=np.sort(rng.integers(0, n_dst, n_e)).astype(np.int32), n_nodes=n_dst)
    announce("tp shared weights")
    got = _run(sp, h, inp)
    ref, scale = _oracle(o, inp, "mul_ir")
    check_scaled(got, ref, scale, "f32", "shared weights")


@pytest.mark.parametrize("idx", ["int32", "int64"])
def test_split_kernel_range_search(idx):
    """The destination-split kernel (multiplicity 32) on a graph of 78,000
    edges (four rounds of the 64-ary range search), with hub nodes of
    in-degree 300 and 700 (range ends past the 64 entries the end search
    probes first, and many edges per lane group), isolated nodes, the first
    and last node with edges, and out-of-range sources spread over the
    graph and inside a hub's range (they add nothing); int32 and int64
    indices."""
    sp = _sp()
    import torch
    in1, in2, filt = "32x0e+32x1o", "0e+1o+2e", "0e+1o+2e"
    o = otp.ChannelwiseTP(in1, in2, filt)
    h = sp.tp_create(in1, in2, filt, layout="mul_ir")
    rng = np.random.default_rng(42)
    n = 3000
    deg = rng.integers(0, 51, n)
    deg[rng.random(n) < 0.1] = 0
    deg[[0, n - 1]] = [5, 9]
    deg[[1000, 2500]] = [300, 700]
    dst = np.repeat(np.arange(n), deg)
    e = dst.shape[0]
    src = rng.integers(0, n, e)
    hub = np.flatnonzero(dst == 2500)
    bad = np.concatenate([rng.choice(e, 40, replace=False), hub[[3, 400, 650]]])
    src[bad] = n + 7
    inp = dict(x=rng.standard_normal((n, o.dim_in1), dtype=np.float32),
               sh=rng.standard_normal((e, o.dim_in2), dtype=np.float32),
               w=rng.standard_normal((e, o.weight_numel), dtype=np.float32),
               src=src, dst=dst, n_nodes=n)
    assert e > 65536
    announce(f"tp split-kernel range search {idx} edges={e}")
    got = _run(sp, h, inp, idx_dtype=getattr(torch, idx))
    ok = src < n
    sub = dict(inp, sh=inp["sh"][ok], w=inp["w"][ok], src=src[ok], dst=dst[ok])
    nodes = np.unique(np.concatenate([rng.choice(n, 300, replace=False), [0, 1, 1000, 2500, n - 2, n - 1]]))
    ref, scale = _oracle(o, sub, "mul_ir", nodes=nodes)
    check_scaled(got[nodes], ref, scale, "f32", f"split search {idx}")
    assert np.count_nonzero(got[deg == 0]) == 0


def test_no_edges_gives_zero_rows():
    sp = _sp()
    import torch
    h = sp.tp_create("32x0e+32x1o", "0e+1o+2e", "0e+1o+2e")
    x = torch.randn(4, h.dim_in1, device="cuda")
    sh = torch.empty(0, h.dim_in2, device="cuda")
    w = torch.empty(0, h.weight_numel, device="cuda")
    e = torch.empty(0, dtype=torch.int32, device="cuda")
    out = torch.full((6, h.dim_out), 7.0, device="cuda")
    announce("tp no edges")
    sp.tp_conv_fwd(h, x, sh, w, e, e, n_nodes=6, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0


@pytest.mark.parametrize("layout", ["mul_ir", "ir_mul"])
def test_integer_plumbing_bit_exact(layout):
    """Identity paths (l x 0e -> l, 0e x l -> l) with small-integer data:
    every partial sum is an exact float32 integer, so gather, layout
    addressing, weight offsets and the segmented sum must match the oracle
    bit for bit.  The descriptor is the registered large-graph one; the
    inputs zero every operand that would reach a non-identity path."""
    sp = _sp()
    wl = workloads.WORKLOADS[4]
    in1 = "16x0e+16x1o+16x2e"
    o = otp.ChannelwiseTP(in1, wl.irreps_in2, wl.irreps_out)
    h = sp.tp_create(in1, wl.irreps_in2, wl.irreps_out, layout=layout)
    assert h.specialized
    for variant in ("sh0_only", "x0e_only"):
        inp = workloads.integer_tp_inputs(n_src=23, n_edges=600, dim1=o.dim_in1, dim2=o.dim_in2,
                                          numel=o.weight_numel, n_nodes=41, seed=5)
        if variant == "sh0_only":
            inp["sh"][:, 1:] = 0.0                 # only l x 0e -> l paths see a non-zero sh
        else:
            from oracle import layout as ol
            parts = ol.split_blocks(inp["x"], o.in1, layout)
            parts[1][:] = 0.0
            parts[2][:] = 0.0                      # only 0e x l -> l paths see a non-zero x
            inp["x"] = ol.join_blocks(parts, layout).astype(np.float32)
        announce(f"tp integer plumbing {layout} {variant}")
        got = _run(sp, h, inp)
        ref = o.conv(inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"], layout=layout)
        assert np.array_equal(got, ref.astype(np.float32)), variant
        assert np.abs(ref).max() > 100            # the data really exercise the sums


def test_deterministic_and_layouts_agree():
    sp = _sp()
    wl = workloads.WORKLOADS[4]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    inp = workloads.tp_inputs(wl, o.weight_fan_in(), n_nodes=200, degree=30)
    sp = _sp()
    h_mul = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout="mul_ir")
    announce("tp determinism")
    a = _run(sp, h_mul, inp)
    b = _run(sp, h_mul, inp)
    assert np.array_equal(a, b)
    from oracle import layout as ol
    h_ir = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout="ir_mul")
    inp_ir = dict(inp, x=ol.transpose(inp["x"], o.in1, "mul_ir", "ir_mul").astype(np.float32))
    c = _run(sp, h_ir, inp_ir)
    assert np.array_equal(ol.transpose(c, o.out, "ir_mul", "mul_ir").astype(np.float32), a)


def test_equivariance_on_gpu():
    """Rotating the node features and the edge vectors rotates the output
    (float64, so the check is tight)."""
    sp = _sp()
    from oracle import sh as osh, wigner
    in1, in2, filt = "8x0e+8x1o+8x2e", "0e+1o+2e+3o", "0e+1o+2e"
    o = otp.ChannelwiseTP(in1, in2, filt)
    h = sp.tp_create(in1, in2, filt, dtype="f64")
    rng = np.random.default_rng(21)
    n, e = 17, 120
    x = rng.standard_normal((n, o.dim_in1))
    vec = rng.standard_normal((e, 3))
    w = rng.standard_normal((e, o.weight_numel))
    src = rng.integers(0, n, e).astype(np.int32)
    dst = np.sort(rng.integers(0, n, e)).astype(np.int32)
    aa = rng.standard_normal(3)
    R = wigner.rotation_matrix(aa)
    base = dict(x=x, sh=osh.real_sh([0, 1, 2, 3], vec), w=w, src=src, dst=dst, n_nodes=n)
    rot = dict(base, x=x @ wigner.wigner_d_irreps(o.in1, aa).T, sh=osh.real_sh([0, 1, 2, 3], vec @ R.T))
    announce("tp equivariance f64")
    a = _run(sp, h, base)
    b = _run(sp, h, rot)
    assert np.allclose(b, a @ wigner.wigner_d_irreps(o.out, aa).T, atol=1e-11)


@pytest.mark.parametrize("force_generic", [False, True])
def test_mean_reduction(force_generic):
    """reduce="mean" on a ragged graph with isolated destinations (those
    rows stay zero), specialised and generic kernels."""
    sp = _sp()
    wl = workloads.WORKLOADS[4]
    in1 = "32x0e+32x1o+32x2e"
    o = otp.ChannelwiseTP(in1, wl.irreps_in2, wl.irreps_out)
    h = sp.tp_create(in1, wl.irreps_in2, wl.irreps_out, layout="ir_mul", reduce="mean",
                     force_generic=force_generic)
    wl2 = workloads.TPWorkload(**{**wl.__dict__, "irreps_in1": in1})
    inp = workloads.tp_inputs(wl2, o.weight_fan_in(), n_nodes=120, degree=20, graph="ragged", seed=77)
    announce(f"tp mean reduction generic={force_generic}")
    got = _run(sp, h, inp)
    args = (inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"])
    ref = o.conv(*args, layout="ir_mul", reduce="mean")
    scale = o.conv(*args, layout="ir_mul", absolute=True, reduce="mean")
    check_scaled(got, ref, scale, "f32", f"mean generic={force_generic}")
    iso = np.bincount(inp["dst"], minlength=120) == 0
    assert iso.any() and np.count_nonzero(got[iso]) == 0


@pytest.mark.parametrize("mul", [32, 128])
def test_no_source_rows(mul):
    """n_src = 0 with edges: no edge has a source row, so the forward is zero
    and the backward gives zero weight and harmonics gradients (x holds no
    rows; the kernels must not read it).  Both kernels of the forward (the
    destination-split one for mul <= 32 and the wave-per-node one)."""
    sp = _sp()
    import torch
    in1, in2, filt = f"{mul}x0e+{mul}x1o", "0e+1o+2e", "0e+1o+2e"
    o = otp.ChannelwiseTP(in1, in2, filt)
    h = sp.tp_create(in1, in2, filt)
    rng = np.random.default_rng(41)
    n_e, n_dst = 50, 7
    dst = np.sort(rng.integers(0, n_dst, n_e)).astype(np.int32)
    src = rng.integers(0, 5, n_e).astype(np.int32)
    x = torch.zeros((0, o.dim_in1), dtype=torch.float32, device="cuda")
    sh = dev(rng.standard_normal((n_e, o.dim_in2), dtype=np.float32))
    w = dev(rng.standard_normal((n_e, o.weight_numel), dtype=np.float32))
    announce(f"tp no source rows mul={mul}")
    out = sp.tp_conv_fwd(h, x, sh, w, dev(src), dev(dst), n_nodes=n_dst)
    g = dev(rng.standard_normal((n_dst, o.dim_out), dtype=np.float32))
    perm = dev(np.argsort(src, kind="stable").astype(np.int32))
    gx, gsh, gw = sp.tp_conv_bwd(h, x, sh, w, g, dev(src), dev(dst), perm, n_nodes=n_dst)
    torch.cuda.synchronize()
    assert out.shape == (n_dst, o.dim_out) and torch.count_nonzero(out) == 0
    assert gx.shape == (0, o.dim_in1)
    assert torch.count_nonzero(gsh) == 0 and torch.count_nonzero(gw) == 0
