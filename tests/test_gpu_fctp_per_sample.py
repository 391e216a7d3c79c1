"""GPU parity of the fully connected (uvw) tensor product with one weight row
per sample (external per-item weights, [n, weight_numel]): forward, both
input gradients and the per-sample weight gradient, called through the C
ABI, against the float64 oracle on the same seeded inputs.  Tolerance:
scaled error (oracle.metrics) <= 1e-5 in float32, <= 1e-12 in float64."""

import numpy as np
import pytest

from oracle import fctp as ofc
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
    w = rng.standard_normal((n, f.weight_numel)).astype(dt)
    g = rng.standard_normal((n, f.dim_out)).astype(dt)
    return x1, x2, w, g


CASES = [
    # (in1, in2, out, n)
    ("8x0e+8x1o", "8x0e+8x1o", "8x0e+8x1o", 37),                      # several channels on both inputs
    ("3x0e+2x1o+1x2e", "2x0e+1x1o+2x1e", "2x0e+3x1o+2x1e+1x2e+1x2o", 29),  # mixed, a block without paths
    ("16x0e+16x1o", "0e+1o+2e", "16x0e+16x1o+16x2e", 40),            # one channel on input 2
    ("4x0e", "3x0e", "100x0e", 9),                                   # two tiles (64 + 36 channels)
    ("2x2e", "3x2e", "2x2e", 11),                                    # five components, two lanes per pair
    ("1x4e", "2x4e", "1x3e+1x4e", 6),                                # many couplings per component
    ("70x0e+5x1o", "2x0e", "3x0e+1x1o", 13),                         # three ragged chunks of pairs
    ("5x1o", "1x1o", "1x0e+1x1e+1x2e", 1),                           # one sample
    ("2x3o", "1x3o", "3x6e", 7),                                     # l = 6 outputs (13 components)
    ("3x2e", "2x4e", "2x6e+1x4e", 5),                                # 13 and 9 components
    ("2x3o", "1x3e", "2x5o+1x4o", 4),                                # 11 components
]


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}|{c[1]}|{c[2]}|n{c[3]}" for c in CASES])
def test_per_sample_parity(case, lay, dtype):
    sp = _sp()
    import torch
    i1, i2, io, n = case
    f = ofc.FullyConnectedTP(i1, i2, io)
    h = sp.fctp_create(i1, i2, io, layout=lay, dtype=dtype)
    x1, x2, w, g = _inputs(f, n, dtype, seed=n + len(i1))
    td = _td(dtype)
    X1, X2, W, G = dev(x1, td), dev(x2, td), dev(w, td), dev(g, td)
    announce(f"fctp per-sample {case} {lay} {dtype}")
    out = sp.fctp_fwd_per_sample(h, X1, X2, W)
    g1, g2, gw = sp.fctp_bwd_per_sample(h, X1, X2, W, G)
    torch.cuda.synchronize()
    check_scaled(out.cpu().numpy(), f.fwd(x1, x2, w, layout=lay), f.fwd(x1, x2, w, layout=lay, absolute=True),
                 dtype, "fwd")
    r1, r2, rw = f.vjp(x1, x2, None, g, layout=lay, edge_weights=w)
    a1, a2, aw = f.vjp(x1, x2, None, g, layout=lay, absolute=True, edge_weights=w)
    assert gw.shape == (n, f.weight_numel)
    check_scaled(g1.cpu().numpy(), r1, a1, dtype, "dx1")
    check_scaled(g2.cpu().numpy(), r2, a2, dtype, "dx2")
    check_scaled(gw.cpu().numpy(), rw, aw, dtype, "dw")


@pytest.mark.parametrize("need", [(True, False, False), (False, True, False), (False, False, True),
                                  (True, True, False)])
def test_gradient_subsets(need):
    """Each requested gradient alone equals the full backward's (bit for
    bit: every sum is taken in the same order)."""
    sp = _sp()
    import torch
    i1, i2, io = "6x0e+4x1o", "3x0e+2x1o", "5x0e+3x1o+2x2e"
    f = ofc.FullyConnectedTP(i1, i2, io)
    h = sp.fctp_create(i1, i2, io, layout="mul_ir", dtype="f32")
    x1, x2, w, g = _inputs(f, 21, "f32", seed=5)
    X1, X2, W, G = dev(x1), dev(x2), dev(w), dev(g)
    announce(f"fctp per-sample gradient subset {need}")
    full = sp.fctp_bwd_per_sample(h, X1, X2, W, G)
    part = sp.fctp_bwd_per_sample(h, X1, X2, W, G, need=need)
    torch.cuda.synchronize()
    for want, a, b in zip(need, full, part):
        if want:
            assert torch.equal(a, b)
        else:
            assert b is None


def test_routing_and_shared_rows():
    """fctp_fwd / fctp_bwd take the per-sample path for [n, numel] weights;
    per-sample rows all equal to one row give the shared product, and the
    per-sample weight gradient summed over the samples gives the shared
    one."""
    sp = _sp()
    import torch
    i1, i2, io = "8x0e+8x1o", "4x0e+2x1o", "8x0e+8x1o+4x2e"
    f = ofc.FullyConnectedTP(i1, i2, io)
    h = sp.fctp_create(i1, i2, io, layout="ir_mul", dtype="f64")
    x1, x2, w, g = _inputs(f, 50, "f64", seed=9)
    X1, X2, W, G = dev(x1), dev(x2), dev(w), dev(g)
    announce("fctp per-sample routing")
    a = sp.fctp_fwd(h, X1, X2, W)
    b = sp.fctp_fwd_per_sample(h, X1, X2, W)
    ga = sp.fctp_bwd(h, X1, X2, W, G)
    gb = sp.fctp_bwd_per_sample(h, X1, X2, W, G)
    W1 = W[:1].contiguous()
    Wrep = W1.expand(50, -1).contiguous()
    shared = sp.fctp_fwd(h, X1, X2, W1)
    rep = sp.fctp_fwd_per_sample(h, X1, X2, Wrep)
    gs = sp.fctp_bwd(h, X1, X2, W1, G)
    gr = sp.fctp_bwd_per_sample(h, X1, X2, Wrep, G)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    for p, q in zip(ga, gb):
        assert torch.equal(p, q)
    scale = torch.from_numpy(f.fwd(x1, x2, w[:1], layout="ir_mul", absolute=True)).cuda()
    assert float(((shared - rep).abs() / scale.clamp_min(1e-300)).max()) <= 1e-12
    for k in range(2):
        assert float((gs[k] - gr[k]).abs().max()) <= 1e-12 * float(gs[k].abs().max() + 1)
    dws = gr[2].sum(0, keepdim=True)
    assert float((dws - gs[2]).abs().max()) <= 1e-11 * float(gs[2].abs().max() + 1)


def test_empty_and_errors():
    sp = _sp()
    import torch
    h = sp.fctp_create("2x0e+1x1o", "1x0e+1x1o", "2x0e+1x1o", dtype="f32")
    f = ofc.FullyConnectedTP("2x0e+1x1o", "1x0e+1x1o", "2x0e+1x1o")
    z1 = torch.empty((0, f.dim_in1), device="cuda")
    z2 = torch.empty((0, f.dim_in2), device="cuda")
    zw = torch.empty((0, f.weight_numel), device="cuda")
    zg = torch.empty((0, f.dim_out), device="cuda")
    announce("fctp per-sample empty batch")
    assert sp.fctp_fwd_per_sample(h, z1, z2, zw).shape == (0, f.dim_out)
    g1, g2, gw = sp.fctp_bwd_per_sample(h, z1, z2, zw, zg)
    assert g1.shape == z1.shape and g2.shape == z2.shape and gw.shape == zw.shape
    x1 = torch.zeros((3, f.dim_in1), device="cuda")
    x2 = torch.zeros((3, f.dim_in2), device="cuda")
    with pytest.raises(ValueError):
        sp.fctp_fwd_per_sample(h, x1, x2, torch.zeros((2, f.weight_numel), device="cuda"))
    with pytest.raises(ValueError):
        sp.fctp_fwd(h, x1, x2, torch.zeros((2, f.weight_numel), device="cuda"))


def test_full_size_workload_sampled():
    """The timed per-sample workload at full size (20k samples, 8,192
    weights each), in the launch configuration the benchmark times:
    sampled rows against the oracle one by one, both layouts."""
    sp = _sp()
    import torch
    import workloads
    wl = workloads.WORKLOADS[10]
    f = ofc.FullyConnectedTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    inp = workloads.fc_inputs(wl, f.weight_numel)
    x1, x2, w = inp["x1"], inp["x2"], inp["w"]
    g = workloads.output_gradient(wl.n, f.dim_out, wl.dtype, seed=2010)
    X1, X2, W, G = dev(x1), dev(x2), dev(w), dev(g)
    rows = np.concatenate([np.random.default_rng(3).choice(wl.n, 24, replace=False), [0, wl.n - 1]])
    for lay in wl.layouts:
        h = sp.fctp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=lay, dtype=wl.dtype)
        announce(f"fctp per-sample full size {wl.name} {lay}")
        out = sp.fctp_fwd(h, X1, X2, W).cpu().numpy()
        g1, g2, gw = (t.cpu().numpy() for t in sp.fctp_bwd(h, X1, X2, W, G))
        torch.cuda.synchronize()
        s = (x1[rows], x2[rows], w[rows])
        check_scaled(out[rows], f.fwd(*s, layout=lay), f.fwd(*s, layout=lay, absolute=True), "f32",
                     f"{lay} fwd rows")
        r = f.vjp(*s[:2], None, g[rows], layout=lay, edge_weights=s[2])
        a = f.vjp(*s[:2], None, g[rows], layout=lay, absolute=True, edge_weights=s[2])
        for got, ref, sc, name in zip((g1, g2, gw), r, a, ("dx1", "dx2", "dw")):
            check_scaled(got[rows], ref, sc, "f32", f"{lay} {name} rows")


def _random_irreps(rng, max_blocks, max_mul, max_l):
    blocks = []
    for _ in range(rng.integers(1, max_blocks + 1)):
        l = int(rng.integers(0, max_l + 1))
        p = "eo"[int(rng.integers(0, 2))]
        blocks.append(f"{int(rng.integers(1, max_mul + 1))}x{l}{p}")
    return "+".join(blocks)


@pytest.mark.parametrize("seed", range(12))
def test_random_descriptors(seed):
    """Seeded random descriptors (up to three blocks per operand, l <= 3,
    1..20 channels, either parity), both layouts, float32: the per-sample
    tables for shapes no hand-picked case covers."""
    sp = _sp()
    import torch
    rng = np.random.default_rng(100 + seed)
    while True:
        i1, i2, io = (_random_irreps(rng, 3, 20, 3) for _ in range(3))
        f = ofc.FullyConnectedTP(i1, i2, io)
        if f.weight_numel > 0:
            break
    n = int(rng.integers(1, 40))
    x1, x2, w, g = _inputs(f, n, "f32", seed=seed)
    X1, X2, W, G = dev(x1), dev(x2), dev(w), dev(g)
    for lay in ("mul_ir", "ir_mul"):
        h = sp.fctp_create(i1, i2, io, layout=lay, dtype="f32")
        announce(f"fctp per-sample random {i1} | {i2} | {io} n={n} {lay}")
        out = sp.fctp_fwd_per_sample(h, X1, X2, W)
        g1, g2, gw = sp.fctp_bwd_per_sample(h, X1, X2, W, G)
        torch.cuda.synchronize()
        check_scaled(out.cpu().numpy(), f.fwd(x1, x2, w, layout=lay), f.fwd(x1, x2, w, layout=lay, absolute=True),
                     "f32", "fwd")
        r = f.vjp(x1, x2, None, g, layout=lay, edge_weights=w)
        a = f.vjp(x1, x2, None, g, layout=lay, absolute=True, edge_weights=w)
        for got, ref, sc, name in zip((g1, g2, gw), r, a, ("dx1", "dx2", "dw")):
            check_scaled(got.cpu().numpy(), ref, sc, "f32", name)
