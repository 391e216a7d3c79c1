"""GPU parity on seeded random descriptors: the channelwise convolution, the
fully connected product with one shared weight row and as a convolution
with per-edge weights, the equivariant linear layer and the symmetric
contraction, forward and backward, both layouts, float32, called through
the C ABI and compared with the float64 oracle (scaled error,
oracle.metrics, <= 1e-5).  The hand-picked cases of the
other GPU tests cover the shapes the pages name; these cover block orders,
channel counts and type sets that none of them picks."""

import numpy as np
import pytest

from oracle import fctp as ofc
from oracle import linear as olin
from oracle import symcon as osym
from oracle import tp as otp
from tests._gpu import announce, check_scaled, dev, need_gpu

pytestmark = pytest.mark.gpu

TYPES = [f"{l}{p}" for l in range(4) for p in "eo"]


def _sp():
    need_gpu()
    import segmented_polynomials_amd as sp
    return sp


def _irreps(rng, max_blocks, max_mul, max_l, mul=None):
    out = []
    for _ in range(int(rng.integers(1, max_blocks + 1))):
        m = mul if mul is not None else int(rng.integers(1, max_mul + 1))
        out.append(f"{m}x{int(rng.integers(0, max_l + 1))}{'eo'[int(rng.integers(0, 2))]}")
    return "+".join(out)


def _f32(rng, shape):
    return rng.standard_normal(shape).astype(np.float32).astype(np.float64)


@pytest.mark.parametrize("seed", range(6))
def test_random_channelwise_convolution(seed):
    sp = _sp()
    import torch
    rng = np.random.default_rng(300 + seed)
    while True:
        in1 = _irreps(rng, 3, 20, 3)
        in2 = "+".join(sorted(set(t for t in (["0e"] + list(rng.choice(["1o", "2e", "3o", "1e"], 2))))))
        filt = "+".join(sorted(set(rng.choice(TYPES, 5))))
        o = otp.ChannelwiseTP(in1, in2, filt)
        if o.weight_numel > 0:
            break
    n_src, n_dst, n_e = 29, 23, int(rng.integers(50, 200))
    src = rng.integers(0, n_src, n_e)
    dst = np.sort(rng.integers(0, n_dst, n_e))
    x, sh, w = _f32(rng, (n_src, o.dim_in1)), _f32(rng, (n_e, o.dim_in2)), _f32(rng, (n_e, o.weight_numel))
    g = _f32(rng, (n_dst, o.dim_out))
    perm = np.argsort(src, kind="stable")
    for lay in ("mul_ir", "ir_mul"):
        h = sp.tp_create(in1, in2, filt, layout=lay)
        announce(f"random channelwise {in1} | {in2} | {filt} {lay} ({h.kernel_name})")
        X, S, W, G = dev(x, torch.float32), dev(sh, torch.float32), dev(w, torch.float32), dev(g, torch.float32)
        I, D, P = dev(src, torch.int32), dev(dst, torch.int32), dev(perm, torch.int32)
        out = sp.tp_conv_fwd(h, X, S, W, I, D, n_nodes=n_dst)
        dx, dsh, dw = sp.tp_conv_bwd(h, X, S, W, G, I, D, P, n_nodes=n_dst)
        torch.cuda.synchronize()
        check_scaled(out.cpu().numpy(), o.conv(x, sh, w, src, dst, n_dst, layout=lay),
                     o.conv(x, sh, w, src, dst, n_dst, layout=lay, absolute=True), "f32", "fwd")
        ref = o.conv_vjp(x, sh, w, src, dst, n_dst, g, layout=lay)
        scale = o.conv_vjp(x, sh, w, src, dst, n_dst, g, layout=lay, absolute=True)
        for got, r, a, name in zip((dx, dsh, dw), ref, scale, ("dx", "dsh", "dw")):
            check_scaled(got.cpu().numpy(), r, a, "f32", name)


@pytest.mark.parametrize("seed", range(6))
def test_random_fully_connected_shared(seed):
    sp = _sp()
    import torch
    rng = np.random.default_rng(400 + seed)
    while True:
        i1, i2, io = (_irreps(rng, 3, 16, 2) for _ in range(3))
        f = ofc.FullyConnectedTP(i1, i2, io)
        if f.weight_numel > 0:
            break
    n = int(rng.integers(1, 150))
    x1, x2, w = _f32(rng, (n, f.dim_in1)), _f32(rng, (n, f.dim_in2)), _f32(rng, (1, f.weight_numel))
    g = _f32(rng, (n, f.dim_out))
    for lay in ("mul_ir", "ir_mul"):
        h = sp.fctp_create(i1, i2, io, layout=lay)
        announce(f"random fully connected {i1} | {i2} | {io} n={n} {lay}")
        X1, X2, W, G = (dev(a, torch.float32) for a in (x1, x2, w, g))
        out = sp.fctp_fwd(h, X1, X2, W)
        g1, g2, gw = sp.fctp_bwd(h, X1, X2, W, G)
        torch.cuda.synchronize()
        check_scaled(out.cpu().numpy(), f.fwd(x1, x2, w, layout=lay), f.fwd(x1, x2, w, layout=lay, absolute=True),
                     "f32", "fwd")
        ref = f.vjp(x1, x2, w, g, layout=lay)
        scale = f.vjp(x1, x2, w, g, layout=lay, absolute=True)
        for got, r, a, name in zip((g1, g2, gw), ref, scale, ("dx1", "dx2", "dw")):
            check_scaled(got.cpu().numpy(), r, a, "f32", name)


@pytest.mark.parametrize("seed", range(6))
def test_random_linear(seed):
    sp = _sp()
    import torch
    rng = np.random.default_rng(500 + seed)
    while True:
        ii = _irreps(rng, 4, 40, 3)
        types = sorted(set(t.split("x")[1] for t in ii.split("+")))
        oo = "+".join(f"{int(rng.integers(1, 40))}x{t}" for t in rng.permutation(types + ["2o"])[:3])
        lin = olin.Linear(ii, oo)
        if lin.weight_numel > 0:
            break
    n = int(rng.integers(1, 300))
    x, w, g = _f32(rng, (n, lin.dim_in)), _f32(rng, (1, lin.weight_numel)), _f32(rng, (n, lin.dim_out))
    for lay in ("mul_ir", "ir_mul"):
        h = sp.linear_create(ii, oo, layout=lay)
        announce(f"random linear {ii} -> {oo} n={n} {lay}")
        X, W, G = (dev(a, torch.float32) for a in (x, w, g))
        out = sp.linear_fwd(h, X, W)
        gx, gw = sp.linear_bwd(h, X, W, G)
        torch.cuda.synchronize()
        check_scaled(out.cpu().numpy(), lin.fwd(x, w, layout=lay), lin.fwd(x, w, layout=lay, absolute=True),
                     "f32", "fwd")
        ref = lin.vjp(x, w, g, layout=lay)
        scale = lin.vjp(x, w, g, layout=lay, absolute=True)
        for got, r, a, name in zip((gx, gw), ref, scale, ("dx", "dw")):
            check_scaled(got.cpu().numpy(), r, a, "f32", name)


@pytest.mark.parametrize("seed", range(6))
def test_random_symmetric_contraction(seed):
    sp = _sp()
    import torch
    rng = np.random.default_rng(600 + seed)
    mul = int(rng.integers(1, 70))
    while True:
        ii = "+".join(sorted(set(f"{mul}x{t}" for t in rng.choice(["0e", "1o", "2e", "1e", "2o"], 3))))
        oo = "+".join(sorted(set(f"{mul}x{t}" for t in rng.choice(["0e", "1o", "1e", "2e"], 2))))
        sc = osym.SymmetricContraction(ii, oo)
        if sc.weight_numel > 0:
            break
    ne, n = 3, int(rng.integers(1, 60))
    x, w = _f32(rng, (n, sc.dim_in)), _f32(rng, (ne, sc.weight_numel))
    g = _f32(rng, (n, sc.dim_out))
    species = rng.integers(0, ne, n).astype(np.int32)
    perm = np.argsort(species, kind="stable").astype(np.int32)
    for lay in ("mul_ir", "ir_mul"):
        h = sp.symcon_create(ii, oo, 3, ne, layout=lay)
        announce(f"random symmetric contraction {ii} -> {oo} n={n} {lay}")
        X, W, G = (dev(a, torch.float32) for a in (x, w, g))
        Sp, P = dev(species), dev(perm)
        out = sp.symcon_fwd(h, X, Sp, W)
        gx, gw = sp.symcon_bwd(h, X, Sp, W, G, P)
        torch.cuda.synchronize()
        check_scaled(out.cpu().numpy(), sc.eval(x, species, w, layout=lay),
                     sc.eval(x, species, w, layout=lay, absolute=True), "f32", "fwd")
        ref = sc.eval_vjp(x, species, w, g, layout=lay)
        scale = sc.eval_vjp(x, species, w, g, layout=lay, absolute=True)
        for got, r, a, name in zip((gx, gw), ref, scale, ("dx", "dw")):
            check_scaled(got.cpu().numpy(), r, a, "f32", name)


@pytest.mark.parametrize("seed", range(6))
def test_random_fully_connected_convolution(seed):
    """The fully connected product as a convolution with one weight row per
    edge (input 2: one channel per degree), sum or mean, ragged graph."""
    sp = _sp()
    import torch
    rng = np.random.default_rng(700 + seed)
    while True:
        i1 = _irreps(rng, 3, 24, 2)
        i2 = "+".join(sorted(set(["0e"] + list(rng.choice(["1o", "2e", "1e"], 2)))))
        io = _irreps(rng, 3, 24, 2)
        f = ofc.FullyConnectedTP(i1, i2, io)
        if f.weight_numel > 0:
            break
    reduce = "mean" if seed % 2 else "sum"
    n_src, n_dst, n_e = 27, 19, int(rng.integers(40, 160))
    src = rng.integers(0, n_src, n_e)
    dst = np.sort(rng.integers(0, n_dst, n_e))
    x, sh, w = _f32(rng, (n_src, f.dim_in1)), _f32(rng, (n_e, f.dim_in2)), _f32(rng, (n_e, f.weight_numel))
    g = _f32(rng, (n_dst, f.dim_out))
    perm = np.argsort(src, kind="stable")
    for lay in ("mul_ir", "ir_mul"):
        h = sp.fctp_create(i1, i2, io, layout=lay, reduce=reduce)
        announce(f"random fully connected conv {i1} | {i2} | {io} {reduce} {lay}")
        X, S, W, G = (dev(a, torch.float32) for a in (x, sh, w, g))
        I, D, P = dev(src, torch.int32), dev(dst, torch.int32), dev(perm, torch.int32)
        out = sp.fctp_conv_fwd(h, X, S, W, I, D, n_dst)
        dx, dsh, dw = sp.fctp_conv_bwd(h, X, S, W, G, I, D, P, n_dst)
        torch.cuda.synchronize()
        check_scaled(out.cpu().numpy(), f.conv(x, sh, w, src, dst, n_dst, layout=lay, reduce=reduce),
                     f.conv(x, sh, w, src, dst, n_dst, layout=lay, reduce=reduce, absolute=True), "f32", "fwd")
        ref = f.conv_vjp(x, sh, w, src, dst, n_dst, g, layout=lay, reduce=reduce)
        scale = f.conv_vjp(x, sh, w, src, dst, n_dst, g, layout=lay, reduce=reduce, absolute=True)
        for got, r, a, name in zip((dx, dsh, dw), ref, scale, ("dx", "dsh", "dw")):
            check_scaled(got.cpu().numpy(), r, a, "f32", name)
