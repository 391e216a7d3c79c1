"""GPU parity of the merged-output option of the channelwise convolution
(SEGPOLY_MERGE_PATHS: the paths of one output type sum into one block):
forward with the generated kernel and with the table-driven one, backward
with the generated kernel, both layouts, against the float64 oracle.
Tolerance: scaled error (oracle.metrics) <= 1e-5 in float32, <= 1e-12 in
float64."""

import numpy as np
import pytest

import workloads
from oracle import tp as otp
from tests._gpu import announce, check_scaled, dev, need_gpu

pytestmark = pytest.mark.gpu

IN1, IN2, OUT = "32x0e+32x1o", "0e+1o+2e", "0e+1o+2e"   # the molecules' irreps (a generated merged kernel)


def _sp():
    need_gpu()
    import segmented_polynomials_amd as sp
    return sp


def _inputs(o, dtype, seed, n_nodes=120, max_degree=14):
    rng = np.random.default_rng(seed)
    dt = np.float32 if dtype == "f32" else np.float64
    deg = rng.integers(0, max_degree + 1, n_nodes)
    deg[rng.random(n_nodes) < 0.2] = 0
    dst = np.repeat(np.arange(n_nodes), deg)
    src = rng.integers(0, n_nodes, dst.shape[0])
    E = dst.shape[0]
    return dict(x=rng.standard_normal((n_nodes, o.dim_in1)).astype(dt),
                sh=rng.standard_normal((E, o.dim_in2)).astype(dt),
                w=rng.standard_normal((E, o.weight_numel)).astype(dt),
                src=src.astype(np.int32), dst=dst.astype(np.int32), n_nodes=n_nodes)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
@pytest.mark.parametrize("generic", [False, True])
def test_merged_forward(generic, lay, dtype):
    import torch
    sp = _sp()
    o = otp.ChannelwiseTP(IN1, IN2, OUT, merge=True)
    h = sp.tp_create(IN1, IN2, OUT, layout=lay, dtype=dtype, merge=True, force_generic=generic)
    assert h.irreps_out == o.irreps_out == "32x0e+32x1o+32x2e"
    assert h.specialized == (not generic)
    inp = _inputs(o, dtype, 40 + generic)
    td = torch.float32 if dtype == "f32" else torch.float64
    announce(f"tp merged forward generic={generic} {lay} {dtype} E={inp['dst'].shape[0]}")
    out = sp.tp_conv_fwd(h, dev(inp["x"], td), dev(inp["sh"], td), dev(inp["w"], td), dev(inp["src"]),
                         dev(inp["dst"]), n_nodes=inp["n_nodes"])
    torch.cuda.synchronize()
    args = (inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"])
    check_scaled(out.cpu().numpy(), o.conv(*args, layout=lay), o.conv(*args, layout=lay, absolute=True), dtype,
                 "merged forward")


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
def test_merged_backward(lay, dtype):
    import torch
    sp = _sp()
    o = otp.ChannelwiseTP(IN1, IN2, OUT, merge=True)
    h = sp.tp_create(IN1, IN2, OUT, layout=lay, dtype=dtype, merge=True)
    inp = _inputs(o, dtype, 50)
    g = workloads.output_gradient(inp["n_nodes"], o.dim_out, dtype, seed=51)
    td = torch.float32 if dtype == "f32" else torch.float64
    announce(f"tp merged backward {lay} {dtype}")
    perm = dev(workloads.src_permutation(inp["src"]))
    got = sp.tp_conv_bwd(h, dev(inp["x"], td), dev(inp["sh"], td), dev(inp["w"], td), dev(g, td), dev(inp["src"]),
                         dev(inp["dst"]), perm, n_nodes=inp["n_nodes"])
    torch.cuda.synchronize()
    args = (inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"], g)
    ref = o.conv_vjp(*args, layout=lay)
    scale = o.conv_vjp(*args, layout=lay, absolute=True)
    for name, a, b, c in zip(("dx", "dsh", "dw"), got, ref, scale):
        check_scaled(a.cpu().numpy(), b, c, dtype, f"merged backward {name}")
