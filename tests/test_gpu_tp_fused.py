"""GPU parity of the convolution with the harmonics computed in the kernel
from the edge vectors (tp_conv_fwd_vec): bitwise equal to the two-call path
(sh_fwd, then tp_conv_fwd) and against the float64 oracle fed the oracle's
harmonics of the same (cast) vectors."""

import numpy as np
import pytest

import workloads
from oracle import sh as osh
from oracle import tp as otp
from tests._gpu import announce, check_scaled, dev, need_gpu

pytestmark = pytest.mark.gpu


def _sp():
    need_gpu()
    import segmented_polynomials_amd as sp
    return sp


@pytest.mark.parametrize("n,layout,normalize,kw", [
    (1, "mul_ir", True, {}),
    (2, "mul_ir", True, {}),
    (3, "ir_mul", False, dict(n_nodes=300, degree=16)),
    (4, "ir_mul", True, dict(n_nodes=300, degree=30)),
    (4, "mul_ir", False, dict(n_nodes=300, degree=30)),
])
def test_fused_harmonics(n, layout, normalize, kw):
    sp = _sp()
    import torch
    wl = workloads.WORKLOADS[n]
    o = otp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=layout, dtype=wl.dtype)
    inp = workloads.tp_inputs(wl, o.weight_fan_in(), **kw)
    td = torch.float32 if wl.dtype == "f32" else torch.float64
    x, w, vec = dev(inp["x"], td), dev(inp["w"], td), dev(inp["vec"], td)
    src = dst = None
    if inp["src"] is not None:
        src, dst = dev(inp["src"], torch.int32), dev(inp["dst"], torch.int32)
    lmax = max(wl.sh_ls)
    announce(f"tp fused harmonics workload {n} {layout} normalize={normalize}")
    fused = sp.tp_conv_fwd_vec(h, x, vec, w, src, dst, n_nodes=inp["n_nodes"], normalize=normalize)
    sh = sp.sh_fwd(vec, lmax, normalize=normalize)
    two = sp.tp_conv_fwd(h, x, sh, w, src, dst, n_nodes=inp["n_nodes"])
    torch.cuda.synchronize()
    fused, two = fused.cpu().numpy(), two.cpu().numpy()
    assert np.array_equal(fused, two)
    shr = osh.real_sh(list(wl.sh_ls), inp["vec"].astype(np.float64), normalize=normalize)
    args = (inp["x"], shr, inp["w"], inp["src"], inp["dst"], inp["n_nodes"])
    check_scaled(fused, o.conv(*args, layout=layout), o.conv(*args, layout=layout, absolute=True), wl.dtype,
                 f"fused workload {n} {layout}")


def test_fused_unsupported():
    sp = _sp()
    import torch
    v = torch.randn(4, 3, device="cuda")
    x = torch.randn(4, 4 * 4, device="cuda")
    for ins2, fg in (("0e+1e", False), ("0e+1o", True)):
        h = sp.tp_create("4x0e+4x1o", ins2, "0e+1o+1e", force_generic=fg)
        w = torch.randn(4, h.weight_numel, device="cuda")
        announce(f"tp fused unsupported {ins2} generic={fg}")
        with pytest.raises(sp.SegpolyError) as e:
            sp.tp_conv_fwd_vec(h, x, v, w)
        assert e.value.code == sp.E_UNSUPPORTED
