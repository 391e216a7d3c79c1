"""GPU check that the hot-path calls can be captured into a HIP graph and
replayed: the convolution forward and backward (with the in-kernel range
searches and with row pointers) on the molecular batch (destination-split
forward, edge-parallel backward) and on a 300-node graph of the large
workload's irreps (two channels per lane, destination-major backward), and
the symmetric contraction forward and backward.  The library launches only
kernels on the caller's stream (no allocation, no memset, no host
synchronisation without VALIDATE), so every replay must reproduce the eager
results bit for bit.  Outputs are overwritten with NaN before each replay
and eager work runs between replays."""

import numpy as np
import pytest

import workloads
from tests._gpu import announce, dev, need_gpu

pytestmark = pytest.mark.gpu


def _sp():
    need_gpu()
    import segmented_polynomials_amd as sp
    return sp


def _conv_calls(sp, torch, h, inp, n_nodes):
    """Closures for forward, backward, row-pointer forward and backward on
    preallocated outputs (everything allocated here, before any capture)."""
    x, sh, w = dev(inp["x"], torch.float32), dev(inp["sh"], torch.float32), dev(inp["w"], torch.float32)
    src, dst = dev(inp["src"], torch.int32), dev(inp["dst"], torch.int32)
    perm = dev(workloads.src_permutation(inp["src"]), torch.int32)
    g = dev(workloads.output_gradient(n_nodes, h.dim_out, "f32", seed=5), torch.float32)
    rp = sp.tp_rowptr_build(dst, n_nodes)
    srp = sp.tp_src_rowptr_build(src, perm, x.shape[0])
    ws = torch.empty(sp.tp_conv_bwd_workspace(h, sh.shape[0]), dtype=torch.uint8, device="cuda")
    outs = {k: torch.empty((n_nodes, h.dim_out), device="cuda") for k in ("out", "out_rp")}
    for k in ("", "_rp"):
        outs["gx" + k], outs["gsh" + k], outs["gw" + k] = torch.empty_like(x), torch.empty_like(sh), torch.empty_like(w)
    calls = [
        lambda: sp.tp_conv_fwd(h, x, sh, w, src, dst, n_nodes=n_nodes, out=outs["out"]),
        lambda: sp.tp_conv_fwd_rowptr(h, x, sh, w, src, rp, out=outs["out_rp"]),
        lambda: sp.tp_conv_bwd(h, x, sh, w, g, src, dst, perm, n_nodes=n_nodes, workspace=ws,
                               grad_x=outs["gx"], grad_sh=outs["gsh"], grad_w=outs["gw"]),
        lambda: sp.tp_conv_bwd_rowptr(h, x, sh, w, g, src, dst, perm, rp, srp, workspace=ws,
                                      grad_x=outs["gx_rp"], grad_sh=outs["gsh_rp"], grad_w=outs["gw_rp"]),
    ]
    return calls, outs


def _replay_matches_eager(torch, calls, outs, what):
    for f in calls:           # eager, which also loads every kernel before the capture
        f()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for f in calls:
            f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for f in calls:
            f()
    scratch = torch.randn(512, 512, device="cuda")
    for r in range(3):
        for v in outs.values():
            v.fill_(float("nan"))
        scratch = scratch @ scratch.T / 512      # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, ref[k]), f"{what}: replay {r} differs from eager in {k}"


@pytest.mark.parametrize("case", ["molecules", "graph_300_nodes"])
def test_conv_graph_replay(case):
    sp = _sp()
    import torch
    if case == "molecules":
        wl = workloads.WORKLOADS[2]
        h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=wl.layouts[0])
        inp = workloads.tp_inputs(wl, workloads.fan_in_from_irreps_out(h.irreps_out))
    else:
        wl = workloads.WORKLOADS[4]
        h = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout="ir_mul")
        inp = workloads.tp_inputs(wl, workloads.fan_in_from_irreps_out(h.irreps_out), n_nodes=300, degree=12,
                                  graph="ragged", seed=31)
    announce(f"graph replay conv {case} ({h.kernel_name}, {inp['sh'].shape[0]} edges)")
    calls, outs = _conv_calls(sp, torch, h, inp, inp["n_nodes"])
    _replay_matches_eager(torch, calls, outs, case)
    for a, b in (("out", "out_rp"), ("gx", "gx_rp"), ("gsh", "gsh_rp"), ("gw", "gw_rp")):
        assert torch.equal(outs[a], outs[b]), f"{case}: row pointers change {a}"


def test_symcon_graph_replay():
    sp = _sp()
    import torch
    s5 = workloads.WORKLOADS[5]
    h = sp.symcon_create(s5.irreps_in, s5.irreps_out, 3, s5.num_elements, layout="ir_mul")
    n = 3000
    rng = np.random.default_rng(41)
    x = dev(rng.standard_normal((n, h.dim_in)).astype(np.float32), torch.float32)
    w = dev(rng.standard_normal((s5.num_elements, h.weight_numel)).astype(np.float32), torch.float32)
    species = rng.integers(0, s5.num_elements, n)
    spc = dev(species, torch.int32)
    perm = dev(np.argsort(species, kind="stable"), torch.int32)
    g = dev(rng.standard_normal((n, h.dim_out)).astype(np.float32), torch.float32)
    ws = torch.empty(sp.symcon_bwd_workspace(h, n), dtype=torch.uint8, device="cuda")
    outs = dict(out=torch.empty((n, h.dim_out), device="cuda"), gx=torch.empty_like(x), gw=torch.empty_like(w))
    calls = [lambda: sp.symcon_fwd(h, x, spc, w, out=outs["out"]),
             lambda: sp.symcon_bwd(h, x, spc, w, g, perm, workspace=ws, grad_x=outs["gx"], grad_w=outs["gw"])]
    announce("graph replay symcon")
    _replay_matches_eager(torch, calls, outs, "symcon")
