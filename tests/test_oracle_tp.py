"""Pins of the channelwise tensor-product oracle: descriptor counts the pages
print, a dense brute force on tiny irreps, the gather/scatter worked example,
layout equivalence and O(3) equivariance.  CPU only."""

import json
import os

import numpy as np
import pytest

from oracle import irreps, layout, sh, tp, wigner
from oracle.cg import real_cg
import workloads


def test_page_descriptor_counts(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "channelwise_descriptor.json")))
    a, b = g["cases"]
    d = tp.ChannelwiseTP(a["irreps_in1"], a["irreps_in2"], a["irreps_out"])
    assert d.num_paths == a["num_paths"]
    assert d.weight_numel == a["weight_numel"]
    assert d.irreps_out == a["irreps_out_actual"]
    assert {2 * l + 1 for _, l, _ in d.out} == set(a["segment_sizes"])
    e = tp.ChannelwiseTP(b["irreps_in1"], b["irreps_in2"], b["irreps_out"])
    assert e.num_paths == b["num_paths"]
    assert b["contains_type"] in e.irreps_out


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_workload_descriptor_sizes(n):
    # (paths, weight_numel, dim_out, sum of CG non-zeros) recomputed for the
    # workloads; a dropped parity or path changes one of them
    expect = {1: (9, 72, 232, 59), 2: (7, 224, 672, 37), 3: (18, 1152, 4096, 207),
              4: (13, 1664, 5504, 125)}[n]
    wl = workloads.WORKLOADS[n]
    d = tp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    nnz = sum(r[3] for r in d.path_table())
    assert (d.num_paths, d.weight_numel, d.dim_out, nnz) == expect


def test_output_order_and_filter():
    d = tp.ChannelwiseTP("2x0e+2x1o+2x2e", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o")
    keys = [irreps.type_key(l, p) for _, l, p in d.out]
    assert keys == sorted(keys)
    # 0o cannot arise from these inputs
    assert all((l, p) != (0, -1) for _, l, p in d.out)
    f = tp.ChannelwiseTP("2x0e+2x1o+2x2e", "0e+1o+2e+3o", "0e+1o+2e")
    assert {(l, p) for _, l, p in f.out} == {(0, 1), (1, -1), (2, 1)}


def _dense_tensor(d):
    """The whole product as a dense [dim1, dim2, dim_out, numel] tensor in
    mul_ir order, built entry by entry from the path list and real_cg."""
    off1 = np.cumsum([0] + [m * (2 * l + 1) for m, l, _ in d.in1])
    off2 = np.cumsum([0] + [m * (2 * l + 1) for m, l, _ in d.in2])
    offo = np.cumsum([0] + [m * (2 * l + 1) for m, l, _ in d.out])
    t = np.zeros((d.dim_in1, d.dim_in2, d.dim_out, d.weight_numel))
    woff = 0
    for p, (i, j, lo, _) in enumerate(d.paths):
        mul, l1, _ = d.in1[i]
        l2 = d.in2[j][1]
        c = real_cg(l1, l2, lo)
        for u in range(mul):
            for a in range(2 * l1 + 1):
                for b in range(2 * l2 + 1):
                    for k in range(2 * lo + 1):
                        t[off1[i] + u * (2 * l1 + 1) + a, off2[j] + b,
                          offo[p] + u * (2 * lo + 1) + k, woff + u] = c[a, b, k]
        woff += mul
    return t


@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
def test_brute_force_dense(lay):
    d = tp.ChannelwiseTP("2x0e+3x1o+2x2e", "0e+1o+2e", "0e+0o+1e+1o+2e+2o")
    t = _dense_tensor(d)
    rng = np.random.default_rng(5)
    n_src, n_e, n_dst = 4, 9, 5
    x = rng.normal(size=(n_src, d.dim_in1))
    s = rng.normal(size=(n_e, d.dim_in2))
    w = rng.normal(size=(n_e, d.weight_numel))
    src = rng.integers(0, n_src, n_e)
    dst = np.sort(rng.integers(0, n_dst, n_e))
    ref = np.zeros((n_dst, d.dim_out))
    for e in range(n_e):
        ref[dst[e]] += np.einsum("abkc,a,b,c->k", t, x[src[e]], s[e], w[e])
    xin = layout.transpose(x, d.in1, "mul_ir", lay)
    got = d.conv(xin, s, w, src, dst, n_dst, layout=lay)
    got = layout.transpose(got, d.out, lay, "mul_ir")
    assert np.allclose(got, ref, atol=1e-12)


def test_shared_weights_and_absolute_mode():
    d = tp.ChannelwiseTP("3x0e+3x1o", "0e+1o", "0e+1o")
    rng = np.random.default_rng(2)
    x = rng.normal(size=(6, d.dim_in1))
    s = rng.normal(size=(10, d.dim_in2))
    w1 = rng.normal(size=(1, d.weight_numel))
    src = rng.integers(0, 6, 10)
    dst = np.sort(rng.integers(0, 4, 10))
    a = d.conv(x, s, w1, src, dst, 4)
    b = d.conv(x, s, np.repeat(w1, 10, axis=0), src, dst, 4)
    assert np.allclose(a, b, atol=1e-14)
    big = d.conv(x, s, w1, src, dst, 4, absolute=True)
    assert np.all(big >= np.abs(a) - 1e-12)


def test_gather_scatter_worked_example(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "gather_scatter_example.json")))
    d = tp.ChannelwiseTP("3x0e+2x1o", "0e+1o", "0e+1o")
    rng = np.random.default_rng(7)
    nodes = rng.normal(size=(g["n_src"], d.dim_in1))
    snd = np.array(g["senders"])
    rcv = np.array(g["receivers"])
    order = np.argsort(rcv, kind="stable")
    s = rng.normal(size=(len(snd), d.dim_in2))
    w = rng.normal(size=(len(snd), d.weight_numel))
    got = d.conv(nodes, s[order], w[order], snd[order], rcv[order], g["n_dst"])
    edges = d.conv(nodes[snd], s, w)                 # batch mode on gathered rows
    ref = np.zeros((g["n_dst"], d.dim_out))
    np.add.at(ref, rcv, edges)                       # index_add_ of the page
    assert np.allclose(got, ref, atol=1e-13)
    for r in g["isolated_rows"]:
        assert np.count_nonzero(got[r]) == 0


def test_node_subset_matches_full():
    wl = workloads.WORKLOADS[3]
    d = tp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
    inp = workloads.tp_inputs(wl, d.weight_fan_in(), n_nodes=40, degree=5)
    full = d.conv(inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"], "ir_mul")
    nodes = np.array([0, 7, 13, 39])
    part = d.conv(inp["x"], inp["sh"], inp["w"], inp["src"], inp["dst"], inp["n_nodes"], "ir_mul",
                  nodes=nodes)
    assert np.allclose(part, full[nodes], atol=1e-13)


@pytest.mark.parametrize("lay", ["mul_ir", "ir_mul"])
def test_equivariance_rotation_and_inversion(lay):
    d = tp.ChannelwiseTP("2x0e+2x1o+2x2e", "0e+1o+2e+3o", "0e+0o+1e+1o+2e+2o")
    rng = np.random.default_rng(11)
    n = 7
    x = rng.normal(size=(n, d.dim_in1))
    vec = rng.normal(size=(n, 3))
    w = rng.normal(size=(n, d.weight_numel))
    src = rng.permutation(n)
    dst = np.sort(rng.integers(0, n, n))
    aa = rng.normal(size=3)
    R = wigner.rotation_matrix(aa)
    ls = [0, 1, 2, 3]

    def run(xm, v):
        xin = layout.transpose(xm, d.in1, "mul_ir", lay)
        o = d.conv(xin, sh.real_sh(ls, v), w, src, dst, n, layout=lay)
        return layout.transpose(o, d.out, lay, "mul_ir")

    base = run(x, vec)
    # rotation: features rotate with D_in1, vectors with R
    rot = run(x @ wigner.wigner_d_irreps(d.in1, aa).T, vec @ R.T)
    assert np.allclose(rot, base @ wigner.wigner_d_irreps(d.out, aa).T, atol=1e-11)
    # inversion: features pick up their parity, vectors flip
    inv = run(x @ wigner.wigner_d_irreps(d.in1, np.zeros(3), parity=-1).T, -vec)
    assert np.allclose(inv, base @ wigner.wigner_d_irreps(d.out, np.zeros(3), parity=-1).T,
                       atol=1e-12)


def test_fan_in_from_string_matches_descriptor():
    for n in (2, 3, 4):
        wl = workloads.WORKLOADS[n]
        d = tp.ChannelwiseTP(wl.irreps_in1, wl.irreps_in2, wl.irreps_out)
        assert np.array_equal(workloads.fan_in_from_irreps_out(d.irreps_out), d.weight_fan_in())


def test_mean_reduction():
    """reduce="mean": a destination with identical incoming messages gets
    that message; in general mean = sum / in-degree, isolated rows zero, and
    the VJP is the sum's VJP with g divided by the in-degree (checked by the
    adjoint identity in x)."""
    d = tp.ChannelwiseTP("3x0e+2x1o", "0e+1o", "0e+1o")
    rng = np.random.default_rng(31)
    x = rng.normal(size=(5, d.dim_in1))
    sh = rng.normal(size=(1, d.dim_in2)).repeat(4, axis=0)
    w = rng.normal(size=(1, d.weight_numel)).repeat(4, axis=0)
    src = np.array([2, 2, 2, 4])
    dst = np.array([0, 0, 0, 3])
    mean = d.conv(x, sh, w, src, dst, 5, reduce="mean")
    one = d.conv(x, sh[:1], w[:1], src[:1], np.array([0]), 1)
    assert np.allclose(mean[0], one[0], atol=1e-13)
    s = d.conv(x, sh, w, src, dst, 5)
    assert np.allclose(mean[3], s[3]) and np.count_nonzero(mean[[1, 2, 4]]) == 0
    assert np.allclose(mean[0] * 3, s[0], atol=1e-13)
    g = rng.normal(size=(5, d.dim_out))
    dx, dsh, dw = d.conv_vjp(x, sh, w, src, dst, 5, g, reduce="mean")
    vx = rng.normal(size=x.shape)
    assert np.isclose(np.sum(g * d.conv(vx, sh, w, src, dst, 5, reduce="mean")), np.sum(dx * vx), rtol=1e-12)
    vw = rng.normal(size=w.shape)
    assert np.isclose(np.sum(g * d.conv(x, sh, vw, src, dst, 5, reduce="mean")), np.sum(dw * vw), rtol=1e-12)


def test_merged_output_sums_paths_of_a_type():
    """merge=True: the output row has one block per type, the sum of the
    unmerged path blocks of that type; with one path per type nothing
    changes; the VJP keeps the adjoint identities; mixed multiplicities
    within a type are rejected."""
    ins, sh_ir, outs = "6x0e+6x1o", "0e+1o+2e", "0e+1o+2e"
    u = tp.ChannelwiseTP(ins, sh_ir, outs)
    m = tp.ChannelwiseTP(ins, sh_ir, outs, merge=True)
    assert m.irreps_out == "6x0e+6x1o+6x2e" and m.weight_numel == u.weight_numel
    rng = np.random.default_rng(20)
    src = rng.integers(0, 5, 14)
    dst = np.sort(rng.integers(0, 4, 14))
    x = rng.normal(size=(5, u.dim_in1))
    sh = rng.normal(size=(14, u.dim_in2))
    w = rng.normal(size=(14, u.weight_numel))
    for lay in ("mul_ir", "ir_mul"):
        yu = layout.split_blocks(u.conv(x, sh, w, src, dst, 4, layout=lay), u.out, lay)
        ym = layout.split_blocks(m.conv(x, sh, w, src, dst, 4, layout=lay), m.out_blocks, lay)
        for t, (mul, lo, po) in enumerate(m.out_blocks):
            want = sum(yu[p] for p, (_, l2, p2) in enumerate(u.out) if (l2, p2) == (lo, po))
            assert np.allclose(ym[t], want, atol=1e-12)
        g = rng.normal(size=(4, m.dim_out))
        dx, dsh, dw = m.conv_vjp(x, sh, w, src, dst, 4, g, layout=lay)
        vx, vs, vw = rng.normal(size=x.shape), rng.normal(size=sh.shape), rng.normal(size=w.shape)
        assert np.isclose(np.sum(g * m.conv(vx, sh, w, src, dst, 4, layout=lay)), np.sum(dx * vx), rtol=1e-11)
        assert np.isclose(np.sum(g * m.conv(x, vs, w, src, dst, 4, layout=lay)), np.sum(dsh * vs), rtol=1e-11)
        assert np.isclose(np.sum(g * m.conv(x, sh, vw, src, dst, 4, layout=lay)), np.sum(dw * vw), rtol=1e-11)
    one = tp.ChannelwiseTP("4x1o", "0e", "1o", merge=True)
    ref = tp.ChannelwiseTP("4x1o", "0e", "1o")
    xx = rng.normal(size=(3, 12))
    ss = rng.normal(size=(3, 1))
    ww = rng.normal(size=(3, 4))
    assert np.allclose(one.conv(xx, ss, ww), ref.conv(xx, ss, ww), atol=1e-13)
    with pytest.raises(ValueError):
        tp.ChannelwiseTP("4x0e+3x0e", "0e", "0e", merge=True)
