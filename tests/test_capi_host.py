"""The C ABI on the host (no GPU needed, no kernel launched): the library
loads and exports every declared symbol; the C++ descriptor builder agrees
with the oracle (paths, output irreps, coefficients, symmetric-contraction
basis); invalid arguments fail closed with the documented status codes."""

import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import segmented_polynomials_amd as sp
from oracle import cg as ocg, fctp as ofctp, irreps as oirreps, symcon as osymcon, tp as otp
import workloads

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "segpoly.h")


def test_one_hip_runtime_per_process():
    # the library must use the HIP runtime PyTorch loaded, not a second copy
    assert len(sp.hip_runtimes_loaded()) == 1, sp.hip_runtimes_loaded()


def test_exports_every_declared_symbol():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"^\s*(?:int|const char\*)\s+(\w+)\s*\(", text, flags=re.M))
    assert names == set(sp.EXPORTS)
    for n in names:
        assert hasattr(sp.lib, n), n
    assert "gfx950" in sp.version()


@pytest.mark.parametrize("l1,l2", [(a, b) for a in range(7) for b in range(7)])
def test_real_cg_matches_oracle(l1, l2):
    """Every coupling the library can build (l1, l2, l3 <= 6) against the
    oracle's exact-arithmetic tensor, entry by entry and in its zero pattern;
    l3 outside the triangle gives zeros, l above 6 fails closed."""
    for l3 in range(0, 7):
        a = sp.real_cg(l1, l2, l3)
        b = ocg.real_cg(l1, l2, l3)
        assert np.abs(a - b).max() <= 2e-16 * max(1, np.abs(b).max()), (l1, l2, l3)
        assert np.array_equal(a != 0, b != 0)
    out = np.zeros(15 * 15 * 15)
    buf = out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    assert sp.lib.segpoly_real_cg(l1, l2, 7, buf) == sp.E_UNSUPPORTED
    assert sp.lib.segpoly_real_cg(7, l2, l1, buf) == sp.E_UNSUPPORTED


def _compare_tp(in1, in2, filt, layout="mul_ir"):
    h = sp.tp_create(in1, in2, filt, layout=layout)
    o = otp.ChannelwiseTP(in1, in2, filt)
    assert h.irreps_out == o.irreps_out
    assert (h.num_paths, h.weight_numel, h.dim_in1, h.dim_in2, h.dim_out) == \
        (o.num_paths, o.weight_numel, o.dim_in1, o.dim_in2, o.dim_out)
    woff = 0
    for p, (i, j, lo, po) in enumerate(o.paths):
        info = h.path_info(p)
        assert (info["in1_block"], info["in2_block"], info["lo"], info["parity"]) == (i, j, lo, po)
        assert info["weight_offset"] == woff
        woff += o.in1[i][0]
        l1, l2 = o.in1[i][1], o.in2[j][1]
        c = ocg.real_cg(l1, l2, lo)
        assert np.abs(h.path_cg(p) - c).max() <= 2e-16
        assert info["nnz"] == np.count_nonzero(c)
    assert h.cg_nnz == sum(r[3] for r in o.path_table())
    return h


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_workload_descriptors_match_oracle_and_are_specialized(n):
    wl = workloads.WORKLOADS[n]
    for lay in wl.layouts:
        h = _compare_tp(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, lay)
        assert h.specialized, h.kernel_name
        g = sp.tp_create(wl.irreps_in1, wl.irreps_in2, wl.irreps_out, layout=lay, force_generic=True)
        assert not g.specialized and g.kernel_name == "tp_conv_generic"


def test_page_descriptor():
    h = _compare_tp("32x0e+32x1o", "0e+1o", "32x0e+32x1o")
    assert h.num_paths == 4 and h.weight_numel == 128
    assert h.irreps_out == "32x0e+32x0e+32x1o+32x1o"


_irrep = st.tuples(st.integers(1, 5), st.integers(0, 6), st.sampled_from("eo"))


@settings(max_examples=60, deadline=None)
@given(st.lists(_irrep, min_size=1, max_size=4), st.lists(st.tuples(st.integers(0, 6), st.sampled_from("eo")),
                                                          min_size=1, max_size=4),
       st.lists(st.tuples(st.integers(0, 6), st.sampled_from("eo")), min_size=1, max_size=6))
def test_fuzz_tp_descriptor(b1, b2, bo):
    in1 = "+".join(f"{m}x{l}{p}" for m, l, p in b1)
    in2 = "+".join(f"{l}{p}" for l, p in b2)
    filt = "+".join(f"{l}{p}" for l, p in bo)
    o = otp.ChannelwiseTP(in1, in2, filt)
    if sum(2 * lo + 1 for _, _, lo, _ in o.paths) * 64 * 4 > 64 * 1024:
        # more output components per channel than the table-driven kernel
        # holds in LDS (and no generated kernel): fails closed
        with pytest.raises(sp.SegpolyError) as err:
            sp.tp_create(in1, in2, filt)
        assert err.value.code == sp.E_UNSUPPORTED
        return
    _compare_tp(in1, in2, filt)


@pytest.mark.parametrize("ins,outs", [
    ("32x0e+32x1o", "32x0e"),
    ("4x0e+4x1o+4x2e+4x3o", "4x0e+4x1o"),
    ("3x0e+3x1o+3x2e", "3x0e+3x1o+3x2e"),
    ("2x0o+2x1e", "2x0e+2x1o"),
])
def test_symcon_basis_matches_oracle(ins, outs):
    h = sp.symcon_create(ins, outs, max_degree=3, num_elements=2)
    o = osymcon.SymmetricContraction(ins, outs)
    assert h.weight_numel == o.weight_numel and h.num_couplings == len(o.segments)
    assert (h.dim_in, h.dim_out) == (o.dim_in, o.dim_out)
    for c, (nu, ob, k) in enumerate(o.segments):
        info = h.coupling_info(c)
        assert (info["degree"], info["out_block"], info["k"]) == (nu, ob, k)
        a = h.coupling_dense(c, o.n)
        b = o.basis[(nu, ob)][k]
        assert np.abs(a - b).max() < 1e-13
    # the span (a basis-free quantity) agrees too
    for (nu, ob), us in o.basis.items():
        if not us:
            continue
        idx = [c for c, s in enumerate(o.segments) if s[:2] == (nu, ob)]
        A = np.stack([h.coupling_dense(c, o.n).ravel() for c in idx], 1)
        B = np.stack([u.ravel() for u in us], 1)
        pa = A @ np.linalg.pinv(A)
        pb = B @ np.linalg.pinv(B)
        assert np.abs(pa - pb).max() < 1e-10


def test_symcon_workload5_specialized():
    wl = workloads.WORKLOADS[5]
    h = sp.symcon_create(wl.irreps_in, wl.irreps_out, 3, wl.num_elements, layout="ir_mul")
    assert h.specialized
    assert h.weight_numel == 3712 and h.num_couplings == 29
    assert h.num_terms == 550
    # the specialised kernel addresses an atom's rows with 32-bit buffer
    # offsets: a row of 2 GiB or more (here 20M channels x 29 weights x 4 B)
    # takes the table-driven kernel
    m = 20_000_000
    big = sp.symcon_create(f"{m}x0e+{m}x1o+{m}x2e+{m}x3o", f"{m}x0e+{m}x1o", 3, wl.num_elements, layout="ir_mul")
    assert not big.specialized
    m = 4_000_000  # 4M x 29 x 4 B < 2 GiB
    ok = sp.symcon_create(f"{m}x0e+{m}x1o+{m}x2e+{m}x3o", f"{m}x0e+{m}x1o", 3, wl.num_elements, layout="ir_mul")
    assert ok.specialized


# ---------------------------------------------------------------- errors

def _raw_create(*args):
    raw = ctypes.c_void_p()
    return sp.lib.tp_create(*args, ctypes.byref(raw)), raw


def test_create_errors():
    assert _raw_create(b"32x1q", b"0e", b"0e", 0, 0, 0)[0] == sp.E_PARSE
    assert _raw_create(b"3x", b"0e", b"0e", 0, 0, 0)[0] == sp.E_PARSE
    assert _raw_create(b"4x0e", b"2x1o", b"1o", 0, 0, 0)[0] == sp.E_UNSUPPORTED
    assert _raw_create(b"4x9e", b"0e", b"9e", 0, 0, 0)[0] == sp.E_UNSUPPORTED
    # the envelope is l <= 6 on every side: 6 builds, 7 anywhere fails closed
    rc, raw = _raw_create(b"4x6e", b"0e+6e", b"0e+6e", 0, 0, 0)
    assert rc == sp.OK
    sp.lib.tp_destroy(raw)
    assert _raw_create(b"4x7o", b"0e", b"7o", 0, 0, 0)[0] == sp.E_UNSUPPORTED
    assert _raw_create(b"4x3o", b"4e", b"7o", 0, 0, 0)[0] == sp.E_UNSUPPORTED
    assert _raw_create(b"4x3o", b"7o", b"4e", 0, 0, 0)[0] == sp.E_UNSUPPORTED
    assert _raw_create(b"4x0e", b"0e", b"0e", 7, 0, 0)[0] == sp.E_INVALID
    assert _raw_create(b"4x0e", b"0e", b"0e", 0, 5, 0)[0] == sp.E_INVALID
    assert _raw_create(b"4x0e", b"0e", b"0e", 0, 0, 64)[0] == sp.E_INVALID
    assert sp.lib.tp_create(None, b"0e", b"0e", 0, 0, 0, None) == sp.E_INVALID
    assert sp.lib.segpoly_last_error()
    with pytest.raises(sp.SegpolyError) as e:
        sp.symcon_create("2x0e+3x1o", "2x0e")
    assert e.value.code == sp.E_UNSUPPORTED
    with pytest.raises(sp.SegpolyError):
        sp.symcon_create("2x0e", "2x0e", max_degree=4)


def test_query_errors():
    h = sp.tp_create("4x0e+4x1o", "0e+1o", "0e+1o")
    v = ctypes.c_int64()
    assert sp.lib.tp_query(h._h, 99, ctypes.byref(v)) == sp.E_INVALID
    assert sp.lib.tp_query(None, 0, ctypes.byref(v)) == sp.E_INVALID
    buf = ctypes.create_string_buffer(3)
    assert sp.lib.tp_irreps_out(h._h, buf, 3) == sp.E_INVALID
    info = (ctypes.c_int64 * 10)()
    assert sp.lib.tp_path_info(h._h, 99, info) == sp.E_INVALID


def test_forward_argument_errors_fail_before_any_gpu_call():
    h = sp.tp_create("4x0e+4x1o", "0e+1o", "0e+1o")
    f = sp.lib.tp_conv_fwd
    p = ctypes.c_void_p(16)   # never dereferenced: every call below fails validation
    assert f(None, p, 1, p, p, p, p, 0, 1, 1, p, None) == sp.E_INVALID
    assert f(h._h, p, -1, p, p, p, p, 0, 1, 1, p, None) == sp.E_INVALID
    assert f(h._h, p, 1, p, p, p, None, 0, 1, 1, p, None) == sp.E_INVALID      # src without dst
    assert f(h._h, p, 1, p, p, None, None, 0, 2, 2, p, None) == sp.E_INVALID   # batch: n_src < n_edges
    assert f(h._h, p, 4, p, p, None, None, 0, 2, 3, p, None) == sp.E_INVALID   # batch: n_edges != n_nodes
    assert f(h._h, p, 1, p, p, p, p, 9, 1, 1, p, None) == sp.E_INVALID         # index dtype
    assert f(h._h, p, 1, p, p, p, p, 0, 1, 1, None, None) == sp.E_INVALID      # null out
    assert f(h._h, p, 1, p, None, p, p, 0, 1, 1, p, None) == sp.E_INVALID      # null w
    assert f(h._h, p, 1, p, p, p, p, 0, 1, 1 << 31, p, None) == sp.E_UNSUPPORTED
    # nothing to do: succeeds without touching a device
    assert f(h._h, None, 0, None, None, None, None, 0, 0, 0, None, None) == sp.OK
    s = sp.symcon_create("2x0e+2x1o", "2x0e", 3, 2)
    g = sp.lib.symcon_fwd
    assert g(s._h, p, p, 0, p, -1, p, None) == sp.E_INVALID
    assert g(s._h, p, None, 0, p, 3, p, None) == sp.E_INVALID
    assert g(s._h, p, p, 3, p, 3, p, None) == sp.E_INVALID
    assert g(s._h, None, None, 0, None, 0, None, None) == sp.OK


def test_destroy_null_is_noop():
    assert sp.lib.tp_destroy(None) == sp.OK
    assert sp.lib.symcon_destroy(None) == sp.OK


def test_backward_argument_errors_fail_before_any_gpu_call():
    h = sp.tp_create("32x0e+32x1o", "0e+1o", "0e+1o")
    assert h.specialized
    n = ctypes.c_size_t()
    r256 = lambda b: (b + 255) // 256 * 256
    # indexed mode: messages, then the int32 sources in src_perm order
    assert sp.lib.tp_conv_bwd_workspace(h._h, 10, 0, ctypes.byref(n)) == sp.OK
    assert n.value == r256(10 * h.dim_in1 * 4) + 10 * 4
    assert sp.lib.tp_conv_bwd_workspace(h._h, 10, 1, ctypes.byref(n)) == sp.OK and n.value == 0
    assert sp.lib.tp_conv_bwd_workspace(h._h, -1, 0, ctypes.byref(n)) == sp.E_INVALID
    # multiplicity 200: four tiles of harmonic-gradient partials
    h2 = sp.tp_create("200x0e+200x1o", "0e+1o", "0e+1o")
    assert sp.lib.tp_conv_bwd_workspace(h2._h, 7, 1, ctypes.byref(n)) == sp.OK
    assert n.value == 4 * 7 * h2.dim_in2 * 4
    assert sp.lib.tp_conv_bwd_workspace(h2._h, 7, 0, ctypes.byref(n)) == sp.OK
    assert n.value == r256(r256(7 * h2.dim_in1 * 4) + 4 * 7 * h2.dim_in2 * 4) + 7 * 4
    f = sp.lib.tp_conv_bwd
    p = ctypes.c_void_p(16)   # never dereferenced: every call below fails validation
    big = 1 << 40
    # h, x, n_src, sh, w, src, dst, perm, idx, n_edges, n_nodes, g, gx, gsh, gw, ws, ws_bytes, stream
    assert f(None, p, 1, p, p, p, p, p, 0, 1, 1, p, p, p, p, p, big, None) == sp.E_INVALID
    assert f(h._h, p, -1, p, p, p, p, p, 0, 1, 1, p, p, p, p, p, big, None) == sp.E_INVALID
    assert f(h._h, p, 1, p, p, p, p, None, 0, 1, 1, p, p, p, p, p, big, None) == sp.E_INVALID  # no perm
    assert f(h._h, p, 1, p, p, p, p, p, 7, 1, 1, p, p, p, p, p, big, None) == sp.E_INVALID     # index dtype
    assert f(h._h, p, 1, p, p, p, p, p, 0, 1, 1, p, None, p, p, p, big, None) == sp.E_INVALID  # grad_x
    assert f(h._h, p, 1, p, p, p, p, p, 0, 1, 1, p, p, p, None, p, big, None) == sp.E_INVALID  # grad_w
    assert f(h._h, p, 1, p, p, p, p, p, 0, 1, 1, None, p, p, p, p, big, None) == sp.E_INVALID  # grad_out
    assert f(h._h, p, 1, p, p, p, p, p, 0, 1, 1, p, p, p, p, p, 8, None) == sp.E_INVALID       # workspace small
    assert f(h._h, p, 1, p, p, p, p, p, 0, 1, 1, p, p, p, p, None, big, None) == sp.E_INVALID  # no workspace
    assert f(h._h, p, 1, p, p, None, None, None, 0, 2, 2, p, p, p, p, None, 0, None) == sp.E_INVALID  # batch
    # shared weights: the workspace adds the per-edge weight gradients and
    # one partial sum per 1024 edges; generic descriptors fail closed
    hs = sp.tp_create("32x0e+32x1o", "0e+1o", "0e+1o", shared_weights=True)
    assert sp.tp_conv_bwd_workspace(hs, 1000) == r256(1000 * hs.dim_in1 * 4 + 1000 * 4) \
        + 1000 * hs.weight_numel * 4 + hs.weight_numel * 4
    assert sp.tp_conv_bwd_workspace(hs, 2049) == r256(r256(2049 * hs.dim_in1 * 4) + 2049 * 4) \
        + r256(2049 * hs.weight_numel * 4) + 3 * hs.weight_numel * 4
    # batch mode with shared weights: no messages and no keys
    assert sp.tp_conv_bwd_workspace(hs, 1000, batch=True) == 1000 * hs.weight_numel * 4 + hs.weight_numel * 4
    assert f(hs._h, p, 1, p, p, p, p, p, 0, 1, 1, p, p, p, p, p, 8, None) == sp.E_INVALID       # workspace small
    # a workspace off the 256-byte alignment fails closed (its shared-weight
    # rows take paired stores), in indexed and in batch mode
    odd = ctypes.c_void_p(256 + 4)
    assert f(hs._h, p, 1, p, p, p, p, p, 0, 1, 1, p, p, p, p, odd, big, None) == sp.E_INVALID
    assert b"aligned" in sp.lib.segpoly_last_error()
    assert f(hs._h, p, 2, p, p, None, None, None, 0, 2, 2, p, p, p, p, odd, big, None) == sp.E_INVALID
    assert b"aligned" in sp.lib.segpoly_last_error()
    assert f(hs._h, p, 1, p, p, p, p, p, 0, 1, 1, p, p, p, None, p, big, None) == sp.E_INVALID  # grad_w
    # table-driven descriptors: no workspace, except the shared-weight rows
    hg = sp.tp_create("32x0e+32x1o", "0e+1o", "0e+1o", force_generic=True)
    assert sp.tp_conv_bwd_workspace(hg, 1000) == 0
    hgs = sp.tp_create("32x0e+32x1o", "0e+1o", "0e+1o", force_generic=True, shared_weights=True)
    assert sp.tp_conv_bwd_workspace(hgs, 2049) == r256(2049 * hgs.weight_numel * 4) + 3 * hgs.weight_numel * 4
    assert f(hgs._h, p, 1, p, p, p, p, p, 0, 1, 1, p, p, p, p, None, 0, None) == sp.E_INVALID  # no workspace
    # more input components per channel than the table-driven backward holds
    # in LDS (float64: 128 components of 64 lanes)
    hbig = sp.tp_create("+".join(["2x6e"] * 10), "1o", "5o", dtype="f64")   # 130 input components
    assert not hbig.specialized
    assert f(hbig._h, p, 1, p, p, p, p, p, 0, 1, 1, p, p, p, p, p, big, None) == sp.E_UNSUPPORTED
    # nothing to do: succeeds without touching a device
    assert f(h._h, None, 0, None, None, None, None, None, 0, 0, 0, None, None, None, None, None, 0,
             None) == sp.OK


def test_symcon_backward_argument_errors_fail_before_any_gpu_call():
    s = sp.symcon_create("32x0e+32x1o", "32x0e", 3, 4)
    assert s.specialized
    n = ctypes.c_size_t()
    assert sp.lib.symcon_bwd_workspace(s._h, 100, ctypes.byref(n)) == sp.OK
    table = (16 * (4 + 3) + 255) // 256 * 256
    assert n.value == table + ((100 + 7) // 8 + 4 + 2) * s.weight_numel * 4
    assert sp.lib.symcon_bwd_workspace(s._h, -1, ctypes.byref(n)) == sp.E_INVALID
    f = sp.lib.symcon_bwd
    p = ctypes.c_void_p(16)   # never dereferenced: every call below fails validation
    big = 1 << 40
    # h, x, species, perm, idx, w, g, n_atoms, gx, gw, ws, ws_bytes, stream
    assert f(None, p, p, p, 0, p, p, 3, p, p, p, big, None) == sp.E_INVALID
    assert f(s._h, p, p, p, 0, p, p, -3, p, p, p, big, None) == sp.E_INVALID
    assert f(s._h, p, p, p, 5, p, p, 3, p, p, p, big, None) == sp.E_INVALID       # index dtype
    assert f(s._h, p, p, None, 0, p, p, 3, p, p, p, big, None) == sp.E_INVALID    # no perm
    assert f(s._h, p, p, p, 0, p, p, 3, p, None, p, big, None) == sp.E_INVALID    # no grad_w
    assert f(s._h, p, p, p, 0, p, p, 3, p, p, p, 16, None) == sp.E_INVALID        # workspace small
    odd = ctypes.c_void_p(512 + 8)
    assert f(s._h, p, p, p, 0, p, p, 3, p, p, odd, big, None) == sp.E_INVALID      # workspace misaligned
    assert b"aligned" in sp.lib.segpoly_last_error()
    assert f(s._h, p, p, p, 0, p, p, 1 << 31, p, p, p, big, None) == sp.E_UNSUPPORTED
    sg = sp.symcon_create("32x0e+32x1o", "32x0e", 3, 4, force_generic=True)
    assert sp.symcon_bwd_workspace(sg, 100) == 0   # the table-driven backward needs none
    assert f(sg._h, p, p, p, 0, p, p, 3, p, None, None, 0, None) == sp.E_INVALID  # no grad_w


def test_linear_descriptor_and_errors():
    h = sp.linear_create("3x0e+2x1o", "2x0e+4x1o")
    assert (h.dim_in, h.dim_out, h.weight_numel, h.num_segments) == (9, 14, 14, 2)
    h2 = sp.linear_create(workloads.CONV4_OUT, "128x0e+128x1o+128x2e")
    assert h2.dim_in == 5504 and h2.weight_numel == 13 * 128 * 128
    # the conv's actual output irreps are what the linear workload takes
    t = sp.tp_create(workloads.WORKLOADS[4].irreps_in1, workloads.WORKLOADS[4].irreps_in2,
                     workloads.WORKLOADS[4].irreps_out)
    assert t.irreps_out == workloads.CONV4_OUT
    raw = ctypes.c_void_p()
    assert sp.lib.linear_create(b"3x0e", b"3x0e", 7, 0, 0, ctypes.byref(raw)) == sp.E_INVALID
    assert sp.lib.linear_create(b"3x0q", b"3x0e", 0, 0, 0, ctypes.byref(raw)) == sp.E_PARSE
    assert sp.lib.linear_create(b"3x0e", b"3x0e", 0, 0, 1, ctypes.byref(raw)) == sp.E_INVALID   # flag
    big = "+".join(["1x0e"] * 40)
    assert sp.lib.linear_create(big.encode(), b"1x0e", 0, 0, 0, ctypes.byref(raw)) == sp.E_UNSUPPORTED
    # rows up to 65536 elements and 2^27 weights (32-bit operand offsets)
    wide = sp.linear_create("65536x0e", "1x0e")
    assert wide.dim_in == 65536
    assert sp.lib.linear_create(b"65537x0e", b"1x0e", 0, 0, 0, ctypes.byref(raw)) == sp.E_UNSUPPORTED
    assert sp.lib.linear_create(b"1x0e", b"21846x1o", 0, 0, 0, ctypes.byref(raw)) == sp.E_UNSUPPORTED
    assert sp.lib.linear_create(b"12000x0e", b"12000x0e", 0, 0, 0, ctypes.byref(raw)) == sp.E_UNSUPPORTED
    assert b"65536" in sp.lib.segpoly_last_error()
    p = ctypes.c_void_p(16)
    f = sp.lib.linear_fwd
    assert f(h._h, p, p, None, 0, 1, -1, p, None) == sp.E_INVALID
    assert f(h._h, p, p, p, 0, 0, 2, p, None) == sp.E_INVALID          # classes without num_classes
    assert f(h._h, p, p, None, 0, 1, 2, None, None) == sp.E_INVALID    # null out
    assert f(h._h, None, None, None, 0, 1, 0, None, None) == sp.OK     # nothing to do
    b = sp.lib.linear_bwd
    assert b(h._h, p, p, p, p, 0, 70000, 2, p, p, p, 1 << 30, None) == sp.E_UNSUPPORTED  # dw, too many classes
    assert b(h._h, p, p, p, None, 0, 1, 2, p, p, p, 8, None) == sp.E_INVALID          # workspace small
    assert b(h._h, p, p, p, p, 0, 3, 2, p, p, p, 8, None) == sp.E_INVALID             # same with classes
    # class-indexed weight gradient: one set of partials per class and two
    # int32 class bounds per row chunk
    w0, w3 = sp.linear_bwd_workspace(h, 5000, 0), sp.linear_bwd_workspace(h, 5000, 3)
    assert w0 > 0 and w3 > 3 * w0 and (w3 - 3 * w0) % 8 == 0
    assert sp.linear_bwd_workspace(h, 0, 3) == 0


@pytest.mark.parametrize("a,b,c", [("0 + 1", "0 + 1", "0 + 1"), ("32x0e+32x1o", "32x0e+32x1o", "32x0e+32x1o"),
                                   ("3x0e+2x1o+1x2e", "2x0e+1x1o+2x1e", "2x0e+3x1o+2x1e+1x2e+1x2o"),
                                   ("2x0e+1x1o", "1x0e", "2x0e+1x1o+2x2e"), ("4x2e+0x1o", "2x2e", "3x0e+0x1e+2x4e")])
def test_fctp_descriptor_matches_oracle(a, b, c):
    h = sp.fctp_create(a, b, c)
    f = ofctp.FullyConnectedTP(a, b, c)
    assert (h.dim_in1, h.dim_in2, h.dim_out, h.weight_numel) == (f.dim_in1, f.dim_in2, f.dim_out, f.weight_numel)
    assert [h.path_info(p) for p in range(h.num_paths)] == [tuple(p) for p in f.paths]


def test_rowptr_errors():
    p = ctypes.c_void_p(16)   # never dereferenced: every call below fails validation
    rb, rf = sp.lib.tp_rowptr_build, sp.lib.tp_conv_fwd_rowptr
    assert rb(None, 0, 5, 3, p, None) == sp.E_INVALID          # null dst with edges
    assert rb(p, 0, 5, 3, None, None) == sp.E_INVALID          # null row_ptr
    assert rb(p, 7, 5, 3, p, None) == sp.E_INVALID             # index dtype
    assert rb(p, 0, -1, 3, p, None) == sp.E_INVALID
    assert rb(p, 0, 1 << 31, 3, p, None) == sp.E_UNSUPPORTED   # int32 pointers
    h = sp.tp_create("8x0e+8x1o", "0e+1o", "0e+1o")
    assert rf(None, p, 4, p, p, p, p, 0, 5, 3, p, None) == sp.E_INVALID
    assert rf(h._h, p, 4, p, p, p, None, 0, 5, 3, p, None) == sp.E_INVALID   # null row_ptr
    assert rf(h._h, p, 4, p, p, None, p, 0, 5, 3, p, None) == sp.E_INVALID   # null src with edges
    assert rf(h._h, p, 4, p, p, p, p, 0, 5, 0, None, None) == sp.OK          # no destinations


def test_bwd_rowptr_errors():
    p = ctypes.c_void_p(16)   # never dereferenced: every call below fails validation or returns early
    sb, bb = sp.lib.tp_src_rowptr_build, sp.lib.tp_conv_bwd_rowptr
    assert sb(None, p, 0, 5, 3, p, None) == sp.E_INVALID          # null src with edges
    assert sb(p, None, 0, 5, 3, p, None) == sp.E_INVALID          # null src_perm with edges
    assert sb(p, p, 0, 5, 3, None, None) == sp.E_INVALID          # null row pointers
    assert sb(p, p, 7, 5, 3, p, None) == sp.E_INVALID             # index dtype
    assert sb(p, p, 0, 5, -1, p, None) == sp.E_INVALID
    assert sb(p, p, 0, 1 << 31, 3, p, None) == sp.E_UNSUPPORTED   # int32 pointers
    h = sp.tp_create("8x0e+8x1o", "0e+1o", "0e+1o")
    args = lambda **k: [k.get(n, d) for n, d in (
        ("h", h._h), ("x", p), ("n_src", 4), ("sh", p), ("w", p), ("src", p), ("dst", p), ("perm", p), ("rp", p),
        ("srp", p), ("idx", 0), ("n_edges", 5), ("n_nodes", 3), ("g", p), ("gx", p), ("gsh", p), ("gw", p),
        ("ws", p), ("wsb", 0), ("stream", None))]
    assert bb(*args(h=None)) == sp.E_INVALID
    assert bb(*args(rp=None)) == sp.E_INVALID                     # null row_ptr
    assert bb(*args(srp=None)) == sp.E_INVALID                    # null src_row_ptr
    assert bb(*args(dst=None)) == sp.E_INVALID                    # the table-driven kernels read dst
    assert bb(*args(perm=None)) == sp.E_INVALID
    assert bb(*args(idx=5)) == sp.E_INVALID
    assert bb(*args(ws=None)) == sp.E_INVALID                     # workspace missing
    assert bb(*args(n_src=0, n_edges=0, n_nodes=0)) == sp.OK      # nothing to do


def test_fctp_errors_and_workspace():
    raw = ctypes.c_void_p()
    c = sp.lib.fctp_create
    assert c(b"2x0e", b"2x0e", b"2x0e", 7, 0, 0, ctypes.byref(raw)) == sp.E_INVALID      # layout
    assert c(b"2x0e", b"2x0e", b"2x0e", 0, 3, 0, ctypes.byref(raw)) == sp.E_INVALID      # dtype
    assert c(b"2x0e", b"2x0e", b"2x0e", 0, 0, 4, ctypes.byref(raw)) == sp.E_INVALID      # flag
    assert c(b"2x0q", b"2x0e", b"2x0e", 0, 0, 0, ctypes.byref(raw)) == sp.E_PARSE
    assert c(b"0 + 1", b"0e", b"0e", 0, 0, 0, ctypes.byref(raw)) == sp.E_PARSE           # SO(3) with O(3)
    assert c(b"1x7o", b"1x0e", b"1x7o", 0, 0, 0, ctypes.byref(raw)) == sp.E_UNSUPPORTED  # l > 6
    # 3 x 3 -> 2 couples up to 10 component pairs per component (the 16-entry class)
    assert c(b"2x3o", b"1x3o", b"2x2e", 0, 0, 0, ctypes.byref(raw)) == sp.OK
    assert sp.lib.fctp_destroy(raw) == sp.OK
    h = sp.fctp_create("32x0e+32x1o", "32x0e+32x1o", "32x0e+32x1o")
    info = (ctypes.c_int64 * 4)()
    assert sp.lib.fctp_path_info(h._h, 4, info) == sp.E_INVALID
    assert sp.lib.fctp_query(h._h, 99, ctypes.byref(ctypes.c_int64())) == sp.E_INVALID
    p = ctypes.c_void_p(16)
    assert sp.lib.fctp_fwd(h._h, p, p, p, -1, p, None) == sp.E_INVALID
    assert sp.lib.fctp_fwd(h._h, p, p, p, 3, None, None) == sp.E_INVALID
    assert sp.lib.fctp_fwd(h._h, None, None, None, 0, None, None) == sp.OK
    assert sp.lib.fctp_fwd(None, p, p, p, 3, p, None) == sp.E_INVALID
    # backward workspace: one partial row of weight_numel per chunk of 1024
    # samples (weight gradient) and two transposed weight copies (input gradients)
    assert sp.fctp_bwd_workspace(h, 0) == 0
    assert sp.fctp_bwd_workspace(h, 1) == (1 + 2) * 131072 * 4
    assert sp.fctp_bwd_workspace(h, 2049) == (3 + 2) * 131072 * 4
    b = sp.lib.fctp_bwd
    assert b(h._h, p, p, p, p, 5000, None, None, p, p, 8, None) == sp.E_INVALID          # workspace small
    assert b(h._h, p, p, p, p, 5000, None, None, p, None, 1 << 30, None) == sp.E_INVALID  # null workspace
    assert b(h._h, p, p, None, p, 5000, p, None, None, None, 0, None) == sp.E_INVALID     # dx1: no workspace
    big = 1 << 30
    assert b(h._h, p, p, None, p, 5000, p, None, None, p, big, None) == sp.E_INVALID      # dx1 needs w
    assert b(h._h, None, None, None, None, 0, None, None, None, None, 0, None) == sp.OK
    # one weight row per sample: no workspace
    pf, pb = sp.lib.fctp_fwd_per_sample, sp.lib.fctp_bwd_per_sample
    assert pf(h._h, p, p, p, -1, p, None) == sp.E_INVALID
    assert pf(h._h, p, p, p, 3, None, None) == sp.E_INVALID
    assert pf(h._h, p, p, None, 3, p, None) == sp.E_INVALID
    assert pf(h._h, None, None, None, 0, None, None) == sp.OK
    assert pf(None, p, p, p, 3, p, None) == sp.E_INVALID
    assert pb(h._h, p, p, p, None, 3, p, None, None, None) == sp.E_INVALID      # no output gradient
    assert pb(h._h, p, p, None, p, 3, p, None, None, None) == sp.E_INVALID      # dx1 needs w
    assert pb(h._h, None, p, p, p, 3, None, None, p, None) == sp.E_INVALID      # dw needs x1
    assert pb(h._h, p, p, p, p, 3, None, None, None, None) == sp.OK             # nothing requested
    assert pb(h._h, p, p, p, p, -2, p, p, p, None) == sp.E_INVALID
    many = "+".join(["1000x0e"] * 5)
    wide = sp.fctp_create(many, many, "1x0e")   # the backward stages 2 (5000 + 5000) floats
    assert pb(wide._h, p, p, p, p, 3, p, None, None, None) == sp.E_UNSUPPORTED
    assert b"64 KB" in sp.lib.segpoly_last_error()
    assert sp.lib.fctp_destroy(None) == sp.OK
    # the convolution form: input 2 with one channel per block, w_rows 1 or n_edges
    cv = sp.lib.fctp_conv_fwd
    assert cv(h._h, p, 4, p, p, 1, p, p, 0, 3, 2, p, None) == sp.E_UNSUPPORTED        # 32x0e+32x1o as input 2
    hc = sp.fctp_create("16x0e+16x1o", "0e+1o+2e", "16x0e+16x1o", reduce="mean")
    assert cv(hc._h, p, 4, p, p, 2, p, p, 0, 3, 2, p, None) == sp.E_INVALID           # w_rows
    assert cv(hc._h, p, 4, p, p, 3, p, p, 5, 3, 2, p, None) == sp.E_INVALID           # index dtype
    assert cv(hc._h, p, 4, p, p, 3, None, p, 0, 3, 2, p, None) == sp.E_INVALID        # null src
    assert cv(hc._h, p, 4, p, p, 3, p, p, 0, 3, 2, None, None) == sp.E_INVALID        # null out
    assert cv(hc._h, p, -4, p, p, 3, p, p, 0, 3, 2, p, None) == sp.E_INVALID
    assert cv(hc._h, None, 0, None, None, 1, None, None, 0, 0, 0, None, None) == sp.OK  # nothing to do
    wide = sp.fctp_create("80x0e", "0e", "8x0e")                                     # > 64 channels:
    assert cv(wide._h, p, 4, p, p, 1, p, p, 0, 3, 2, None, None) == sp.E_INVALID     # accepted (null out)
    assert c(b"2x0e", b"2x0e", b"2x0e", 0, 0, 8 | 16, ctypes.byref(raw)) == sp.E_INVALID  # unknown flag
    # its backward: workspace of the per-edge messages, plus per-edge weight
    # gradients and their partial sums per 1024 edges with one shared row
    bw = sp.lib.fctp_conv_bwd
    assert sp.fctp_conv_bwd_workspace(hc, 1000) == 1000 * hc.dim_in1 * 4
    assert sp.fctp_conv_bwd_workspace(hc, 1000, 1) == 1000 * hc.dim_in1 * 4 \
        + (1000 * hc.weight_numel * 4 + 255) // 256 * 256 + hc.weight_numel * 4
    assert sp.fctp_conv_bwd_workspace(hc, 1, 1) == (hc.dim_in1 * 4 + 255) // 256 * 256  # one edge: its own row
    assert bw(hc._h, p, 4, p, p, 2, p, p, p, 0, 3, 2, p, p, p, p, p, 1 << 30, None) == sp.E_INVALID      # w_rows
    assert bw(hc._h, p, 4, p, p, 1, p, p, p, 0, 3, 2, p, p, p, p, p, 8, None) == sp.E_INVALID            # shared: workspace
    assert bw(hc._h, p, 4, p, p, 3, p, p, p, 0, 3, 2, p, p, p, p, p, 8, None) == sp.E_INVALID            # workspace
    assert bw(hc._h, p, 4, p, p, 3, p, p, None, 0, 3, 2, p, p, p, p, p, 1 << 30, None) == sp.E_INVALID   # no perm
    assert bw(hc._h, p, 4, p, p, 3, p, p, p, 0, 3, 2, p, p, None, p, p, 1 << 30, None) == sp.E_INVALID   # no dsh


def test_merged_descriptor():
    h = sp.tp_create("32x0e+32x1o", "0e+1o+2e", "0e+1o+2e", merge=True)
    o = otp.ChannelwiseTP("32x0e+32x1o", "0e+1o+2e", "0e+1o+2e", merge=True)
    assert h.irreps_out == o.irreps_out and h.dim_out == o.dim_out and h.weight_numel == o.weight_numel
    assert h.specialized and h.num_paths == o.num_paths
    raw = ctypes.c_void_p()
    assert sp.lib.tp_create(b"4x0e+3x0e", b"0e", b"0e", 0, 0, sp.MERGE_PATHS, ctypes.byref(raw)) == sp.E_UNSUPPORTED
    assert sp.lib.tp_create(b"4x0e", b"0e", b"0e", 0, 0, 32, ctypes.byref(raw)) == sp.E_INVALID


def test_edge_scalars_argument_errors():
    p = ctypes.c_void_p(16)
    f, b = sp.lib.edge_scalars_fwd, sp.lib.edge_scalars_bwd
    assert f(3, p, 4, p, 2, p, 2, p, p, 0, 5, 3, 3, p, None) == sp.E_INVALID          # dtype
    assert f(0, p, 4, p, 2, p, 2, p, p, 7, 5, 3, 3, p, None) == sp.E_INVALID          # index dtype
    assert f(0, p, 4, p, 2, p, 2, p, p, 0, -5, 3, 3, p, None) == sp.E_INVALID         # negative
    assert f(0, p, 4, None, 2, p, 2, p, p, 0, 5, 3, 3, p, None) == sp.E_INVALID       # src scalars
    assert f(0, p, 4, None, 0, None, 0, None, None, 0, 0, 0, 0, None, None) == sp.OK  # nothing to do
    assert b(0, p, 4, 2, 2, p, p, None, 0, 5, 3, 3, p, p, p, None) == sp.E_INVALID    # no src_perm
    assert b(0, p, 4, 2, 2, p, p, p, 0, 5, 3, 3, p, None, p, None) == sp.E_INVALID    # no grad_src


def test_sh_argument_errors():
    p = ctypes.c_void_p(16)
    assert sp.lib.sh_fwd(7, 1, 0, p, 4, p, None) == sp.E_UNSUPPORTED
    assert sp.lib.sh_fwd(-1, 1, 0, p, 4, p, None) == sp.E_UNSUPPORTED
    assert sp.lib.sh_fwd(3, 1, 5, p, 4, p, None) == sp.E_INVALID
    assert sp.lib.sh_fwd(3, 1, 0, p, -4, p, None) == sp.E_INVALID
    assert sp.lib.sh_fwd(3, 1, 0, None, 4, p, None) == sp.E_INVALID
    assert sp.lib.sh_bwd(3, 1, 0, p, None, 4, p, None) == sp.E_INVALID
    assert sp.lib.sh_fwd(3, 1, 0, None, 0, None, None) == sp.OK


def test_bench_traffic_replay_rejects_other_shapes_before_any_gpu_call():
    """The benchmark's traffic-replay probe (its own library, loaded only by
    bench.py) replays the large graph's shape alone; anything else, and
    missing buffers, are refused before a launch."""
    path = os.path.join(os.path.dirname(sp.__file__), "libsegpoly_bench.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    lib = ctypes.CDLL(path)
    fn = lib.segpoly_bench_traffic_replay
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_int64,
                                                                          ctypes.c_int] + [ctypes.c_int64] * 4 + [
        ctypes.c_void_p]
    p = ctypes.c_void_p(16)
    shape = (1664, 1152, 16, 5504)
    assert fn(0, 0, p, p, p, p, p, 10, 10, 30, 1663, 1152, 16, 5504, None) == -1   # weights per edge
    assert fn(0, 0, p, p, p, p, p, 10, 10, 30, 1664, 1152, 9, 5504, None) == -1    # harmonics
    assert fn(2, 0, p, None, p, p, p, 10, 10, 30, *shape, None) == -1              # gather without x
    assert fn(0, 0, p, p, p, p, p, 0, 10, 30, *shape, None) == -1                  # no nodes
    assert fn(0, 0, p, p, p, p, p, 10, 10, 0, *shape, None) == -1                  # no edges per node
    assert fn(7, 0, p, p, p, p, p, 10, 10, 30, *shape, None) == -1                 # mode


def test_fctp_coupling_entry_limit_matches_oracle():
    """The fully connected product compiles coupling classes of up to 16
    non-zero entries per component (along each of the three axes: output,
    and the two input gradients).  Every SO(3) coupling with l1, l2, l3 <= 6
    builds exactly when the oracle's tensor stays within that, and fails
    closed (E_UNSUPPORTED) otherwise, e.g. 5 x 1 -> 5 (18 entries)."""
    for l1 in range(7):
        for l2 in range(7):
            for l3 in range(abs(l1 - l2), min(l1 + l2, 6) + 1):
                nz = np.abs(ocg.real_cg(l1, l2, l3)) > 1e-13
                most = max(nz.sum(axis=(1, 2)).max(), nz.sum(axis=(0, 2)).max(), nz.sum(axis=(0, 1)).max())
                raw = ctypes.c_void_p()
                rc = sp.lib.fctp_create(f"1x{l1}".encode(), f"1x{l2}".encode(), f"1x{l3}".encode(), 0, 0, 0,
                                        ctypes.byref(raw))
                if most > 16:
                    assert rc == sp.E_UNSUPPORTED, (l1, l2, l3, most)
                    assert b"couplings per component" in sp.lib.segpoly_last_error()
                else:
                    assert rc == sp.OK, (l1, l2, l3, sp.lib.segpoly_last_error())
                    sp.lib.fctp_destroy(raw)
    with pytest.raises(sp.SegpolyError) as err:
        sp.fctp_create("1x5o", "1x1o", "1x5e")
    assert err.value.code == sp.E_UNSUPPORTED
