"""The allocation-free symmetric-contraction backward (symcon_bwd_noalloc,
workspace in the library's fixed device scratch) against the entry point
with a caller workspace (symcon_bwd), called through the C ABI.

The two run the same kernels, and those kernels are deterministic (fixed
summation order, no atomics), so the results must agree bit for bit, which
is stronger than the float32 bar of the parity tests (scaled error 1e-5).
Calls in a row share the scratch: the first call is the 50,000-atom bench
shape (the largest the scratch holds at 128 channels), the next ones are
smaller and use the scratch the previous call left behind.  The host-side
refusals (sizes above the scratch, VALIDATE handles) run without a GPU."""

import ctypes

import numpy as np
import pytest

import workloads
from oracle import metrics


def _sp():
    import segmented_polynomials_amd as sp
    return sp


def _inputs(torch, hs, n, seed, idx_dtype):
    rng = np.random.default_rng(seed)
    dev = torch.device("cuda")
    x = torch.from_numpy(rng.standard_normal((n, hs.dim_in), dtype=np.float32)).to(dev)
    w = torch.from_numpy(rng.standard_normal((hs.num_elements, hs.weight_numel), dtype=np.float32)).to(dev)
    g = torch.from_numpy(rng.standard_normal((n, hs.dim_out), dtype=np.float32)).to(dev)
    species = torch.from_numpy(rng.integers(0, hs.num_elements, n).astype(np.int64)).to(dev).to(idx_dtype)
    perm = torch.argsort(species, stable=True).to(idx_dtype)
    return x, species, w, g, perm


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_on_calls_in_a_row():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    sp = _sp()
    s5 = workloads.WORKLOADS[5]
    ha = sp.symcon_create(s5.irreps_in, s5.irreps_out, 3, s5.num_elements, layout="ir_mul")
    hb = sp.symcon_create(s5.irreps_in, s5.irreps_out, 3, s5.num_elements, layout="mul_ir")
    assert sp.symcon_bwd_workspace(ha, s5.n_atoms) <= sp.NOALLOC_SCRATCH_BYTES
    calls = [(ha, s5.n_atoms, 501, torch.int32), (ha, 1200, 502, torch.int32), (hb, 700, 503, torch.int64)]
    for h, n, seed, it in calls:
        print(f"\n[gpu case] symcon_bwd_noalloc {h.layout} n_atoms={n} {it}", flush=True)
        x, species, w, g, perm = _inputs(torch, h, n, seed, it)
        ref_x, ref_w = sp.symcon_bwd(h, x, species, w, g, perm)
        got_x, got_w = sp.symcon_bwd_noalloc(h, x, species, w, g, perm)
        torch.cuda.synchronize()
        for got, ref, name in ((got_x, ref_x, "grad_x"), (got_w, ref_w, "grad_w")):
            a, b = got.cpu().numpy(), ref.cpu().numpy()
            err = metrics.scaled_error(a, b, np.abs(b) + np.abs(b).max() * 1e-30)
            assert err <= 1e-5, f"{name}: scaled error {err}"
            assert np.array_equal(a, b), f"{name} differs from symcon_bwd at n_atoms={n}"
        del x, species, w, g, perm, ref_x, ref_w, got_x, got_w


def test_noalloc_refusals_before_any_launch():
    """Sizes beyond the scratch and VALIDATE handles fail closed on the
    host; the pointers are never read (no GPU needed)."""
    sp = _sp()
    s5 = workloads.WORKLOADS[5]
    h = sp.symcon_create(s5.irreps_in, s5.irreps_out, 3, s5.num_elements, layout="ir_mul")
    fake = ctypes.c_void_p(256)    # never dereferenced: the call returns first
    big = 200000
    assert sp.symcon_bwd_workspace(h, big) > sp.NOALLOC_SCRATCH_BYTES
    args = (fake, fake, fake, sp.I32, fake, fake, big, fake, fake, None)
    assert sp.lib.symcon_bwd_noalloc(h._h, *args) == sp.E_UNSUPPORTED
    assert b"scratch" in sp.lib.segpoly_last_error()
    hv = sp.symcon_create(s5.irreps_in, s5.irreps_out, 3, s5.num_elements, layout="ir_mul", validate=True)
    assert sp.lib.symcon_bwd_noalloc(hv._h, fake, fake, fake, sp.I32, fake, fake, 10, fake, fake,
                                     None) == sp.E_UNSUPPORTED
    assert sp.lib.symcon_bwd_noalloc(None, *args) == sp.E_INVALID
    assert sp.lib.symcon_bwd_noalloc(h._h, fake, fake, fake, sp.I32, fake, fake, -1, fake, fake,
                                     None) == sp.E_INVALID
