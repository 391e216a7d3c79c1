"""GPU parity of the edge-embedding assembly of the convolution layer (edge
embedding with gathered src/dst scalars, and its backward), through the C
ABI, against the oracle.  Gathers and slices are exact (bit-equal); the
backward sums are compared at the float tolerance of the other tests."""

import numpy as np
import pytest

from oracle import edge_scalars as es
from tests._gpu import announce, check_scaled, dev, need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("idx", ["int32", "int64"])
@pytest.mark.parametrize("parts", [(16, 8, 8), (5, 0, 3), (0, 70, 0), (33, 2, 0)])
def test_forward_and_backward(parts, idx, dtype):
    import torch
    need_gpu()
    import segmented_polynomials_amd as sp
    d_emb, d_src, d_dst = parts
    rng = np.random.default_rng(sum(parts))
    n_src, n_dst = 37, 29
    deg = rng.integers(0, 9, n_dst)
    deg[::5] = 0
    dst = np.repeat(np.arange(n_dst), deg)
    E = dst.shape[0]
    src = rng.integers(0, n_src, E)
    dt = np.float32 if dtype == "f32" else np.float64
    emb = rng.standard_normal((E, d_emb)).astype(dt)
    ssc = rng.standard_normal((n_src, d_src)).astype(dt) if d_src else None
    dsc = rng.standard_normal((n_dst, d_dst)).astype(dt) if d_dst else None
    it = torch.int32 if idx == "int32" else torch.int64
    S, D = dev(src).to(it), dev(dst).to(it)
    announce(f"edge scalars {parts} {idx} {dtype} E={E}")
    out = sp.edge_scalars_fwd(dev(emb), S, D, None if ssc is None else dev(ssc), None if dsc is None else dev(dsc))
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), es.concat(emb, ssc, dsc, src, dst).astype(dt))
    g = rng.standard_normal((E, d_emb + d_src + d_dst)).astype(dt)
    perm = dev(np.argsort(src, kind="stable")).to(it)
    ge, gs, gd = sp.edge_scalars_bwd(dev(g), d_emb, d_src, d_dst, S, D, perm, n_src, n_dst)
    torch.cuda.synchronize()
    re_, rs, rd = es.concat_vjp(g, d_emb, d_src, d_dst, src, dst, n_src, n_dst)
    ae, as_, ad = es.concat_vjp(np.abs(g), d_emb, d_src, d_dst, src, dst, n_src, n_dst)
    assert np.array_equal(ge.cpu().numpy(), re_.astype(dt))
    if d_src:
        check_scaled(gs.cpu().numpy(), rs, as_, dtype, "grad src scalars")
    if d_dst:
        check_scaled(gd.cpu().numpy(), rd, ad, dtype, "grad dst scalars")
