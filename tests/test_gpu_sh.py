"""GPU parity of the spherical harmonics of vectors (forward and
vector-Jacobian product), called through the C ABI, against the float64
oracle.  Tolerance: scaled error (oracle.metrics, scale = the oracle on
|operands| where one exists, else the magnitude of the reference) <= 1e-5
in float32, <= 1e-12 in float64."""

import numpy as np
import pytest

import workloads
from oracle import sh as osh
from tests._gpu import announce, check_scaled, dev, need_gpu

pytestmark = pytest.mark.gpu


def _sp():
    need_gpu()
    import segmented_polynomials_amd as sp
    return sp


def _scale_fwd(ls, v, normalize):
    # a bound of every partial sum: the harmonics of (|x|, |y|, |z|) with all
    # coefficients made positive is not available from the oracle, so the
    # scale is the degree-wise norm sqrt(sum_m Y^2) = sqrt(2l+1) |v|^l (or
    # sqrt(2l+1) normalised), spread over the block
    r = np.linalg.norm(v, axis=1, keepdims=True)
    cols = []
    for l in ls:
        s = np.sqrt(2 * l + 1) * (np.ones_like(r) if normalize else r ** l)
        cols.append(np.repeat(s, 2 * l + 1, axis=1))
    return np.concatenate(cols, axis=1)


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("lmax", [0, 1, 2, 3, 4, 6])
def test_forward(dtype, normalize, lmax):
    sp = _sp()
    import torch
    rng = np.random.default_rng(10 + lmax)
    n = 1000 + 37                     # several workgroups and a partial one
    v = rng.standard_normal((n, 3))
    v[:5] *= 1e-3                     # short and long vectors
    v[5:10] *= 50.0
    td = torch.float32 if dtype == "f32" else torch.float64
    vv = v.astype(np.float32).astype(np.float64) if dtype == "f32" else v
    announce(f"sh fwd lmax={lmax} normalize={normalize} {dtype}")
    got = sp.sh_fwd(dev(vv, td), lmax, normalize=normalize).cpu().numpy()
    ls = list(range(lmax + 1))
    ref = osh.real_sh(ls, vv, normalize=normalize)
    check_scaled(got, ref, _scale_fwd(ls, vv, normalize), dtype, f"sh fwd lmax={lmax} norm={normalize}")


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("lmax", [1, 2, 3, 4])
def test_backward(dtype, normalize, lmax):
    sp = _sp()
    import torch
    rng = np.random.default_rng(20 + lmax)
    n = 700
    v = rng.standard_normal((n, 3))
    nc = (lmax + 1) ** 2
    g = rng.standard_normal((n, nc))
    td = torch.float32 if dtype == "f32" else torch.float64
    if dtype == "f32":
        v, g = v.astype(np.float32).astype(np.float64), g.astype(np.float32).astype(np.float64)
    announce(f"sh bwd lmax={lmax} normalize={normalize} {dtype}")
    got = sp.sh_bwd(dev(v, td), dev(g, td), lmax, normalize=normalize).cpu().numpy()
    ls = list(range(lmax + 1))
    ref = osh.real_sh_vjp(ls, v, g, normalize=normalize)
    # scale: |g| against the gradient magnitude of each degree (sum_m |dY|
    # is at most l sqrt(2l+1) |v|^(l-1) per unit direction, or that over |v|
    # with normalisation), summed over degrees
    r = np.linalg.norm(v, axis=1)
    sc = np.zeros(n)
    for l in ls[1:]:
        blk = np.abs(g[:, l * l:(l + 1) * (l + 1)]).sum(1)
        sc += blk * l * np.sqrt(2 * l + 1) * ((1 / r) if normalize else r ** (l - 1))
    check_scaled(got, ref, np.repeat(sc[:, None], 3, axis=1), dtype, f"sh bwd lmax={lmax} norm={normalize}")


def test_workload_harmonics_and_zero_vector():
    """The workloads' edge harmonics (l <= 3 of random unit vectors) match
    the kernel; a zero vector with normalisation gives Y_0 = 1, zeros and a
    zero gradient."""
    sp = _sp()
    import torch
    rng = np.random.default_rng(3)
    v = rng.standard_normal((500, 3))
    ref = workloads.edge_harmonics(v, (0, 1, 2, 3))
    announce("sh workload harmonics")
    got = sp.sh_fwd(dev(v, torch.float64), 3).cpu().numpy()
    assert np.allclose(got, ref, atol=1e-13)
    z = torch.zeros(3, 3, dtype=torch.float64, device="cuda")
    y = sp.sh_fwd(z, 3).cpu().numpy()
    assert np.all(y[:, 0] == 1) and np.count_nonzero(y[:, 1:]) == 0
    gz = sp.sh_bwd(z, torch.ones(3, 16, dtype=torch.float64, device="cuda"), 3).cpu().numpy()
    assert np.count_nonzero(gz) == 0
