"""GPU parity of the spherical harmonics of vectors (forward and
vector-Jacobian product), called through the C ABI, against the float64
oracle, for every degree the library accepts (0..6).  Tolerance: scaled
error (oracle.metrics) <= 1e-5 in float32, <= 1e-12 in float64, the scale
being the oracle's sum of absolute terms of each harmonic
(oracle.sh.real_sh_abs) and of each gradient (oracle.sh.real_sh_vjp_abs)."""

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


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("lmax", [0, 1, 2, 3, 4, 5, 6])
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
    check_scaled(got, ref, osh.real_sh_abs(ls, vv, normalize=normalize), dtype,
                 f"sh fwd lmax={lmax} norm={normalize}")


@pytest.mark.parametrize("dtype", ["f32", "f64"])
@pytest.mark.parametrize("normalize", [True, False])
@pytest.mark.parametrize("lmax", [1, 2, 3, 4, 5, 6])
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
    check_scaled(got, ref, osh.real_sh_vjp_abs(ls, v, g, normalize=normalize), dtype,
                 f"sh bwd lmax={lmax} norm={normalize}")


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
