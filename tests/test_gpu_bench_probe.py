"""The benchmark's traffic-replay probe (libsegpoly_bench.so) reads and
writes what the benchmark says it does: per destination node the weight
rows of its edges, the gathered source rows and the harmonics, and one
output row, checked on a small graph of the large graph's shape against the
same sums in NumPy (float64)."""

import ctypes
import os

import numpy as np
import pytest

from tests._gpu import announce, dev, need_gpu

pytestmark = pytest.mark.gpu

WN, XN, SHN, ON = 1664, 1152, 16, 5504


def _fn():
    import segmented_polynomials_amd as sp
    path = os.path.join(os.path.dirname(sp.__file__), "libsegpoly_bench.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    fn = ctypes.CDLL(path).segpoly_bench_traffic_replay
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 5 + [ctypes.c_int64, ctypes.c_int64,
                                                                          ctypes.c_int] + [ctypes.c_int64] * 4 + [
        ctypes.c_void_p]
    return fn


@pytest.mark.parametrize("mode,nt", [(1, 0), (1, 1), (2, 0), (2, 1)])
def test_traffic_replay_sums(mode, nt):
    import torch
    need_gpu()
    fn = _fn()
    n, deg, n_src = 40, 30, 37
    rng = np.random.default_rng(5 + mode)
    w = rng.standard_normal((n * deg, WN), dtype=np.float32)
    x = rng.standard_normal((n_src, XN), dtype=np.float32)
    sh = rng.standard_normal((n * deg, SHN), dtype=np.float32)
    src = rng.integers(0, n_src, n * deg).astype(np.int32)
    W, X, S, I = dev(w, torch.float32), dev(x, torch.float32), dev(sh, torch.float32), dev(src, torch.int32)
    out = torch.zeros((n, ON), dtype=torch.float32, device="cuda")
    announce(f"traffic replay mode {mode} nt {nt}")
    rc = fn(mode, nt, W.data_ptr(), X.data_ptr(), S.data_ptr(), I.data_ptr(), out.data_ptr(), n, n_src, deg,
            WN, XN, SHN, ON, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    got = out.cpu().numpy().astype(np.float64)
    # per node and channel c (lane c // 2): a[c] = sum over edges of the weight row's channel c in
    # every 128-wide segment, plus (mode 2) the gathered row's channel c times the edge's harmonics sum
    wd = w.astype(np.float64).reshape(n, deg, WN // 128, 128).sum(axis=(1, 2))
    a = wd
    if mode == 2:
        xs = x.astype(np.float64)[src].reshape(n, deg, XN // 128, 128).sum(axis=2)
        hs = sh.astype(np.float64).sum(axis=1).reshape(n, deg, 1)
        a = a + (xs * hs).sum(axis=1)
    k = np.arange(ON // 128).reshape(1, -1, 1)
    sign = np.where(np.arange(128) % 2 == 0, 1.0, -1.0).reshape(1, 1, 128)
    want = a.reshape(n, 1, 128) + sign * k
    scale = np.abs(want).max()
    assert np.abs(got.reshape(n, ON // 128, 128) - want).max() <= 1e-5 * scale
