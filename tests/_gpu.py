"""Helpers of the GPU parity tests: device transfer, the oracle side of a
comparison, and the tolerance check (scaled error, see oracle.metrics)."""

import sys

import numpy as np
import pytest

from oracle import layout as olayout
from oracle import metrics

F32_TOL = 1e-5     # max |g - o| / A in float32
F64_TOL = 1e-12    # max |g - o| / A in float64


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def announce(what):
    """Name the case before a GPU step (so a crash log says which)."""
    print(f"\n[gpu case] {what}", flush=True)
    sys.stdout.flush()


def dev(a, torch_dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if torch_dtype is not None:
        t = t.to(torch_dtype)
    return t.cuda()


def tol(dtype):
    return F32_TOL if dtype == "f32" else F64_TOL


def check_scaled(got, ref, scale, dtype, what=""):
    err = metrics.scaled_error(got, ref, scale)
    nw = metrics.normwise_error(got, ref)
    print(f"[parity] {what} scaled={err:.3e} normwise={nw:.3e}", flush=True)
    assert err <= tol(dtype), f"{what}: scaled error {err:.3e} > {tol(dtype):.1e}"
    return err


def to_layout(x, blocks, src, dst):
    return olayout.transpose(x, blocks, src, dst)
