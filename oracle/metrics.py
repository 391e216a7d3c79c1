"""Error metric of the parity tests (oracle side).

The tolerance asked for is a maximum relative error (1e-5 in float32; the
pages compare float64 results at atol 1e-12 in the cuequivariance-torch skill
document, "Spherical harmonics and a NumPy reference" and "Channelwise
product with external per-example weights").  A plain |g - o| / |o| is
ill-posed where a sum cancels to about zero, so the error of each output is
scaled by A_i, the same output evaluated with the absolute values of every
operand and coefficient (the standard forward-error scale of a sum of
products):

    err = max_i |g_i - o_i| / A_i,   with g_i == o_i required where A_i == 0.
"""

import numpy as np


def scaled_error(got, ref, scale):
    """max_i |got_i - ref_i| / scale_i (inf if scale_i == 0 and got_i != ref_i)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.asarray(scale, dtype=np.float64)
    if got.shape != ref.shape or ref.shape != scale.shape:
        raise ValueError(f"shape mismatch {got.shape} {ref.shape} {scale.shape}")
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    diff = np.abs(got - ref)
    zero = scale == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    s = np.where(zero, 1.0, scale)
    return float(np.max(diff / s))


def normwise_error(got, ref):
    """||got - ref||_inf / ||ref||_inf (reported beside the scaled error)."""
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    if den == 0:
        return float(np.max(np.abs(got))) if np.size(got) else 0.0
    return float(np.max(np.abs(np.asarray(got, dtype=np.float64) - ref)) / den)
