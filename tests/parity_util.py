"""Shared helpers of the parity tests: tolerance checks and the documented
exemptions for sampled decisions.  Nothing here computes the method; expected
values come from the oracle (or from numpy/scipy where stated)."""
import numpy as np
import torch
from scipy.special import softmax

ATTN_REL, ATTN_ABS = 1e-2, 1e-3      # bf16 inputs, fp32 accumulation
F32_REL, F32_ABS = 1e-5, 1e-6        # fp32 path
U_EXEMPT = 1e-6                      # sampled decisions within this of the threshold


def to64(t):
    return t.detach().cpu().double().numpy() if t.is_floating_point() else t.detach().cpu().numpy()


def assert_close_scaled(got, ref, rel, abs_, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref).max() if got.size else 0.0
    bound = rel * np.abs(ref).max() + abs_ if ref.size else abs_
    assert err <= bound, f"{what}: max|err| {err:.3e} > {bound:.3e}"
    return err, bound


def draw_boundary_ok(z_row, T, u, got, ref, residual_q=None, residual_exclude=None):
    """A categorical draw may differ from the oracle only when u * S lies within
    1e-6 * S of a CDF boundary between the two indices (weights in fp64 by scipy).
    residual_exclude: token removed from p (the residual of a deterministic draft)."""
    if got == ref:
        return True
    if residual_exclude is not None:
        w = softmax(np.asarray(z_row, dtype=np.float64) / T)
        w[int(residual_exclude)] = 0.0
    elif residual_q is None:
        w = softmax(np.asarray(z_row, dtype=np.float64) / T)
    else:
        p = softmax(np.asarray(z_row, dtype=np.float64) / T)
        q = softmax(np.asarray(residual_q, dtype=np.float64) / T)
        w = np.maximum(p - q, 0.0)
        if w.sum() <= 0:
            w = p
    c = np.cumsum(w) / w.sum()
    lo, hi = min(got, ref), max(got, ref)
    # every boundary between the two indices must be within the exemption of u
    bounds = c[lo:hi]
    return bool(np.all(np.abs(bounds - u) < U_EXEMPT)) and w[got] > 0


def cuda():
    return torch.device("cuda:0")
