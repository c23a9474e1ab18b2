"""Shared helpers for the GPU parity tests (tolerances and conversions)."""
import numpy as np
import pytest
import torch

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(),
                               reason="no GPU visible")


def dev():
    return torch.device("cuda", 0)


def to_np(t):
    return t.detach().cpu().numpy()


def fp16_ulp(z):
    """Spacing of binary16 at |z| (subnormal spacing 2^-24 near zero)."""
    a = np.minimum(np.abs(np.asarray(z, np.float64)), 65504.0)
    return np.spacing(a.astype(np.float16)).astype(np.float64)


def assert_fp16_close_to_oracle(y_gpu, z_oracle, what=""):
    """|y - z| <= 1 fp16 ulp(z) + 1e-3 for every element."""
    y = np.asarray(y_gpu, np.float64)
    z = np.asarray(z_oracle, np.float64)
    err = np.abs(y - z)
    tol = fp16_ulp(z) + 1e-3
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outside ulp+1e-3; worst at "
            f"{i}: gpu {y[i]!r} oracle {z[i]!r}")


def assert_codes_within_one(q_gpu, q_oracle, frac=1e-3, what=""):
    """Fused LN+quant: codes differ by at most 1, in at most `frac` of them."""
    d = np.abs(q_gpu.astype(np.int32) - q_oracle.astype(np.int32))
    assert d.max() <= 1, f"{what}: code difference {d.max()}"
    assert (d != 0).mean() <= frac, f"{what}: {(d != 0).mean():.3%} codes differ"


def assert_ln_close(h_gpu, h_oracle, what=""):
    """LN output within 2e-3 relative, floor of 1 fp16 ulp for |h| < 2^-14."""
    h = np.asarray(h_gpu, np.float64)
    r = np.asarray(h_oracle, np.float64)
    tol = np.maximum(2e-3 * np.abs(r), np.where(np.abs(r) < 2.0 ** -14,
                                                2.0 ** -24, 0.0))
    bad = np.abs(h - r) > tol
    assert not bad.any(), f"{what}: {bad.sum()} LN outputs outside 2e-3"
