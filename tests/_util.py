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


def assert_linear_matches_oracle(y, qx, sx, ref, q, sw, G, act, ln, what=""):
    """One quantized linear of the HIP path (its codes qx, scales sx and
    output y) against the oracle's linear computed from the same CPU inputs
    (``ref`` = oracle.linear(...), ``q`` the oracle's int8 weight codes).

    * Codes: with LayerNorm, within 1 of the oracle's and different in at
      most 0.1% of them, scales within 2e-3 relative; without LayerNorm
      (identical quantizer inputs) bit-exact.
    * y: in every token row whose codes and scale equal the oracle's, within
      1 fp16 ulp + 1e-3 of the oracle's fp64 epilogue.  In a row where LN
      moved a code or the scale, the tolerance widens by the derived bound
      L * sw[n/G] * (|sx - sx_ref| * (|acc_ref| + D) + sx * D) with
      D = sum over moved codes of |dq| * |q[n, k]| (L = 1.13 bounds the GeLU
      slope; 1 without GeLU)."""
    qx = np.asarray(qx)
    sx = np.asarray(sx, np.float32)
    dq = qx.astype(np.int64) - ref["qx"].astype(np.int64)
    if ln:
        assert_codes_within_one(qx, ref["qx"], 1e-3, what + " codes")
        assert np.allclose(sx, ref["sx"], rtol=2e-3, atol=0), what + " scales"
    else:
        assert np.array_equal(qx, ref["qx"]), what + " codes"
        assert np.array_equal(sx, ref["sx"]), what + " scales"
    z = ref["z"]
    tol = fp16_ulp(z) + 1e-3
    moved = (dq != 0).any(axis=1) | (sx != ref["sx"])
    if moved.any():
        rows = np.nonzero(moved)[0]
        D = np.abs(dq[rows]).astype(np.float64) @ np.abs(q.astype(np.float64)).T
        swn = np.repeat(np.asarray(sw, np.float64), G)[None, :]
        dsx = np.abs(sx[rows].astype(np.float64) - ref["sx"][rows])[:, None]
        L = 1.13 if act == 1 else 1.0
        acc = np.abs(ref["acc"][rows].astype(np.float64))
        tol[rows] += L * swn * (dsx * (acc + D) + sx[rows, None] * D)
    err = np.abs(np.asarray(y, np.float64) - z)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outputs outside the tolerance; "
            f"worst at {i}: gpu {float(np.asarray(y)[i])!r} oracle {z[i]!r} "
            f"(row moved: {bool(moved[i[0]])})")
