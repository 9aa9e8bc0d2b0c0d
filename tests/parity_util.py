"""Comparison helpers and the tolerances the parity tests apply.

Tolerances (stated for this method's outputs; the pages give none):
  * bf16 inputs, fp32 accumulation: max|x - x*| <= 2e-2 and mean|x - x*| <= 2e-3
    for O and LSE;
  * fp32 inputs: max|x - x*| <= 1e-4;
  * gradients dQ, dK, dV: the same bounds applied to |g - g*| / max|g*|.
x* is the fp64 oracle evaluated on exactly the values the GPU received.
"""

from __future__ import annotations

import numpy as np

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
FP32_MAX = 1e-4


def to64(t) -> np.ndarray:
    """Exact widening of a (GPU or CPU) torch tensor to a float64 NumPy array."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def err_stats(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    fin = np.isfinite(ref)
    # both sides must agree on which entries are infinite (LSE of empty rows)
    assert np.array_equal(np.isfinite(got), fin), "finite/infinite pattern differs"
    if not np.any(fin):
        return 0.0, 0.0
    e = np.abs(got[fin] - ref[fin])
    return float(e.max()), float(e.mean())


def assert_bf16_close(got, ref, what=""):
    mx, mean = err_stats(got, ref)
    assert mx <= BF16_MAX and mean <= BF16_MEAN, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def assert_fp32_close(got, ref, what=""):
    mx, mean = err_stats(got, ref)
    assert mx <= FP32_MAX, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def assert_grad_close(got, ref, what="", max_tol=BF16_MAX, mean_tol=BF16_MEAN):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = float(np.max(np.abs(ref)))
    if scale == 0.0:
        assert float(np.max(np.abs(got))) == 0.0, f"{what}: expected all zeros"
        return 0.0, 0.0
    e = np.abs(got - ref) / scale
    mx, mean = float(e.max()), float(e.mean())
    assert mx <= max_tol and mean <= mean_tol, f"{what}: rel max {mx:.3e} rel mean {mean:.3e}"
    return mx, mean
