"""Comparison helpers and the tolerances the parity tests apply.

Tolerances (stated for this method's outputs; the pages give none):
  * bf16 inputs, fp32 accumulation: max|x - x*| <= 2e-2 and mean|x - x*| <= 2e-3
    for O and LSE;
  * fp32 inputs: max|x - x*| <= 1e-4;
  * gradients dQ, dK, dV: the same bounds applied to |g - g*| / max|g*|;
  * LSE with bf16 inputs: |LSE - LSE*| <= 4.5e-3 + 2^-17 |LSE*|, derived from
    the arithmetic rather than borrowed from O.  The kernels sum the same
    bf16-rounded probabilities that enter P V.  bf16 carries 8 significant
    bits, so rounding to nearest has relative error at most 2^-8; all terms
    are positive, so the row sum is off by a factor within 1 +- 2^-8, i.e. at
    most ln(1 + 2^-8) = 3.90e-3 in the LSE (reached when one rounded term
    dominates a row).  fp32 accumulation of the sum (a lane chain of at most
    N/2 terms, N <= 16K: below 5e-4 relative) and of the scores (exact bf16
    products, d terms) add less than 6e-4 at unit-variance inputs.  The
    relative term covers the fp32 rounding of the running maximum and of
    m ln 2 + ln l for large |LSE|.
x* is the fp64 oracle evaluated on exactly the values the GPU received.
"""

from __future__ import annotations

import numpy as np

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
FP32_MAX = 1e-4
LSE_ABS, LSE_REL = 4.5e-3, 2.0 ** -17


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


def score_error_bound(q, k, scale):
    """Per query row, the worst-case error of an fp32-accumulated score
    scale * q.k of bf16 inputs: every product is exact in fp32 and d of them are
    summed, so |error| <= d 2^-24 scale max_j sum_e |q_e k_je| (recursive
    summation bound).  It enters the LSE at most once.  q [B,H,N,d],
    k [B,Hkv,N,d] as float64; returns [B,H,N]."""
    q = np.abs(np.asarray(q, dtype=np.float64))
    k = np.abs(np.asarray(k, dtype=np.float64))
    G = q.shape[1] // k.shape[1]
    k = np.repeat(k, G, axis=1)
    d = q.shape[-1]
    return d * 2.0 ** -24 * scale * np.max(q @ np.swapaxes(k, -1, -2), axis=-1)


def assert_lse_close(got, ref, what="", extra=None):
    """LSE of bf16 inputs against the oracle, within the bound derived above
    (plus ``extra``, e.g. ``score_error_bound`` for inputs with large scores)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mx, mean = err_stats(got, ref)
    fin = np.isfinite(ref)
    if np.any(fin):
        allow = LSE_ABS + LSE_REL * np.abs(ref)
        if extra is not None:
            allow = allow + np.broadcast_to(np.asarray(extra, dtype=np.float64), ref.shape)
        excess = np.abs(got[fin] - ref[fin]) - allow[fin]
        assert float(excess.max()) <= 0.0, f"{what}: max {mx:.3e} mean {mean:.3e} (bound {LSE_ABS:.1e} + 2^-17|LSE|)"
    return mx, mean


def assert_fp32_close(got, ref, what=""):
    mx, mean = err_stats(got, ref)
    assert mx <= FP32_MAX, f"{what}: max {mx:.3e} mean {mean:.3e}"
    return mx, mean


def one_key_grad_bound(x, v, do, scale):
    """Bound on |dQ| (x = K) or |dK| (x = Q) when every query sees one key.

    Then P = 1 and dS = P (dP - D) is exactly 0, so the true dQ and dK vanish
    and a bound relative to their max-abs scale is undefined.  On the GPU, dP
    (a matrix product) and D = rowsum(dO * O) (O = V exactly, with one key) are
    the same fp32 sum of d exact bf16 products in two orders; each is within
    d 2^-24 sum_e |dO_e V_e| of the exact value, so |dS| <= 2 d 2^-24
    max_i sum_e |dO_ie V_e|, and the gradient is at most scale |dS| max|x|
    (times 1 + 2^-8 for its bf16 rounding)."""
    x, v, do = (np.abs(np.asarray(t, dtype=np.float64)) for t in (x, v, do))
    d = do.shape[-1]
    ds = 2.0 * d * 2.0 ** -24 * float(np.max(np.sum(do * v, axis=-1)))
    return (1 + 2.0 ** -8) * scale * ds * float(np.max(x))


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
