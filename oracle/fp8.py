"""fp64 CPU oracle for the fp8 (e4m3) forward -- test infrastructure only.

Only the test suite may import it.  It shares nothing with the HIP path.

The pages name an FP8 variant of the method ("Flash Attention uitgelegd", FA3
section: FP8 support, lower precision for more throughput) but give no
number format, scaling or rounding convention.  The reading used here:

* Inputs are OCP FP8 E4M3 codes (1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits; exponent field 0 holds subnormals of spacing 2^-9; the code
  S.1111.111 is NaN; no infinities; largest finite 448), each tensor with a
  dequantisation factor: the real inputs are Q = q_scale * q, K = k_scale * k,
  V = v_scale * v.  ``e4m3_decode`` and ``fp8_dequantize`` are that
  definition; ``e4m3_round`` is the format's round-to-nearest-even.
* What the method should produce is still the exact result for those real
  inputs: ``ref_fwd`` of the attention oracle on the decoded values.  The
  oracle holds nothing else for fp8: how a kernel rounds its intermediate
  probabilities is that kernel's choice, and the tolerance that choice needs
  is derived next to the tests, not here.
"""

from __future__ import annotations

import numpy as np

from .attention import _f64

__all__ = ["E4M3_MAX", "e4m3_decode", "e4m3_round", "fp8_dequantize"]

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """OCP FP8 E4M3 codes (uint8) -> float64 values, from the format definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def e4m3_round(x) -> np.ndarray:
    """Nearest E4M3 value of each element (ties to even), as float64.

    Normal numbers in [2^e, 2^(e+1)), e >= -6, have spacing 2^(e-3); below 2^-6
    the spacing is 2^-9 (subnormals).  Magnitudes above 448 are rejected.
    """
    x = _f64(x)
    a = np.abs(x)
    if np.any(a > E4M3_MAX):
        raise ValueError("value beyond the largest finite e4m3 (448)")
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    spacing = np.exp2(np.maximum(e, -6.0) - 3.0)
    return np.sign(x) * (np.round(a / spacing) * spacing)    # np.round: half to even


def fp8_dequantize(q8, k8, vt8, q_scale, k_scale, v_scale):
    """Real-valued Q [B,H,N,d], K and V [B,Hkv,N,d] (V from its transpose) in float64."""
    q = e4m3_decode(q8) * float(q_scale)
    k = e4m3_decode(k8) * float(k_scale)
    v = np.swapaxes(e4m3_decode(vt8), -1, -2) * float(v_scale)
    return q, k, np.ascontiguousarray(v)
