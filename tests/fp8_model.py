"""Error model of the fp8 forward's own rounding -- a tolerance derivation
for the GPU tests, not part of the oracle.

The oracle (``oracle/``) fixes only what the fp8 forward must compute: the
exact attention of the dequantised inputs.  The pages give no rounding rule
for FP8 ("Flash Attention uitgelegd", FA3 section), so the kernel makes its own
choice, and the two functions here describe that choice in float64 so that
the tests can say how far from the exact result the kernel may land:

* ``ref_fwd_fp8`` takes the online-softmax steps over key tiles of ``bc`` keys
  ("FlashAttention (EL)", tiling and online-softmax sections) with the
  kernel's two choices: the reference max is the running max rounded up to an
  integer in base-2 units, so every probability is at most 1 and every rescale
  a power of two; and the probabilities enter P V as e4m3 after multiplication
  by 2^8 (nearest even).  The row sum and the LSE use the unrounded values.
  The GPU tests report the kernel's distance to it as a diagnostic only.
* ``fp8_p_rounding_sigma`` bounds the RMS deviation from the exact result that
  this rounding introduces: with relative rounding errors of at most half an
  e4m3 spacing (spacing/value <= 2^-3 for normal numbers), each uniform, the
  variance of output element (i, e) is at most
      sum_j [ (2^-3)^2 / 12 * w_ij^2 + 4 * (2^-17)^2 / 12 / l_i^2 ] * v_je^2,
  w_ij = softmax weight, l_i = sum_j 2^(s_ij - max_j s_ij) (log2 units); the
  second term covers subnormal codes (spacing 2^-9 after the 2^8 scaling, and
  a reference max at most one unit above the row max).  The GPU tests gate
  the kernel's RMS error against the exact result on this sigma.
"""

from __future__ import annotations

import math

import numpy as np

import oracle.fp8 as F8
from oracle import causal_visible, fp8_dequantize, kv_head

__all__ = ["ref_fwd_fp8", "fp8_p_rounding_sigma"]


def ref_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, causal: bool, scale: float,
                bc: int = 64, round_p: bool = True):
    """The fp8 forward's steps in float64 (the choices in the module docstring).

    q8 [B,H,N,d], k8 [B,Hkv,N,d] and vt8 [B,Hkv,d,N] are e4m3 codes (uint8).
    Per row, over key tiles of ``bc`` keys, in log2 units (s = scale q.k / ln 2):

        m_new = max(m, ceil(rowmax(s_tile)))     # integer reference
        alpha = 2^(m - m_new)
        e     = 2^(s_tile - m_new + 8)           # 2^8 p, at most 2^8
        l     = alpha l + rowsum(e)
        acc   = alpha acc + e4m3(e) V_tile       # e unrounded if round_p is False

    At the end O = acc / l and LSE = ln 2 (m - 8) + ln l.  Returns float64 O
    [B,H,N,d] and LSE [B,H,N]; a row with nothing visible gives O = 0, LSE = -inf.
    """
    q, k, v = fp8_dequantize(q8, k8, vt8, q_scale, k_scale, v_scale)
    B, H, N, d = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    o = np.zeros((B, H, N, d))
    lse = np.full((B, H, N), -np.inf)
    vis = causal_visible(np.arange(N), nk) if causal else None
    rnd = F8.e4m3_round if round_p else (lambda t: t)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            s = (scale / math.log(2.0)) * (q[b, h] @ k[b, g].T)
            if vis is not None:
                s = np.where(vis, s, -np.inf)
            m = np.full(N, -np.inf)
            l = np.zeros(N)
            acc = np.zeros((N, d))
            for c0 in range(0, nk, bc):
                blk = s[:, c0:c0 + bc]
                m_new = np.maximum(m, np.ceil(np.max(blk, axis=1)))
                ref = np.where(np.isfinite(m_new), m_new, 0.0)
                alpha = np.where(np.isfinite(m), np.exp2(m - ref), 0.0)
                e = np.exp2(blk - ref[:, None] + 8.0)
                l = alpha * l + np.sum(e, axis=1)
                acc = alpha[:, None] * acc + rnd(e) @ v[b, g, c0:c0 + bc]
                m = m_new
            live = l > 0
            o[b, h] = np.where(live[:, None], acc / np.where(live, l, 1.0)[:, None], 0.0)
            lse[b, h] = np.where(live, math.log(2.0) * (m - 8.0) + np.log(np.where(live, l, 1.0)), -np.inf)
    return o, lse


def fp8_p_rounding_sigma(q8, k8, vt8, q_scale, k_scale, v_scale, causal: bool, scale: float) -> float:
    """Upper model of the RMS (over all elements of O) of the deviation that
    rounding 2^8 p to e4m3 causes (formula in the module docstring)."""
    q, k, v = fp8_dequantize(q8, k8, vt8, q_scale, k_scale, v_scale)
    B, H, N, d = q.shape
    Hkv, nk = k.shape[1], k.shape[2]
    vis = causal_visible(np.arange(N), nk) if causal else None
    rel = (2.0 ** -3) ** 2 / 12.0
    sub = 4.0 * (2.0 ** -17) ** 2 / 12.0
    total = 0.0
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            s = (scale / math.log(2.0)) * (q[b, h] @ k[b, g].T)
            if vis is not None:
                s = np.where(vis, s, -np.inf)
            mx = np.max(s, axis=1, keepdims=True)
            p = np.exp2(s - mx)                   # <= 1, exactly 1 at the max
            l = np.sum(p, axis=1, keepdims=True)
            w = p / l
            v2 = v[b, g] ** 2
            seen = np.ones_like(w) if vis is None else vis.astype(np.float64)
            var = rel * ((w ** 2) @ v2) + (sub / l ** 2) * (seen @ v2)
            total += float(np.sum(var))
    return math.sqrt(total / (B * H * N * d))
