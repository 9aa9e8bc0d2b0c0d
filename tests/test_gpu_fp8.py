"""GPU parity of the fp8 forward (fa_fwd_fp8) against the exact oracle.

The gate is the definition: ``ref_fwd`` of the oracle on the dequantised
inputs.  Its tolerances come from the kernel's one rounding step (P rounded
to e4m3 before the second product; the derivation is in tests/fp8_model.py):
* RMS error over O within sigma_p, the rounding model's expected RMS,
  combined with the bf16 rounding of the output.  sigma_p is an expectation
  over independent rounding events (one per visible query-key pair); with n
  of them the mean square of a sample fluctuates by a relative sqrt(2/n)
  (chi-square with n degrees of freedom), so the gate allows 4 such standard
  deviations: about 1% at the smallest whole-tile case (N = 64, n = 2080),
  and a factor 2.6 on a single key (N = 1, one event), where the worst-case
  element-wise bound below is the sharper check;
* every element within the worst case max|V| (2^-4 + N 2^-17), plus the
  output rounding (relative error 2^-4 of each weight, plus subnormal codes);
* LSE: the kernel's row sum uses the unrounded probabilities, so the LSE
  matches the exact one to fp32 accumulation error, 5e-4 relative.
The distance to the kernel's own rounding recipe (``fp8_model.ref_fwd_fp8``)
is printed as a diagnostic and is not a pass/fail criterion.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import fa_workloads as W
from fp8_model import fp8_p_rounding_sigma, ref_fwd_fp8
from oracle import fp8_dequantize, ref_fwd

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _fa():
    import exact_io_aware_11_amd as fa
    return fa


def say(msg):
    print(msg, flush=True)


def _codes(t):
    return t.view(torch.uint8).cpu().numpy()


def _check(o, lse, args, causal, scale, out_bf16, heads=None):
    """Compare kernel outputs (numpy, float64) with the exact result; report the
    distance to the kernel's rounding recipe."""
    q8, k8, vt8, qs, ks, vs = args
    if heads is not None:                     # sampled (b, h) pairs with their K/V heads
        H, Hkv = q8.shape[1], k8.shape[1]
        G = H // Hkv
        for b, h in heads:
            sub = (q8[b:b + 1, h:h + 1], k8[b:b + 1, h // G:h // G + 1], vt8[b:b + 1, h // G:h // G + 1], qs, ks, vs)
            _check(o[b:b + 1, h:h + 1], lse[b:b + 1, h:h + 1], sub, causal, scale, out_bf16)
        return
    c = (q8, k8, vt8, qs, ks, vs)
    q, k, v = fp8_dequantize(*c)
    exact, lse_exact = ref_fwd(q, k, v, causal, scale)
    method, _ = ref_fwd_fp8(*c, causal, scale)
    sigma_p = fp8_p_rounding_sigma(*c, causal, scale)
    rms_o = math.sqrt(np.mean(exact ** 2))
    sigma_out = (2.0 ** -8) / math.sqrt(12.0) * rms_o if out_bf16 else 1e-7 * rms_o
    rms_exact = math.sqrt(np.mean((o - exact) ** 2))
    rms_method = math.sqrt(np.mean((o - method) ** 2))
    say(f"  rms vs exact {rms_exact / sigma_p:.3f} sigma_p, vs the method {rms_method / sigma_p:.4f} sigma_p "
        f"(sigma_p {sigma_p:.2e}, bf16 output {sigma_out:.1e})")
    n = k.shape[2]
    nq = q.shape[2]
    events = q.shape[0] * q.shape[1] * (nq * (nq + 1) // 2 if causal else nq * n)
    allow = 1.0 + 4.0 * math.sqrt(2.0 / events)
    assert rms_exact <= math.sqrt(allow * sigma_p ** 2 + sigma_out ** 2), (rms_exact, sigma_p, sigma_out, events)
    bound = np.max(np.abs(v)) * (2.0 ** -4 + n * 2.0 ** -17) + (2.0 ** -8 if out_bf16 else 1e-6) * np.abs(exact) + 1e-6
    assert np.all(np.abs(o - exact) <= bound)
    assert np.max(np.abs(lse - lse_exact) / np.maximum(1.0, np.abs(lse_exact))) <= 5e-4


CASES = [
    # (B, H, Hkv, N, d, causal, out)
    (1, 1, 1, 64, 64, False, "bf16"),
    (1, 2, 1, 192, 128, True, "bf16"),
    (2, 4, 2, 256, 64, True, "fp32"),
    (1, 8, 8, 320, 128, False, "bf16"),
    (1, 4, 1, 512, 128, True, "fp32"),
    (3, 2, 2, 128, 128, True, "bf16"),
    # ragged N: tails masked; N % 4 != 0 takes the byte-gathered V^T path
    (1, 1, 1, 1, 64, True, "bf16"),
    (1, 1, 1, 1, 128, False, "fp32"),
    (1, 2, 1, 65, 128, True, "bf16"),
    (2, 4, 2, 100, 64, False, "fp32"),
    (1, 2, 2, 130, 128, True, "bf16"),
    (1, 4, 1, 333, 128, False, "bf16"),
    (1, 2, 1, 1001, 64, True, "fp32"),
    (1, 3, 3, 700, 128, True, "bf16"),
]


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,out", CASES)
def test_fwd_fp8(B, H, Hkv, N, d, causal, out):
    fa = _fa()
    q8, k8, vt8, qs, ks, vs = W.make_fp8(B, H, Hkv, N, d, seed=5000 + N + H, device=DEV)
    scale = 1.0 / math.sqrt(d)
    out_dt = torch.bfloat16 if out == "bf16" else torch.float32
    say(f"fa_fwd_fp8 B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal} out={out}")
    o, lse = fa.attention_fp8(q8, k8, vt8, qs, ks, vs, is_causal=causal, scale=scale, out_dtype=out_dt)
    torch.cuda.synchronize()
    _check(o.double().cpu().numpy(), lse.double().cpu().numpy(),
           (_codes(q8), _codes(k8), _codes(vt8), qs, ks, vs), causal, scale, out == "bf16")


def test_fwd_fp8_peaked_scores_and_scales():
    # scale x4 makes the softmax peaked (few keys carry the weight) and the
    # dequantisation factors are set far from 1
    fa = _fa()
    B, H, Hkv, N, d = 1, 2, 1, 384, 128
    q8, k8, vt8, _, _, _ = W.make_fp8(B, H, Hkv, N, d, seed=5101, device=DEV)
    qs, ks, vs = 3.0e-3, 0.17, 41.0
    # scores with a standard deviation of 4: a few keys carry most of each row
    raw_std = float(q8.float().std()) * float(k8.float().std()) * math.sqrt(d)
    scale = 4.0 / (qs * ks * raw_std)
    say("fa_fwd_fp8 peaked scores, non-unit scales")
    o, lse = fa.attention_fp8(q8, k8, vt8, qs, ks, vs, is_causal=True, scale=scale)
    torch.cuda.synchronize()
    _check(o.double().cpu().numpy(), lse.double().cpu().numpy(),
           (_codes(q8), _codes(k8), _codes(vt8), qs, ks, vs), True, scale, True)


def test_fwd_fp8_b4h16n2048d128_sampled_heads():
    fa = _fa()
    B, H, Hkv, N, d = 4, 16, 16, 2048, 128
    q8, k8, vt8, qs, ks, vs = W.make_fp8(B, H, Hkv, N, d, seed=5200, device=DEV)
    scale = 1.0 / math.sqrt(d)
    say("fa_fwd_fp8 B4 H16 N2048 d128 causal")
    o, lse = fa.attention_fp8(q8, k8, vt8, qs, ks, vs, is_causal=True, scale=scale)
    torch.cuda.synchronize()
    _check(o.double().cpu().numpy(), lse.double().cpu().numpy(),
           (_codes(q8), _codes(k8), _codes(vt8), qs, ks, vs), True, scale, True,
           heads=[(0, 0), (1, 7), (3, 15)])


def test_fwd_fp8_deterministic():
    fa = _fa()
    q8, k8, vt8, qs, ks, vs = W.make_fp8(2, 4, 2, 512, 128, seed=5300, device=DEV)
    say("fa_fwd_fp8 determinism")
    a = fa.attention_fp8(q8, k8, vt8, qs, ks, vs, is_causal=True)
    b = fa.attention_fp8(q8, k8, vt8, qs, ks, vs, is_causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
