"""Pins of the fp8 oracle (oracle/fp8.py) and of the test-side rounding
model (tests/fp8_model.py) against things other than themselves.

* The e4m3 decoding and rounding against PyTorch's own float8_e4m3fn type
  (an independent implementation of the same OCP format).
* The model's online steps with the rounding of P switched off against the
  exact attention definition (ref_fwd).
* The rounding-noise model against the deviation the rounding actually
  causes, and its power to reject plausible mistakes (mutants planted in the
  model on the CPU).
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import fa_workloads as W
import fp8_model as M
import oracle.fp8 as F8
from fp8_model import fp8_p_rounding_sigma, ref_fwd_fp8
from oracle import e4m3_decode, e4m3_round, fp8_dequantize, ref_fwd


def _codes(t):
    return t.view(torch.uint8).cpu().numpy()


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert np.nanmax(got) == 448.0 and np.sum(np.isnan(got)) == 2


def test_e4m3_round_matches_torch_cast():
    g = torch.Generator().manual_seed(11)
    mags = torch.exp2(torch.rand(20000, generator=g) * 22 - 13)          # 2^-13 .. 2^9
    x = (mags * torch.where(torch.rand(20000, generator=g) < 0.5, -1.0, 1.0)).clamp(-448, 448)
    want = x.to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_round(x.numpy())
    assert np.array_equal(got, want)


def test_e4m3_round_grid_and_midpoints():
    vals = np.unique(np.abs(e4m3_decode(np.arange(0, 127, dtype=np.uint8))))   # finite non-negative
    assert np.array_equal(e4m3_round(vals), vals)
    mids = (vals[:-1] + vals[1:]) / 2
    r = e4m3_round(mids)
    want = torch.tensor(mids, dtype=torch.float64).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(r, want)            # ties to the even code
    with pytest.raises(ValueError):
        e4m3_round(np.array([449.0]))


@pytest.mark.parametrize("B,H,Hkv,N,d,causal,bc", [
    (1, 2, 1, 200, 64, True, 64),
    (2, 2, 2, 130, 32, False, 64),
    (1, 4, 2, 96, 64, True, 32),
])
def test_fp8_steps_without_rounding_equal_the_definition(B, H, Hkv, N, d, causal, bc):
    q8, k8, vt8, qs, ks, vs = W.make_fp8(B, H, Hkv, N, d, seed=300 + N)
    scale = 1.0 / math.sqrt(d)
    o, lse = ref_fwd_fp8(_codes(q8), _codes(k8), _codes(vt8), qs, ks, vs, causal, scale, bc=bc, round_p=False)
    q, k, v = fp8_dequantize(_codes(q8), _codes(k8), _codes(vt8), qs, ks, vs)
    o_ref, lse_ref = ref_fwd(q, k, v, causal, scale)
    assert np.max(np.abs(o - o_ref)) <= 1e-12 * max(1.0, np.max(np.abs(v)))
    assert np.max(np.abs(lse - lse_ref)) <= 1e-12 * max(1.0, np.max(np.abs(lse_ref)))


def _fp8_case(seed, N=256, d=64, H=2, Hkv=1, causal=True, sigma=1.0, scale_mul=1.0):
    q8, k8, vt8, qs, ks, vs = W.make_fp8(1, H, Hkv, N, d, seed=seed, sigma=sigma)
    args = (_codes(q8), _codes(k8), _codes(vt8), qs, ks, vs)
    scale = scale_mul / math.sqrt(d)
    exact, lse_exact = ref_fwd(*fp8_dequantize(*args), causal, scale)
    sigma_p = fp8_p_rounding_sigma(*args, causal, scale)
    return args, scale, exact, lse_exact, sigma_p


@pytest.mark.parametrize("seed,scale_mul", [(401, 1.0), (402, 4.0), (403, 0.25)])
def test_fp8_rounding_noise_is_within_the_model(seed, scale_mul):
    # peaked (scale x4), ordinary and flat (x1/4) attention
    args, scale, exact, lse_exact, sigma_p = _fp8_case(seed, scale_mul=scale_mul)
    o, lse = ref_fwd_fp8(*args, True, scale)
    rms = math.sqrt(np.mean((o - exact) ** 2))
    # the model assumes the largest relative spacing; the real rounding error
    # averages over the spacings of a binade, about 0.74 of the model
    assert 0.4 * sigma_p <= rms <= 1.0 * sigma_p, (rms, sigma_p)
    # the LSE uses the unrounded sum: exact up to float64
    assert np.max(np.abs(lse - lse_exact)) <= 1e-12 * np.max(np.abs(lse_exact))


def test_fp8_noise_criterion_rejects_mutants(monkeypatch):
    args, scale, exact, _, sigma_p = _fp8_case(404, N=512)

    def rms_of(o):
        return math.sqrt(np.mean((o - exact) ** 2))

    # 1. one key tile dropped from the product (its keys still in the sum)
    real_round = F8.e4m3_round
    calls = {"n": 0}

    def drop_third_tile(t):
        calls["n"] += 1
        r = real_round(t)
        return np.zeros_like(r) if calls["n"] % 8 == 3 else r
    monkeypatch.setattr(F8, "e4m3_round", drop_third_tile)
    o_bad, _ = M.ref_fwd_fp8(*args, True, scale)
    assert rms_of(o_bad) > 3.0 * sigma_p

    # 2. P rounded with two mantissa bits instead of three
    def coarse(t):
        a = np.abs(t)
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        sp = np.exp2(np.maximum(e, -6.0) - 2.0)
        return np.sign(t) * np.round(a / sp) * sp
    monkeypatch.setattr(F8, "e4m3_round", coarse)
    o_bad, _ = M.ref_fwd_fp8(*args, True, scale)
    assert rms_of(o_bad) > 1.0 * sigma_p
