"""Seeded random shapes through forward, backward and decode, each checked
against the fp64 oracle at the bf16 tolerances of the parity suite.

The shapes are drawn once from a fixed seed (so a failure names a
reproducible case): batch 1-3, 1-8 query heads with a random divisor as the
number of K/V heads, sequence lengths 1-700 (mostly off the tile grid),
head dim 64 or 128, causal or not; decode with cache lengths 1-2000 and an
automatic or random split count; paged decode with random page sizes and
ragged lengths; the fp8 forward at random lengths (any residue mod 4 and 64).
"""

from __future__ import annotations

import math
import random

import pytest
import torch

import fa_workloads as W
from oracle import ref_bwd, ref_decode, ref_decode_paged, ref_fwd
from parity_util import assert_bf16_close, assert_grad_close, assert_lse_close, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _fa():
    import exact_io_aware_11_amd as fa
    return fa


def say(msg):
    print(msg, flush=True)


def _draw_attention_cases(n, seed=8800):
    rng = random.Random(seed)
    cases = []
    for _ in range(n):
        H = rng.randint(1, 8)
        Hkv = rng.choice([h for h in range(1, H + 1) if H % h == 0])
        cases.append((rng.randint(1, 3), H, Hkv, rng.randint(1, 700), rng.choice([64, 128]), rng.random() < 0.6))
    return cases


def _draw_decode_cases(n, seed=8900):
    rng = random.Random(seed)
    cases = []
    for _ in range(n):
        H = rng.randint(1, 32)
        Hkv = rng.choice([h for h in range(1, H + 1) if H % h == 0])
        L = rng.randint(1, 2000)
        cases.append((rng.randint(1, 6), H, Hkv, L, rng.choice([64, 128]), rng.choice([0, 0, 1, rng.randint(1, 40)])))
    return cases


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", _draw_attention_cases(16))
def test_random_shape_forward_backward(B, H, Hkv, N, d, causal):
    fa = _fa()
    q, k, v, do = W.make_gqa(B, H, Hkv, N, d, "bf16", seed=9000 + 7 * N + H + d, with_dout=True, device=DEV)
    scale = 1.0 / math.sqrt(d)
    say(f"sweep fwd+bwd B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    o, lse = fa.attention(q, k, v, is_causal=causal, scale=scale)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, is_causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_fwd(to64(q), to64(k), to64(v), causal, scale)
    assert_bf16_close(to64(o), o_ref, "O")
    assert_lse_close(to64(lse), lse_ref, "LSE")
    rq, rk, rv = ref_bwd(to64(q), to64(k), to64(v), to64(do), causal, scale)
    assert_grad_close(to64(dq), rq, "dQ")
    assert_grad_close(to64(dk), rk, "dK")
    assert_grad_close(to64(dv), rv, "dV")


@pytest.mark.parametrize("B,H,Hkv,L,d,splits", _draw_decode_cases(10))
def test_random_shape_decode(B, H, Hkv, L, d, splits):
    fa = _fa()
    q, kc, vc = W.make_gqa(B, H, Hkv, 1, d, "bf16", seed=9500 + L + H, device=DEV, Nk=L)
    scale = 1.0 / math.sqrt(d)
    splits = min(splits, L)
    say(f"sweep decode B{B} H{H} Hkv{Hkv} L{L} d{d} splits={splits}")
    o, lse = fa.decode(q, kc, vc, scale=scale, num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_decode(to64(q), to64(kc), to64(vc), scale)
    assert_bf16_close(to64(o), o_ref, "O")
    assert_lse_close(to64(lse), lse_ref, "LSE")


def _draw_small_group_cases(n, seed=9600):
    # groups of 2 or 4 with enough (batch, cache head) pairs for the
    # small-group decode kernel (B * Hkv >= 64 for groups of 4)
    rng = random.Random(seed)
    cases = []
    for _ in range(n):
        G = rng.choice([2, 4])
        Hkv = rng.choice([4, 8, 16])
        B = max(rng.randint(1, 8), -(-64 // Hkv)) if G == 4 else rng.randint(1, 8)
        cases.append((B, G * Hkv, Hkv, rng.randint(1, 1500), rng.choice([64, 128, 256]),
                      rng.choice([0, 0, 1, rng.randint(1, 40)])))
    return cases


@pytest.mark.parametrize("B,H,Hkv,L,d,splits", _draw_small_group_cases(8))
def test_random_shape_small_group_decode(B, H, Hkv, L, d, splits):
    test_random_shape_decode(B, H, Hkv, L, d, splits)


def _draw_paged_cases(n, seed=9100):
    rng = random.Random(seed)
    cases = []
    for _ in range(n):
        H = rng.randint(1, 16)
        Hkv = rng.choice([h for h in range(1, H + 1) if H % h == 0])
        B = rng.randint(1, 4)
        lens = [rng.choice([0, rng.randint(1, 40), rng.randint(1, 1500)]) for _ in range(B)]
        cases.append((B, H, Hkv, rng.choice([32, 64, 128, 256]), tuple(lens), rng.choice([64, 128]),
                      rng.choice([0, 0, 1, rng.randint(1, 20)])))
    return cases


@pytest.mark.parametrize("B,H,Hkv,ps,lens,d,splits", _draw_paged_cases(8))
def test_random_shape_paged_decode(B, H, Hkv, ps, lens, d, splits):
    fa = _fa()
    g = torch.Generator().manual_seed(9200 + ps + sum(lens))
    n_pg = [-(-n // ps) for n in lens]
    pool = sum(n_pg) + 3
    max_pages = max(max(n_pg), 1)
    slots = torch.randperm(pool, generator=g).tolist()
    q = torch.randn((B, H, 1, d), generator=g).to(torch.bfloat16)
    kp = torch.randn((pool, Hkv, ps, d), generator=g).to(torch.bfloat16)
    vp = torch.randn((pool, Hkv, ps, d), generator=g).to(torch.bfloat16)
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    i = 0
    for b in range(B):
        for j in range(n_pg[b]):
            table[b, j] = slots[i]
            i += 1
    sl = torch.tensor(lens, dtype=torch.int32)
    scale = 1.0 / math.sqrt(d)
    say(f"sweep paged decode B{B} H{H} Hkv{Hkv} page{ps} lens{lens} d{d} splits={splits}")
    o_ref, lse_ref = ref_decode_paged(to64(q), to64(kp), to64(vp), table.numpy(), sl.numpy(), scale)
    o, lse = fa.decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), sl.to(DEV), scale=scale,
                             num_splits=min(splits, max_pages * ps))
    torch.cuda.synchronize()
    assert_bf16_close(to64(o), o_ref, "O")
    assert_lse_close(to64(lse), lse_ref, "LSE")


def _draw_fp8_cases(n, seed=9300):
    rng = random.Random(seed)
    cases = []
    for _ in range(n):
        H = rng.randint(1, 6)
        Hkv = rng.choice([h for h in range(1, H + 1) if H % h == 0])
        cases.append((rng.randint(1, 2), H, Hkv, rng.randint(1, 520), rng.choice([64, 128]), rng.random() < 0.6))
    return cases


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", _draw_fp8_cases(8))
def test_random_shape_fp8_forward(B, H, Hkv, N, d, causal):
    from test_gpu_fp8 import _check, _codes
    fa = _fa()
    q8, k8, vt8, qs, ks, vs = W.make_fp8(B, H, Hkv, N, d, seed=9400 + N + H, device=DEV)
    scale = 1.0 / math.sqrt(d)
    say(f"sweep fp8 fwd B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    o, lse = fa.attention_fp8(q8, k8, vt8, qs, ks, vs, is_causal=causal, scale=scale)
    torch.cuda.synchronize()
    _check(o.double().cpu().numpy(), lse.double().cpu().numpy(),
           (_codes(q8), _codes(k8), _codes(vt8), qs, ks, vs), causal, scale, True)
