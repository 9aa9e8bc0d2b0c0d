"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case draws seeded inputs, runs the library on the GPU, widens exactly
the values the GPU received to fp64 and compares element by element with the
oracle under the tolerances of ``parity_util``.  Full-size workloads that the
oracle cannot finish in seconds are checked on sampled rows / heads / batches
that the oracle computes one by one, at the same launch configuration the
benchmark times.
"""

from __future__ import annotations

import math
import sys

import numpy as np
import pytest
import torch

import fa_workloads as W
from oracle import ref_bwd, ref_decode, ref_decode_paged, ref_fwd, ref_fwd_rows
from parity_util import (assert_bf16_close, assert_fp32_close, assert_grad_close, assert_lse_close,
                         one_key_grad_bound, score_error_bound, to64)

pytestmark = pytest.mark.gpu


def _fa():
    import exact_io_aware_11_amd as fa
    return fa


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


DEV = "cuda:0"


# ----------------------------------------------------------------------------
# forward: the five workloads' forward parts
# ----------------------------------------------------------------------------

def test_fwd_fp32_b1h1n128d64():
    fa = _fa()
    w = W.WORKLOADS["fwd_fp32_b1h1n128d64"]
    q, k, v = W.make_inputs(w, DEV)
    say(f"fa_fwd fp32 {tuple(q.shape)} causal={w.causal}")
    o, lse = fa.attention(q, k, v, is_causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_fwd(to64(q), to64(k), to64(v), w.causal, w.scale)
    assert_fp32_close(to64(o), o_ref, "O")
    assert_fp32_close(to64(lse), lse_ref, "LSE")


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32], ids=["o_bf16", "o_fp32"])
def test_fwd_causal_bf16_b4h16n2048d128(out_dtype):
    fa = _fa()
    w = W.WORKLOADS["fwd_causal_bf16_b4h16n2048d128"]
    q, k, v = W.make_inputs(w, DEV)
    say(f"fa_fwd bf16 {tuple(q.shape)} causal out={out_dtype}")
    o, lse = fa.attention(q, k, v, is_causal=True, scale=w.scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_fwd(to64(q), to64(k), to64(v), True, w.scale)
    assert_bf16_close(to64(o), o_ref, "O")
    assert_lse_close(to64(lse), lse_ref, "LSE")


def test_fwd_causal_bf16_b1h32n16384d128_sampled_rows():
    fa = _fa()
    w = W.WORKLOADS["fwd_causal_bf16_b1h32n16384d128"]
    q, k, v = W.make_inputs(w, DEV)
    say(f"fa_fwd bf16 {tuple(q.shape)} causal (64 sampled rows per head + edge rows)")
    o, lse = fa.attention(q, k, v, is_causal=True, scale=w.scale)
    torch.cuda.synchronize()
    rows = W.sample_rows(w.N, w.extra["sample_rows"], w.extra["row_seed"])
    edge = [0, 1, 127, 128, w.N - 1]
    for name, rr in (("sampled", rows), ("edge", edge)):
        o_ref, lse_ref = ref_fwd_rows(to64(q), to64(k), to64(v), True, w.scale, rr)
        assert_bf16_close(to64(o[:, :, rr]), o_ref, f"O {name}")
        assert_lse_close(to64(lse[:, :, rr]), lse_ref, f"LSE {name}")


# ----------------------------------------------------------------------------
# forward: ragged and small shapes against the full oracle
# ----------------------------------------------------------------------------

SMALL = [
    # (B, H, N, d, dtype, causal)
    (1, 1, 1, 64, "bf16", False),
    (1, 1, 1, 128, "bf16", True),
    (1, 2, 17, 64, "bf16", True),
    (2, 1, 63, 128, "bf16", False),
    (1, 2, 127, 128, "bf16", True),
    (1, 1, 128, 128, "bf16", True),
    (2, 2, 129, 64, "bf16", True),
    (1, 3, 200, 128, "bf16", False),
    (1, 2, 1000, 128, "bf16", True),
    (1, 1, 1000, 64, "bf16", False),
    # d = 128 streams 32-key tiles: lengths at and just past tile edges
    (1, 2, 32, 128, "bf16", True),
    (1, 1, 33, 128, "bf16", True),
    (2, 1, 96, 128, "bf16", False),
    (1, 2, 161, 128, "bf16", True),
    (1, 1, 1, 64, "fp32", False),
    (1, 2, 33, 128, "fp32", True),
    (2, 1, 129, 64, "fp32", True),
    # fp32: the four waves of a 32-row workgroup take every fourth key tile,
    # so these give each wave two or three tiles (the prefetch path)
    (1, 2, 300, 64, "fp32", False),
    (1, 1, 257, 128, "fp32", False),
    (1, 1, 300, 128, "fp32", False),
    # head dim 256 (bf16 only)
    (1, 2, 300, 256, "bf16", True),
    (2, 1, 129, 256, "bf16", False),
    (1, 2, 1000, 256, "bf16", True),
    (1, 1, 1, 256, "bf16", True),
]


@pytest.mark.parametrize("B,H,N,d,dtype,causal", SMALL)
def test_fwd_small_shapes(B, H, N, d, dtype, causal):
    fa = _fa()
    q, k, v = W.make_custom(B, H, N, d, dtype, seed=1000 + N + d, device=DEV)
    scale = 1.0 / math.sqrt(d)
    say(f"fa_fwd {dtype} {(B, H, N, d)} causal={causal}")
    o, lse = fa.attention(q, k, v, is_causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_fwd(to64(q), to64(k), to64(v), causal, scale)
    check = assert_fp32_close if dtype == "fp32" else assert_bf16_close
    check(to64(o), o_ref, "O")
    (assert_fp32_close if dtype == "fp32" else assert_lse_close)(to64(lse), lse_ref, "LSE")


def test_fwd_closed_form_uniform_scores():
    # Q = 0: row i of a causal head is the mean of V_0..V_i and LSE_i = ln(i+1)
    fa = _fa()
    B, H, N, d = 1, 2, 300, 128
    _, k, v = W.make_custom(B, H, N, d, "bf16", seed=77, device=DEV)
    q = torch.zeros_like(k)
    say("fa_fwd closed form Q=0 causal")
    o, lse = fa.attention(q, k, v, is_causal=True, scale=0.125)
    torch.cuda.synchronize()
    vv = to64(v)
    counts = np.arange(1, N + 1, dtype=np.float64)
    expect = np.cumsum(vv, axis=2) / counts[None, None, :, None]
    assert_bf16_close(to64(o), expect, "O")
    assert_lse_close(to64(lse), np.broadcast_to(np.log(counts), (B, H, N)), "LSE")


def test_fwd_large_scores_stay_finite():
    # Q and K scaled x8 make scores of O(100): the running max must keep exp
    # finite.  V stays N(0, 1) so that O's own bf16 rounding stays below the
    # absolute tolerance.
    fa = _fa()
    q, k = W.make_custom(1, 2, 257, 128, "bf16", seed=78, sigma=8.0, n_tensors=2, device=DEV)
    (v,) = W.make_custom(1, 2, 257, 128, "bf16", seed=178, n_tensors=1, device=DEV)
    say("fa_fwd large logits")
    o, lse = fa.attention(q, k, v, is_causal=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
    o_ref, lse_ref = ref_fwd(to64(q), to64(k), to64(v), True, 1 / math.sqrt(128))
    # scores of magnitude ~100: the fp32 accumulation of each score adds its
    # own worst-case error to the LSE bound
    assert_bf16_close(to64(o), o_ref, "O")
    assert_lse_close(to64(lse), lse_ref, "LSE", extra=score_error_bound(to64(q), to64(k), 1 / math.sqrt(128)))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_rising_scores_rescale(causal, d):
    # K rows scaled by a ramp growing along the keys: every later key tile
    # raises the row maximum, so the output accumulated so far must be
    # rescaled again and again (and some tiles overflow the kept-sum bound
    # while each of their values alone would not).
    fa = _fa()
    B, H, N = 1, 2, 700
    q, k, v = W.make_custom(B, H, N, d, "bf16", seed=79, device=DEV)
    ramp = torch.linspace(1.0, 6.0, N, device=DEV).view(1, 1, N, 1)
    k = (k.float() * ramp).to(torch.bfloat16)
    say(f"fa_fwd rising scores causal={causal} d={d}")
    o, lse = fa.attention(q, k, v, is_causal=causal)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_fwd(to64(q), to64(k), to64(v), causal, 1 / math.sqrt(d))
    assert_bf16_close(to64(o), o_ref, "O")
    assert_lse_close(to64(lse), lse_ref, "LSE", extra=score_error_bound(to64(q), to64(k), 1 / math.sqrt(d)))


def test_fwd_deterministic_and_allocation_free():
    fa = _fa()
    q, k, v = W.make_custom(2, 4, 1000, 128, "bf16", seed=79, device=DEV)
    o1 = torch.empty_like(q)
    o2 = torch.empty_like(q)
    l1 = torch.empty((2, 4, 1000), dtype=torch.float32, device=DEV)
    l2 = torch.empty_like(l1)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    stream = torch.cuda.current_stream().cuda_stream
    say("fa_fwd determinism / no allocation")
    for o, l in ((o1, l1), (o2, l2)):
        st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), fa.FA_BF16, l.data_ptr(),
                       2, 4, 4, 1000, 128, fa.FA_BF16, 1, 1 / math.sqrt(128), stream)
        assert st == fa.FA_OK
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == before
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ----------------------------------------------------------------------------
# backward
# ----------------------------------------------------------------------------

BWD_SMALL = [
    # (B, H, N, d, causal, o_dtype)
    (1, 1, 1, 64, True, "bf16"),
    (1, 2, 17, 128, True, "bf16"),
    (1, 1, 64, 64, False, "bf16"),
    (2, 1, 127, 128, True, "fp32"),
    (1, 2, 128, 128, False, "bf16"),
    (1, 1, 129, 64, True, "bf16"),
    (1, 2, 300, 128, True, "bf16"),
    (1, 1, 515, 128, False, "fp32"),
    # non-causal with N a multiple of the key and query tiles: the dK/dV
    # kernel runs its unmasked loop for the whole launch
    (1, 2, 512, 128, False, "bf16"),
    (2, 1, 256, 64, False, "bf16"),
    # head dim 256: one 32-row query block per step, 32-key dQ tiles
    (1, 1, 1, 256, True, "bf16"),
    (1, 2, 33, 256, True, "bf16"),
    (1, 1, 129, 256, False, "fp32"),
    (2, 1, 300, 256, True, "bf16"),
    (1, 2, 256, 256, False, "bf16"),
    (1, 1, 515, 256, True, "fp32"),
]


def _bwd_case(B, H, N, d, causal, o_dtype, seed, sigma=1.0):
    fa = _fa()
    q, k, v, do = W.make_custom(B, H, N, d, "bf16", seed=seed, sigma=sigma, n_tensors=4, device=DEV)
    scale = 1.0 / math.sqrt(d)
    odt = torch.bfloat16 if o_dtype == "bf16" else torch.float32
    o, lse = fa.attention(q, k, v, is_causal=causal, scale=scale, out_dtype=odt)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, is_causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (q, k, v, do), (dq, dk, dv)


@pytest.mark.parametrize("B,H,N,d,causal,o_dtype", BWD_SMALL)
def test_bwd_small_shapes(B, H, N, d, causal, o_dtype):
    say(f"fa_bwd {(B, H, N, d)} causal={causal} o={o_dtype}")
    (q, k, v, do), (dq, dk, dv) = _bwd_case(B, H, N, d, causal, o_dtype, seed=2000 + N + d)
    rq, rk, rv = ref_bwd(to64(q), to64(k), to64(v), to64(do), causal, 1 / math.sqrt(d))
    if N == 1:
        # one key: the true dQ and dK are exactly zero; the GPU's are fp32
        # rounding of dP - D, bounded by the derivation in parity_util
        assert np.max(np.abs(rq)) == 0.0 and np.max(np.abs(rk)) == 0.0
        assert np.max(np.abs(to64(dq))) <= one_key_grad_bound(to64(k), to64(v), to64(do), 1 / math.sqrt(d))
        assert np.max(np.abs(to64(dk))) <= one_key_grad_bound(to64(q), to64(v), to64(do), 1 / math.sqrt(d))
    else:
        assert_grad_close(to64(dq), rq, "dQ")
        assert_grad_close(to64(dk), rk, "dK")
    assert_grad_close(to64(dv), rv, "dV")


def test_bwd_noncausal_ragged_with_very_negative_scores():
    # Scores around -181 (Q = -4 + N(0,1), K = 4 + N(0,1)), so LSE < -88.
    # The non-causal dK/dV kernel runs unmasked: a key past N (zero K and V)
    # gets P = exp(-LSE), which overflows to inf, but only in that key's own
    # dK/dV columns, which are never stored.  The live keys' gradients must
    # still match the oracle.  (The unit noise keeps dQ well conditioned: the
    # constant part of K cancels from dQ exactly, since each row of dS sums
    # to zero.)
    fa = _fa()
    B, H, N, d = 1, 2, 200, 128
    g = torch.Generator().manual_seed(2500)
    q = torch.full((B, H, N, d), -4.0) + torch.randn((B, H, N, d), generator=g)
    k = torch.full((B, H, N, d), 4.0) + torch.randn((B, H, N, d), generator=g)
    v = torch.randn((B, H, N, d), generator=g)
    do = torch.randn((B, H, N, d), generator=g)
    q, k, v, do = (t.to(torch.bfloat16).to(DEV) for t in (q, k, v, do))
    scale = 1.0 / math.sqrt(d)
    say("fa_bwd non-causal N200 with scores near -181")
    o, lse = fa.attention(q, k, v, is_causal=False, scale=scale)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, is_causal=False, scale=scale)
    torch.cuda.synchronize()
    assert float(lse.max()) < -88.0
    for t in (dq, dk, dv):
        assert torch.isfinite(t.float()).all()
    rq, rk, rv = ref_bwd(to64(q), to64(k), to64(v), to64(do), False, scale)
    assert_grad_close(to64(dq), rq, "dQ")
    assert_grad_close(to64(dk), rk, "dK")
    assert_grad_close(to64(dv), rv, "dV")


def test_bwd_causal_bf16_b2h16n4096d128_sampled_heads():
    fa = _fa()
    w = W.WORKLOADS["bwd_causal_bf16_b2h16n4096d128"]
    q, k, v, do = W.make_inputs(w, DEV)
    say(f"fa_fwd+fa_bwd bf16 {tuple(q.shape)} causal")
    o, lse = fa.attention(q, k, v, is_causal=True, scale=w.scale)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, is_causal=True, scale=w.scale)
    torch.cuda.synchronize()
    heads = [(0, 0), (0, 9), (1, 4), (1, 15)]
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = ref_bwd(to64(q[sl]), to64(k[sl]), to64(v[sl]), to64(do[sl]), True, w.scale)
        assert_grad_close(to64(dq[sl]), rq, f"dQ head {(b, h)}")
        assert_grad_close(to64(dk[sl]), rk, f"dK head {(b, h)}")
        assert_grad_close(to64(dv[sl]), rv, f"dV head {(b, h)}")
    # invariants over every head: sum_j dV_j = sum_i dO_i, sum_j dK_j = 0
    dv_sum = dv.float().sum(dim=2)
    do_sum = do.float().sum(dim=2)
    scale_v = dv.float().abs().amax().item()
    assert (dv_sum - do_sum).abs().max().item() <= 2e-2 * scale_v * math.sqrt(w.N)
    scale_k = dk.float().abs().amax().item()
    assert dk.float().sum(dim=2).abs().max().item() <= 2e-2 * scale_k * math.sqrt(w.N)


def test_bwd_deterministic():
    # no atomics anywhere in the backward: two runs agree bit for bit
    fa = _fa()
    q, k, v, do = W.make_custom(2, 3, 700, 128, "bf16", seed=2100, n_tensors=4, device=DEV)
    say("fa_bwd determinism")
    o, lse = fa.attention(q, k, v, is_causal=True)
    a = fa.attention_backward(q, k, v, o, lse, do, is_causal=True)
    b = fa.attention_backward(q, k, v, o, lse, do, is_causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


# ----------------------------------------------------------------------------
# decode
# ----------------------------------------------------------------------------

def test_decode_bf16_b64h32l8192d128_sampled_batches():
    fa = _fa()
    w = W.WORKLOADS["decode_bf16_b64h32l8192d128"]
    q, kc, vc = W.make_inputs(w, DEV)
    say(f"fa_decode bf16 q{tuple(q.shape)} cache{tuple(kc.shape)} splits=auto")
    o, lse = fa.decode(q, kc, vc, scale=w.scale)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(505)
    batches = torch.randperm(w.B, generator=g)[:6].tolist() + [0, w.B - 1]
    for b in sorted(set(batches)):
        o_ref, lse_ref = ref_decode(to64(q[b:b + 1]), to64(kc[b:b + 1]), to64(vc[b:b + 1]), w.scale)
        assert_bf16_close(to64(o[b:b + 1]), o_ref, f"O batch {b}")
        assert_lse_close(to64(lse[b:b + 1]), lse_ref, f"LSE batch {b}")


@pytest.mark.parametrize("L", [1, 7, 100, 1000, 4097])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_split_counts_agree(L, d):
    fa = _fa()
    B, H = 3, 5
    q, kc, vc = W.make_custom(B, H, 1, d, "bf16", seed=3000 + L + d, Nk=L, device=DEV)
    scale = 1 / math.sqrt(d)
    o_ref, lse_ref = ref_decode(to64(q), to64(kc), to64(vc), scale)
    outs = []
    for s in (0, 1, 2, 4, 8, 16):
        if s > L:
            continue
        say(f"fa_decode {(B, H, L, d)} splits={s}")
        o, lse = fa.decode(q, kc, vc, scale=scale, num_splits=s)
        torch.cuda.synchronize()
        assert_bf16_close(to64(o), o_ref, f"O splits={s}")
        assert_lse_close(to64(lse), lse_ref, f"LSE splits={s}")
        outs.append((to64(o), to64(lse)))
    o0, l0 = outs[0]
    for o, lse in outs[1:]:
        # split counts change only the fp32 summation order: LSEs agree to fp32
        # level, bf16 outputs at most one rounding step apart
        assert np.max(np.abs(lse - l0)) <= 1e-4
        assert np.all(np.abs(o - o0) <= np.maximum(np.abs(o), np.abs(o0)) * 2.0 ** -7 + 1e-6)


@pytest.mark.parametrize("B,H,Hkv,L,d", [
    (2, 4, 4, 300, 128),     # per-head kernel
    (2, 16, 8, 500, 64),     # small-group kernel, groups of 2
    (16, 32, 8, 700, 128),   # small-group kernel, groups of 4
    (2, 16, 2, 600, 128),    # MFMA grouped kernel (groups of 8), which keeps the merge
])
def test_decode_one_split_without_lse(B, H, Hkv, L, d):
    # With one split the per-head and small-group kernels write O and the LSE
    # themselves (no merge launch).  A null LSE pointer must leave O as it is
    # with an LSE, and both must meet the oracle.
    fa = _fa()
    q, kc, vc = W.make_gqa(B, H, Hkv, 1, d, "bf16", seed=3300 + L, Nk=L, device=DEV)
    scale = 1 / math.sqrt(d)
    say(f"fa_decode one split B{B} H{H} Hkv{Hkv} L{L} d{d}, with and without LSE")
    o_ref, lse_ref = fa.decode(q, kc, vc, scale=scale, num_splits=1)
    o = torch.full_like(o_ref, float("nan"))
    nb = fa.fa_decode_workspace_bytes(B, H, Hkv, L, d, 1)
    ws = torch.empty((nb,), dtype=torch.uint8, device=DEV)
    st = fa.fa_decode(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(), 0, ws.data_ptr(), nb,
                      B, H, Hkv, L, d, fa.FA_BF16, 1, scale, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    o64, l64 = ref_decode(to64(q), to64(kc), to64(vc), scale)
    assert_bf16_close(to64(o_ref), o64, "O")
    assert_lse_close(to64(lse_ref), l64, "LSE")


def test_decode_deterministic():
    fa = _fa()
    q, kc, vc = W.make_custom(4, 8, 1, 128, "bf16", seed=3100, Nk=3000, device=DEV)
    say("fa_decode determinism")
    a = fa.decode(q, kc, vc)
    b = fa.decode(q, kc, vc)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ----------------------------------------------------------------------------
# grouped-query / multi-query attention: K and V carry Hkv < H heads
# ----------------------------------------------------------------------------

GQA_FWD = [
    # (B, H, Hkv, N, d, dtype, causal)
    (1, 8, 2, 300, 128, "bf16", True),
    (2, 4, 1, 130, 64, "bf16", False),
    (1, 6, 3, 257, 128, "bf16", False),
    (1, 8, 1, 1000, 128, "bf16", True),
    (2, 16, 8, 129, 64, "bf16", True),
    (1, 4, 2, 200, 64, "fp32", True),
    (1, 6, 2, 97, 128, "fp32", False),
    (1, 8, 2, 257, 256, "bf16", True),
]


@pytest.mark.parametrize("B,H,Hkv,N,d,dtype,causal", GQA_FWD)
def test_fwd_gqa(B, H, Hkv, N, d, dtype, causal):
    fa = _fa()
    q, k, v = W.make_gqa(B, H, Hkv, N, d, dtype, seed=4000 + N + H + Hkv, device=DEV)
    scale = 1.0 / math.sqrt(d)
    say(f"fa_fwd gqa {dtype} B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    o, lse = fa.attention(q, k, v, is_causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_fwd(to64(q), to64(k), to64(v), causal, scale)
    check = assert_fp32_close if dtype == "fp32" else assert_bf16_close
    check(to64(o), o_ref, "O")
    (assert_fp32_close if dtype == "fp32" else assert_lse_close)(to64(lse), lse_ref, "LSE")


GQA_BWD = [
    # (B, H, Hkv, N, d, causal)
    (1, 8, 2, 256, 128, True),
    (2, 4, 1, 190, 64, False),
    (1, 6, 3, 129, 128, True),
    (1, 4, 1, 700, 128, True),
    (1, 8, 4, 65, 64, True),
    (1, 4, 2, 200, 128, False),
    (1, 4, 2, 200, 256, True),
    (2, 6, 1, 97, 256, False),
]


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", GQA_BWD)
def test_bwd_gqa(B, H, Hkv, N, d, causal):
    fa = _fa()
    q, k, v, do = W.make_gqa(B, H, Hkv, N, d, "bf16", seed=4100 + N + H + Hkv, with_dout=True, device=DEV)
    scale = 1.0 / math.sqrt(d)
    say(f"fa_bwd gqa B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    o, lse = fa.attention(q, k, v, is_causal=causal, scale=scale)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, is_causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert tuple(dk.shape) == tuple(k.shape) and tuple(dv.shape) == tuple(v.shape)
    rq, rk, rv = ref_bwd(to64(q), to64(k), to64(v), to64(do), causal, scale)
    assert_grad_close(to64(dq), rq, "dQ")
    assert_grad_close(to64(dk), rk, "dK")
    assert_grad_close(to64(dv), rv, "dV")


def test_bwd_gqa_large_grid_sums_in_registers():
    # 2 key tiles x 512 K/V heads = 1024 dK/dV workgroups: enough work for the
    # kernel to sum each group in registers (the workspace has no partials).
    # The small grouped shapes above split the query heads instead.
    fa = _fa()
    B, H, Hkv, N, d = 64, 16, 8, 256, 64
    G = H // Hkv
    assert fa.fa_bwd_workspace_bytes(B, H, Hkv, N, d) == 2 * B * H * N * 4
    q, k, v, do = W.make_gqa(B, H, Hkv, N, d, "bf16", seed=4300, with_dout=True, device=DEV)
    scale = 1.0 / math.sqrt(d)
    say(f"fa_bwd gqa large grid B{B} H{H} Hkv{Hkv} N{N} d{d} causal")
    o, lse = fa.attention(q, k, v, is_causal=True, scale=scale)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, is_causal=True, scale=scale)
    torch.cuda.synchronize()
    for b, hk in [(0, 0), (17, 5), (63, 7)]:
        qs = (slice(b, b + 1), slice(hk * G, hk * G + G))
        ks = (slice(b, b + 1), slice(hk, hk + 1))
        rq, rk, rv = ref_bwd(to64(q[qs]), to64(k[ks]), to64(v[ks]), to64(do[qs]), True, scale)
        assert_grad_close(to64(dq[qs]), rq, f"dQ {(b, hk)}")
        assert_grad_close(to64(dk[ks]), rk, f"dK {(b, hk)}")
        assert_grad_close(to64(dv[ks]), rv, f"dV {(b, hk)}")


def test_bwd_d256_grouped_without_split_sampled_heads():
    # 8 key tiles x 64 K/V heads = 512 dK/dV workgroups: the kernel sums each
    # group of 2 in registers; sampled (batch, K/V head) pairs against the oracle
    fa = _fa()
    B, H, Hkv, N, d = 16, 8, 4, 1000, 256
    G = H // Hkv
    assert fa.fa_bwd_workspace_bytes(B, H, Hkv, N, d) == 2 * ((B * H * N * 4 + 255) // 256 * 256)
    q, k, v, do = W.make_gqa(B, H, Hkv, N, d, "bf16", seed=4400, with_dout=True, device=DEV)
    scale = 1.0 / math.sqrt(d)
    say(f"fa_bwd d256 gqa B{B} H{H} Hkv{Hkv} N{N} causal")
    o, lse = fa.attention(q, k, v, is_causal=True, scale=scale)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, is_causal=True, scale=scale)
    torch.cuda.synchronize()
    for b, hk in [(0, 0), (9, 3), (15, 1)]:
        qs = (slice(b, b + 1), slice(hk * G, hk * G + G))
        ks = (slice(b, b + 1), slice(hk, hk + 1))
        rq, rk, rv = ref_bwd(to64(q[qs]), to64(k[ks]), to64(v[ks]), to64(do[qs]), True, scale)
        assert_grad_close(to64(dq[qs]), rq, f"dQ {(b, hk)}")
        assert_grad_close(to64(dk[ks]), rk, f"dK {(b, hk)}")
        assert_grad_close(to64(dv[ks]), rv, f"dV {(b, hk)}")


def test_bwd_d256_b2h8n4096_sampled_heads():
    # the head-dim-256 backward at a long sequence, causal, two heads checked
    fa = _fa()
    B, H, N, d = 2, 8, 4096, 256
    q, k, v, do = W.make_custom(B, H, N, d, "bf16", seed=4500, n_tensors=4, device=DEV)
    scale = 1.0 / math.sqrt(d)
    say(f"fa_bwd d256 B{B} H{H} N{N} causal")
    o, lse = fa.attention(q, k, v, is_causal=True, scale=scale)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, is_causal=True, scale=scale)
    torch.cuda.synchronize()
    for b, h in [(0, 3), (1, 7)]:
        sl = (slice(b, b + 1), slice(h, h + 1))
        rq, rk, rv = ref_bwd(to64(q[sl]), to64(k[sl]), to64(v[sl]), to64(do[sl]), True, scale)
        assert_grad_close(to64(dq[sl]), rq, f"dQ {(b, h)}")
        assert_grad_close(to64(dk[sl]), rk, f"dK {(b, h)}")
        assert_grad_close(to64(dv[sl]), rv, f"dV {(b, h)}")


def test_bwd_d256_deterministic():
    fa = _fa()
    q, k, v, do = W.make_gqa(1, 4, 2, 333, 256, "bf16", seed=4600, with_dout=True, device=DEV)
    say("fa_bwd d256 determinism")
    o, lse = fa.attention(q, k, v, is_causal=True)
    a = fa.attention_backward(q, k, v, o, lse, do, is_causal=True)
    b = fa.attention_backward(q, k, v, o, lse, do, is_causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", [
    (4, 16, 4, 2048, 128, True),     # 256 (K/V head, key tile) pairs: groups of 2 query heads
    (4, 32, 4, 2048, 128, True),     # G = 8: groups of 4
    (4, 16, 4, 2000, 64, False),     # groups of 2, ragged, no mask
    (4, 16, 4, 2048, 256, True),     # groups of 2 at d = 256
])
def test_bwd_gqa_head_groups_sampled(B, H, Hkv, N, d, causal):
    # Few (K/V head, key tile) pairs: the dK/dV kernel splits each K/V head's
    # query heads into groups and sums the groups' fp32 partials afterwards.
    # The workspace size shows the group size; sampled (batch, K/V head)
    # pairs are checked against the oracle.
    fa = _fa()
    G, pairs = H // Hkv, -(-N // 128) * B * Hkv
    s = next((t for t in range(G // 2, 1, -1) if G % t == 0 and pairs * (G // t) >= 512), 1)
    assert s > 1
    rows = 2 * ((B * H * N * 4 + 255) // 256 * 256)
    assert fa.fa_bwd_workspace_bytes(B, H, Hkv, N, d) == rows + 2 * (B * H // s) * N * d * 4
    q, k, v, do = W.make_gqa(B, H, Hkv, N, d, "bf16", seed=4500 + G + d, with_dout=True, device=DEV)
    scale = 1.0 / math.sqrt(d)
    say(f"fa_bwd gqa head groups of {s} B{B} H{H} Hkv{Hkv} N{N} d{d} causal={causal}")
    o, lse = fa.attention(q, k, v, is_causal=causal, scale=scale)
    dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, is_causal=causal, scale=scale)
    torch.cuda.synchronize()
    for b, hk in [(0, 0), (B - 1, Hkv - 1)]:
        qs = (slice(b, b + 1), slice(hk * G, hk * G + G))
        ks = (slice(b, b + 1), slice(hk, hk + 1))
        rq, rk, rv = ref_bwd(to64(q[qs]), to64(k[ks]), to64(v[ks]), to64(do[qs]), causal, scale)
        assert_grad_close(to64(dq[qs]), rq, f"dQ {(b, hk)}")
        assert_grad_close(to64(dk[ks]), rk, f"dK {(b, hk)}")
        assert_grad_close(to64(dv[ks]), rv, f"dV {(b, hk)}")
    # deterministic: the groups are summed in a fixed order
    again = fa.attention_backward(q, k, v, o, lse, do, is_causal=causal, scale=scale)
    torch.cuda.synchronize()
    for x, y in zip((dq, dk, dv), again):
        assert torch.equal(x, y)


def test_bwd_gqa_deterministic():
    fa = _fa()
    q, k, v, do = W.make_gqa(1, 8, 2, 600, 128, "bf16", seed=4200, with_dout=True, device=DEV)
    say("fa_bwd gqa determinism")
    o, lse = fa.attention(q, k, v, is_causal=True)
    a = fa.attention_backward(q, k, v, o, lse, do, is_causal=True)
    b = fa.attention_backward(q, k, v, o, lse, do, is_causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


GQA_DEC = [
    # (B, H, Hkv, L, d): groups of 2 and 3, and of 4 over at least 64 (batch, cache
    # head) pairs, take the small-group kernel; other groups up to 32 the MFMA
    # grouped kernel; G = 1 and G > 32 the per-head kernel
    (8, 32, 8, 700, 64),
    (4, 16, 8, 513, 256),
    (2, 4, 2, 65, 64),
    (16, 8, 4, 1029, 128),
    (8, 32, 8, 300, 256),
    (4, 24, 8, 1000, 128),
    (2, 3, 1, 517, 256),
    (3, 8, 2, 1000, 128),
    (2, 8, 1, 777, 64),
    (1, 32, 8, 4097, 128),
    (2, 6, 3, 1, 128),
    # caches shorter than one 32-key tile: the MFMA grouped kernel (groups of
    # 8; groups of 4 over fewer than 64 pairs) and the small-group kernel
    (1, 8, 1, 1, 128),
    (2, 16, 4, 31, 64),
    (16, 32, 8, 17, 128),
    (2, 4, 4, 300, 64),
    (1, 32, 1, 2049, 128),
    (1, 64, 1, 500, 64),
    (2, 12, 4, 33, 64),
    (2, 8, 2, 777, 256),
    (2, 4, 4, 300, 256),
]


@pytest.mark.parametrize("B,H,Hkv,L,d", GQA_DEC)
def test_decode_gqa(B, H, Hkv, L, d):
    fa = _fa()
    q, kc, vc = W.make_gqa(B, H, Hkv, 1, d, "bf16", seed=4300 + L + H + Hkv, device=DEV, Nk=L)
    scale = 1.0 / math.sqrt(d)
    o_ref, lse_ref = ref_decode(to64(q), to64(kc), to64(vc), scale)
    for s in (0, 1, 2, 4, 7):
        if s > L:
            continue
        say(f"fa_decode gqa B{B} H{H} Hkv{Hkv} L{L} d{d} splits={s}")
        o, lse = fa.decode(q, kc, vc, scale=scale, num_splits=s)
        torch.cuda.synchronize()
        assert_bf16_close(to64(o), o_ref, f"O splits={s}")
        assert_lse_close(to64(lse), lse_ref, f"LSE splits={s}")


@pytest.mark.parametrize("B,H,Hkv,L,d,rising", [(16, 8, 4, 3000, 128, True), (8, 32, 8, 1500, 64, True),
                                                  (16, 8, 4, 3000, 128, False)])
def test_decode_small_groups_with_drifting_scores(B, H, Hkv, L, d, rising):
    # keys carry a common offset that ramps over the cache and every query a
    # positive mean, so the scores drift by about +-3*sqrt(d) along the keys:
    # rising, the small-group kernel's reference maximum is raised many times
    # inside one chunk; falling, the early keys dominate
    fa = _fa()
    g = torch.Generator().manual_seed(4350 + L + H)
    q = (torch.randn((B, H, 1, d), generator=g) + 1.0).to(torch.bfloat16)
    ramp = torch.linspace(-3.0, 3.0, L) if rising else torch.linspace(3.0, -3.0, L)
    kc = (torch.randn((B, Hkv, L, d), generator=g) + ramp[:, None]).to(torch.bfloat16)
    vc = torch.randn((B, Hkv, L, d), generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(d)
    o_ref, lse_ref = ref_decode(to64(q), to64(kc), to64(vc), scale)
    for s in (0, 1, 3):
        say(f"fa_decode drifting scores B{B} H{H} Hkv{Hkv} L{L} d{d} rising={rising} splits={s}")
        o, lse = fa.decode(q.to(DEV), kc.to(DEV), vc.to(DEV), scale=scale, num_splits=s)
        torch.cuda.synchronize()
        assert_bf16_close(to64(o), o_ref, f"O splits={s}")
        assert_lse_close(to64(lse), lse_ref, f"LSE splits={s}")


def test_decode_gqa_b64h32kv8l8192d128_sampled_batches():
    # the cache workload's shape with 8 cache heads (groups of 4), at the
    # launch configuration the grouped kernel picks
    fa = _fa()
    B, H, Hkv, L, d = 64, 32, 8, 8192, 128
    q, kc, vc = W.make_gqa(B, H, Hkv, 1, d, "bf16", seed=4400, device=DEV, Nk=L)
    scale = 1.0 / math.sqrt(d)
    say(f"fa_decode gqa B{B} H{H} Hkv{Hkv} L{L} splits=auto")
    o, lse = fa.decode(q, kc, vc, scale=scale)
    torch.cuda.synchronize()
    for b in (0, 17, 40, B - 1):
        o_ref, lse_ref = ref_decode(to64(q[b:b + 1]), to64(kc[b:b + 1]), to64(vc[b:b + 1]), scale)
        assert_bf16_close(to64(o[b:b + 1]), o_ref, f"O batch {b}")
        assert_lse_close(to64(lse[b:b + 1]), lse_ref, f"LSE batch {b}")



# ----------------------------------------------------------------------------
# paged KV cache: pool [P, Hkv, page_size, d], block table, ragged lengths
# ----------------------------------------------------------------------------

def _paged_inputs(B, H, Hkv, ps, lens, d, seed, extra_pages=5):
    """Seeded q and a page pool whose every row that no sequence owns is NaN,
    so any read of an unowned row would show up in the output."""
    g = torch.Generator().manual_seed(seed)
    n_pg = [-(-n // ps) for n in lens]
    total = sum(n_pg) + extra_pages
    max_pages = max(max(n_pg), 1) + 1
    slots = torch.randperm(total, generator=g).tolist()
    q = torch.randn((B, H, 1, d), generator=g).to(torch.bfloat16)
    kp = torch.full((total, Hkv, ps, d), float("nan"), dtype=torch.bfloat16)
    vp = torch.full((total, Hkv, ps, d), float("nan"), dtype=torch.bfloat16)
    table = torch.full((B, max_pages), 1 << 30, dtype=torch.int32)   # unused entries: out of range
    i = 0
    for b in range(B):
        for j in range(n_pg[b]):
            rows = min(ps, lens[b] - j * ps)
            kp[slots[i], :, :rows] = torch.randn((Hkv, rows, d), generator=g).to(torch.bfloat16)
            vp[slots[i], :, :rows] = torch.randn((Hkv, rows, d), generator=g).to(torch.bfloat16)
            table[b, j] = slots[i]
            i += 1
    return q, kp, vp, table, torch.tensor(lens, dtype=torch.int32)


PAGED = [
    # (B, H, Hkv, page_size, lens, d): grouped kernels for 2 <= H/Hkv <= 32
    # (the small-group one for groups of 2 and 3, and of 4 from B*Hkv = 64),
    # per-head kernel otherwise
    (8, 32, 8, 32, [100, 0, 1, 33, 257, 64, 500, 31], 128),
    (3, 8, 4, 64, [300, 129, 2], 64),
    (16, 16, 4, 64, [70, 0, 1, 640, 63, 64, 65, 300, 2, 129, 31, 500, 7, 256, 1000, 33], 64),
    (2, 4, 2, 32, [300, 77], 256),
    (3, 12, 4, 64, [500, 1, 130], 64),
    (3, 8, 2, 32, [1000, 1, 33], 128),
    (2, 8, 8, 64, [700, 64], 128),
    (4, 32, 8, 256, [4097, 0, 31, 2048], 128),
    (2, 4, 1, 128, [300, 129], 64),
    (2, 64, 1, 32, [100, 45], 64),
    (1, 6, 3, 1024, [3000], 128),
    (2, 8, 2, 64, [500, 33], 256),
    (2, 4, 4, 32, [100, 1], 256),
    # one split: 132 and 65 pages in one chunk, so the grouped kernel's table
    # window (64 entries) is read again at pages 64 and 128
    (2, 8, 2, 32, [4200, 2080], 64),
]


@pytest.mark.parametrize("B,H,Hkv,ps,lens,d", PAGED)
def test_decode_paged(B, H, Hkv, ps, lens, d):
    fa = _fa()
    q, kp, vp, table, sl = _paged_inputs(B, H, Hkv, ps, lens, d, seed=5000 + ps + H + sum(lens))
    scale = 1.0 / math.sqrt(d)
    o_ref, lse_ref = ref_decode_paged(to64(q), to64(kp), to64(vp), table.numpy(), sl.numpy(), scale)
    qd, kpd, vpd, td, sld = (x.to(DEV) for x in (q, kp, vp, table, sl))
    for s in (0, 1, 3):
        say(f"fa_decode_paged B{B} H{H} Hkv{Hkv} ps{ps} lens{lens} d{d} splits={s}")
        o, lse = fa.decode_paged(qd, kpd, vpd, td, sld, scale=scale, num_splits=s)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all(), "an unowned (NaN) cache row reached the output"
        assert_bf16_close(to64(o), o_ref, f"O splits={s}")
        assert_lse_close(to64(lse), lse_ref, f"LSE splits={s}")


def test_decode_paged_matches_contiguous():
    # the same cache once contiguous and once scattered over a shuffled pool
    fa = _fa()
    B, H, Hkv, L, d, ps = 4, 16, 4, 1500, 128, 64
    q, kc, vc = W.make_gqa(B, H, Hkv, 1, d, "bf16", seed=5100, device="cpu", Nk=L)
    n_pg = -(-L // ps)
    g = torch.Generator().manual_seed(5101)
    slots = torch.randperm(B * n_pg, generator=g)
    kp = torch.zeros((B * n_pg, Hkv, ps, d), dtype=torch.bfloat16)
    vp = torch.zeros_like(kp)
    table = torch.empty((B, n_pg), dtype=torch.int32)
    for b in range(B):
        for j in range(n_pg):
            rows = min(ps, L - j * ps)
            kp[slots[b * n_pg + j], :, :rows] = kc[b, :, j * ps:j * ps + rows]
            vp[slots[b * n_pg + j], :, :rows] = vc[b, :, j * ps:j * ps + rows]
            table[b, j] = slots[b * n_pg + j]
    sl = torch.full((B,), L, dtype=torch.int32)
    say("fa_decode_paged vs fa_decode")
    o1, l1 = fa.decode(q.to(DEV), kc.to(DEV), vc.to(DEV))
    o2, l2 = fa.decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table.to(DEV), sl.to(DEV))
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_decode(to64(q), to64(kc), to64(vc), 1 / math.sqrt(d))
    assert_bf16_close(to64(o2), o_ref, "O paged")
    assert_lse_close(to64(l2), lse_ref, "LSE paged")
    # same split plan and key order inside each chunk: the two layouts agree closely
    assert (l1 - l2).abs().max().item() <= 1e-3
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2


@pytest.mark.parametrize("n_pages,bad,splits", [
    (5, [2], 0),
    # one chunk of 140 pages: bad entries in the second and third 64-entry
    # window of the grouped kernel's table read
    (140, [70, 129, 139], 1),
])
def test_decode_paged_skips_pages_outside_the_pool(n_pages, bad, splits):
    # a page index outside [0, num_pages) is skipped: the result is the decode
    # over the remaining tokens
    fa = _fa()
    B, H, Hkv, ps, d = 1, 8, 2, 32, 128
    lens = [32 * n_pages]
    q, kp, vp, table, sl = _paged_inputs(B, H, Hkv, ps, lens, d, seed=5200 + n_pages)
    keep = [j for j in range(n_pages) if j not in bad]
    table_bad = table.clone()
    for j in bad:
        table_bad[0, j] = kp.shape[0] + 7 if j % 2 else -3
    say(f"fa_decode_paged with out-of-pool pages {bad} of {n_pages}, splits={splits}")
    o, lse = fa.decode_paged(q.to(DEV), kp.to(DEV), vp.to(DEV), table_bad.to(DEV), sl.to(DEV), num_splits=splits)
    torch.cuda.synchronize()
    kk = torch.cat([kp[int(table[0, j])] for j in keep], dim=1)[None]
    vv = torch.cat([vp[int(table[0, j])] for j in keep], dim=1)[None]
    o_ref, lse_ref = ref_decode(to64(q), to64(kk), to64(vv), 1 / math.sqrt(d))
    assert_bf16_close(to64(o), o_ref, "O")
    assert_lse_close(to64(lse), lse_ref, "LSE")



def test_fwd_d256_fp32_output():
    fa = _fa()
    q, k, v = W.make_custom(2, 2, 333, 256, "bf16", seed=6000, device=DEV)
    say("fa_fwd d256 causal, O in fp32")
    o, lse = fa.attention(q, k, v, is_causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, lse_ref = ref_fwd(to64(q), to64(k), to64(v), True, 1 / 16.0)
    assert_bf16_close(to64(o), o_ref, "O")
    assert_lse_close(to64(lse), lse_ref, "LSE")
