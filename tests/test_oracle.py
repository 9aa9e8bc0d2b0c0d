"""Pins for the fp64 oracle: facts fixed by the pages and by mathematics.

None of these retypes the oracle's formula.  Each checks the oracle against
something independent of it: values derived by hand (tests/golden), closed
forms, invariants the definition implies, brute force of the tiled method
against the definition, finite differences, and PyTorch's CPU float64
``scaled_dot_product_attention`` (the routine the pages point users to:
datacamp "PyTorch-integratie"; Slovak page section 6).

A final group plants plausible mistakes into copies of the oracle and checks
that at least one pin catches each of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import (attention_probs, ref_bwd, ref_decode, ref_fwd, ref_fwd_rows,
                    ref_fwd_tiled, ref_merge_partials)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_derived.json")


def rng(seed):
    return np.random.default_rng(seed)


def rand_qkv(seed, B=1, H=2, N=9, d=4, Nk=None, scale=1.0):
    r = rng(seed)
    nk = N if Nk is None else Nk
    q = r.standard_normal((B, H, N, d)) * scale
    k = r.standard_normal((B, H, nk, d)) * scale
    v = r.standard_normal((B, H, nk, d))
    return q, k, v


# ----------------------------------------------------------------------------
# pins written as functions of the implementation under test, so that the
# mutation tests at the bottom can run them against broken copies
# ----------------------------------------------------------------------------

def pin_golden(fwd, bwd):
    with open(GOLDEN) as f:
        g = json.load(f)
    for c in g["cases"]:
        q = np.array(c["q"])[None, None]
        k = np.array(c["k"])[None, None]
        v = np.array(c["v"])[None, None]
        o, lse = fwd(q, k, v, c["causal"], c["scale"])
        if "o" in c:
            np.testing.assert_allclose(o[0, 0], c["o"], atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[0, 0], c["lse"], atol=1e-12, rtol=0)
        if "o_row0" in c:
            np.testing.assert_allclose(o[0, 0, 0], c["o_row0"], atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[0, 0, 0], c["lse_row0"], atol=1e-12, rtol=0)
        if "dq" in c:
            do = np.array(c["dout"])[None, None]
            dq, dk, dv = bwd(q, k, v, do, c["causal"], c["scale"])[:3]
            np.testing.assert_allclose(dq[0, 0], c["dq"], atol=1e-12, rtol=0)
            np.testing.assert_allclose(dk[0, 0], c["dk"], atol=1e-12, rtol=0)
            np.testing.assert_allclose(dv[0, 0], c["dv"], atol=1e-12, rtol=0)


def pin_equal_values(fwd, bwd):
    # all V rows equal -> every output row equals that row (weights sum to 1)
    for causal in (False, True):
        q, k, _ = rand_qkv(11, N=13, d=5)
        row = rng(12).standard_normal(5)
        v = np.broadcast_to(row, q.shape[:3] + (5,)).copy()
        o, _ = fwd(q, k, v, causal, 0.7)
        np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), atol=1e-12, rtol=0)


def pin_uniform_scores(fwd, bwd):
    # Q = 0: row i averages the visible values; LSE = ln(#visible)
    N = 11
    _, k, v = rand_qkv(13, N=N, d=3)
    q = np.zeros_like(k)
    o, lse = fwd(q, k, v, False, 0.3)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(axis=2, keepdims=True), o.shape),
                               atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, np.full(lse.shape, math.log(N)), atol=1e-12, rtol=0)
    o, lse = fwd(q, k, v, True, 0.3)
    counts = np.arange(1, N + 1, dtype=np.float64)
    expect = np.cumsum(v, axis=2) / counts[None, None, :, None]
    np.testing.assert_allclose(o, expect, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(counts), lse.shape), atol=1e-12, rtol=0)


def pin_first_causal_row(fwd, bwd):
    q, k, v = rand_qkv(14, N=7, d=6)
    s = 0.45
    o, lse = fwd(q, k, v, True, s)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse[:, :, 0], s * np.sum(q[:, :, 0] * k[:, :, 0], axis=-1),
                               atol=1e-12, rtol=0)


def pin_permutation(fwd, bwd):
    # non-causal: permuting keys together with their values changes nothing
    q, k, v = rand_qkv(15, N=10, Nk=10, d=4)
    perm = rng(16).permutation(10)
    o1, l1 = fwd(q, k, v, False, 0.8)
    o2, l2 = fwd(q, k[:, :, perm], v[:, :, perm], False, 0.8)
    np.testing.assert_allclose(o1, o2, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l1, l2, atol=1e-12, rtol=0)


def pin_one_hot_selection(fwd, bwd):
    # K = I (N <= d), Q_i = alpha e_pi(i) with scale*alpha = 60: row i selects V_pi(i)
    N, d, s = 6, 8, 0.5
    alpha = 60.0 / s
    k = np.eye(N, d)[None, None]
    r = rng(17)
    v = r.standard_normal((1, 1, N, 3))
    tol = N * math.exp(-60.0) * np.max(np.abs(v)) * 4 + 1e-15
    for causal in (False, True):
        if causal:
            pi = np.array([r.integers(0, i + 1) for i in range(N)])
        else:
            pi = r.permutation(N)
        q = np.zeros((1, 1, N, d))
        q[0, 0, np.arange(N), pi] = alpha
        o, _ = fwd(q, k, v, causal, s)
        np.testing.assert_allclose(o[0, 0], v[0, 0, pi], atol=tol, rtol=0)


def pin_shift_invariance(fwd, bwd):
    # K -> K + 1 c^T: O unchanged, LSE_i shifts by scale * q_i . c
    q, k, v = rand_qkv(18, N=9, d=4)
    c = rng(19).standard_normal(4)
    s = 0.6
    for causal in (False, True):
        o1, l1 = fwd(q, k, v, causal, s)
        o2, l2 = fwd(q, k + c, v, causal, s)
        np.testing.assert_allclose(o1, o2, atol=1e-12, rtol=0)
        np.testing.assert_allclose(l2 - l1, s * (q @ c), atol=1e-12, rtol=0)


def pin_sdpa_fwd(fwd, bwd):
    for causal in (False, True):
        q, k, v = rand_qkv(20, B=2, H=3, N=17, d=8)
        s = 0.37
        o, lse = fwd(q, k, v, causal, s)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=s)
        np.testing.assert_allclose(o, ot.numpy(), atol=1e-10, rtol=0)
        # LSE: logsumexp of the masked scores, via torch's own routine
        sc = s * (tq @ tk.transpose(-1, -2))
        if causal:
            sc = sc.masked_fill(~torch.ones(17, 17, dtype=torch.bool).tril(), float("-inf"))
        np.testing.assert_allclose(lse, torch.logsumexp(sc, dim=-1).numpy(), atol=1e-10, rtol=0)


def pin_sdpa_bwd(fwd, bwd):
    for causal in (False, True):
        q, k, v = rand_qkv(21, B=1, H=2, N=12, d=6)
        do = rng(22).standard_normal(q.shape)
        s = 0.5
        dq, dk, dv = bwd(q, k, v, do, causal, s)[:3]
        tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
        ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=s)
        ot.backward(torch.from_numpy(do))
        np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-10, rtol=0)
        np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-10, rtol=0)
        np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-10, rtol=0)


def pin_finite_differences(fwd, bwd):
    # loss = <dO, O>; central differences in fp64, eps = 1e-6
    eps = 1e-6
    for causal in (False, True):
        q, k, v = rand_qkv(23, B=1, H=1, N=5, d=3)
        do = rng(24).standard_normal(q.shape)
        s = 0.9
        grads = bwd(q, k, v, do, causal, s)[:3]
        for which, g in zip(range(3), grads):
            base = [q, k, v]
            num = np.zeros_like(base[which])
            it = np.nditer(base[which], flags=["multi_index"])
            for _ in it:
                idx = it.multi_index
                plus = [x.copy() for x in base]
                minus = [x.copy() for x in base]
                plus[which][idx] += eps
                minus[which][idx] -= eps
                lp = np.sum(do * fwd(*plus, causal, s)[0])
                lm = np.sum(do * fwd(*minus, causal, s)[0])
                num[idx] = (lp - lm) / (2 * eps)
            err = np.max(np.abs(num - g)) / max(np.max(np.abs(g)), 1e-30)
            assert err <= 1e-6, (which, causal, err)


def pin_bwd_invariants(fwd, bwd):
    for causal in (False, True):
        q, k, v = rand_qkv(25, B=2, H=2, N=10, d=4)
        do = rng(26).standard_normal(q.shape)
        dq, dk, dv, ds = bwd(q, k, v, do, causal, 0.7, return_ds=True)
        # rows of P sum to 1 -> sum over keys of dV equals sum over queries of dO
        np.testing.assert_allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-10, rtol=0)
        # O is invariant to K -> K + 1 c^T -> dK sums to zero over keys
        np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-10, rtol=0)
        # rows of dS sum to zero
        np.testing.assert_allclose(ds.sum(axis=-1), 0.0, atol=1e-10, rtol=0)


def pin_tiled_equals_naive(fwd, bwd):
    # the pages' blockwise online-softmax algorithm reproduces the definition
    for N in (1, 2, 3, 5, 8, 17):
        for d in (1, 4):
            q, k, v = rand_qkv(100 + N * 10 + d, B=1, H=1, N=N, d=d, scale=1.5)
            for causal in (False, True):
                o_ref, l_ref = fwd(q, k, v, causal, 0.9)
                for br in range(1, N + 1):
                    for bc in range(1, N + 1):
                        o_t, l_t = ref_fwd_tiled(q, k, v, causal, 0.9, br, bc)
                        np.testing.assert_allclose(o_t, o_ref, atol=1e-12, rtol=0)
                        np.testing.assert_allclose(l_t, l_ref, atol=1e-12, rtol=0)
    # with shared K/V heads the blockwise form reads each query head's own
    # K/V head (groups of 2 and MQA), also for tiles that cut the rows
    for (B, H, Hkv) in ((1, 4, 2), (2, 3, 1)):
        q, k, v, _ = _gqa_inputs(70 + H, B, H, Hkv, 7, 3)
        for causal in (False, True):
            o_ref, l_ref = fwd(q, k, v, causal, 0.7)
            for br, bc in ((1, 1), (3, 2), (7, 7), (2, 5)):
                o_t, l_t = ref_fwd_tiled(q, k, v, causal, 0.7, br, bc)
                np.testing.assert_allclose(o_t, o_ref, atol=1e-12, rtol=0)
                np.testing.assert_allclose(l_t, l_ref, atol=1e-12, rtol=0)


def _gqa_inputs(seed, B, H, Hkv, N, d):
    r = rng(seed)
    q = r.standard_normal((B, H, N, d))
    k = r.standard_normal((B, Hkv, N, d))
    v = r.standard_normal((B, Hkv, N, d))
    do = r.standard_normal((B, H, N, d))
    return q, k, v, do


GQA_SHAPES = [(2, 4, 2), (1, 6, 3), (1, 4, 1)]      # (B, H, Hkv): groups of 2, 2 and MQA


def pin_sdpa_gqa_fwd(fwd, bwd):
    # grouped-query attention against torch's own enable_gqa path (fp64, CPU)
    for i, (B, H, Hkv) in enumerate(GQA_SHAPES):
        q, k, v, _ = _gqa_inputs(40 + i, B, H, Hkv, 11, 5)
        for causal in (False, True):
            o, lse = fwd(q, k, v, causal, 0.45)
            tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
            ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                                  scale=0.45, enable_gqa=True)
            np.testing.assert_allclose(o, ot.numpy(), atol=1e-10, rtol=0)


def pin_sdpa_gqa_bwd(fwd, bwd):
    for i, (B, H, Hkv) in enumerate(GQA_SHAPES):
        q, k, v, do = _gqa_inputs(50 + i, B, H, Hkv, 9, 4)
        for causal in (False, True):
            dq, dk, dv = bwd(q, k, v, do, causal, 0.55)[:3]
            tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
            ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                                                  scale=0.55, enable_gqa=True)
            ot.backward(torch.from_numpy(do))
            np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-10, rtol=0)
            np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-10, rtol=0)
            np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-10, rtol=0)


def pin_gqa_group_sum(fwd, bwd):
    # sharing a K/V head among G query heads is the same as giving each query
    # head its own copy: outputs equal, and the shared head's gradients are the
    # sums of the copies' gradients (linearity of the chain rule)
    B, H, Hkv, N, d = 1, 6, 2, 8, 3
    q, k, v, do = _gqa_inputs(60, B, H, Hkv, N, d)
    G = H // Hkv
    k_rep, v_rep = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    for causal in (False, True):
        o1, l1 = fwd(q, k, v, causal, 0.8)
        o2, l2 = fwd(q, k_rep, v_rep, causal, 0.8)
        np.testing.assert_allclose(o1, o2, atol=1e-12, rtol=0)
        np.testing.assert_allclose(l1, l2, atol=1e-12, rtol=0)
        dq1, dk1, dv1 = bwd(q, k, v, do, causal, 0.8)[:3]
        dq2, dk2, dv2 = bwd(q, k_rep, v_rep, do, causal, 0.8)[:3]
        np.testing.assert_allclose(dq1, dq2, atol=1e-12, rtol=0)
        np.testing.assert_allclose(dk1, dk2.reshape(B, Hkv, G, N, d).sum(axis=2), atol=1e-12, rtol=0)
        np.testing.assert_allclose(dv1, dv2.reshape(B, Hkv, G, N, d).sum(axis=2), atol=1e-12, rtol=0)


PINS = [pin_golden, pin_equal_values, pin_uniform_scores, pin_first_causal_row,
        pin_permutation, pin_one_hot_selection, pin_shift_invariance, pin_sdpa_fwd,
        pin_sdpa_bwd, pin_finite_differences, pin_bwd_invariants,
        pin_sdpa_gqa_fwd, pin_sdpa_gqa_bwd, pin_gqa_group_sum]


@pytest.mark.parametrize("pin", PINS + [pin_tiled_equals_naive], ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(ref_fwd, ref_bwd)


# ----------------------------------------------------------------------------
# further facts
# ----------------------------------------------------------------------------

def test_rows_of_p_sum_to_one():
    for causal in (False, True):
        q, k, _ = rand_qkv(30, B=2, H=2, N=33, d=7, scale=3.0)
        p = attention_probs(q, k, causal, 0.4)
        np.testing.assert_allclose(p.sum(axis=-1), 1.0, atol=1e-12, rtol=0)
        if causal:
            assert np.all(np.triu(p[0, 0], 1) == 0.0)


def test_counting_n_squared():
    with open(GOLDEN) as f:
        pairs = json.load(f)["counting"]["pairs"]
    n, entries = pairs[0]
    q, k, _ = rand_qkv(31, B=1, H=1, N=n, d=2)
    assert attention_probs(q, k, False, 1.0).size == entries
    n2, entries2 = pairs[1]
    assert n2 * n2 == entries2


def test_rows_helper_equals_full():
    q, k, v = rand_qkv(32, B=2, H=2, N=40, d=5)
    rows = [0, 1, 7, 20, 39]
    for causal in (False, True):
        o, lse = ref_fwd(q, k, v, causal, 0.5)
        o_r, lse_r = ref_fwd_rows(q, k, v, causal, 0.5, rows)
        np.testing.assert_allclose(o_r, o[:, :, rows], atol=1e-13, rtol=0)
        np.testing.assert_allclose(lse_r, lse[:, :, rows], atol=1e-13, rtol=0)


def test_decode_is_one_query_forward_and_merge_rule():
    r = rng(33)
    q = r.standard_normal((3, 2, 1, 6))
    kc = r.standard_normal((3, 2, 50, 6))
    vc = r.standard_normal((3, 2, 50, 6))
    o, lse = ref_decode(q, kc, vc, 0.4)
    tq, tk, tv = (torch.from_numpy(x) for x in (q, kc, vc))
    ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.4)
    np.testing.assert_allclose(o, ot.numpy(), atol=1e-12, rtol=0)
    # split the cache into uneven disjoint chunks, attend to each, merge by LSE
    bounds = [0, 7, 8, 31, 50]
    parts_o, parts_l = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        oo, ll = ref_decode(q, kc[:, :, a:b], vc[:, :, a:b], 0.4)
        parts_o.append(oo[:, :, 0])
        parts_l.append(ll)
    # an empty split contributes nothing
    parts_o.append(np.zeros_like(parts_o[0]))
    parts_l.append(np.full_like(parts_l[0], -np.inf))
    mo, ml = ref_merge_partials(np.stack(parts_o, axis=2), np.stack(parts_l, axis=2))
    np.testing.assert_allclose(mo, o[:, :, 0], atol=1e-12, rtol=0)
    np.testing.assert_allclose(ml, lse, atol=1e-12, rtol=0)


def test_fully_masked_rows_convention():
    # more queries than keys with causal top-left alignment never masks row 0;
    # a zero-length key set is the only fully masked case the oracle can see
    q = rng(34).standard_normal((1, 1, 3, 2))
    k = np.zeros((1, 1, 0, 2))
    v = np.zeros((1, 1, 0, 2))
    o, lse = ref_fwd(q, k, v, False, 1.0)
    assert np.all(o == 0.0) and np.all(np.isneginf(lse))


def test_large_logits_stay_finite():
    # scores of +-1e4 must not overflow (max subtraction in the softmax)
    q, k, v = rand_qkv(35, N=8, d=2)
    o, lse = ref_fwd(q * 100, k * 100, v, True, 1.0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    p = attention_probs(q * 100, k * 100, True, 1.0)
    np.testing.assert_allclose(o, p @ v, atol=1e-12, rtol=0)


# ----------------------------------------------------------------------------
# mutation checks: plausible mistakes planted into copies of the oracle (CPU)
# ----------------------------------------------------------------------------

def _mut_fwd(kind):
    def fwd(q, k, v, causal, scale):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        B, H, nq, _ = q.shape
        nk = k.shape[2]
        o = np.zeros(q.shape[:3] + (v.shape[-1],))
        lse = np.zeros((B, H, nq))
        for b in range(B):
            for h in range(H):
                s = scale * (q[b, h] @ k[b, h].T)
                if kind == "scale_sqrt":
                    s = math.sqrt(scale) * (q[b, h] @ k[b, h].T)
                if causal:
                    i = np.arange(nq)[:, None]
                    j = np.arange(nk)[None, :]
                    vis = j <= i
                    if kind == "strict_mask":        # diagonal hidden (row 0 kept alive)
                        vis = (j < i) | ((i == 0) & (j == 0))
                    if kind == "mask_transposed":
                        vis = j >= i
                    s = np.where(vis, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                l = e.sum(axis=1, keepdims=True)
                p = e / l
                if kind == "no_normalise":
                    p = e
                vv = v[b, h]
                if kind == "v_reversed":
                    vv = vv[::-1]
                o[b, h] = p @ vv
                lse[b, h] = (m + np.log(l))[:, 0]
                if kind == "lse_no_max":
                    lse[b, h] = np.log(l)[:, 0]
        return o, lse
    return fwd


def _mut_bwd(kind):
    def bwd(q, k, v, do, causal, scale, return_ds=False):
        dq, dk, dv, ds = ref_bwd(q, k, v, do, causal, scale, return_ds=True)
        q64, k64 = np.asarray(q, np.float64), np.asarray(k, np.float64)
        p = attention_probs(q, k, causal, scale)
        if kind == "drop_D":
            dp = np.asarray(do, np.float64) @ np.swapaxes(np.asarray(v, np.float64), -1, -2)
            ds = p * dp
            dq = scale * ds @ k64
            dk = scale * np.swapaxes(ds, -1, -2) @ q64
        if kind == "dk_not_transposed":
            dk = scale * ds @ q64
        if kind == "dq_no_scale":
            dq = ds @ k64
        if kind == "dv_wrong_side":
            dv = p @ np.asarray(do, np.float64)
        if return_ds:
            return dq, dk, dv, ds
        return dq, dk, dv
    return bwd


def _mut_gqa_fwd(kind):
    # K/V head of query head h taken as h % Hkv instead of h // (H / Hkv)
    def fwd(q, k, v, causal, scale):
        H, Hkv = np.shape(q)[1], np.shape(k)[1]
        idx = [h % Hkv for h in range(H)]
        return ref_fwd(q, np.asarray(k)[:, idx], np.asarray(v)[:, idx], causal, scale)
    return fwd


def _mut_gqa_bwd(kind):
    # a shared K/V head keeps the gradient of one query head instead of the sum
    def bwd(q, k, v, do, causal, scale, return_ds=False):
        H, Hkv = np.shape(q)[1], np.shape(k)[1]
        G = H // Hkv
        rep = [h // G for h in range(H)]
        dq, dk, dv, ds = ref_bwd(q, np.asarray(k)[:, rep], np.asarray(v)[:, rep], do, causal,
                                 scale, return_ds=True)
        last = [g * G + G - 1 for g in range(Hkv)]
        dk, dv = dk[:, last], dv[:, last]
        if return_ds:
            return dq, dk, dv, ds
        return dq, dk, dv
    return bwd


FWD_MUTANTS = ["scale_sqrt", "strict_mask", "mask_transposed", "no_normalise",
               "v_reversed", "lse_no_max"]
BWD_MUTANTS = ["drop_D", "dk_not_transposed", "dq_no_scale", "dv_wrong_side"]


def _caught(fwd, bwd):
    for pin in PINS:
        try:
            pin(fwd, bwd)
        except Exception:       # a wrong value or a shape error both count
            return pin.__name__
    return None


@pytest.mark.parametrize("kind", FWD_MUTANTS)
def test_pins_catch_forward_mutant(kind):
    assert _caught(_mut_fwd(kind), ref_bwd) is not None, kind


@pytest.mark.parametrize("kind", BWD_MUTANTS)
def test_pins_catch_backward_mutant(kind):
    assert _caught(ref_fwd, _mut_bwd(kind)) is not None, kind


def test_pins_catch_gqa_head_mapping_mutant():
    assert _caught(_mut_gqa_fwd("kv_modulo"), ref_bwd) == "pin_sdpa_gqa_fwd"


def test_pins_catch_gqa_gradient_sum_mutant():
    assert _caught(ref_fwd, _mut_gqa_bwd("kv_grad_one_head")) == "pin_sdpa_gqa_bwd"


def test_kv_head_mapping_and_divisibility():
    assert [oracle.kv_head(h, 8, 2) for h in range(8)] == [0, 0, 0, 0, 1, 1, 1, 1]
    assert [oracle.kv_head(h, 4, 1) for h in range(4)] == [0, 0, 0, 0]
    with pytest.raises(ValueError):
        oracle.kv_head(0, 6, 4)


def test_gqa_decode_is_one_query_forward():
    B, H, Hkv, L, d = 2, 8, 2, 37, 5
    q, k, v, _ = _gqa_inputs(70, B, H, Hkv, L, d)
    q1 = q[:, :, :1]
    o, lse = ref_decode(q1, k, v, 0.3)
    tq, tk, tv = (torch.from_numpy(x) for x in (q1, k, v))
    ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.3, enable_gqa=True)
    np.testing.assert_allclose(o, ot.numpy(), atol=1e-10, rtol=0)
    assert lse.shape == (B, H)



# ----------------------------------------------------------------------------
# paged KV cache (next row f2)
# ----------------------------------------------------------------------------

def _scatter_to_pool(k, v, lens, ps, seed, extra_pages=3):
    """Test-side construction of a paged pool from contiguous caches [B,Hkv,L,d]:
    the pages of all sequences are placed at shuffled pool slots."""
    B, Hkv, L, d = k.shape
    n_pg = [-(-int(n) // ps) for n in lens]
    total = sum(n_pg) + extra_pages
    slots = rng(seed).permutation(total)
    kp = rng(seed + 1).standard_normal((total, Hkv, ps, d))   # garbage in unused rows
    vp = rng(seed + 2).standard_normal((total, Hkv, ps, d))
    table = np.full((B, max(max(n_pg), 1)), -1, dtype=np.int64)
    i = 0
    for b in range(B):
        for j in range(n_pg[b]):
            t0, t1 = j * ps, min(int(lens[b]), (j + 1) * ps)
            kp[slots[i], :, :t1 - t0] = k[b, :, t0:t1]
            vp[slots[i], :, :t1 - t0] = v[b, :, t0:t1]
            table[b, j] = slots[i]
            i += 1
    return kp, vp, table


def pin_paged_equals_contiguous(decode_paged):
    B, H, Hkv, L, d, ps = 3, 4, 2, 23, 5, 4
    q, k, v, _ = _gqa_inputs(80, B, H, Hkv, L, d)
    q1 = q[:, :, :1]
    lens = np.array([23, 9, 1])
    kp, vp, table = _scatter_to_pool(k, v, lens, ps, seed=81)
    o, lse = decode_paged(q1, kp, vp, table, lens, 0.6)
    for b in range(B):
        n = int(lens[b])
        tq, tk, tv = (torch.from_numpy(x) for x in (q1[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n]))
        ot = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=0.6, enable_gqa=True)
        np.testing.assert_allclose(o[b:b + 1], ot.numpy(), atol=1e-10, rtol=0)
        o_ref, lse_ref = ref_decode(q1[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], 0.6)
        np.testing.assert_allclose(lse[b:b + 1], lse_ref, atol=1e-12, rtol=0)


def test_paged_decode_pin():
    pin_paged_equals_contiguous(oracle.ref_decode_paged)


def test_paged_decode_empty_sequence():
    q, k, v, _ = _gqa_inputs(82, 2, 2, 1, 8, 3)
    kp, vp, table = _scatter_to_pool(k, v, [8, 0], 4, seed=83)
    o, lse = oracle.ref_decode_paged(q[:, :, :1], kp, vp, table, [8, 0], 0.5)
    assert np.all(o[1] == 0.0) and np.all(np.isneginf(lse[1]))
    assert np.all(np.isfinite(lse[0]))


def test_paged_pin_catches_ignored_block_table():
    # a paged decode that reads pages in pool order instead of through the table
    def wrong(q, kp, vp, table, lens, scale):
        ident = np.arange(np.asarray(table).size).reshape(np.shape(table))
        return oracle.ref_decode_paged(q, kp, vp, ident, lens, scale)
    with pytest.raises(AssertionError):
        pin_paged_equals_contiguous(wrong)
