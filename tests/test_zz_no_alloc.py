"""fa_decode_noalloc against fa_decode, through the C ABI.

fa_decode_noalloc runs fa_decode's kernels with the split partials in the
library's static scratch array instead of a caller's workspace, so with the
same num_splits its outputs must equal fa_decode's bit for bit.  Two calls in a
row, the second smaller, then the first again: whatever a call leaves in the
shared array must not leak into the next one.  The noalloc calls must not
allocate device memory (torch's allocator is checked around them).
"""

from __future__ import annotations

import math

import pytest
import torch

import fa_workloads as W
from oracle import ref_decode
from parity_util import assert_bf16_close, assert_lse_close, to64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def say(msg):
    print(msg, flush=True)


def _pair(B, H, Hkv, L, d, splits, seed):
    """(fa_decode outputs, fa_decode_noalloc outputs) on the same inputs."""
    import exact_io_aware_11_amd as fa
    q, kc, vc = W.make_gqa(B, H, Hkv, 1, d, "bf16", seed=seed, Nk=L, device=DEV)
    scale = 1.0 / math.sqrt(d)
    o_ref, lse_ref = fa.decode(q, kc, vc, scale=scale, num_splits=splits)
    o = torch.full((B, H, 1, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    st = fa.fa_decode_noalloc(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              B, H, Hkv, L, d, fa.FA_BF16, splits, scale,
                              torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.fa_status_string(st)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return (q, kc, vc, scale), (o_ref, lse_ref), (o, lse)


CASES = [
    # (B, H, Hkv, L, d, num_splits): the per-head kernel, the small-group
    # kernel (groups of 4) and the MFMA grouped kernel (groups of 8)
    (8, 32, 32, 3000, 128, 0),
    (16, 32, 8, 2048, 128, 0),
    (2, 16, 2, 1500, 64, 5),
]


def test_noalloc_equals_decode_two_calls_second_smaller():
    big = (16, 32, 32, 4100, 128, 0)
    small = (2, 4, 4, 700, 64, 3)
    say(f"fa_decode_noalloc call 1 {big}")
    _, (o_ref1, l_ref1), (o1, l1) = _pair(*big, seed=9101)
    assert torch.equal(o1, o_ref1) and torch.equal(l1, l_ref1)
    say(f"fa_decode_noalloc call 2 (smaller) {small}")
    inp, (o_ref2, l_ref2), (o2, l2) = _pair(*small, seed=9102)
    assert torch.equal(o2, o_ref2) and torch.equal(l2, l_ref2)
    # the smaller call also meets the oracle's tolerance
    q, kc, vc, scale = inp
    o64, l64 = ref_decode(to64(q), to64(kc), to64(vc), scale)
    assert_bf16_close(to64(o2), o64, "O")
    assert_lse_close(to64(l2), l64, "LSE")
    say("fa_decode_noalloc call 3 (the first shape again)")
    _, (o_ref3, l_ref3), (o3, l3) = _pair(*big, seed=9101)
    assert torch.equal(o3, o_ref3) and torch.equal(l3, l_ref3)


@pytest.mark.parametrize("B,H,Hkv,L,d,splits", CASES)
def test_noalloc_equals_decode(B, H, Hkv, L, d, splits):
    say(f"fa_decode_noalloc B{B} H{H} Hkv{Hkv} L{L} d{d} splits={splits}")
    _, (o_ref, l_ref), (o, l) = _pair(B, H, Hkv, L, d, splits, seed=9200 + L)
    assert torch.equal(o, o_ref) and torch.equal(l, l_ref)


def test_noalloc_rejects_beyond_the_scratch_limit():
    import exact_io_aware_11_amd as fa
    B, H, L, d = 64, 32, 8192, 128
    q = torch.zeros((B, H, 1, d), dtype=torch.bfloat16, device=DEV)
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
    kc = torch.zeros((1, 1, 1, d), dtype=torch.bfloat16, device=DEV)   # never read: rejected first
    say("fa_decode_noalloc over the scratch limit")
    st = fa.fa_decode_noalloc(q.data_ptr(), kc.data_ptr(), kc.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              B, H, H, L, d, fa.FA_BF16, 32, 0.1, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_ERR_SCRATCH_LIMIT
