"""The entry points inside a captured HIP graph.

The library allocates, frees and synchronises nothing and clears no memory with
memset nodes, so a caller can capture its launches (through torch's CUDAGraph,
which is hipGraph on ROCm) and replay them; small-batch decode is
launch-bound and is where that pays.  Each test replays its graph several
times, with new inputs copied into the captured buffers by eager work between
the replays, and compares every replay with an eager call on the same inputs:
the kernels are deterministic, so the two must agree bit for bit.  (The eager
calls themselves are checked against the oracle in test_gpu_parity.py.)
"""

from __future__ import annotations

import pytest
import torch

import fa_workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
REPLAYS = 4


def _fa():
    import exact_io_aware_11_amd as fa
    return fa


def say(msg):
    print(msg, flush=True)


def _capture(fn):
    """Warm fn up on a side stream, then capture one call of it; returns the
    graph and the tensors the captured call produced (static across replays)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = fn()
    torch.cuda.synchronize()
    return g, out


@pytest.mark.parametrize("Hkv", [8, 16])
def test_decode_replays_in_a_graph(Hkv):
    # Hkv = 8: groups of 4 at B*Hkv = 16 (MFMA grouped kernel); Hkv = 16:
    # groups of 2 (small-group kernel)
    fa = _fa()
    B, H, L, d = 2, 32, 1500, 128
    q, kc, vc = W.make_gqa(B, H, Hkv, 1, d, "bf16", seed=7000 + Hkv, device=DEV, Nk=L)
    qs = q.clone()
    say(f"graph: fa_decode B{B} H{H} Hkv{Hkv} L{L} d{d}")
    g, (o_g, lse_g) = _capture(lambda: fa.decode(qs, kc, vc))
    for i in range(REPLAYS):
        qs.copy_(W.make_gqa(B, H, Hkv, 1, d, "bf16", seed=7001 + i, device=DEV, Nk=1)[0])
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = fa.decode(qs, kc, vc)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {i}: O differs from the eager call"
        assert torch.equal(lse_g, lse_e), f"replay {i}: LSE differs from the eager call"


def test_paged_decode_replays_in_a_graph():
    fa = _fa()
    B, H, Hkv, d, ps, n_pg = 3, 16, 4, 128, 32, 70
    g0 = torch.Generator(device=DEV).manual_seed(7100)
    pool = B * n_pg
    kp = torch.randn((pool, Hkv, ps, d), generator=g0, device=DEV).to(torch.bfloat16)
    vp = torch.randn((pool, Hkv, ps, d), generator=g0, device=DEV).to(torch.bfloat16)
    table = torch.randperm(pool, generator=g0, device=DEV).to(torch.int32).reshape(B, n_pg)
    lens = torch.tensor([ps * n_pg, 1000, 33], dtype=torch.int32, device=DEV)
    qs = torch.randn((B, H, 1, d), generator=g0, device=DEV).to(torch.bfloat16)
    say(f"graph: fa_decode_paged B{B} H{H} Hkv{Hkv} page{ps} pages{n_pg}")
    g, (o_g, lse_g) = _capture(lambda: fa.decode_paged(qs, kp, vp, table, lens, num_splits=1))
    for i in range(REPLAYS):
        qs.copy_(torch.randn((B, H, 1, d), generator=g0, device=DEV).to(torch.bfloat16))
        lens.copy_(torch.tensor([ps * n_pg - 5 * i, 1000 + i, 33 * i], dtype=torch.int32, device=DEV))
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = fa.decode_paged(qs, kp, vp, table, lens, num_splits=1)
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e), f"replay {i}: O differs from the eager call"
        assert torch.equal(lse_g, lse_e), f"replay {i}: LSE differs from the eager call"


@pytest.mark.parametrize("Hkv", [4, 1])
def test_forward_backward_replay_in_a_graph(Hkv):
    # Hkv = 1 with H = 4 and a small grid takes the backward's split path
    # (fp32 partials in the workspace, then the reduce kernel)
    fa = _fa()
    B, H, N, d = 1, 4, 640, 128
    q, k, v, do = W.make_gqa(B, H, Hkv, N, d, "bf16", seed=7200 + Hkv, with_dout=True, device=DEV)

    def step():
        o, lse = fa.attention(q, k, v, is_causal=True)
        dq, dk, dv = fa.attention_backward(q, k, v, o, lse, do, is_causal=True)
        return o, lse, dq, dk, dv

    say(f"graph: fa_fwd + fa_bwd B{B} H{H} Hkv{Hkv} N{N} d{d} causal")
    g, outs_g = _capture(step)
    for i in range(REPLAYS):
        new = W.make_gqa(B, H, Hkv, N, d, "bf16", seed=7210 + 10 * Hkv + i, with_dout=True, device=DEV)
        for dst, src in zip((q, k, v, do), new):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        outs_e = step()
        torch.cuda.synchronize()
        for name, a, b in zip(("O", "LSE", "dQ", "dK", "dV"), outs_g, outs_e):
            assert torch.equal(a, b), f"replay {i}: {name} differs from the eager call"
