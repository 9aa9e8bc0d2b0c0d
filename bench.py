"""Benchmark of the exact-attention hot path on one MI355X.

One step runs every stage of the path once, on resident synthetic inputs:
  * fa_fwd on the 2K-token causal bf16 workload (B=4, H=16, N=2048, d=128),
  * fa_bwd on the same batch, consuming that forward's O and LSE,
  * fa_decode on the KV-cache workload (B=64, H=32, L=8192, d=128).
HIP events on the library's stream time each call inside the step.

``value`` is the metric's first clause: attention forward+backward TFLOP/s on
the 2K workload (4*B*H*N^2*d, halved for causal; backward 2.5x that), taken
over the fwd and bwd calls inside the timed steps.  The decode leg of the same
steps is reported as achieved HBM GB/s (K and V read once: 2*B*H*L*d*2 bytes).
A sweep over N = 2K..16K (H=32, B=16384/N, causal) reports forward and
backward TFLOP/s as the metric's range asks, and the oracle's CPU time on a
bounded sample is reported as ``cpu_baseline``.

After the sweep, ``next_rows`` reports grouped-query attention (decode with
8 cache heads for 32 query heads, fwd/bwd with groups of 4), paged-cache
decodes, batch-1 decode latency, head dim 256 (forward and decode) and the
fp8 (e4m3) forward.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep]
                       [--no-next] [--no-cpu-baseline]
       python bench.py --reduce-counters DIR... [--write-traffic]   (host only)
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk)
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA (spec)


def fwd_flops(B, H, N, d, causal=True):
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the grouped-query, paged-cache and head-dim-256 measurements")
    ap.add_argument("--reduce-counters", nargs="+", metavar="DIR",
                    help="host only: summarise rocprofv3 --pmc output of this script and exit")
    ap.add_argument("--write-traffic", action="store_true",
                    help="with --reduce-counters: write profiles/traffic.json")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class Buffers:
    """Resident inputs, outputs and workspaces for one step (raw pointers for the C ABI)."""

    def __init__(self, torch, fa, W, dev):
        self.w_tr = W.WORKLOADS["fwd_causal_bf16_b4h16n2048d128"]
        self.w_dec = W.WORKLOADS["decode_bf16_b64h32l8192d128"]
        t = self.w_tr
        self.q, self.k, self.v, self.do = W.draw([(t.B, t.H, t.N, t.d)] * 4, t.seed, torch.bfloat16,
                                                 device="cpu")
        self.q, self.k, self.v, self.do = (x.to(dev) for x in (self.q, self.k, self.v, self.do))
        self.o = torch.empty_like(self.q)
        self.lse = torch.empty((t.B, t.H, t.N), dtype=torch.float32, device=dev)
        self.dq = torch.empty_like(self.q)
        self.dk = torch.empty_like(self.q)
        self.dv = torch.empty_like(self.q)
        self.bwd_ws_bytes = fa.fa_bwd_workspace_bytes(t.B, t.H, t.H, t.N, t.d)
        self.bwd_ws = torch.empty((self.bwd_ws_bytes,), dtype=torch.uint8, device=dev)
        dcfg = self.w_dec
        self.dq_in, self.kc, self.vc = W.make_inputs(dcfg, dev)
        self.do_out = torch.empty_like(self.dq_in)
        self.dlse = torch.empty((dcfg.B, dcfg.H), dtype=torch.float32, device=dev)
        self.splits = fa.fa_decode_num_splits(dcfg.B, dcfg.H, dcfg.H, dcfg.N, dcfg.d)
        self.dec_ws_bytes = fa.fa_decode_workspace_bytes(dcfg.B, dcfg.H, dcfg.H, dcfg.N, dcfg.d, 0)
        self.dec_ws = torch.empty((self.dec_ws_bytes,), dtype=torch.uint8, device=dev)


def run_fwd(fa, b, stream):
    t = b.w_tr
    st = fa.fa_fwd(b.q.data_ptr(), b.k.data_ptr(), b.v.data_ptr(), b.o.data_ptr(), fa.FA_BF16,
                   b.lse.data_ptr(), t.B, t.H, t.H, t.N, t.d, fa.FA_BF16, 1, t.scale, stream)
    if st != fa.FA_OK:
        raise RuntimeError(fa.fa_status_string(st))


def run_bwd(fa, b, stream):
    t = b.w_tr
    st = fa.fa_bwd(b.q.data_ptr(), b.k.data_ptr(), b.v.data_ptr(), b.o.data_ptr(), fa.FA_BF16,
                   b.lse.data_ptr(), b.do.data_ptr(), b.dq.data_ptr(), b.dk.data_ptr(), b.dv.data_ptr(),
                   b.bwd_ws.data_ptr(), b.bwd_ws_bytes, t.B, t.H, t.H, t.N, t.d, fa.FA_BF16, 1, t.scale,
                   stream)
    if st != fa.FA_OK:
        raise RuntimeError(fa.fa_status_string(st))


def run_decode(fa, b, stream):
    t = b.w_dec
    st = fa.fa_decode(b.dq_in.data_ptr(), b.kc.data_ptr(), b.vc.data_ptr(), b.do_out.data_ptr(),
                      b.dlse.data_ptr(), b.dec_ws.data_ptr(), b.dec_ws_bytes, t.B, t.H, t.H, t.N, t.d,
                      fa.FA_BF16, 0, t.scale, stream)
    if st != fa.FA_OK:
        raise RuntimeError(fa.fa_status_string(st))


def timed_ms(torch, fn, iters, warm_ms=50.0):
    """Mean milliseconds per call of ``fn`` over ``iters`` back-to-back calls on
    the current stream, after untimed calls worth at least ``warm_ms`` (the
    chip's clocks need tens of milliseconds of load to settle)."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    for _ in range(min(500, max(3, math.ceil(warm_ms / max(e0.elapsed_time(e1), 1e-3))))):
        fn()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(iters):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


def sweep(torch, fa, W, dev, iters=10):
    """fwd and bwd TFLOP/s at N = 2K..16K, H = 32, B = 16384/N, causal bf16, d = 128."""
    out = []
    stream = torch.cuda.current_stream().cuda_stream
    for N in (2048, 4096, 8192, 16384):
        B, H, d = 16384 // N, 32, 128
        scale = 1.0 / math.sqrt(d)
        seed = 10 + int(math.log2(N // 1024))
        q, k, v, do = W.draw([(B, H, N, d)] * 4, seed, torch.bfloat16, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        nb = fa.fa_bwd_workspace_bytes(B, H, H, N, d)
        ws = torch.empty((nb,), dtype=torch.uint8, device=dev)

        def f():
            fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), fa.FA_BF16, lse.data_ptr(),
                      B, H, H, N, d, fa.FA_BF16, 1, scale, stream)

        def g():
            fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), fa.FA_BF16, lse.data_ptr(),
                      do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), nb,
                      B, H, H, N, d, fa.FA_BF16, 1, scale, stream)

        res = {"N": N, "B": B, "H": H, "d": d}
        for name, fn, mult in (("fwd", f, 1.0), ("bwd", g, 2.5)):
            f()
            ms = timed_ms(torch, fn, iters)
            tf = mult * fwd_flops(B, H, N, d) / (ms * 1e-3) / 1e12
            res[name] = {"ms": round(ms, 4), "tflops": round(tf, 1),
                         "frac_mfma_peak": round(tf / PEAK_BF16_TFLOPS, 4)}
        log(f"sweep N={N}: fwd {res['fwd']['tflops']} TFLOP/s, bwd {res['bwd']['tflops']} TFLOP/s")
        out.append(res)
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return out


def gqa_measure(torch, fa, W, dev, iters=20):
    """Grouped-query attention (K/V heads shared by groups of query heads).

    decode: B64 H32 Hkv8 L8192 d128 (groups of 4); each cache head is read
    once per group, so the algorithmic bytes are 2*B*Hkv*L*d*2.
    fwd/bwd: B4 H16 Hkv4 N2048 d128 causal; same flops as multi-head.
    """
    stream = torch.cuda.current_stream().cuda_stream
    out = {}

    def timed(fn):
        return timed_ms(torch, fn, iters)

    B, H, Hkv, L, d = 64, 32, 8, 8192, 128
    q, kc, vc = W.make_gqa(B, H, Hkv, 1, d, "bf16", seed=20, device=dev, Nk=L)
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    nb = fa.fa_decode_workspace_bytes(B, H, Hkv, L, d, 0)
    ws = torch.empty((nb,), dtype=torch.uint8, device=dev)
    scale = 1.0 / math.sqrt(d)
    ms = timed(lambda: fa.fa_decode(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    ws.data_ptr(), nb, B, H, Hkv, L, d, fa.FA_BF16, 0, scale, stream))
    byt = 2.0 * B * Hkv * L * d * 2
    gbs = byt / (ms * 1e-3) / 1e9
    out["decode"] = {"workload": f"B{B} H{H} Hkv{Hkv} L{L} d{d}", "ms": round(ms, 4), "GBps": round(gbs, 1),
                     "bound": "hbm", "frac": round(gbs / PEAK_HBM_GBPS, 4), "algorithmic_bytes": byt,
                     "splits": fa.fa_decode_num_splits(B, H, Hkv, L, d)}
    log(f"gqa decode {out['decode']['workload']}: {ms:.4f} ms, {gbs:.1f} GB/s")
    del q, kc, vc, o, ws

    B, H, Hkv, N = 4, 16, 4, 2048
    q, k, v, do = W.make_gqa(B, H, Hkv, N, d, "bf16", seed=21, with_dout=True, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nb = fa.fa_bwd_workspace_bytes(B, H, Hkv, N, d)
    ws = torch.empty((nb,), dtype=torch.uint8, device=dev)

    def f():
        fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), fa.FA_BF16, lse.data_ptr(),
                  B, H, Hkv, N, d, fa.FA_BF16, 1, scale, stream)

    def g():
        fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), fa.FA_BF16, lse.data_ptr(),
                  do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), nb,
                  B, H, Hkv, N, d, fa.FA_BF16, 1, scale, stream)

    ff = fwd_flops(B, H, N, d)
    for name, fn, mult in (("fwd", f, 1.0), ("bwd", g, 2.5)):
        f()
        ms = timed(fn)
        tf = mult * ff / (ms * 1e-3) / 1e12
        out[name] = {"workload": f"B{B} H{H} Hkv{Hkv} N{N} d{d} causal", "ms": round(ms, 4),
                     "tflops": round(tf, 1), "bound": "mfma", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
        log(f"gqa {name} {out[name]['workload']}: {ms:.4f} ms, {tf:.1f} TFLOP/s")
    return out


def paged_measure(torch, fa, dev, iters=20):
    """Decode against a paged cache: B64 H32 L8192 d128, 64-token pages of one
    pool in shuffled order, every sequence full length; multi-head (32 cache
    heads, per-head kernel) and grouped (8 cache heads, grouped kernel).
    Algorithmic bytes: the K and V rows read, 2*B*Hkv*L*d*2."""
    stream = torch.cuda.current_stream().cuda_stream
    B, H, L, d, ps = 64, 32, 8192, 128, 64
    scale = 1.0 / math.sqrt(d)
    g = torch.Generator(device=dev)
    g.manual_seed(30)
    out = {}
    for name, Hkv in (("mha", 32), ("gqa", 8)):
        pages = B * (L // ps)
        q = torch.randn((B, H, 1, d), generator=g, device=dev).to(torch.bfloat16)
        kp = torch.randn((pages, Hkv, ps, d), generator=g, device=dev).to(torch.bfloat16)
        vp = torch.randn((pages, Hkv, ps, d), generator=g, device=dev).to(torch.bfloat16)
        table = torch.randperm(pages, generator=g, device=dev).to(torch.int32).reshape(B, L // ps)
        lens = torch.full((B,), L, dtype=torch.int32, device=dev)
        o = torch.empty_like(q)
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        nb = fa.fa_decode_workspace_bytes(B, H, Hkv, L, d, 0)
        ws = torch.empty((nb,), dtype=torch.uint8, device=dev)

        def fn():
            st = fa.fa_decode_paged(q.data_ptr(), kp.data_ptr(), vp.data_ptr(), table.data_ptr(), lens.data_ptr(),
                                    o.data_ptr(), lse.data_ptr(), ws.data_ptr(), nb, B, H, Hkv, pages, ps,
                                    L // ps, d, fa.FA_BF16, 0, scale, stream)
            if st != fa.FA_OK:
                raise RuntimeError(fa.fa_status_string(st))
        ms = timed_ms(torch, fn, iters)
        byt = 2.0 * B * Hkv * L * d * 2
        gbs = byt / (ms * 1e-3) / 1e9
        out[name] = {"workload": f"B{B} H{H} Hkv{Hkv} L{L} d{d} page{ps}", "ms": round(ms, 4),
                     "GBps": round(gbs, 1), "bound": "hbm", "frac": round(gbs / PEAK_HBM_GBPS, 4),
                     "algorithmic_bytes": byt}
        log(f"paged decode {out[name]['workload']}: {ms:.4f} ms, {gbs:.1f} GB/s")
        del q, kp, vp, table, lens, o, lse, ws
        torch.cuda.empty_cache()
    return out


def fp8_measure(torch, fa, W, dev, iters=30):
    """FP8 (e4m3) forward, causal, d = 128, at the 2K workload (B4 H16 N2048) and
    the long-context one (B1 H32 N16384); same flop formula, against the fp8
    MFMA peak."""
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for key, (B, H, N) in (("n2048", (4, 16, 2048)), ("n16384", (1, 32, 16384))):
        d = 128
        scale = 1.0 / math.sqrt(d)
        q8, k8, vt8, qs, ks, vs = W.make_fp8(B, H, H, N, d, seed=50 + N // 2048, device=dev, gen_device=dev)
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)

        def f():
            st = fa.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), qs, ks, vs, o.data_ptr(), fa.FA_BF16,
                               lse.data_ptr(), B, H, H, N, d, 1, scale, stream)
            assert st == fa.FA_OK, fa.fa_status_string(st)
        ms = timed_ms(torch, f, iters)
        tf = fwd_flops(B, H, N, d) / (ms * 1e-3) / 1e12
        out[key] = {"workload": f"B{B} H{H} N{N} d{d} causal, e4m3 in, bf16 out", "ms": round(ms, 4),
                    "tflops": round(tf, 1), "bound": "mfma", "frac": round(tf / PEAK_FP8_TFLOPS, 4)}
        log(f"fp8 fwd {out[key]['workload']}: {ms:.4f} ms, {tf:.1f} TFLOP/s")
        del q8, k8, vt8, o, lse
    return out


def small_batch_decode_measure(torch, fa, W, dev, iters=200):
    """Decode steps at batch 1 (latency-bound: a few MB of cache), with 8
    cache heads (grouped kernel) and 32 (per-head kernel), L = 4K and 16K."""
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for key, (Hkv, L) in (("gqa_l4096", (8, 4096)), ("gqa_l16384", (8, 16384)), ("mha_l16384", (32, 16384))):
        B, H, d = 1, 32, 128
        q, kc, vc = W.make_gqa(B, H, Hkv, 1, d, "bf16", seed=61 + L // 4096 + Hkv, device=dev, Nk=L)
        o = torch.empty_like(q)
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        nb = fa.fa_decode_workspace_bytes(B, H, Hkv, L, d, 0)
        ws = torch.empty((nb,), dtype=torch.uint8, device=dev)
        scale = 1.0 / math.sqrt(d)
        ms = timed_ms(torch, lambda: fa.fa_decode(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(),
                                                  lse.data_ptr(), ws.data_ptr(), nb, B, H, Hkv, L, d, fa.FA_BF16,
                                                  0, scale, stream), iters)
        byt = 2.0 * B * Hkv * L * d * 2
        out[key] = {"workload": f"B{B} H{H} Hkv{Hkv} L{L} d{d}", "us": round(ms * 1e3, 2),
                    "GBps": round(byt / (ms * 1e-3) / 1e9, 1),
                    "splits": fa.fa_decode_num_splits(B, H, Hkv, L, d)}
        log(f"small-batch decode {out[key]['workload']}: {out[key]['us']} us, {out[key]['GBps']} GB/s")
    return out


def d256_measure(torch, fa, W, dev, iters=10):
    """Head dim 256: causal bf16 forward at B4 H16 N4096 and decode at
    B64 H16 L4096 (multi-head) -- same flop formula / bytes as at d = 128."""
    stream = torch.cuda.current_stream().cuda_stream
    out = {}

    def timed(fn):
        return timed_ms(torch, fn, iters)

    B, H, N, d = 4, 16, 4096, 256
    scale = 1.0 / math.sqrt(d)
    q, k, v = W.make_custom(B, H, N, d, "bf16", seed=40, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    ms = timed(lambda: fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), fa.FA_BF16,
                                 lse.data_ptr(), B, H, H, N, d, fa.FA_BF16, 1, scale, stream))
    tf = fwd_flops(B, H, N, d) / (ms * 1e-3) / 1e12
    out["fwd"] = {"workload": f"B{B} H{H} N{N} d{d} causal", "ms": round(ms, 4), "tflops": round(tf, 1),
                  "bound": "mfma", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    log(f"d256 fwd {out['fwd']['workload']}: {ms:.4f} ms, {tf:.1f} TFLOP/s")
    del q, k, v, o, lse

    B, H, L = 64, 16, 4096
    q, kc, vc = W.make_custom(B, H, 1, d, "bf16", seed=41, device=dev, Nk=L)
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    nb = fa.fa_decode_workspace_bytes(B, H, H, L, d, 0)
    ws = torch.empty((nb,), dtype=torch.uint8, device=dev)
    ms = timed(lambda: fa.fa_decode(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                    ws.data_ptr(), nb, B, H, H, L, d, fa.FA_BF16, 0, scale, stream))
    byt = 2.0 * B * H * L * d * 2
    gbs = byt / (ms * 1e-3) / 1e9
    out["decode"] = {"workload": f"B{B} H{H} L{L} d{d}", "ms": round(ms, 4), "GBps": round(gbs, 1),
                     "bound": "hbm", "frac": round(gbs / PEAK_HBM_GBPS, 4), "algorithmic_bytes": byt}
    log(f"d256 decode {out['decode']['workload']}: {ms:.4f} ms, {gbs:.1f} GB/s")
    return out


def cpu_baseline(W, min_seconds=10.0, max_passes=8):
    """The fp64 oracle, as it stands, on the 2K training workload.

    One pass is ref_fwd + ref_bwd over all B*H = 64 heads of B4 H16 N2048 d128
    (causal); passes repeat until ``min_seconds`` have elapsed, and the rate is
    the mean over them.
    """
    import numpy as np
    import torch

    from oracle import ref_bwd, ref_fwd
    t = W.WORKLOADS["fwd_causal_bf16_b4h16n2048d128"]
    q, k, v, do = W.draw([(t.B, t.H, t.N, t.d)] * 4, t.seed, torch.bfloat16, device="cpu")
    q, k, v, do = (x.float().numpy().astype(np.float64) for x in (q, k, v, do))
    threads = None
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=None)
    except Exception:
        pass
    passes = 0
    t0 = time.perf_counter()
    while passes < max_passes:
        ref_fwd(q, k, v, True, t.scale)
        ref_bwd(q, k, v, do, True, t.scale)
        passes += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    secs = time.perf_counter() - t0
    flops = passes * 3.5 * fwd_flops(t.B, t.H, t.N, t.d)
    return {
        "value": round(flops / secs / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": threads or os.cpu_count(),
        "kind": "oracle",
        "sample": f"oracle ref_fwd + ref_bwd (fp64, full N x N scores) on the whole B4 H16 N2048 d128 "
                  f"causal workload, {passes} pass(es) in {secs:.2f} s; rate uses the same causal flop "
                  "count as the GPU",
        "seconds": round(secs, 3),
        "affinity_cores": len(os.sched_getaffinity(0)),
    }


# Kernels of one step as they appear in rocprofv3 output: key -> (name
# substring, source file, algorithmic HBM bytes per launch on the step's
# workloads).  Algorithmic bytes count each tensor the kernel must touch once:
# bf16 [B,H,N,d] tensors at 2 bytes an element, fp32 row statistics at 4.
def _step_kernels():
    B, H, N, d = 4, 16, 2048, 128          # training workload
    Bd, Hd, L = 64, 32, 8192                # decode workload
    t, r = B * H * N * d * 2, B * H * N * 4
    return {
        "fwd": ("fwd_bf16_kernel", "fa_fwd.hip", "B4 H16 N2048 d128 causal", 4 * t + r,
                "read Q, K, V; write O, LSE"),
        "bwd_prep": ("bwd_prep_kernel", "fa_bwd.hip", "B4 H16 N2048 d128 causal", 2 * t + r,
                     "read O, dO; write D"),
        "bwd_dkdv": ("bwd_dkdv_kernel", "fa_bwd.hip", "B4 H16 N2048 d128 causal", 6 * t + 2 * r,
                     "read Q, K, V, dO, LSE, D; write dK, dV"),
        "bwd_dq": ("bwd_dq_kernel", "fa_bwd.hip", "B4 H16 N2048 d128 causal", 5 * t + 2 * r,
                   "read Q, K, V, dO, LSE, D; write dQ"),
        "decode": ("decode_split_kernel", "fa_decode.hip", "B64 H32 L8192 d128",
                   2 * Bd * Hd * L * d * 2, "read the K and V caches"),
        "decode_merge": ("decode_merge_kernel", "fa_decode.hip", "B64 H32 L8192 d128", None,
                         "read the split partials; write O, LSE"),
    }


def kernel_digest(src, csrc=None):
    """SHA-256 of what a kernel is compiled from: its .hip file and the two
    shared headers, with comments and whitespace removed (so a comment edit
    keeps a traffic record valid, while any code change in the file or the
    headers invalidates it)."""
    import hashlib
    import re
    csrc = csrc or os.path.join(ROOT, "exact_io_aware_11_amd", "csrc")
    h = hashlib.sha256()
    for name in (src, "fa_common.hpp", "fa_internal.hpp"):
        with open(os.path.join(csrc, name)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(name.encode())
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


COPY_KERNEL = "copyBuffer"            # the 256 MiB device copy main() runs at set-up
COPY_BYTES = 256 * 1024 * 1024


def reduce_counters(dirs, write_traffic):
    """Turn rocprofv3 ``--pmc`` CSV output of this script into per-kernel means.

    Every ``*counter_collection.csv`` under ``dirs`` is read; each counter is
    averaged per dispatch of a kernel, leaving out the first (cold) dispatch.
    With FETCH_SIZE and WRITE_SIZE present, both are scaled by what they read
    for the 256 MiB copy, and ``write_traffic`` writes profiles/traffic.json
    with each kernel's HBM bytes per launch.  Prints a markdown summary.
    """
    import csv
    import glob
    from collections import defaultdict

    kern = _step_kernels()
    names = {k: v[0] for k, v in kern.items()} | {"copy": COPY_KERNEL}
    vals = defaultdict(lambda: defaultdict(list))   # key -> counter -> [(dispatch, value)]
    for d in dirs:
        for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    for key, pat in names.items():
                        if pat in row["Kernel_Name"]:
                            vals[key][row["Counter_Name"]].append(
                                (int(row["Dispatch_Id"]), float(row["Counter_Value"])))
    mean = {}
    for key, cs in vals.items():
        mean[key] = {}
        for c, xs in cs.items():
            xs = [v for _, v in sorted(xs)]
            xs = xs[1:] if len(xs) > 1 else xs
            mean[key][c] = sum(xs) / len(xs)

    print("| kernel | counter | mean per dispatch |\n|---|---|---:|")
    for key in list(kern) + ["copy"]:
        for c in sorted(mean.get(key, {})):
            print(f"| {names[key]} | {c} | {mean[key][c]:.6g} |")

    derived = []
    for key in kern:
        m = mean.get(key, {})
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m and "GRBM_GUI_ACTIVE" in m:
            # GRBM_GUI_ACTIVE sums the 8 XCDs' clocks; MFMA busy cycles sum the 1024 SIMDs
            cyc = m["GRBM_GUI_ACTIVE"] / 8
            derived.append(f"| {names[key]} | MFMA busy | {100 * m['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / cyc:.1f}% "
                           f"of {cyc:.4g} cycles |")
        if "SQ_WAIT_ANY" in m and "SQ_WAVE_CYCLES" in m:
            derived.append(f"| {names[key]} | waves waiting | {100 * m['SQ_WAIT_ANY'] / m['SQ_WAVE_CYCLES']:.0f}% "
                           "of wave cycles |")
        if "SQ_LDS_BANK_CONFLICT" in m and "SQ_LDS_IDX_ACTIVE" in m and m["SQ_LDS_IDX_ACTIVE"] > 0:
            derived.append(f"| {names[key]} | LDS bank conflicts | "
                           f"{100 * m['SQ_LDS_BANK_CONFLICT'] / m['SQ_LDS_IDX_ACTIVE']:.2f}% of LDS cycles |")
    if derived:
        print("\n| kernel | derived | value |\n|---|---|---|")
        print("\n".join(derived))

    cm = mean.get("copy", {})
    if not ("FETCH_SIZE" in cm and "WRITE_SIZE" in cm):
        if write_traffic:
            raise SystemExit("no FETCH_SIZE and WRITE_SIZE for the calibration copy in the given runs")
        return
    ff = COPY_BYTES / 1024 / cm["FETCH_SIZE"]
    wf = COPY_BYTES / 1024 / cm["WRITE_SIZE"]
    rec = {"_about": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (separate passes "
                     "over bench.py), each scaled by what the counter reads for bench.py's 256 MiB device "
                     "copy; valid while source_digest matches the kernel's code (its .hip file and the "
                     "shared headers, comments and whitespace removed)",
           "copy_calibration": {"bytes": COPY_BYTES, "fetch_kib": cm["FETCH_SIZE"], "write_kib": cm["WRITE_SIZE"],
                                "fetch_factor": ff, "write_factor": wf}}
    print(f"\nCalibration: the {COPY_BYTES >> 20} MiB copy reads FETCH_SIZE {cm['FETCH_SIZE']:.0f} KiB and "
          f"WRITE_SIZE {cm['WRITE_SIZE']:.0f} KiB: factors {ff:.3f} and {wf:.3f}.\n")
    print("| entry | kernel | workload | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (scaled) | "
          "algorithmic bytes | ratio |\n|---|---|---|---:|---:|---:|---:|---:|")
    for key, (pat, src, wl, alg, what) in kern.items():
        m = mean.get(key, {})
        if not ("FETCH_SIZE" in m and "WRITE_SIZE" in m):
            continue
        hbm = m["FETCH_SIZE"] * 1024 * ff + m["WRITE_SIZE"] * 1024 * wf
        rec[key] = {"kernel": pat, "workload": wl, "source": src, "source_digest": kernel_digest(src),
                    "fetch_kib": m["FETCH_SIZE"], "write_kib": m["WRITE_SIZE"],
                    "bytes_per_launch": hbm, "algorithmic_bytes": alg, "algorithmic": what}
        ratio = f"{hbm / alg:.3f}" if alg else "—"
        print(f"| {key} | `{pat}` | {wl} | {m['FETCH_SIZE']:.0f} | {m['WRITE_SIZE']:.0f} | {hbm:.4g} | "
              f"{alg if alg else '—'} | {ratio} |")
    if write_traffic:
        with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as fh:
            json.dump(rec, fh, indent=1)
            fh.write("\n")


def traffic_record(kernel_key):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/traffic.json).

    Returns None when there is no record or when the kernel's code has
    changed since the counters were taken.
    """
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except OSError:
        return None
    ent = rec.get(kernel_key)
    if not ent:
        return None
    try:
        d = kernel_digest(ent["source"])
    except OSError:
        return None
    return round(ent["bytes_per_launch"]) if d == ent.get("source_digest") else None


def main():
    args = parse()
    if args.reduce_counters:
        reduce_counters(args.reduce_counters, args.write_traffic)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(every (batch, head) is independent; see the sharding notes in DESIGN.md)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import exact_io_aware_11_amd as fa
    import fa_workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    b = Buffers(torch, fa, W, dev)
    # A plain 256 MiB device-to-device copy (outside the timed region): the
    # reference against which rocprofv3's FETCH_SIZE / WRITE_SIZE counters are
    # calibrated when this script runs under the profiler.
    cal_src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
    torch.empty_like(cal_src).copy_(cal_src)
    del cal_src
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    stages = {"fwd": run_fwd, "bwd": run_bwd, "decode": run_decode}
    active = list(stages)

    log(f"warmup {args.warmup} steps ({', '.join(active)})")
    for _ in range(args.warmup):
        for name in active:
            stages[name](fa, b, stream)
    torch.cuda.synchronize()

    ev = {n: [] for n in active}
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for name in active:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            stages[name](fa, b, stream)
            e1.record()
            ev[name].append((e0, e1))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = {n: sum(a.elapsed_time(c) for a, c in ev[n]) / args.steps for n in active}
    log("per-call ms: " + ", ".join(f"{n} {ms[n]:.4f}" for n in active))

    t, dc = b.w_tr, b.w_dec
    f_fwd = fwd_flops(t.B, t.H, t.N, t.d)
    f_bwd = 2.5 * f_fwd
    dec_bytes = 2.0 * dc.B * dc.H * dc.N * dc.d * 2
    parts = {}
    roofs = []
    if "fwd" in ms:
        tf = f_fwd / (ms["fwd"] * 1e-3) / 1e12
        parts["fwd"] = {"ms": round(ms["fwd"], 4), "tflops": round(tf, 1)}
        roofs.append({"kernel": "fwd_bf16_kernel<128,causal>", "bound": "mfma", "achieved": round(tf, 1),
                      "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                      "traffic": traffic_record("fwd"), "ms": ms["fwd"],
                      "per_launch": f"{f_fwd:.4g} flop (4*B*H*N^2*d/2 at B4 H16 N2048 d128)"})
    if "bwd" in ms:
        tf = f_bwd / (ms["bwd"] * 1e-3) / 1e12
        parts["bwd"] = {"ms": round(ms["bwd"], 4), "tflops": round(tf, 1)}
        tr = [traffic_record("bwd_dkdv"), traffic_record("bwd_dq")]
        roofs.append({"kernel": "fa_bwd (bwd_prep + bwd_dkdv_kernel<128,causal> + bwd_dq_kernel<128,causal>)",
                      "bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                      "traffic": None if None in tr else sum(tr),
                      "ms": ms["bwd"], "per_launch": f"{f_bwd:.4g} flop (2.5x forward)"})
    if "decode" in ms:
        gbs = dec_bytes / (ms["decode"] * 1e-3) / 1e9
        parts["decode"] = {"ms": round(ms["decode"], 4), "GBps": round(gbs, 1), "splits": b.splits}
        roofs.append({"kernel": "fa_decode (decode_split_kernel<128> + merge)", "bound": "hbm",
                      "achieved": round(gbs, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                      "frac": round(gbs / PEAK_HBM_GBPS, 4), "traffic": traffic_record("decode"),
                      "ms": ms["decode"], "per_launch": f"{dec_bytes:.4g} B (K and V caches read once)"})
    dominant = max(roofs, key=lambda r: r["ms"])

    tr_ms = ms.get("fwd", 0.0) + ms.get("bwd", 0.0)
    tr_flops = (f_fwd if "fwd" in ms else 0.0) + (f_bwd if "bwd" in ms else 0.0)
    value = tr_flops / (tr_ms * 1e-3) / 1e12 if tr_ms > 0 else 0.0

    sweep_res = None
    if not args.no_sweep:
        log("sweep N=2K..16K")
        sweep_res = sweep(torch, fa, W, dev)

    next_rows = None
    if not args.no_next:
        log("grouped-query attention")
        next_rows = {"gqa": gqa_measure(torch, fa, W, dev)}
        log("paged KV cache")
        next_rows["paged_decode"] = paged_measure(torch, fa, dev)
        log("small-batch decode")
        next_rows["small_batch_decode"] = small_batch_decode_measure(torch, fa, W, dev)
        log("head dim 256")
        next_rows["head_dim_256"] = d256_measure(torch, fa, W, dev)
        log("fp8 forward")
        next_rows["fp8_forward"] = fp8_measure(torch, fa, W, dev)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(W)

    line = {
        "metric": "attn fwd/bwd TFLOP/s bf16 causal (N=2K–16K) + % MFMA peak; decode HBM GB/s",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "attention step: fa_fwd + fa_bwd on causal B4 H16 N2048 d128, "
                               "then fa_decode on B64 H32 L8192 d128",
                   "B": t.B, "H": t.H, "N": t.N, "d": t.d, "causal": True,
                   "decode": {"B": dc.B, "H": dc.H, "L": dc.N, "d": dc.d, "splits": b.splits}},
        "value_basis": "fwd+bwd flops / fwd+bwd event time inside the timed steps",
        "frac_mfma_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "parts": parts,
        "roofline": {k: dominant[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic")}
                    | {"kernel": dominant["kernel"]},
        "rooflines": roofs,
        "sweep": sweep_res,
        "next_rows": next_rows,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
