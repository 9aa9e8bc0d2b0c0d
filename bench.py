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

Every other measurement warms up for at least 50 ms, then times single calls
with HIP events until at least 20 calls and 200 ms have passed, and reports
the median and the minimum:
  * ``configs``: the five workloads at their own shapes -- the fp32 128-token
    forward (latency, us), the 16K-token forward against its target of
    <= 1.75 ms, the 4K-token backward; the 2K forward/backward and the decode
    come from the step;
  * ``sweep``: forward and backward TFLOP/s at N = 2K..16K (H=32, B=16384/N);
  * ``next_rows``: grouped-query attention, paged-cache and batch-1 decodes,
    head dim 256 (forward, backward, decode) and the fp8 forward;
  * ``ceilings``: what the chip delivers, from the probe library
    (libfa_probe.so): MFMA loops on random and constant operands and with one
    exponential per product, each with the shader clock it ran at, a streaming
    read, and the clock the library's own forward kernel runs at;
  * ``cpu_baseline``: the fp64 oracle on the host cores (bounded samples).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-sweep]
                       [--no-next] [--no-configs] [--no-ceilings] [--no-cpu-baseline]
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
PEAK_FP32_MATRIX_TFLOPS = 157.3   # MI355X dense fp32 matrix (spec), for the fp32 workload only
SPEC_CLOCK_GHZ = 2.4          # the clock the published peaks assume


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
                    help="skip the grouped-query, paged-cache, head-dim-256 and fp8 measurements")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-workload measurements")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the probe-library calibration")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed whole steps for at least this long before the warm-up steps (0: none)")
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


def timed_stats(torch, fn, min_calls=20, min_ms=200.0, max_calls=4000, warm_ms=50.0):
    """Median and minimum milliseconds of single calls of ``fn``.

    Untimed calls worth at least ``warm_ms`` come first (the clocks need tens of
    milliseconds of load to settle).  Then each call is bracketed by its own
    pair of HIP events on the current stream, in batches between host
    synchronisations, until at least ``min_calls`` calls and ``min_ms``
    milliseconds have been timed (at most ``max_calls``).
    """
    import statistics
    fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn()
    e1.record()
    torch.cuda.synchronize()
    est = max(e0.elapsed_time(e1), 1e-3)
    for _ in range(min(500, max(3, math.ceil(warm_ms / est)))):
        fn()
    torch.cuda.synchronize()
    times = []
    while len(times) < max_calls and (len(times) < min_calls or sum(times) < min_ms):
        batch = min(64, max_calls - len(times))
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(batch)]
        for a, b in evs:
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        times += [a.elapsed_time(b) for a, b in evs]
    return {"median_ms": statistics.median(times), "min_ms": min(times), "calls": len(times)}


def rate_entry(st, work, unit, peak, workload, **extra):
    """A measurement record: median and min time, the rate at both, and the
    fraction of ``peak`` at the median.  ``work`` is flops (unit TFLOP/s) or
    bytes (unit GB/s)."""
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    med = work / (st["median_ms"] * 1e-3) / scale
    best = work / (st["min_ms"] * 1e-3) / scale
    key = "tflops" if unit == "TFLOP/s" else "GBps"
    return {"workload": workload, "ms": round(st["median_ms"], 4), "ms_min": round(st["min_ms"], 4),
            "calls": st["calls"], key: round(med, 1), key + "_best": round(best, 1),
            "frac": round(med / peak, 4), **extra}


def _ok(fa, st):
    if st != fa.FA_OK:
        raise RuntimeError(fa.fa_status_string(st))


def _fwd_bwd_calls(torch, fa, q, k, v, do, causal, scale, stream):
    """Closures calling fa_fwd and fa_bwd through the C ABI on resident buffers."""
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nb = fa.fa_bwd_workspace_bytes(B, H, Hkv, N, d)
    ws = torch.empty((max(nb, 1),), dtype=torch.uint8, device=q.device)

    def f():
        _ok(fa, fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), fa.FA_BF16, lse.data_ptr(),
                          B, H, Hkv, N, d, fa.FA_BF16, int(causal), scale, stream))

    def g():
        _ok(fa, fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), fa.FA_BF16, lse.data_ptr(),
                          do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), nb,
                          B, H, Hkv, N, d, fa.FA_BF16, int(causal), scale, stream))
    return f, g


def _decode_call(torch, fa, q, kc, vc, scale, stream):
    B, H, _, d = q.shape
    Hkv, L = kc.shape[1], kc.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    nb = fa.fa_decode_workspace_bytes(B, H, Hkv, L, d, 0)
    ws = torch.empty((max(nb, 1),), dtype=torch.uint8, device=q.device)

    def f():
        _ok(fa, fa.fa_decode(q.data_ptr(), kc.data_ptr(), vc.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             ws.data_ptr(), nb, B, H, Hkv, L, d, fa.FA_BF16, 0, scale, stream))
    return f


def sweep(torch, fa, W, dev):
    """fwd and bwd TFLOP/s at N = 2K..16K, H = 32, B = 16384/N, causal bf16, d = 128."""
    out = []
    stream = torch.cuda.current_stream().cuda_stream
    for N in (2048, 4096, 8192, 16384):
        B, H, d = 16384 // N, 32, 128
        scale = 1.0 / math.sqrt(d)
        seed = 10 + int(math.log2(N // 1024))
        q, k, v, do = W.draw([(B, H, N, d)] * 4, seed, torch.bfloat16, device=dev)
        f, g = _fwd_bwd_calls(torch, fa, q, k, v, do, True, scale, stream)
        res = {"N": N, "B": B, "H": H, "d": d}
        wl = f"B{B} H{H} N{N} d{d} causal"
        f()
        for name, fn, mult in (("fwd", f, 1.0), ("bwd", g, 2.5)):
            res[name] = rate_entry(timed_stats(torch, fn), mult * fwd_flops(B, H, N, d), "TFLOP/s",
                                   PEAK_BF16_TFLOPS, wl)
        log(f"sweep N={N}: fwd {res['fwd']['tflops']} TFLOP/s, bwd {res['bwd']['tflops']} TFLOP/s")
        out.append(res)
        del q, k, v, do, f, g
        torch.cuda.empty_cache()
    return out


def configs_measure(torch, fa, W, dev):
    """The workloads at their own shapes: the fp32 128-token forward (latency),
    the 16K-token forward (target <= 1.75 ms, >= 50% of the bf16 MFMA peak) and
    the 4K-token backward (O and LSE from fa_fwd).  The 2K forward/backward and
    the 8K-cache decode are the step's own legs."""
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    w = W.WORKLOADS["fwd_fp32_b1h1n128d64"]
    q, k, v = W.make_inputs(w, dev)
    o, lse = torch.empty_like(q), torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    st = timed_stats(torch, lambda: _ok(fa, fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                                      fa.FA_FP32, lse.data_ptr(), w.B, w.H, w.H, w.N, w.d,
                                                      fa.FA_FP32, 0, w.scale, stream)), max_calls=2000)
    fl = fwd_flops(w.B, w.H, w.N, w.d, causal=False)
    out["C1"] = {"workload": "fwd fp32 B1 H1 N128 d64 non-causal", "us": round(st["median_ms"] * 1e3, 2),
                 "us_min": round(st["min_ms"] * 1e3, 2), "calls": st["calls"],
                 "tflops": round(fl / (st["median_ms"] * 1e-3) / 1e12, 3),
                 "note": "latency-bound: 4.19 MFLOP on four workgroups of 32 query rows, whose four waves take "
                         "one 32-key tile each and merge through LDS (the kernel itself takes ~6.5 us, about 2 us "
                         "of it the 64 fp32 MFMAs per wave, the rest loads, the merge and the dispatch); the fp32 "
                         f"matrix peak is {PEAK_FP32_MATRIX_TFLOPS} TFLOP/s, for information only"}
    log(f"C1 {out['C1']['workload']}: {out['C1']['us']} us")

    w = W.WORKLOADS["fwd_causal_bf16_b1h32n16384d128"]
    q, k, v = W.make_inputs(w, dev)
    f, _ = _fwd_bwd_calls(torch, fa, q, k, v, q, True, w.scale, stream)
    e = rate_entry(timed_stats(torch, f), fwd_flops(w.B, w.H, w.N, w.d), "TFLOP/s", PEAK_BF16_TFLOPS,
                   "fwd causal bf16 B1 H32 N16384 d128 (inputs N(0,1)*0.5)")
    e["target_ms"] = 1.75
    e["target_met"] = e["ms"] <= 1.75
    out["C3"] = e
    log(f"C3 {e['workload']}: {e['ms']} ms (min {e['ms_min']}), {e['tflops']} TFLOP/s")
    del q, k, v, f

    w = W.WORKLOADS["bwd_causal_bf16_b2h16n4096d128"]
    q, k, v, do = W.make_inputs(w, dev)
    f, g = _fwd_bwd_calls(torch, fa, q, k, v, do, True, w.scale, stream)
    f()
    out["C4"] = rate_entry(timed_stats(torch, g), 2.5 * fwd_flops(w.B, w.H, w.N, w.d), "TFLOP/s",
                           PEAK_BF16_TFLOPS, "bwd causal bf16 B2 H16 N4096 d128 (O, LSE from fa_fwd)")
    out["C4_fwd"] = rate_entry(timed_stats(torch, f), fwd_flops(w.B, w.H, w.N, w.d), "TFLOP/s",
                               PEAK_BF16_TFLOPS, "fwd causal bf16 B2 H16 N4096 d128")
    log(f"C4 {out['C4']['workload']}: {out['C4']['ms']} ms, {out['C4']['tflops']} TFLOP/s")
    del q, k, v, do, f, g
    torch.cuda.empty_cache()
    return out


def gqa_measure(torch, fa, W, dev):
    """Grouped-query attention (K/V heads shared by groups of query heads).

    decode: B64 H32 Hkv8 L8192 d128 (groups of 4); each cache head is read
    once per group, so the algorithmic bytes are 2*B*Hkv*L*d*2.
    fwd/bwd: B4 H16 Hkv4 N2048 d128 causal; same flops as multi-head.
    """
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    B, H, Hkv, L, d = 64, 32, 8, 8192, 128
    scale = 1.0 / math.sqrt(d)
    q, kc, vc = W.make_gqa(B, H, Hkv, 1, d, "bf16", seed=20, device=dev, Nk=L)
    out["decode"] = rate_entry(timed_stats(torch, _decode_call(torch, fa, q, kc, vc, scale, stream)),
                               2.0 * B * Hkv * L * d * 2, "GB/s", PEAK_HBM_GBPS, f"B{B} H{H} Hkv{Hkv} L{L} d{d}",
                               bound="hbm", splits=fa.fa_decode_num_splits(B, H, Hkv, L, d))
    log(f"gqa decode {out['decode']['workload']}: {out['decode']['ms']} ms, {out['decode']['GBps']} GB/s")
    del q, kc, vc

    B, H, Hkv, N = 4, 16, 4, 2048
    q, k, v, do = W.make_gqa(B, H, Hkv, N, d, "bf16", seed=21, with_dout=True, device=dev)
    f, g = _fwd_bwd_calls(torch, fa, q, k, v, do, True, scale, stream)
    f()
    for name, fn, mult in (("fwd", f, 1.0), ("bwd", g, 2.5)):
        out[name] = rate_entry(timed_stats(torch, fn), mult * fwd_flops(B, H, N, d), "TFLOP/s", PEAK_BF16_TFLOPS,
                               f"B{B} H{H} Hkv{Hkv} N{N} d{d} causal", bound="mfma")
        log(f"gqa {name} {out[name]['workload']}: {out[name]['ms']} ms, {out[name]['tflops']} TFLOP/s")
    return out


def paged_measure(torch, fa, dev):
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
            _ok(fa, fa.fa_decode_paged(q.data_ptr(), kp.data_ptr(), vp.data_ptr(), table.data_ptr(),
                                       lens.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(), nb, B, H, Hkv,
                                       pages, ps, L // ps, d, fa.FA_BF16, 0, scale, stream))
        out[name] = rate_entry(timed_stats(torch, fn), 2.0 * B * Hkv * L * d * 2, "GB/s", PEAK_HBM_GBPS,
                               f"B{B} H{H} Hkv{Hkv} L{L} d{d} page{ps}", bound="hbm")
        log(f"paged decode {out[name]['workload']}: {out[name]['ms']} ms, {out[name]['GBps']} GB/s")
        del q, kp, vp, table, lens, o, lse, ws
        torch.cuda.empty_cache()
    return out


def fp8_measure(torch, fa, W, dev):
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
            _ok(fa, fa.fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), vt8.data_ptr(), qs, ks, vs, o.data_ptr(),
                                  fa.FA_BF16, lse.data_ptr(), B, H, H, N, d, 1, scale, stream))
        out[key] = rate_entry(timed_stats(torch, f), fwd_flops(B, H, N, d), "TFLOP/s", PEAK_FP8_TFLOPS,
                              f"B{B} H{H} N{N} d{d} causal, e4m3 in, bf16 out", bound="mfma")
        log(f"fp8 fwd {out[key]['workload']}: {out[key]['ms']} ms, {out[key]['tflops']} TFLOP/s")
        del q8, k8, vt8, o, lse
    return out


def small_batch_decode_measure(torch, fa, W, dev):
    """Decode steps at batch 1 (latency-bound: a few MB of cache), with 8
    cache heads (grouped kernel) and 32 (per-head kernel), L = 4K and 16K."""
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    for key, (Hkv, L) in (("gqa_l4096", (8, 4096)), ("gqa_l16384", (8, 16384)), ("mha_l16384", (32, 16384))):
        B, H, d = 1, 32, 128
        q, kc, vc = W.make_gqa(B, H, Hkv, 1, d, "bf16", seed=61 + L // 4096 + Hkv, device=dev, Nk=L)
        st = timed_stats(torch, _decode_call(torch, fa, q, kc, vc, 1.0 / math.sqrt(d), stream), max_calls=2000)
        byt = 2.0 * B * Hkv * L * d * 2
        out[key] = {"workload": f"B{B} H{H} Hkv{Hkv} L{L} d{d}", "us": round(st["median_ms"] * 1e3, 2),
                    "us_min": round(st["min_ms"] * 1e3, 2), "calls": st["calls"],
                    "GBps": round(byt / (st["median_ms"] * 1e-3) / 1e9, 1),
                    "splits": fa.fa_decode_num_splits(B, H, Hkv, L, d)}
        log(f"small-batch decode {out[key]['workload']}: {out[key]['us']} us, {out[key]['GBps']} GB/s")
    return out


def d256_measure(torch, fa, W, dev):
    """Head dim 256: causal bf16 forward and backward at B4 H16 N4096, and
    decode at B64 H16 L4096 (multi-head) -- same flop formula / bytes as at
    d = 128."""
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    B, H, N, d = 4, 16, 4096, 256
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = W.make_custom(B, H, N, d, "bf16", seed=40, n_tensors=4, device=dev)
    f, g = _fwd_bwd_calls(torch, fa, q, k, v, do, True, scale, stream)
    f()
    for name, fn, mult in (("fwd", f, 1.0), ("bwd", g, 2.5)):
        out[name] = rate_entry(timed_stats(torch, fn), mult * fwd_flops(B, H, N, d), "TFLOP/s", PEAK_BF16_TFLOPS,
                               f"B{B} H{H} N{N} d{d} causal", bound="mfma")
        log(f"d256 {name} {out[name]['workload']}: {out[name]['ms']} ms, {out[name]['tflops']} TFLOP/s")
    del q, k, v, do, f, g

    B, H, L = 64, 16, 4096
    q, kc, vc = W.make_custom(B, H, 1, d, "bf16", seed=41, device=dev, Nk=L)
    out["decode"] = rate_entry(timed_stats(torch, _decode_call(torch, fa, q, kc, vc, scale, stream)),
                               2.0 * B * H * L * d * 2, "GB/s", PEAK_HBM_GBPS, f"B{B} H{H} L{L} d{d}", bound="hbm")
    log(f"d256 decode {out['decode']['workload']}: {out['decode']['ms']} ms, {out['decode']['GBps']} GB/s")
    return out


def ceilings(torch, dev, fwd_q=None):
    """Calibration with the probe library (outside every timed step).

    MFMA: a register-only v_mfma_f32_32x32x16_bf16 loop at two waves per SIMD
    on every CU, on random bf16 operands, on the same with one v_exp_f32 per
    product, and on constant operands; each with the shader clock the chip ran
    at (s_memtime cycles over the 100 MHz s_memrealtime, per workgroup).  HBM:
    a streaming read of 4 GiB.  Clock of the library's own forward kernel at
    B1 H32 N16384 d128 causal (its per-workgroup clock record on), and its
    MFMA utilisation at that clock.
    """
    import ctypes
    import statistics
    path = os.path.join(ROOT, "exact_io_aware_11_amd", "libfa_probe.so")
    if not os.path.exists(path):
        log(f"no {path}: ceilings skipped (build with exact_io_aware_11_amd/build.py)")
        return None
    lib = ctypes.CDLL(path)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_probe_mfma.argtypes = [I, P, I, I, P, P, P]
    lib.fa_probe_stream_read.argtypes = [P, Z, I, P, P]
    lib.fa_probe_fwd_clock.argtypes = [P, P, P, P, P, I, I, I, F, P, P]
    stream = torch.cuda.current_stream().cuda_stream
    out = {}
    grid = 512                                   # two workgroups of 4 waves per CU
    nops = grid * 256 * 8 * 8                    # 8 operand vectors of 8 bf16 per lane
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    ops_rand = torch.randn((nops,), generator=g, device=dev).to(torch.bfloat16)
    ops_const = torch.full((nops,), 1.0, dtype=torch.bfloat16, device=dev)
    sink = torch.empty((grid * 256,), dtype=torch.float32, device=dev)
    clk = torch.zeros((2 * grid,), dtype=torch.int64, device=dev)

    def clock_ghz(c):
        c = c.view(-1, 2).double()
        return float(c[:, 0].sum() / c[:, 1].sum()) * 0.1

    # random e4m3 codes (no NaN codes: drawn through the format's own cast)
    ops_fp8 = (torch.randn((nops * 2,), generator=g, device=dev) * 8).to(torch.float8_e4m3fn).view(torch.uint8)
    for mode, name, ops, iters, kdim, peak in (
            (0, "mfma_bf16_random", ops_rand, 60000, 16, PEAK_BF16_TFLOPS),
            (1, "mfma_bf16_random_exp", ops_rand, 60000, 16, PEAK_BF16_TFLOPS),
            (2, "mfma_bf16_constant", ops_const, 60000, 16, PEAK_BF16_TFLOPS),
            (3, "mfma_fp8_random", ops_fp8, 30000, 64, PEAK_FP8_TFLOPS)):
        run = lambda: lib.fa_probe_mfma(mode, ops.data_ptr(), iters, grid, sink.data_ptr(), clk.data_ptr(), stream)
        st = timed_stats(torch, run, min_calls=5, min_ms=100.0, max_calls=50, warm_ms=100.0)
        flops = grid * 4.0 * iters * 4 * 2 * 32 * 32 * kdim
        tf = flops / (st["median_ms"] * 1e-3) / 1e12
        ghz = clock_ghz(clk)
        out[name] = {"tflops": round(tf, 1), "frac_spec": round(tf / peak, 4), "clock_ghz": round(ghz, 3),
                     "ms": round(st["median_ms"], 3)}
        log(f"ceiling {name}: {tf:.1f} TFLOP/s at {ghz:.3f} GHz")

    nbytes = 4 << 30
    buf = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    rsink = torch.empty((2048 * 256,), dtype=torch.int32, device=dev)
    st = timed_stats(torch, lambda: lib.fa_probe_stream_read(buf.data_ptr(), nbytes, 2048, rsink.data_ptr(), stream),
                     min_calls=20, min_ms=100.0)
    gbs = nbytes / (st["median_ms"] * 1e-3) / 1e9
    out["stream_read"] = {"GBps": round(gbs, 1), "frac_spec": round(gbs / PEAK_HBM_GBPS, 4),
                          "bytes": nbytes, "ms": round(st["median_ms"], 3)}
    log(f"ceiling stream read: {gbs:.1f} GB/s")
    del buf, ops_rand, ops_const, ops_fp8

    if fwd_q is not None:
        q, k, v = fwd_q
        B, H, N, d = q.shape
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        fclk = torch.zeros((2 * ((N + 127) // 128) * B * H,), dtype=torch.int64, device=dev)
        scale = 1.0 / math.sqrt(d)
        run = lambda: lib.fa_probe_fwd_clock(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                             lse.data_ptr(), B, H, N, scale, fclk.data_ptr(), stream)
        st = timed_stats(torch, run)
        ghz = clock_ghz(fclk)
        tf = fwd_flops(B, H, N, d) / (st["median_ms"] * 1e-3) / 1e12
        at_clock = PEAK_BF16_TFLOPS * ghz / SPEC_CLOCK_GHZ
        out["fwd_clock"] = {"workload": f"fwd causal bf16 B{B} H{H} N{N} d{d}", "tflops": round(tf, 1),
                            "clock_ghz": round(ghz, 3), "peak_at_clock": round(at_clock, 1),
                            "mfma_util_at_clock": round(tf / at_clock, 4)}
        log(f"forward clock: {ghz:.3f} GHz, {tf:.1f} TFLOP/s, {100 * tf / at_clock:.1f}% of the peak at that clock")
    return out


def annotate_ceilings(ceil, configs, sweep_res, next_rows):
    """Add ``frac_of_measured_ceiling`` to every rate record: bf16 forwards
    against the MFMA + exponential loop, bf16 backwards against the MFMA-only
    loop, the fp8 forward against the fp8 loop, decodes against the streaming
    read."""
    def ref(kind):
        key = {"fwd": "mfma_bf16_random_exp", "bwd": "mfma_bf16_random", "fp8": "mfma_fp8_random",
               "hbm": "stream_read"}[kind]
        e = ceil.get(key) or {}
        return e.get("GBps") if kind == "hbm" else e.get("tflops")

    def mark(rec, kind):
        r = ref(kind)
        val = rec.get("GBps") if kind == "hbm" else rec.get("tflops")
        if rec is not None and r and val:
            rec["frac_of_measured_ceiling"] = round(val / r, 4)

    for s_ in sweep_res or []:
        mark(s_["fwd"], "fwd")
        mark(s_["bwd"], "bwd")
    if configs:
        mark(configs.get("C3", {}), "fwd")
        mark(configs.get("C4", {}), "bwd")
        mark(configs.get("C4_fwd", {}), "fwd")
    if next_rows:
        for grp, recs in next_rows.items():
            for name, rec in recs.items():
                if grp == "fp8_forward":
                    mark(rec, "fp8")
                elif "GBps" in rec and "tflops" not in rec:
                    mark(rec, "hbm")
                elif name in ("fwd", "bwd"):
                    mark(rec, name)


def host_info():
    """CPU model, core counts and the BLAS thread count the oracle runs with."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=None)
    except Exception:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "blas_threads": threads}


def cpu_baseline(W, c3_inputs=None, c5_inputs=None, c5_slices=8):
    """The fp64 oracle, as it stands, on the host cores (about 20-30 s in all).

    Every call materialises the full N x N scores (the oracle's definition), so
    rates use the same causal flop count as the GPU.
      C1: ref_fwd on the fp32 128-token head, on all cores and on one.
      C2: ref_fwd and ref_bwd over the whole 2K workload (64 heads); the
          headline ``value`` is its fwd+bwd TFLOP/s.
      C4: ref_fwd and ref_bwd over the whole 4K backward workload (32 heads).
      C3: the parity check's 64 sampled rows for all 32 heads (ref_fwd_rows),
          and one whole head, reported times 32 as *extrapolated*.
      C5: ref_decode on ``c5_slices`` batch slices of the 8K cache (read back
          from the device), reported times 64 / c5_slices as *extrapolated*.
    """
    import numpy as np
    import torch

    from oracle import ref_bwd, ref_decode, ref_fwd, ref_fwd_rows

    def to64(x):
        return x.float().cpu().numpy().astype(np.float64)

    def secs(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    def per_call(fn, min_s=0.3):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            if time.perf_counter() - t0 >= min_s:
                return (time.perf_counter() - t0) / n

    info = host_info()
    res = {}
    t_all = time.perf_counter()

    w = W.WORKLOADS["fwd_fp32_b1h1n128d64"]
    q, k, v = (to64(x) for x in W.make_inputs(w, "cpu"))
    c1 = {"all_cores_us": round(1e6 * per_call(lambda: ref_fwd(q, k, v, False, w.scale)), 1)}
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(1):
            c1["one_core_us"] = round(1e6 * per_call(lambda: ref_fwd(q, k, v, False, w.scale)), 1)
    except ImportError:
        c1["one_core_us"] = None
    res["C1"] = c1
    log(f"cpu oracle C1: {c1}")

    for key, name in (("C2", "fwd_causal_bf16_b4h16n2048d128"), ("C4", "bwd_causal_bf16_b2h16n4096d128")):
        w = W.WORKLOADS[name]
        q, k, v, do = (to64(x) for x in W.make_inputs(w, "cpu", with_dout=True))
        tf = secs(lambda: ref_fwd(q, k, v, True, w.scale))
        tb = secs(lambda: ref_bwd(q, k, v, do, True, w.scale))
        fl = fwd_flops(w.B, w.H, w.N, w.d)
        res[key] = {"workload": f"B{w.B} H{w.H} N{w.N} d{w.d} causal", "fwd_s": round(tf, 3), "bwd_s": round(tb, 3),
                    "fwd_tflops": round(fl / tf / 1e12, 5), "fwd_bwd_tflops": round(3.5 * fl / (tf + tb) / 1e12, 5)}
        log(f"cpu oracle {key}: {res[key]}")
        del q, k, v, do

    if c3_inputs is not None:
        w = W.WORKLOADS["fwd_causal_bf16_b1h32n16384d128"]
        q, k, v = (to64(x) for x in c3_inputs)
        rows = W.sample_rows(w.N, w.extra["sample_rows"], w.extra["row_seed"])
        tr = secs(lambda: ref_fwd_rows(q, k, v, True, w.scale, rows))
        th = secs(lambda: ref_fwd(q[:, :1], k[:, :1], v[:, :1], True, w.scale))
        fl = fwd_flops(w.B, w.H, w.N, w.d)
        res["C3"] = {"workload": f"B{w.B} H{w.H} N{w.N} d{w.d} causal", "rows_check_s": round(tr, 3),
                     "rows": len(rows), "one_head_s": round(th, 3), "whole_s_extrapolated": round(32 * th, 2),
                     "fwd_tflops_extrapolated": round(fl / (32 * th) / 1e12, 5),
                     "note": "whole-workload time extrapolated from one head x 32"}
        log(f"cpu oracle C3: {res['C3']}")
        del q, k, v

    if c5_inputs is not None:
        w = W.WORKLOADS["decode_bf16_b64h32l8192d128"]
        qd, kc, vc = c5_inputs
        n = min(c5_slices, w.B)
        t = 0.0
        for bi in range(n):
            t += secs(lambda: ref_decode(to64(qd[bi:bi + 1]), to64(kc[bi:bi + 1]), to64(vc[bi:bi + 1]), w.scale))
        whole = t * w.B / n
        byt = 2.0 * w.B * w.H * w.N * w.d * 2
        res["C5"] = {"workload": f"B{w.B} H{w.H} L{w.N} d{w.d}", "slices_timed": n, "slices_s": round(t, 3),
                     "whole_s_extrapolated": round(whole, 2), "GBps_extrapolated": round(byt / whole / 1e9, 3),
                     "note": f"per batch slice (device read-back, fp64 widening, ref_decode), "
                             f"{n} of {w.B} slices timed and scaled"}
        log(f"cpu oracle C5: {res['C5']}")

    total = time.perf_counter() - t_all
    c2 = res["C2"]
    return {
        "value": c2["fwd_bwd_tflops"],
        "unit": "TFLOP/s",
        "cores": info["blas_threads"] or info["affinity_cores"],
        "kind": "oracle",
        "sample": "fp64 oracle (full N x N scores): ref_fwd + ref_bwd once over the whole B4 H16 N2048 d128 causal "
                  "workload (the headline value, counted with the GPU's causal flops); per-workload figures in "
                  "configs (C3 and C5 partly extrapolated, as labelled)",
        "seconds": round(total, 2),
        **info,
        "configs": res,
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
        "bwd_dkdv": ("bwd_dkdv_kernel", "fa_bwd.hip", "B4 H16 N2048 d128 causal", 6 * t + 2 * r,
                     "read Q, K, V, dO, LSE, D; write dK, dV"),
        "bwd_dq": ("bwd_dq_kernel", "fa_bwd.hip", "B4 H16 N2048 d128 causal", 6 * t + 3 * r,
                   "read Q, K, V, dO, O, LSE; write dQ, D, LSE log2 e"),
        "decode": ("decode_split_kernel", "fa_decode.hip", "B64 H32 L8192 d128",
                   2 * Bd * Hd * L * d * 2, "read the K and V caches"),
        "decode_merge": ("decode_merge_kernel", "fa_decode.hip", "B64 H32 L8192 d128", None,
                         "read the split partials; write O, LSE"),
    }


def kernel_digest(src, csrc=None):
    """SHA-256 of what a kernel is compiled from: its .hip file (with the
    forward's kernel header) and the two shared headers, with comments and
    whitespace removed (so a comment edit
    keeps a traffic record valid, while any code change in the file or the
    headers invalidates it)."""
    import hashlib
    import re
    csrc = csrc or os.path.join(ROOT, "exact_io_aware_11_amd", "csrc")
    h = hashlib.sha256()
    extra = ("fa_fwd_kernel.hpp",) if src == "fa_fwd.hip" else ()
    for name in (src,) + extra + ("fa_common.hpp", "fa_internal.hpp"):
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

    # The chip reaches the timed loop at a lower clock when only a few steps
    # precede it: measured on MI355X with 20 timed steps, 5 warm-up steps gave
    # 650-664 TFLOP/s, 20 gave 683-686 and 50 gave 701.  So before the W warm-up
    # steps, whole steps run untimed (each synchronised) until --settle-ms of
    # wall time have passed; the timed region is still exactly K steps.
    settle_steps, t_s = 0, time.perf_counter()
    while (time.perf_counter() - t_s) * 1e3 < args.settle_ms:
        for name in active:
            stages[name](fa, b, stream)
        torch.cuda.synchronize()
        settle_steps += 1
    settle_ms = (time.perf_counter() - t_s) * 1e3
    log(f"settle {settle_steps} steps ({settle_ms:.0f} ms)")
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
    import statistics
    per = {n: [a.elapsed_time(c) for a, c in ev[n]] for n in active}
    ms = {n: sum(per[n]) / args.steps for n in active}
    med = {n: statistics.median(per[n]) for n in active}
    mins = {n: min(per[n]) for n in active}
    log("per-call ms: " + ", ".join(f"{n} {ms[n]:.4f}" for n in active))

    t, dc = b.w_tr, b.w_dec
    f_fwd = fwd_flops(t.B, t.H, t.N, t.d)
    f_bwd = 2.5 * f_fwd
    dec_bytes = 2.0 * dc.B * dc.H * dc.N * dc.d * 2
    parts = {}
    roofs = []
    if "fwd" in ms:
        tf = f_fwd / (ms["fwd"] * 1e-3) / 1e12
        parts["fwd"] = {"ms": round(ms["fwd"], 4), "ms_median": round(med["fwd"], 4), "ms_min": round(mins["fwd"], 4),
                        "tflops": round(tf, 1)}
        roofs.append({"kernel": "fwd_bf16_kernel<128,causal>", "bound": "mfma", "achieved": round(tf, 1),
                      "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                      "traffic": traffic_record("fwd"), "ms": ms["fwd"],
                      "per_launch": f"{f_fwd:.4g} flop (4*B*H*N^2*d/2 at B4 H16 N2048 d128)"})
    if "bwd" in ms:
        tf = f_bwd / (ms["bwd"] * 1e-3) / 1e12
        parts["bwd"] = {"ms": round(ms["bwd"], 4), "ms_median": round(med["bwd"], 4), "ms_min": round(mins["bwd"], 4),
                        "tflops": round(tf, 1)}
        tr = [traffic_record("bwd_dkdv"), traffic_record("bwd_dq")]
        roofs.append({"kernel": "fa_bwd (bwd_dq_kernel<128,causal> + bwd_dkdv_kernel<128,causal>)",
                      "bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                      "traffic": None if None in tr else sum(tr),
                      "ms": ms["bwd"], "per_launch": f"{f_bwd:.4g} flop (2.5x forward)"})
    if "decode" in ms:
        gbs = dec_bytes / (ms["decode"] * 1e-3) / 1e9
        parts["decode"] = {"ms": round(ms["decode"], 4), "ms_median": round(med["decode"], 4),
                           "ms_min": round(mins["decode"], 4), "GBps": round(gbs, 1), "splits": b.splits}
        roofs.append({"kernel": "fa_decode (decode_split_kernel<128> + merge)", "bound": "hbm",
                      "achieved": round(gbs, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                      "frac": round(gbs / PEAK_HBM_GBPS, 4), "traffic": traffic_record("decode"),
                      "ms": ms["decode"], "per_launch": f"{dec_bytes:.4g} B (K and V caches read once)"})
    dominant = max(roofs, key=lambda r: r["ms"])

    tr_ms = ms.get("fwd", 0.0) + ms.get("bwd", 0.0)
    tr_flops = (f_fwd if "fwd" in ms else 0.0) + (f_bwd if "bwd" in ms else 0.0)
    value = tr_flops / (tr_ms * 1e-3) / 1e12 if tr_ms > 0 else 0.0

    configs = None
    if not args.no_configs:
        log("workloads at their own shapes")
        configs = configs_measure(torch, fa, W, dev)

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

    c3_inputs = None
    if not (args.no_ceilings and args.no_cpu_baseline):
        c3_inputs = W.make_inputs(W.WORKLOADS["fwd_causal_bf16_b1h32n16384d128"], dev)
    ceil = None
    if not args.no_ceilings:
        log("ceilings (probe library)")
        ceil = ceilings(torch, dev, fwd_q=c3_inputs)
        if ceil:
            for r in roofs:
                ref = ceil.get("stream_read", {}).get("GBps") if r["bound"] == "hbm" else \
                    ceil.get("mfma_bf16_random_exp" if r["kernel"].startswith("fwd") else "mfma_bf16_random",
                             {}).get("tflops")
                if ref:
                    r["frac_of_measured_ceiling"] = round(r["achieved"] / ref, 4)

    if ceil:
        annotate_ceilings(ceil, configs, sweep_res, next_rows)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(W, c3_inputs=c3_inputs, c5_inputs=(b.dq_in, b.kc, b.vc))

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
                    | {"kernel": dominant["kernel"]}
                    | ({"frac_of_measured_ceiling": dominant["frac_of_measured_ceiling"]}
                       if "frac_of_measured_ceiling" in dominant else {}),
        "rooflines": roofs,
        "timing": "step: untimed settle steps for >= settle_ms, then the warm-up steps, then per-call HIP events "
                  "over the timed steps (mean; median and min in parts); every other figure: >= 50 ms warm-up, then "
                  ">= 20 single calls and >= 200 ms, median (min as *_best)",
        "settle": {"steps": settle_steps, "ms": round(settle_ms, 1)},
        "configs": configs,
        "sweep": sweep_res,
        "next_rows": next_rows,
        "ceilings": ceil,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
