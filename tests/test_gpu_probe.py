"""The benchmark's probe library (libfa_probe.so) on the GPU.

* Its clock-recording instantiation of the bf16 forward must compute exactly
  what the library's fa_fwd computes (bit for bit), so that the clock the
  bench reports is that of the same kernel code.
* The MFMA and streaming-read probes run and report a plausible clock.
"""

from __future__ import annotations

import ctypes
import math
import os

import pytest
import torch

import fa_workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _probe():
    import exact_io_aware_11_amd  # noqa: F401  (torch's HIP runtime first)
    lib = ctypes.CDLL(os.path.join(ROOT, "exact_io_aware_11_amd", "libfa_probe.so"))
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.fa_probe_mfma.argtypes = [I, P, I, I, P, P, P]
    lib.fa_probe_stream_read.argtypes = [P, Z, I, P, P]
    lib.fa_probe_fwd_clock.argtypes = [P, P, P, P, P, I, I, I, F, P, P]
    return lib


def _ghz(clk):
    c = clk.view(-1, 2).double()
    return float(c[:, 0].sum() / c[:, 1].sum()) * 0.1


@pytest.mark.parametrize("B,H,N", [(1, 4, 1000), (2, 3, 2048), (1, 1, 1)])
def test_clock_forward_equals_fa_fwd(B, H, N):
    import exact_io_aware_11_amd as fa
    lib = _probe()
    d = 128
    q, k, v = W.make_custom(B, H, N, d, "bf16", seed=9500 + N, device=DEV)
    scale = 1.0 / math.sqrt(d)
    print(f"probe forward B{B} H{H} N{N}", flush=True)
    o_ref, l_ref = fa.attention(q, k, v, is_causal=True, scale=scale)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    clk = torch.zeros((2 * ((N + 127) // 128) * B * H,), dtype=torch.int64, device=DEV)
    st = lib.fa_probe_fwd_clock(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N,
                                scale, clk.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
    assert 0.3 < _ghz(clk) < 3.5


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_mfma_probe_runs(mode):
    lib = _probe()
    grid = 8
    ops = torch.ones((grid * 256 * 8 * 8,), dtype=torch.bfloat16, device=DEV)   # e4m3 code 0x80 0x3f pairs: finite
    sink = torch.empty((grid * 256,), dtype=torch.float32, device=DEV)
    clk = torch.zeros((2 * grid,), dtype=torch.int64, device=DEV)
    print(f"mfma probe mode {mode}", flush=True)
    st = lib.fa_probe_mfma(mode, ops.data_ptr(), 200, grid, sink.data_ptr(), clk.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    assert 0.3 < _ghz(clk) < 3.5
    assert lib.fa_probe_mfma(4, ops.data_ptr(), 1, grid, sink.data_ptr(), clk.data_ptr(), 0) != 0   # refused


def test_stream_read_probe_runs():
    lib = _probe()
    buf = torch.zeros((1 << 20,), dtype=torch.uint8, device=DEV)
    sink = torch.ones((16 * 256,), dtype=torch.int32, device=DEV)
    print("stream read probe", flush=True)
    assert lib.fa_probe_stream_read(buf.data_ptr(), buf.numel(), 16, sink.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    assert int(sink.abs().sum()) == 0        # XOR of zeros
    assert lib.fa_probe_stream_read(buf.data_ptr(), 15, 16, sink.data_ptr(), 0) != 0   # not a multiple of 16
