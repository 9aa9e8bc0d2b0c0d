"""Host-only checks of the C ABI: the library loads, exports every function
``include/fa.h`` declares, sizes workspaces, and rejects every invalid call
with its status code before anything is enqueued.

No kernel is launched here.  The fake device "pointers" are plain integers
that every tested call rejects during validation, so they are never touched.
"""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import exact_io_aware_11_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

A = 1 << 20          # an aligned fake address (never dereferenced)
MIS = A + 4          # a misaligned one


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted([
        "fa_bwd", "fa_bwd_workspace_bytes", "fa_decode", "fa_decode_noalloc", "fa_decode_num_splits",
        "fa_decode_paged",
        "fa_decode_workspace_bytes", "fa_fwd", "fa_fwd_fp8", "fa_status_string"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fa.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_single_hip_runtime_in_process():
    # importing the binding must not map a second libamdhip64 next to torch's
    import subprocess
    import sys
    code = ("import exact_io_aware_11_amd, torch; "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    libs = eval(out.stdout.strip().splitlines()[-1])
    assert len(libs) == 1, libs


def test_status_strings():
    for s in range(8):
        assert fa.fa_status_string(s).startswith("FA_")
    assert "FA_NOALLOC_SCRATCH_BYTES" in fa.fa_status_string(fa.FA_ERR_SCRATCH_LIMIT)
    assert "unknown" in fa.fa_status_string(99)


def fwd(**kw):
    args = dict(q=A, k=A, v=A, o=A, o_dtype=fa.FA_BF16, lse=A, B=1, H=4, Hkv=None, N=16, d=64,
                in_dtype=fa.FA_BF16, causal=0, scale=0.125)
    args.update(kw)
    hkv = args["H"] if args["Hkv"] is None else args["Hkv"]
    return fa.fa_fwd(args["q"], args["k"], args["v"], args["o"], args["o_dtype"], args["lse"],
                     args["B"], args["H"], hkv, args["N"], args["d"], args["in_dtype"], args["causal"],
                     args["scale"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_NULL),
    (dict(k=0), fa.FA_ERR_NULL),
    (dict(v=0), fa.FA_ERR_NULL),
    (dict(o=0), fa.FA_ERR_NULL),
    (dict(lse=0), fa.FA_ERR_NULL),
    (dict(B=0), fa.FA_ERR_ARG),
    (dict(H=-1), fa.FA_ERR_ARG),
    (dict(N=0), fa.FA_ERR_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_ARG),
    (dict(scale=0.0), fa.FA_ERR_ARG),
    (dict(scale=-0.5), fa.FA_ERR_ARG),
    (dict(B=1 << 16, H=1 << 16, N=16), fa.FA_ERR_ARG),
    (dict(Hkv=3), fa.FA_ERR_ARG),        # 3 K/V heads do not divide 4 query heads
    (dict(Hkv=0), fa.FA_ERR_ARG),
    (dict(Hkv=8), fa.FA_ERR_ARG),        # more K/V heads than query heads
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=512), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256, in_dtype=fa.FA_FP32, o_dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),   # d = 256: bf16 only
    (dict(in_dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(o_dtype=5), fa.FA_ERR_UNSUPPORTED),
    (dict(in_dtype=fa.FA_FP32, o_dtype=fa.FA_BF16), fa.FA_ERR_UNSUPPORTED),
    (dict(N=1 << 24, d=128), fa.FA_ERR_UNSUPPORTED),     # one bf16 head of 2^32 bytes
    (dict(q=MIS), fa.FA_ERR_ALIGN),
    (dict(o=MIS), fa.FA_ERR_ALIGN),
    (dict(lse=MIS), fa.FA_ERR_ALIGN),
])
def test_fwd_rejects(kw, status):
    assert fwd(**kw) == status


def fwd8(**kw):
    args = dict(q=A, k=A, vt=A, qs=1.0, ks=1.0, vs=1.0, o=A, o_dtype=fa.FA_BF16, lse=A, B=1, H=4, Hkv=2, N=128,
                d=128, causal=1, scale=0.125)
    args.update(kw)
    return fa.fa_fwd_fp8(args["q"], args["k"], args["vt"], args["qs"], args["ks"], args["vs"], args["o"],
                         args["o_dtype"], args["lse"], args["B"], args["H"], args["Hkv"], args["N"], args["d"],
                         args["causal"], args["scale"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_NULL),
    (dict(vt=0), fa.FA_ERR_NULL),
    (dict(lse=0), fa.FA_ERR_NULL),
    (dict(Hkv=3), fa.FA_ERR_ARG),
    (dict(B=0), fa.FA_ERR_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_ARG),
    (dict(qs=0.0), fa.FA_ERR_ARG),
    (dict(ks=-1.0), fa.FA_ERR_ARG),
    (dict(vs=float("nan")), fa.FA_ERR_ARG),
    (dict(N=0), fa.FA_ERR_ARG),
    (dict(N=1 << 25, d=128), fa.FA_ERR_UNSUPPORTED),   # one head of 2^32 bytes or more
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(o_dtype=5), fa.FA_ERR_UNSUPPORTED),
    (dict(vt=MIS), fa.FA_ERR_ALIGN),
    (dict(o=MIS), fa.FA_ERR_ALIGN),
])
def test_fwd_fp8_rejects(kw, status):
    assert fwd8(**kw) == status


def bwd(ws_bytes=None, **kw):
    B, H, N, d = kw.get("B", 1), kw.get("H", 4), kw.get("N", 16), kw.get("d", 64)
    need = fa.fa_bwd_workspace_bytes(B, H, kw.get("Hkv", 2), N, d)
    args = dict(q=A, k=A, v=A, o=A, o_dtype=fa.FA_BF16, lse=A, dout=A, dq=A, dk=A, dv=A, ws=A,
                B=B, H=H, Hkv=2, N=N, d=d, in_dtype=fa.FA_BF16, causal=1, scale=0.125)
    args.update(kw)
    return fa.fa_bwd(args["q"], args["k"], args["v"], args["o"], args["o_dtype"], args["lse"],
                     args["dout"], args["dq"], args["dk"], args["dv"], args["ws"],
                     need if ws_bytes is None else ws_bytes, args["B"], args["H"], args["Hkv"], args["N"],
                     args["d"], args["in_dtype"], args["causal"], args["scale"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(dout=0), fa.FA_ERR_NULL),
    (dict(Hkv=3), fa.FA_ERR_ARG),
    (dict(dq=0), fa.FA_ERR_NULL),
    (dict(lse=0), fa.FA_ERR_NULL),
    (dict(N=0), fa.FA_ERR_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_ARG),
    (dict(in_dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=512), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256, in_dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(N=1 << 23, d=256), fa.FA_ERR_UNSUPPORTED),     # one bf16 head of 2^32 bytes
    (dict(o_dtype=3), fa.FA_ERR_UNSUPPORTED),
    (dict(N=1 << 24, d=128), fa.FA_ERR_UNSUPPORTED),
    (dict(dk=MIS), fa.FA_ERR_ALIGN),
    (dict(ws=0), fa.FA_ERR_WORKSPACE),
    (dict(ws=MIS), fa.FA_ERR_ALIGN),
])
def test_bwd_rejects(kw, status):
    assert bwd(**kw) == status


def test_bwd_rejects_small_workspace():
    need = fa.fa_bwd_workspace_bytes(1, 4, 2, 16, 64)
    assert bwd(ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE
    # the fp32 row statistic alone is not enough when the grouped-head split is taken
    assert bwd(ws_bytes=256) == fa.FA_ERR_WORKSPACE


def test_bwd_workspace_size():
    # two fp32 row statistics per query row, D = rowsum(dO * O) and LSE log2 e:
    # O(N), no N^2 term
    B, H, N, d = 2, 16, 4096, 128
    assert fa.fa_bwd_workspace_bytes(B, H, H, N, d) == 2 * B * H * N * 4
    assert fa.fa_bwd_workspace_bytes(1, 3, 3, 5, 64) == 2 * 256      # each padded to 256 bytes
    assert fa.fa_bwd_workspace_bytes(0, 1, 1, 1, 64) == 0
    assert fa.fa_bwd_workspace_bytes(1, 4, 3, 16, 64) == 0           # Hkv must divide H


@pytest.mark.parametrize("B,H,Hkv,N,s", [
    (4, 16, 4, 2048, 2),         # 16 key tiles x 16 K/V heads = 256 pairs; 2 groups of 2 -> 512
    (4, 32, 4, 2048, 4),         # 256 pairs, G = 8: 2 groups of 4 -> 512
    (2, 32, 4, 2048, 2),         # 128 pairs, G = 8: 4 groups of 2 -> 512
    (1, 32, 1, 2048, 1),         # MQA, 16 pairs: even single heads give only 512
    (4, 32, 8, 2048, 0),         # 512 pairs: enough workgroups, sum in registers
    (64, 16, 8, 256, 0),         # 2 key tiles x 512 = 1024
    (63, 16, 8, 128, 1),         # 1 key tile x 504, G = 2: single heads
    (64, 16, 8, 128, 0),         # 1 key tile x 512
    (21, 16, 8, 384, 1),         # 3 key tiles x 168 = 504
    (21, 16, 8, 385, 0),         # ragged: 4 key tiles x 168 = 672
    (4, 16, 16, 2048, 0),        # no grouping: never split
])
def test_bwd_workspace_grouped_split(B, H, Hkv, N, s):
    # the grouped-head split (s query heads per workgroup) adds fp32 partial
    # dK and dV, [B*H/s, N, d] each; s is the largest divisor of G below G
    # that reaches 512 workgroups, else 1
    d = 64
    G, pairs = H // Hkv, -(-N // 128) * B * Hkv
    if Hkv == H or pairs >= 512:
        assert s == 0
    else:
        assert s == next((t for t in range(G // 2, 1, -1) if G % t == 0 and pairs * (G // t) >= 512), 1)
    rows = 2 * ((B * H * N * 4 + 255) // 256 * 256)
    want = rows + (2 * (B * H // s) * N * d * 4 if s else 0)
    assert fa.fa_bwd_workspace_bytes(B, H, Hkv, N, d) == want


def dec(ws_bytes=None, **kw):
    B, H, L, d, s = kw.get("B", 2), kw.get("H", 2), kw.get("L", 100), kw.get("d", 128), kw.get("splits", 0)
    need = fa.fa_decode_workspace_bytes(B, H, 1, L, d, max(s, 0))
    args = dict(q=A, k=A, v=A, o=A, lse=A, ws=A, B=B, H=H, Hkv=1, L=L, d=d, dtype=fa.FA_BF16,
                splits=s, scale=0.1)
    args.update(kw)
    return fa.fa_decode(args["q"], args["k"], args["v"], args["o"], args["lse"], args["ws"],
                        need if ws_bytes is None else ws_bytes, args["B"], args["H"], args["Hkv"],
                        args["L"], args["d"], args["dtype"], args["splits"], args["scale"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_NULL),
    (dict(k=0), fa.FA_ERR_NULL),
    (dict(o=0), fa.FA_ERR_NULL),
    (dict(L=0), fa.FA_ERR_ARG),
    (dict(Hkv=3), fa.FA_ERR_ARG),
    (dict(splits=-1), fa.FA_ERR_ARG),
    (dict(splits=101), fa.FA_ERR_ARG),
    (dict(scale=-1.0), fa.FA_ERR_ARG),
    (dict(dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(d=512), fa.FA_ERR_UNSUPPORTED),
    (dict(v=MIS), fa.FA_ERR_ALIGN),
    (dict(lse=MIS), fa.FA_ERR_ALIGN),
    (dict(ws=0), fa.FA_ERR_WORKSPACE),
])
def test_decode_rejects(kw, status):
    assert dec(**kw) == status


def test_decode_rejects_small_workspace():
    need = fa.fa_decode_workspace_bytes(2, 2, 1, 100, 128, 4)
    assert dec(ws_bytes=need - 1, splits=4) == fa.FA_ERR_WORKSPACE


def dec_noalloc(**kw):
    args = dict(q=A, k=A, v=A, o=A, lse=A, B=2, H=2, Hkv=1, L=100, d=128, dtype=fa.FA_BF16, splits=0, scale=0.1)
    args.update(kw)
    return fa.fa_decode_noalloc(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"], args["H"],
                                args["Hkv"], args["L"], args["d"], args["dtype"], args["splits"], args["scale"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(q=0), fa.FA_ERR_NULL),
    (dict(v=0), fa.FA_ERR_NULL),
    (dict(L=0), fa.FA_ERR_ARG),
    (dict(Hkv=3), fa.FA_ERR_ARG),
    (dict(splits=101), fa.FA_ERR_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_ARG),
    (dict(dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(o=MIS), fa.FA_ERR_ALIGN),
    # partials of B*H*S*(d+1) floats beyond the 16 MiB static array: rejected
    # before anything touches the device
    (dict(B=64, H=32, Hkv=32, L=8192, splits=32), fa.FA_ERR_SCRATCH_LIMIT),
    (dict(B=1, H=64, Hkv=64, L=1 << 20, d=256, splits=256), fa.FA_ERR_SCRATCH_LIMIT),
])
def test_decode_noalloc_rejects(kw, status):
    assert dec_noalloc(**kw) == status


def test_decode_noalloc_limit_matches_the_workspace_size():
    # every call whose workspace fits the static array is accepted by the size
    # check: with num_splits = S the scratch need equals fa_decode's workspace
    cap = fa.FA_NOALLOC_SCRATCH_BYTES
    assert fa.fa_decode_workspace_bytes(64, 32, 32, 8192, 128, 32) > cap
    assert fa.fa_decode_workspace_bytes(64, 32, 32, 8192, 128, 8) <= cap


def test_decode_split_plan():
    # the automatic split count never exceeds L and never leaves a chunk empty
    for (B, H, L) in [(64, 32, 8192), (1, 1, 1), (1, 32, 16384), (2, 3, 700), (1, 1, 513)]:
        s = fa.fa_decode_num_splits(B, H, H, L, 128)
        assert 1 <= s <= L
        chunk = -(-L // s)
        assert (s - 1) * chunk < L
    # a workspace holds d + 1 floats per (b, h, split)
    s = fa.fa_decode_num_splits(64, 32, 32, 8192, 128)
    parts = 64 * 32 * s
    assert fa.fa_decode_workspace_bytes(64, 32, 32, 8192, 128, 0) == ((parts * 128 * 4 + 255) // 256) * 256 + parts * 4
    # an invalid grouping sizes nothing
    assert fa.fa_decode_workspace_bytes(64, 32, 5, 8192, 128, 0) == 0


def test_decode_split_plan_grouped():
    # grouped path (2 <= H/Hkv <= 32): splits sized by the B*Hkv units
    for (B, H, Hkv, L) in [(64, 32, 8, 8192), (1, 32, 1, 100), (2, 8, 2, 255), (4, 6, 3, 1)]:
        s = fa.fa_decode_num_splits(B, H, Hkv, L, 128)
        assert 1 <= s <= L
        chunk = -(-L // s)
        assert (s - 1) * chunk < L
        # num_splits = 0 sizes room for both calls' automatic plans: at least
        # fa_decode's, and exactly some split count's layout
        auto = fa.fa_decode_workspace_bytes(B, H, Hkv, L, 128, 0)
        assert auto >= fa.fa_decode_workspace_bytes(B, H, Hkv, L, 128, s)
        assert any(auto == ((B * H * t * 128 * 4 + 255) // 256) * 256 + B * H * t * 4 for t in range(1, 257))
    # small-group kernel (groups of 2 and 3; of 4 from 64 (batch, cache head)
    # pairs): about 512 workgroups, chunks of 256 keys or more, at most 32
    assert fa.fa_decode_num_splits(64, 32, 8, 8192, 128) == 1
    # the paged call makes the same choice, and the automatic workspace is
    # exactly that plan's
    assert fa.fa_decode_workspace_bytes(64, 32, 8, 8192, 128, 0) == \
        fa.fa_decode_workspace_bytes(64, 32, 8, 8192, 128, 1)
    assert fa.fa_decode_num_splits(16, 32, 8, 8192, 128) == 4
    assert fa.fa_decode_num_splits(4, 24, 8, 8192, 128) == 16
    assert fa.fa_decode_num_splits(1, 32, 16, 8192, 128) == 32
    assert fa.fa_decode_num_splits(1, 32, 16, 1000, 128) == 4
    # MFMA grouped kernel, batch 1, 8 cache heads (groups of 4): chunks down
    # to 64 keys, at most 64 of them
    assert fa.fa_decode_num_splits(1, 32, 8, 4096, 128) == 64
    assert fa.fa_decode_num_splits(1, 32, 8, 16384, 128) == 64
    assert fa.fa_decode_num_splits(1, 32, 8, 1000, 128) == 16
    # the per-head path keeps chunks of 512 keys or more
    assert fa.fa_decode_num_splits(1, 32, 32, 16384, 128) == 32


def test_decode_rejects_cache_head_of_4gib():
    assert dec(L=1 << 24, d=128) == fa.FA_ERR_UNSUPPORTED



def paged(ws_bytes=None, **kw):
    args = dict(q=A, kp=A, vp=A, bt=A, sl=A, o=A, lse=A, ws=A, B=2, H=8, Hkv=2, num_pages=10, ps=64,
                max_pages=4, d=128, dtype=fa.FA_BF16, splits=0, scale=0.1)
    args.update(kw)
    need = fa.fa_decode_workspace_bytes(args["B"], args["H"], args["Hkv"], max(args["max_pages"], 1) *
                                        max(args["ps"], 1), args["d"], max(args["splits"], 0))
    return fa.fa_decode_paged(args["q"], args["kp"], args["vp"], args["bt"], args["sl"], args["o"], args["lse"],
                              args["ws"], need if ws_bytes is None else ws_bytes, args["B"], args["H"],
                              args["Hkv"], args["num_pages"], args["ps"], args["max_pages"], args["d"],
                              args["dtype"], args["splits"], args["scale"], 0)


@pytest.mark.parametrize("kw,status", [
    (dict(bt=0), fa.FA_ERR_NULL),
    (dict(sl=0), fa.FA_ERR_NULL),
    (dict(kp=0), fa.FA_ERR_NULL),
    (dict(ps=48), fa.FA_ERR_ARG),            # not a power of two
    (dict(ps=16), fa.FA_ERR_ARG),            # below one 32-key tile
    (dict(ps=1 << 17), fa.FA_ERR_ARG),
    (dict(num_pages=0), fa.FA_ERR_ARG),
    (dict(max_pages=0), fa.FA_ERR_ARG),
    (dict(Hkv=3), fa.FA_ERR_ARG),
    (dict(splits=-1), fa.FA_ERR_ARG),
    (dict(splits=4 * 64 + 1), fa.FA_ERR_ARG),
    (dict(scale=0.0), fa.FA_ERR_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=fa.FA_FP32), fa.FA_ERR_UNSUPPORTED),
    (dict(kp=MIS), fa.FA_ERR_ALIGN),
    (dict(bt=A + 2), fa.FA_ERR_ALIGN),
    (dict(ws=0), fa.FA_ERR_WORKSPACE),
])
def test_decode_paged_rejects(kw, status):
    assert paged(**kw) == status


def test_decode_paged_rejects_small_workspace():
    need = fa.fa_decode_workspace_bytes(2, 8, 2, 4 * 64, 128, 0)
    assert paged(ws_bytes=need - 1) == fa.FA_ERR_WORKSPACE



def test_builder_loads_without_importing_the_package():
    # the build must work on a fresh checkout, where importing the package
    # (which loads libfa.so) is impossible
    import subprocess
    import sys
    code = ("import sys, __graft_entry__ as g; b = g.load_builder(); "
            "assert callable(b.build); print('exact_io_aware_11_amd' in sys.modules)")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "False"
