"""Seeded synthetic inputs for the attention workloads (shared by tests and bench).

This module only draws random numbers and names shapes.  It holds none of the
attention arithmetic, so both the HIP path's tests and the fp64 oracle can use
it without sharing any of the method.

Recipe (the same for every workload): one ``torch.Generator`` per workload,
seeded with the workload's seed; tensors drawn in the order Q, K, V, dO, each
as ``torch.randn(shape, dtype=float32)``, multiplied by ``sigma`` and then cast
with ``.to(dtype)`` (round-to-nearest-even for bf16).  Small workloads are drawn
on the CPU; the two large ones (16K-token prefill, 8K-token KV cache over 2048
heads) are drawn on the device with a seeded device generator, which avoids
billions of CPU draws; tests read the device values back for the oracle.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "fwd", "bwd" or "decode"
    B: int
    H: int
    N: int               # query/key length; for decode: the KV-cache length L
    d: int
    dtype: str           # "fp32" or "bf16"
    causal: bool
    seed: int
    sigma: float = 1.0
    device_gen: bool = False
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "fp32" else torch.bfloat16


WORKLOADS = {
    # Forward only, non-causal, fp32, one head of 128 tokens.
    "fwd_fp32_b1h1n128d64": Workload("fwd_fp32_b1h1n128d64", "fwd", 1, 1, 128, 64,
                                     "fp32", False, seed=1),
    # Forward, causal, bf16 inputs with fp32 accumulation.
    "fwd_causal_bf16_b4h16n2048d128": Workload("fwd_causal_bf16_b4h16n2048d128", "fwd",
                                               4, 16, 2048, 128, "bf16", True, seed=2),
    # Long-context forward, causal, bf16, inputs scaled by 0.5; checked on
    # 64 sampled query rows per head (row sample seed 103).
    "fwd_causal_bf16_b1h32n16384d128": Workload("fwd_causal_bf16_b1h32n16384d128", "fwd",
                                                1, 32, 16384, 128, "bf16", True, seed=3,
                                                sigma=0.5, device_gen=True,
                                                extra={"sample_rows": 64, "row_seed": 103}),
    # Backward with recomputation, causal, bf16; O and LSE come from the forward.
    "bwd_causal_bf16_b2h16n4096d128": Workload("bwd_causal_bf16_b2h16n4096d128", "bwd",
                                               2, 16, 4096, 128, "bf16", True, seed=4),
    # KV-cache decode, bf16: 64 sequences x 32 heads, one query token each,
    # 8192 cached tokens per sequence, contiguous [B,H,L,d], no mask.
    "decode_bf16_b64h32l8192d128": Workload("decode_bf16_b64h32l8192d128", "decode",
                                            64, 32, 8192, 128, "bf16", False, seed=5,
                                            device_gen=True),
}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def draw(shapes, seed: int, dtype: torch.dtype, sigma: float = 1.0,
         device: str | torch.device = "cpu"):
    """Draw one N(0, sigma^2) tensor per shape, in order, from one seeded generator.

    The generator lives on ``device``; values are drawn as float32, scaled by
    sigma, then cast to ``dtype``.
    """
    g = _gen(seed, device)
    out = []
    for shp in shapes:
        t = torch.randn(shp, dtype=torch.float32, generator=g, device=device)
        if sigma != 1.0:
            t.mul_(sigma)
        out.append(t.to(dtype))
    return out


def make_inputs(w: Workload, device: str | torch.device = "cpu", with_dout: bool | None = None):
    """Q, K, V (and dO for backward workloads) for workload ``w`` on ``device``.

    CPU-drawn workloads are copied to ``device``; device-drawn ones are drawn
    there directly (``device`` must then be a GPU).  Decode returns
    q [B,H,1,d], k_cache and v_cache [B,H,L,d].
    """
    if with_dout is None:
        with_dout = w.kind == "bwd"
    if w.kind == "decode":
        shapes = [(w.B, w.H, 1, w.d), (w.B, w.H, w.N, w.d), (w.B, w.H, w.N, w.d)]
    else:
        shapes = [(w.B, w.H, w.N, w.d)] * (4 if with_dout else 3)
    gen_dev = device if w.device_gen else "cpu"
    ts = draw(shapes, w.seed, w.torch_dtype, w.sigma, device=gen_dev)
    return [t.to(device) for t in ts]


def make_custom(B: int, H: int, N: int, d: int, dtype: str, seed: int,
                sigma: float = 1.0, n_tensors: int = 3, device="cpu", Nk: int | None = None):
    """Ad-hoc seeded tensors: Q [B,H,N,d] then (n_tensors-1) tensors [B,H,Nk,d].

    When Nk is None every tensor is [B,H,N,d] (the last one doubling as dO for
    backward tests).
    """
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    nk = N if Nk is None else Nk
    shapes = [(B, H, N, d)] + [(B, H, nk, d)] * (n_tensors - 1)
    return [t.to(device) for t in draw(shapes, seed, tdt, sigma, device="cpu")]


def make_gqa(B: int, H: int, Hkv: int, N: int, d: int, dtype: str, seed: int,
             with_dout: bool = False, device="cpu", Nk: int | None = None):
    """Seeded grouped-query inputs: Q [B,H,N,d], K and V [B,Hkv,Nk,d] (and dO [B,H,N,d])."""
    tdt = torch.float32 if dtype == "fp32" else torch.bfloat16
    nk = N if Nk is None else Nk
    shapes = [(B, H, N, d), (B, Hkv, nk, d), (B, Hkv, nk, d)] + ([(B, H, N, d)] if with_dout else [])
    return [t.to(device) for t in draw(shapes, seed, tdt, 1.0, device="cpu")]


def make_fp8(B: int, H: int, Hkv: int, N: int, d: int, seed: int, sigma: float = 1.0, device="cpu",
             gen_device: str = "cpu"):
    """Seeded fp8 (e4m3) inputs for ``fa_fwd_fp8``.

    Q [B,H,N,d], K and V [B,Hkv,N,d] are drawn like the other inputs (float32
    N(0, sigma^2)); each tensor gets the per-tensor factor s = max|x| / 256 and
    is stored as the e4m3 codes of x / s (torch's round-to-nearest cast), V
    transposed to [B,Hkv,d,N].  Returns (q8, k8, vt8, q_scale, k_scale,
    v_scale); the real inputs are s * codes.
    """
    q, k, v = draw([(B, H, N, d), (B, Hkv, N, d), (B, Hkv, N, d)], seed, torch.float32, sigma,
                   device=gen_device)
    out, scales = [], []
    for x in (q, k, v):
        s = float(x.abs().max()) / 256.0
        out.append((x / s).to(torch.float8_e4m3fn))
        scales.append(s)
    q8, k8, v8 = out
    vt8 = v8.transpose(-1, -2).contiguous()
    return q8.to(device), k8.to(device), vt8.to(device), scales[0], scales[1], scales[2]


def sample_rows(n: int, count: int, seed: int):
    """``count`` distinct query rows drawn uniformly from [0, n) with a seeded generator."""
    g = _gen(seed, "cpu")
    perm = torch.randperm(n, generator=g)
    return torch.sort(perm[:count]).values.tolist()
