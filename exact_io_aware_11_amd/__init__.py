"""Python binding of the exact IO-aware attention library (``libfa.so``).

Argument marshalling only: every step of forward, backward and decode runs in
the HIP kernels behind the C ABI of ``include/fa.h``.  PyTorch is used for two
things, device memory (``torch.empty``) and the current HIP stream.  There is
no fallback: if the library is missing, importing this package fails.

Entry points with the C names (raw pointers, sizes, stream handle):
``fa_fwd``, ``fa_fwd_fp8``, ``fa_bwd``, ``fa_bwd_workspace_bytes``, ``fa_decode``,
``fa_decode_workspace_bytes``, ``fa_decode_num_splits``, ``fa_decode_noalloc``,
``fa_decode_paged``, ``fa_status_string``.

Tensor-level helpers with the same semantics:
``attention(q, k, v, is_causal=False, scale=None, out_dtype=None) -> (o, lse)``
(the call shape of PyTorch's scaled_dot_product_attention that the pages show),
``attention_fp8(q, k, vt, q_scale, k_scale, v_scale, is_causal=False,
scale=None, out_dtype=None) -> (o, lse)`` on e4m3 inputs,
``attention_backward(q, k, v, o, lse, do, is_causal=False, scale=None)``
``-> (dq, dk, dv)`` and ``decode(q, k_cache, v_cache, scale=None,
num_splits=0) -> (o, lse)``, ``decode_noalloc(q, k_cache, v_cache, o, lse,
scale=None, num_splits=0)`` (writes the caller's o and lse, allocates nothing)
and ``decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale=None,
num_splits=0) -> (o, lse)``.
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "LIB_PATH", "FA_OK", "FA_ERR_NULL", "FA_ERR_ARG", "FA_ERR_UNSUPPORTED", "FA_ERR_ALIGN",
    "FA_ERR_WORKSPACE", "FA_ERR_HIP", "FA_ERR_SCRATCH_LIMIT", "FA_NOALLOC_SCRATCH_BYTES", "FA_FP32", "FA_BF16",
    "FaError",
    "fa_fwd", "fa_fwd_fp8", "fa_bwd", "fa_bwd_workspace_bytes", "fa_decode", "fa_decode_workspace_bytes",
    "fa_decode_num_splits", "fa_decode_noalloc", "fa_decode_paged", "fa_status_string",
    "attention", "attention_fp8", "attention_backward", "decode", "decode_noalloc", "decode_paged", "lib",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

(FA_OK, FA_ERR_NULL, FA_ERR_ARG, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_WORKSPACE, FA_ERR_HIP,
 FA_ERR_SCRATCH_LIMIT) = range(8)
FA_NOALLOC_SCRATCH_BYTES = 16 << 20     # the static scratch array of fa_decode_noalloc (fa.h)
FA_FP32, FA_BF16 = 0, 1


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)}")


def _load() -> ctypes.CDLL:
    # libfa.so needs libamdhip64.so.7.  PyTorch ships its own copy under the
    # same soname; if libfa.so were loaded first, the dynamic loader would map
    # the system copy as well and the process would hold two HIP runtimes,
    # whose streams and allocations the other cannot use.  Importing torch
    # first makes the loader resolve libfa.so's dependency to torch's runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python exact_io_aware_11_amd/build.py). "
            "There is no fallback implementation.")
    lib_ = ctypes.CDLL(LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib_.fa_fwd.argtypes = [P, P, P, P, I, P, I, I, I, I, I, I, I, F, P]
    lib_.fa_fwd.restype = I
    lib_.fa_fwd_fp8.argtypes = [P, P, P, F, F, F, P, I, P, I, I, I, I, I, I, F, P]
    lib_.fa_fwd_fp8.restype = I
    lib_.fa_bwd_workspace_bytes.argtypes = [I, I, I, I, I]
    lib_.fa_bwd_workspace_bytes.restype = Z
    lib_.fa_bwd.argtypes = [P, P, P, P, I, P, P, P, P, P, P, Z, I, I, I, I, I, I, I, F, P]
    lib_.fa_bwd.restype = I
    lib_.fa_decode_num_splits.argtypes = [I, I, I, I, I]
    lib_.fa_decode_num_splits.restype = I
    lib_.fa_decode_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib_.fa_decode_workspace_bytes.restype = Z
    lib_.fa_decode.argtypes = [P, P, P, P, P, P, Z, I, I, I, I, I, I, I, F, P]
    lib_.fa_decode.restype = I
    lib_.fa_decode_noalloc.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, F, P]
    lib_.fa_decode_noalloc.restype = I
    lib_.fa_decode_paged.argtypes = [P, P, P, P, P, P, P, P, Z, I, I, I, I, I, I, I, I, I, F, P]
    lib_.fa_decode_paged.restype = I
    lib_.fa_status_string.argtypes = [I]
    lib_.fa_status_string.restype = ctypes.c_char_p
    return lib_


lib = _load()

# ----------------------------------------------------------------------------
# C-named entry points (plain integers for pointers and the stream)
# ----------------------------------------------------------------------------


def fa_status_string(status: int) -> str:
    return lib.fa_status_string(int(status)).decode()


def fa_fwd(q, k, v, o, o_dtype, lse, B, H, Hkv, N, d, in_dtype, causal, scale, stream=0) -> int:
    return lib.fa_fwd(q, k, v, o, o_dtype, lse, B, H, Hkv, N, d, in_dtype, int(causal), scale, stream)


def fa_fwd_fp8(q, k, vt, q_scale, k_scale, v_scale, o, o_dtype, lse, B, H, Hkv, N, d, causal, scale,
               stream=0) -> int:
    return lib.fa_fwd_fp8(q, k, vt, q_scale, k_scale, v_scale, o, o_dtype, lse, B, H, Hkv, N, d, int(causal),
                          scale, stream)


def fa_bwd_workspace_bytes(B, H, Hkv, N, d) -> int:
    return lib.fa_bwd_workspace_bytes(B, H, Hkv, N, d)


def fa_bwd(q, k, v, o, o_dtype, lse, dout, dq, dk, dv, workspace, workspace_bytes,
           B, H, Hkv, N, d, in_dtype, causal, scale, stream=0) -> int:
    return lib.fa_bwd(q, k, v, o, o_dtype, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                      B, H, Hkv, N, d, in_dtype, int(causal), scale, stream)


def fa_decode_num_splits(B, H, Hkv, L, d) -> int:
    return lib.fa_decode_num_splits(B, H, Hkv, L, d)


def fa_decode_workspace_bytes(B, H, Hkv, L, d, num_splits=0) -> int:
    return lib.fa_decode_workspace_bytes(B, H, Hkv, L, d, num_splits)


def fa_decode(q, k_cache, v_cache, o, lse, workspace, workspace_bytes, B, H, Hkv, L, d, dtype,
              num_splits, scale, stream=0) -> int:
    return lib.fa_decode(q, k_cache, v_cache, o, lse, workspace, workspace_bytes, B, H, Hkv, L, d,
                         dtype, num_splits, scale, stream)


def fa_decode_noalloc(q, k_cache, v_cache, o, lse, B, H, Hkv, L, d, dtype, num_splits, scale, stream=0) -> int:
    return lib.fa_decode_noalloc(q, k_cache, v_cache, o, lse, B, H, Hkv, L, d, dtype, num_splits, scale, stream)


def fa_decode_paged(q, k_pool, v_pool, block_table, seq_lens, o, lse, workspace, workspace_bytes,
                    B, H, Hkv, num_pages, page_size, max_pages_per_seq, d, dtype, num_splits, scale,
                    stream=0) -> int:
    return lib.fa_decode_paged(q, k_pool, v_pool, block_table, seq_lens, o, lse, workspace, workspace_bytes,
                               B, H, Hkv, num_pages, page_size, max_pages_per_seq, d, dtype, num_splits,
                               scale, stream)


# ----------------------------------------------------------------------------
# tensor helpers (torch: allocation and stream only)
# ----------------------------------------------------------------------------


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check(t, name, shape=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(t) -> int:
    torch = _torch()
    return torch.cuda.current_stream(t.device).cuda_stream


def _raise(status: int, where: str):
    if status != FA_OK:
        raise FaError(status, where)


def attention(q, k, v, is_causal: bool = False, scale: float | None = None, out_dtype=None):
    """O = softmax(scale Q K^T [causal]) V and the per-row LSE, via ``fa_fwd``.

    q: contiguous [B,H,N,d] bf16 or fp32 GPU tensor; k, v: [B,Hkv,N,d] with
    Hkv dividing H (grouped-query attention when Hkv < H).  Returns
    (o [B,H,N,d] of ``out_dtype`` (default: q's dtype), lse [B,H,N] fp32).
    """
    torch = _torch()
    _check(q, "q")
    B, H, N, d = q.shape
    _check(k, "k")
    Hkv = k.shape[1]
    _check(k, "k", (B, Hkv, N, d))
    _check(v, "v", (B, Hkv, N, d))
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    o = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _dtype_code(o), lse.data_ptr(),
                B, H, Hkv, N, d, _dtype_code(q), is_causal, scale, _stream(q))
    _raise(st, "fa_fwd")
    return o, lse


def attention_fp8(q, k, vt, q_scale: float, k_scale: float, v_scale: float, is_causal: bool = False,
                  scale: float | None = None, out_dtype=None):
    """``attention`` on fp8 inputs, via ``fa_fwd_fp8``.

    q: contiguous [B,H,N,d] ``torch.float8_e4m3fn`` GPU tensor; k: [B,Hkv,N,d];
    vt: V transposed, [B,Hkv,d,N]; all e4m3.  The inputs' real values are
    q_scale * q, k_scale * k, v_scale * v.  Returns (o [B,H,N,d] of
    ``out_dtype`` (default bf16), lse [B,H,N] fp32).
    """
    torch = _torch()
    _check(q, "q")
    B, H, N, d = q.shape
    _check(k, "k")
    Hkv = k.shape[1]
    _check(k, "k", (B, Hkv, N, d))
    _check(vt, "vt", (B, Hkv, d, N))
    for t, n in ((q, "q"), (k, "k"), (vt, "vt")):
        if t.dtype != torch.float8_e4m3fn:
            raise TypeError(f"{n} must be torch.float8_e4m3fn")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    out_dtype = torch.bfloat16 if out_dtype is None else out_dtype
    o = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    st = fa_fwd_fp8(q.data_ptr(), k.data_ptr(), vt.data_ptr(), float(q_scale), float(k_scale), float(v_scale),
                    o.data_ptr(), _dtype_code(o), lse.data_ptr(), B, H, Hkv, N, d, is_causal, scale, _stream(q))
    _raise(st, "fa_fwd_fp8")
    return o, lse


def attention_backward(q, k, v, o, lse, do, is_causal: bool = False, scale: float | None = None):
    """dQ, dK, dV of ``attention`` by recomputation from (q, k, v, o, lse), via ``fa_bwd``.

    dk and dv have k's shape [B,Hkv,N,d]; a shared K/V head gets the sum over
    its query heads.
    """
    torch = _torch()
    _check(q, "q")
    B, H, N, d = q.shape
    _check(k, "k")
    Hkv = k.shape[1]
    for t, n in ((o, "o"), (do, "do")):
        _check(t, n, q.shape)
    for t, n in ((k, "k"), (v, "v")):
        _check(t, n, (B, Hkv, N, d))
    _check(lse, "lse", (B, H, N))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    nbytes = fa_bwd_workspace_bytes(B, H, Hkv, N, d)
    ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=q.device)
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), _dtype_code(o), lse.data_ptr(),
                do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), nbytes,
                B, H, Hkv, N, d, _dtype_code(q), is_causal, scale, _stream(q))
    _raise(st, "fa_bwd")
    return dq, dk, dv


def decode(q, k_cache, v_cache, scale: float | None = None, num_splits: int = 0):
    """One decode step: q [B,H,1,d] against caches [B,Hkv,L,d] (bf16), via ``fa_decode``.

    Returns (o [B,H,1,d] bf16, lse [B,H] fp32).
    """
    torch = _torch()
    _check(q, "q")
    B, H, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per (batch, head)")
    _check(k_cache, "k_cache")
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    _check(k_cache, "k_cache", (B, Hkv, L, d))
    _check(v_cache, "v_cache", (B, Hkv, L, d))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty((B, H, 1, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    nbytes = fa_decode_workspace_bytes(B, H, Hkv, L, d, num_splits)
    ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=q.device)
    st = fa_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(), lse.data_ptr(),
                   ws.data_ptr(), nbytes, B, H, Hkv, L, d, _dtype_code(q), num_splits, scale, _stream(q))
    _raise(st, "fa_decode")
    return o, lse


def decode_noalloc(q, k_cache, v_cache, o, lse, scale: float | None = None, num_splits: int = 0):
    """``decode`` into caller-provided outputs, via ``fa_decode_noalloc``.

    Allocates nothing (no torch allocation either): the split partials live in
    the library's static scratch array.  q [B,H,1,d], caches [B,Hkv,L,d], o
    [B,H,1,d] bf16, lse [B,H] fp32 (or None).  Raises ``FaError`` with
    FA_ERR_SCRATCH_LIMIT when the call needs more than
    FA_NOALLOC_SCRATCH_BYTES of scratch.  Calls that overlap on one GPU race
    on that array.
    """
    torch = _torch()
    _check(q, "q")
    B, H, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per (batch, head)")
    _check(k_cache, "k_cache")
    Hkv, L = k_cache.shape[1], k_cache.shape[2]
    _check(k_cache, "k_cache", (B, Hkv, L, d))
    _check(v_cache, "v_cache", (B, Hkv, L, d))
    _check(o, "o", (B, H, 1, d))
    if o.dtype != q.dtype:
        raise TypeError("o must have q's dtype")
    lse_ptr = 0
    if lse is not None:
        _check(lse, "lse", (B, H))
        if lse.dtype != torch.float32:
            raise TypeError("lse must be float32")
        lse_ptr = lse.data_ptr()
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = fa_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(), lse_ptr,
                           B, H, Hkv, L, d, _dtype_code(q), num_splits, scale, _stream(q))
    _raise(st, "fa_decode_noalloc")


def decode_paged(q, k_pool, v_pool, block_table, seq_lens, scale: float | None = None, num_splits: int = 0):
    """One decode step against a paged cache, via ``fa_decode_paged``.

    q [B,H,1,d] bf16; k_pool, v_pool [num_pages, Hkv, page_size, d] bf16;
    block_table [B, max_pages] int32 and seq_lens [B] int32 on the GPU.
    Returns (o [B,H,1,d] bf16, lse [B,H] fp32).
    """
    torch = _torch()
    _check(q, "q")
    B, H, one, d = q.shape
    if one != 1:
        raise ValueError("decode takes one query token per (batch, head)")
    _check(k_pool, "k_pool")
    num_pages, Hkv, page_size = k_pool.shape[0], k_pool.shape[1], k_pool.shape[2]
    _check(k_pool, "k_pool", (num_pages, Hkv, page_size, d))
    _check(v_pool, "v_pool", (num_pages, Hkv, page_size, d))
    _check(block_table, "block_table")
    _check(seq_lens, "seq_lens", (B,))
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise TypeError("block_table and seq_lens must be int32")
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError("block_table must be [B, max_pages_per_seq]")
    max_pages = block_table.shape[1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    o = torch.empty((B, H, 1, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    nbytes = fa_decode_workspace_bytes(B, H, Hkv, max_pages * page_size, d, num_splits)
    ws = torch.empty((max(nbytes, 1),), dtype=torch.uint8, device=q.device)
    st = fa_decode_paged(q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(), block_table.data_ptr(),
                         seq_lens.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(), nbytes,
                         B, H, Hkv, num_pages, page_size, max_pages, d, _dtype_code(q), num_splits, scale,
                         _stream(q))
    _raise(st, "fa_decode_paged")
    return o, lse
