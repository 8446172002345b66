"""Exact tiled attention for AMD Instinct MI355X (gfx950).

A thin binding of ``libfa.so`` (C ABI in ``include/fa.h``). The functions
``fa_fwd``, ``fa_bwd``, ``fa_fwd_ex``, ``fa_bwd_ex``, ``fa_bwd_noalloc``,
``fa_key_mass``, ``fa_quantize_e4m3``, ``fa_fwd_fp8``, ``fa_quantize_mx_e4m3``,
``fa_fwd_mxfp8`` and ``fa_status_string`` mirror the C
entry points one to one (raw device pointers as Python ints, ``stream`` as a
hipStream_t handle). ``forward``, ``backward``, ``key_mass``,
``quantize_e4m3``, ``forward_fp8``, ``quantize_mx_e4m3`` and ``forward_mxfp8`` are
conveniences over torch tensors:
they check dtypes and shapes, allocate outputs with torch and pass
``data_ptr()`` and the current stream; every step of the computation runs in
the library's HIP kernels. There is no fallback: if the library is missing
or cannot be loaded, every call raises.

Tensor layout is [batch, heads, seq_len, head_dim] as on "RTX Flash Attention
Implementation COMPLETE" (Usage Examples), bf16 or float16 (the page's Mixed
Precision feature), contiguous; the LSE is float32 [batch, heads, seq_len].
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = ["fa_fwd", "fa_bwd", "fa_fwd_ex", "fa_bwd_ex", "fa_bwd_noalloc", "fa_key_mass",
           "fa_quantize_e4m3", "FA_NOALLOC_MAX_ROWS",
           "fa_fwd_fp8", "fa_quantize_mx_e4m3", "fa_fwd_mxfp8", "fa_status_string", "fa_last_hip_error",
           "forward", "backward", "key_mass", "quantize_e4m3", "forward_fp8", "quantize_mx_e4m3",
           "forward_mxfp8", "load", "FAError", "LIB_PATH", "FA_DTYPE_BF16", "FA_DTYPE_F16"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_OK = 0
FA_ERR_INVALID_ARG = 1
FA_ERR_UNSUPPORTED = 2
FA_ERR_HIP = 3
FA_ERR_OUT_OF_MEMORY = 4
FA_ERR_TOO_LARGE = 5

FA_NOALLOC_MAX_ROWS = 2097152  # query rows (B * H * N) of fa_bwd_noalloc's static workspace

FA_DTYPE_BF16 = 0
FA_DTYPE_F16 = 1

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = f"{where}: {fa_status_string(status)}"
        if status in (FA_ERR_HIP, FA_ERR_OUT_OF_MEMORY):
            msg += f" ({fa_last_hip_error()})"
        super().__init__(msg)


def load(path: str | None = None) -> ctypes.CDLL:
    """Loads libfa.so once and declares its exported signatures.

    torch is imported first: torch ships its own HIP runtime under the same
    soname as the system one, and libfa.so must bind to the runtime instance
    that owns the caller's device memory and streams (a second runtime in the
    same process sees no device).
    """
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (binds libamdhip64 to torch's runtime)
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing; build it with `python -m exact_tiled_attention_17_amd.build`")
    lib = ctypes.CDLL(path)
    vp, ci, cf = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, vp]
    lib.fa_fwd.restype = ci
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, cf, vp]
    lib.fa_bwd.restype = ci
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, vp]
    lib.fa_fwd_ex.restype = ci
    lib.fa_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci,
                              vp]
    lib.fa_bwd_ex.restype = ci
    lib.fa_bwd_noalloc.argtypes = lib.fa_bwd_ex.argtypes
    lib.fa_bwd_noalloc.restype = ci
    lib.fa_key_mass.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, ci, vp]
    lib.fa_key_mass.restype = ci
    lib.fa_quantize_e4m3.argtypes = [vp, vp, vp, ci, ci, ci, ci, vp]
    lib.fa_quantize_e4m3.restype = ci
    lib.fa_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp]
    lib.fa_fwd_fp8.restype = ci
    lib.fa_quantize_mx_e4m3.argtypes = [vp, vp, vp, ci, ci, ci, ci, vp]
    lib.fa_quantize_mx_e4m3.restype = ci
    lib.fa_fwd_mxfp8.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, cf, vp]
    lib.fa_fwd_mxfp8.restype = ci
    lib.fa_status_string.argtypes = [ci]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_last_hip_error.argtypes = []
    lib.fa_last_hip_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def fa_last_hip_error() -> str:
    return load().fa_last_hip_error().decode()


def fa_fwd(Q, K, V, O, LSE, B, H, N, d, causal, softmax_scale, stream) -> int:
    """C ``fa_fwd``: pointers as ints (LSE may be 0 / None); returns the status."""
    return load().fa_fwd(Q, K, V, O, LSE or None, B, H, N, d, int(causal),
                         float(softmax_scale), stream or None)


def fa_bwd(Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, N, d, causal, softmax_scale, stream) -> int:
    """C ``fa_bwd``: pointers as ints; returns the status."""
    return load().fa_bwd(Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, N, d, int(causal),
                         float(softmax_scale), stream or None)


def fa_fwd_ex(Q, K, V, O, LSE, B, H, Hkv, N, d, causal, softmax_scale, dtype, stream) -> int:
    """C ``fa_fwd_ex``: as ``fa_fwd`` with Hkv K/V heads and the element type (FA_DTYPE_*)."""
    return load().fa_fwd_ex(Q, K, V, O, LSE or None, B, H, Hkv, N, d, int(causal),
                            float(softmax_scale), int(dtype), stream or None)


def fa_bwd_ex(Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, Hkv, N, d, causal, softmax_scale, dtype,
              stream) -> int:
    """C ``fa_bwd_ex``: as ``fa_bwd`` with Hkv K/V heads and the element type (FA_DTYPE_*)."""
    return load().fa_bwd_ex(Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, Hkv, N, d, int(causal),
                            float(softmax_scale), int(dtype), stream or None)


def fa_bwd_noalloc(Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, Hkv, N, d, causal, softmax_scale,
                   dtype, stream) -> int:
    """C ``fa_bwd_noalloc``: ``fa_bwd_ex`` with its scratch in the library's static per-device
    workspace (no allocation; B * H * N <= FA_NOALLOC_MAX_ROWS); returns the status."""
    return load().fa_bwd_noalloc(Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, Hkv, N, d, int(causal),
                                 float(softmax_scale), int(dtype), stream or None)


def fa_key_mass(Q, K, LSE, mass, B, H, Hkv, N, d, causal, softmax_scale, dtype, stream) -> int:
    """C ``fa_key_mass``: per-key attention mass summed over heads; returns the status."""
    return load().fa_key_mass(Q, K, LSE, mass, B, H, Hkv, N, d, int(causal), float(softmax_scale),
                              int(dtype), stream or None)


def fa_quantize_e4m3(X, codes, scales, R, N, d, dtype, stream) -> int:
    """C ``fa_quantize_e4m3``: E4M3 codes and power-of-two scales per 16 x 16 block."""
    return load().fa_quantize_e4m3(X, codes, scales, R, N, d, int(dtype), stream or None)


def fa_fwd_fp8(Q, K, V, O, LSE, B, H, Hkv, N, d, causal, softmax_scale, stream) -> int:
    """C ``fa_fwd_fp8``: the forward with Q and K quantised to E4M3 per 16 x 16 block."""
    return load().fa_fwd_fp8(Q, K, V, O, LSE or None, B, H, Hkv, N, d, int(causal),
                             float(softmax_scale), stream or None)


def fa_quantize_mx_e4m3(X, codes, scales, R, N, d, dtype, stream) -> int:
    """C ``fa_quantize_mx_e4m3``: E4M3 codes and E8M0 scale bytes per 1 x 32 block."""
    return load().fa_quantize_mx_e4m3(X, codes, scales, R, N, d, int(dtype), stream or None)


def fa_fwd_mxfp8(Q, K, V, O, LSE, B, H, Hkv, N, d, causal, softmax_scale, stream) -> int:
    """C ``fa_fwd_mxfp8``: the forward with Q and K quantised to E4M3 per 1 x 32 block."""
    return load().fa_fwd_mxfp8(Q, K, V, O, LSE or None, B, H, Hkv, N, d, int(causal),
                               float(softmax_scale), stream or None)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return FA_DTYPE_BF16
    if t.dtype == torch.float16:
        return FA_DTYPE_F16
    raise TypeError(f"tensors must be bfloat16 or float16, got {t.dtype}")


def _check(name, t, shape, dtype, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _kv_heads(H, k):
    Hkv = int(k.shape[1])
    if Hkv < 1 or H % Hkv != 0:
        raise ValueError(f"k/v have {Hkv} heads, which must divide the {H} query heads")
    return Hkv


def _scale(scale, d):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def forward(q, k, v, causal: bool = False, scale: float | None = None, *, out=None, lse=None,
            need_lse: bool = True):
    """O, LSE = attention(q, k, v) on one GPU: q bf16 or float16 [B, H, N, d]; k, v of the
    same dtype, [B, Hkv, N, d] with Hkv dividing H (query head h uses K/V head h // (H // Hkv))."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [batch, heads, seq_len, head_dim]")
    B, H, N, d = q.shape
    Hkv = _kv_heads(H, k)
    dev = q.device
    code = _dtype_code(q)
    _check("q", q, (B, H, N, d), q.dtype, dev)
    for name, t in (("k", k), ("v", v)):
        _check(name, t, (B, Hkv, N, d), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _check("out", out, (B, H, N, d), q.dtype, dev)
    if need_lse:
        if lse is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        _check("lse", lse, (B, H, N), torch.float32, dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                       lse.data_ptr() if need_lse else None, B, H, Hkv, N, d, causal,
                       _scale(scale, d), code, stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_ex")
    return out, lse


def backward(do, q, k, v, o, lse, causal: bool = False, scale: float | None = None, *,
             dq=None, dk=None, dv=None):
    """dQ, dK, dV of attention given dO, the inputs, and the forward's O and LSE (shapes as in
    ``forward``; dK, dV are summed over the query heads that share a K/V head)."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [batch, heads, seq_len, head_dim]")
    B, H, N, d = q.shape
    Hkv = _kv_heads(H, k)
    dev = q.device
    code = _dtype_code(q)
    for name, t in (("do", do), ("q", q), ("o", o)):
        _check(name, t, (B, H, N, d), q.dtype, dev)
    for name, t in (("k", k), ("v", v)):
        _check(name, t, (B, Hkv, N, d), q.dtype, dev)
    _check("lse", lse, (B, H, N), torch.float32, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check("dq", dq, (B, H, N, d), q.dtype, dev)
    for name, t in (("dk", dk), ("dv", dv)):
        _check(name, t, (B, Hkv, N, d), q.dtype, dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                       B, H, Hkv, N, d, causal, _scale(scale, d), code, stream)
    if st != FA_OK:
        raise FAError(st, "fa_bwd_ex")
    return dq, dk, dv


def key_mass(q, k, lse, causal: bool = False, scale: float | None = None, *, out=None):
    """mass[b, j] = sum over heads and query rows of the attention probability key j gets
    (float32 [B, N]), from q, k (as in ``forward``) and the forward's LSE."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k must be [batch, heads, seq_len, head_dim]")
    B, H, N, d = q.shape
    Hkv = _kv_heads(H, k)
    dev = q.device
    code = _dtype_code(q)
    _check("q", q, (B, H, N, d), q.dtype, dev)
    _check("k", k, (B, Hkv, N, d), q.dtype, dev)
    _check("lse", lse, (B, H, N), torch.float32, dev)
    if out is None:
        out = torch.empty((B, N), dtype=torch.float32, device=dev)
    _check("out", out, (B, N), torch.float32, dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = fa_key_mass(q.data_ptr(), k.data_ptr(), lse.data_ptr(), out.data_ptr(), B, H, Hkv, N, d,
                         causal, _scale(scale, d), code, stream)
    if st != FA_OK:
        raise FAError(st, "fa_key_mass")
    return out


def quantize_e4m3(x):
    """E4M3 codes (uint8, same shape) and block scales (float32 [..., ceil(N/16), d/16]) of a
    bf16 or float16 tensor [..., N, d], quantised per 16 x 16 block of each [N, d] matrix."""
    import torch
    if x.dim() < 2:
        raise ValueError("x must be [..., seq_len, head_dim]")
    N, d = int(x.shape[-2]), int(x.shape[-1])
    R = int(x.numel() // (N * d)) if x.numel() else 0
    code = _dtype_code(x)
    _check("x", x, tuple(x.shape), x.dtype, x.device)
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty((*x.shape[:-2], (N + 15) // 16, d // 16), dtype=torch.float32,
                         device=x.device)
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        st = fa_quantize_e4m3(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), R, N, d, code, stream)
    if st != FA_OK:
        raise FAError(st, "fa_quantize_e4m3")
    return codes, scales


def forward_fp8(q, k, v, causal: bool = False, scale: float | None = None, *, out=None, lse=None,
                need_lse: bool = True):
    """O, LSE of the FP8 path: q, k quantised to E4M3 per 16 x 16 block, then attention (bf16
    tensors shaped as in ``forward``)."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [batch, heads, seq_len, head_dim]")
    B, H, N, d = q.shape
    Hkv = _kv_heads(H, k)
    dev = q.device
    if q.dtype != torch.bfloat16:
        raise TypeError(f"the FP8 path takes bfloat16 tensors, got {q.dtype}")
    _check("q", q, (B, H, N, d), q.dtype, dev)
    for name, t in (("k", k), ("v", v)):
        _check(name, t, (B, Hkv, N, d), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _check("out", out, (B, H, N, d), q.dtype, dev)
    if need_lse:
        if lse is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        _check("lse", lse, (B, H, N), torch.float32, dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                        lse.data_ptr() if need_lse else None, B, H, Hkv, N, d, causal,
                        _scale(scale, d), stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_fp8")
    return out, lse


def quantize_mx_e4m3(x):
    """E4M3 codes (uint8, same shape) and E8M0 scale bytes (uint8 [..., N, d/32]; byte s
    means 2^(s - 127)) of a bf16 or float16 tensor [..., N, d], quantised per 1 x 32 block
    (one row, 32 consecutive columns)."""
    import torch
    if x.dim() < 2:
        raise ValueError("x must be [..., seq_len, head_dim]")
    N, d = int(x.shape[-2]), int(x.shape[-1])
    R = int(x.numel() // (N * d)) if x.numel() else 0
    code = _dtype_code(x)
    _check("x", x, tuple(x.shape), x.dtype, x.device)
    codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    scales = torch.empty((*x.shape[:-1], d // 32), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        stream = torch.cuda.current_stream(x.device).cuda_stream
        st = fa_quantize_mx_e4m3(x.data_ptr(), codes.data_ptr(), scales.data_ptr(), R, N, d, code,
                                 stream)
    if st != FA_OK:
        raise FAError(st, "fa_quantize_mx_e4m3")
    return codes, scales


def forward_mxfp8(q, k, v, causal: bool = False, scale: float | None = None, *, out=None, lse=None,
                  need_lse: bool = True):
    """O, LSE of the FP8 path under the 1 x 32 block reading: q, k quantised to E4M3 per row
    and 32 columns, S = Q K^T on the scaled FP8 matrix instruction (bf16 tensors shaped as in
    ``forward``)."""
    import torch
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [batch, heads, seq_len, head_dim]")
    B, H, N, d = q.shape
    Hkv = _kv_heads(H, k)
    dev = q.device
    if q.dtype != torch.bfloat16:
        raise TypeError(f"the FP8 path takes bfloat16 tensors, got {q.dtype}")
    _check("q", q, (B, H, N, d), q.dtype, dev)
    for name, t in (("k", k), ("v", v)):
        _check(name, t, (B, Hkv, N, d), q.dtype, dev)
    if out is None:
        out = torch.empty_like(q)
    _check("out", out, (B, H, N, d), q.dtype, dev)
    if need_lse:
        if lse is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        _check("lse", lse, (B, H, N), torch.float32, dev)
    with torch.cuda.device(dev):
        stream = torch.cuda.current_stream(dev).cuda_stream
        st = fa_fwd_mxfp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                          lse.data_ptr() if need_lse else None, B, H, Hkv, N, d, causal,
                          _scale(scale, d), stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_mxfp8")
    return out, lse
