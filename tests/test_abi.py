"""The C ABI on the CPU: the library loads, exports every entry point the header
declares, and rejects invalid arguments on the host before any HIP call (so
these calls are safe without a GPU: nothing is enqueued)."""
import ctypes
import os
import re

import pytest

import exact_tiled_attention_17_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# A fake but 16-byte aligned, non-null "device pointer": validation never
# dereferences pointers and every call below fails validation first.
P = 0x10000


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert header_functions() == ["fa_bwd", "fa_bwd_ex", "fa_bwd_noalloc", "fa_fwd", "fa_fwd_ex",
                                  "fa_fwd_fp8", "fa_fwd_mxfp8", "fa_key_mass", "fa_last_hip_error",
                                  "fa_quantize_e4m3", "fa_quantize_mx_e4m3", "fa_status_string"]


def test_library_exports_every_declared_symbol():
    lib = fa.load()
    for name in header_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_strings():
    assert fa.fa_status_string(fa.FA_OK).startswith("FA_OK")
    for st in (fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_HIP, fa.FA_ERR_OUT_OF_MEMORY,
               fa.FA_ERR_TOO_LARGE):
        assert fa.fa_status_string(st).startswith("FA_ERR")
    assert str(fa.FA_NOALLOC_MAX_ROWS) in fa.fa_status_string(fa.FA_ERR_TOO_LARGE)
    assert fa.fa_status_string(12345) == "unknown fa_status"
    assert fa.fa_last_hip_error() == "hipSuccess"


GOOD = dict(B=1, H=2, N=16, d=128, causal=0, softmax_scale=0.125)


def fwd(**kw):
    a = dict(GOOD, Q=P, K=P, V=P, O=P, LSE=P, stream=None)
    a.update(kw)
    return fa.fa_fwd(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["N"], a["d"],
                     a["causal"], a["softmax_scale"], a["stream"])


def bwd(**kw):
    a = dict(GOOD, Q=P, K=P, V=P, O=P, LSE=P, dO=P, dQ=P, dK=P, dV=P, stream=None)
    a.update(kw)
    return fa.fa_bwd(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["dO"], a["dQ"], a["dK"], a["dV"],
                     a["B"], a["H"], a["N"], a["d"], a["causal"], a["softmax_scale"], a["stream"])


BAD_SHAPES = [
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(d=0), fa.FA_ERR_UNSUPPORTED),
    (dict(causal=2), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(N=1 << 24, d=128), fa.FA_ERR_INVALID_ARG),          # N * d >= 2^31
    (dict(B=1 << 16, H=1 << 16, N=64), fa.FA_ERR_INVALID_ARG),  # grid too large
]


@pytest.mark.parametrize("kw,want", BAD_SHAPES, ids=lambda x: str(x))
def test_fwd_rejects_bad_shapes(kw, want):
    assert fwd(**kw) == want


@pytest.mark.parametrize("kw,want", BAD_SHAPES, ids=lambda x: str(x))
def test_bwd_rejects_bad_shapes(kw, want):
    assert bwd(**kw) == want


@pytest.mark.parametrize("name", ["Q", "K", "V", "O"])
def test_fwd_rejects_null_and_misaligned(name):
    assert fwd(**{name: None}) == fa.FA_ERR_INVALID_ARG
    assert fwd(**{name: P + 8}) == fa.FA_ERR_INVALID_ARG


def test_fwd_lse_alignment():
    assert fwd(LSE=P + 2) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("name", ["Q", "K", "V", "O", "dO", "dQ", "dK", "dV", "LSE"])
def test_bwd_rejects_null_and_misaligned(name):
    assert bwd(**{name: None}) == fa.FA_ERR_INVALID_ARG
    assert bwd(**{name: P + 2}) == fa.FA_ERR_INVALID_ARG


def test_torch_wrapper_checks_before_calling():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        fa.forward(q.float(), q, q)
    with pytest.raises(ValueError):
        fa.forward(q, q[:, :, :2], q)
    with pytest.raises(ValueError):
        fa.forward(q[..., ::2], q[..., ::2], q[..., ::2])


@pytest.mark.parametrize("dtype", [-1, 2, 99])
def test_ex_entry_points_reject_unknown_dtype(dtype):
    assert fa.fa_fwd_ex(P, P, P, P, P, 1, 2, 2, 16, 128, 0, 0.125, dtype, None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_bwd_ex(P, P, P, P, P, P, P, P, P, 1, 2, 2, 16, 128, 0, 0.125, dtype, None) == \
        fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", [0, 1])
def test_ex_entry_points_validate_like_the_plain_ones(dtype):
    # same host-side checks as fa_fwd / fa_bwd for either element type
    assert fa.fa_fwd_ex(P, P, P, P, P, 1, 2, 2, 16, 96, 0, 0.125, dtype, None) == fa.FA_ERR_UNSUPPORTED
    assert fa.fa_fwd_ex(P, P, P, P, P, 1, 2, 2, 16, 128, 2, 0.125, dtype, None) == fa.FA_ERR_INVALID_ARG
    assert fa.fa_fwd_ex(P + 8, P, P, P, P, 1, 2, 2, 16, 128, 0, 0.125, dtype, None) == \
        fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_ex(P, P, P, P, None, P, P, P, P, 1, 2, 2, 16, 128, 0, 0.125, dtype, None) == \
        fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_ex(P, P, P, P, P, P, P, P, P, 0, 2, 2, 16, 128, 0, 0.125, dtype, None) == \
        fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("dtype", [0, 1])
@pytest.mark.parametrize("H,Hkv", [(4, 0), (4, -1), (4, 3), (6, 4), (2, 4)])
def test_ex_entry_points_reject_kv_heads_not_dividing_query_heads(dtype, H, Hkv):
    assert fa.fa_fwd_ex(P, P, P, P, P, 1, H, Hkv, 16, 128, 0, 0.125, dtype, None) == \
        fa.FA_ERR_INVALID_ARG
    assert fa.fa_bwd_ex(P, P, P, P, P, P, P, P, P, 1, H, Hkv, 16, 128, 0, 0.125, dtype, None) == \
        fa.FA_ERR_INVALID_ARG


def test_torch_wrapper_checks_kv_heads():
    import torch
    q = torch.zeros(1, 6, 4, 64, dtype=torch.bfloat16)
    kv4 = torch.zeros(1, 4, 4, 64, dtype=torch.bfloat16)
    kv2 = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    kv3 = torch.zeros(1, 3, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):   # 4 does not divide 6
        fa.forward(q, kv4, kv4)
    with pytest.raises(ValueError):   # k and v head counts differ
        fa.forward(q, kv2, kv3)
    with pytest.raises(ValueError):
        fa.backward(q, q, kv4, kv4, q, torch.zeros(1, 6, 4))


def mass(**kw):
    a = dict(GOOD, Q=P, K=P, LSE=P, mass=P, Hkv=2, dtype=0, stream=None)
    a.update(kw)
    return fa.fa_key_mass(a["Q"], a["K"], a["LSE"], a["mass"], a["B"], a["H"], a["Hkv"], a["N"],
                          a["d"], a["causal"], a["softmax_scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("name", ["Q", "K", "LSE", "mass"])
def test_key_mass_rejects_null_and_misaligned(name):
    assert mass(**{name: None}) == fa.FA_ERR_INVALID_ARG
    assert mass(**{name: P + 2}) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), "FA_ERR_UNSUPPORTED"), (dict(dtype=5), "FA_ERR_UNSUPPORTED"),
    (dict(N=0), "FA_ERR_INVALID_ARG"), (dict(B=0), "FA_ERR_INVALID_ARG"),
    (dict(Hkv=3), "FA_ERR_INVALID_ARG"), (dict(causal=2), "FA_ERR_INVALID_ARG"),
    (dict(softmax_scale=0.0), "FA_ERR_INVALID_ARG"), (dict(softmax_scale=float("nan")), "FA_ERR_INVALID_ARG"),
])
def test_key_mass_validates(kw, status):
    assert mass(**kw) == getattr(fa, status)


def test_torch_key_mass_checks_before_calling():
    import torch
    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):   # lse of the wrong shape
        fa.key_mass(q, q, torch.zeros(1, 2, 5))
    with pytest.raises(TypeError):    # lse not float32
        fa.key_mass(q, q, torch.zeros(1, 2, 4, dtype=torch.float64))


def quant(**kw):
    a = dict(X=P, codes=P, scales=P, R=2, N=16, d=128, dtype=0, stream=None)
    a.update(kw)
    return fa.fa_quantize_e4m3(a["X"], a["codes"], a["scales"], a["R"], a["N"], a["d"], a["dtype"],
                               a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), "FA_ERR_INVALID_ARG"), (dict(X=P + 2), "FA_ERR_INVALID_ARG"),
    (dict(codes=None), "FA_ERR_INVALID_ARG"), (dict(codes=P + 4), "FA_ERR_INVALID_ARG"),
    (dict(scales=None), "FA_ERR_INVALID_ARG"), (dict(scales=P + 2), "FA_ERR_INVALID_ARG"),
    (dict(R=0), "FA_ERR_INVALID_ARG"), (dict(N=0), "FA_ERR_INVALID_ARG"),
    (dict(N=1 << 24, d=128), "FA_ERR_INVALID_ARG"),
    (dict(d=96), "FA_ERR_UNSUPPORTED"), (dict(dtype=3), "FA_ERR_UNSUPPORTED"),
])
def test_quantize_validates(kw, status):
    assert quant(**kw) == getattr(fa, status)


def fwd8(**kw):
    a = dict(GOOD, Q=P, K=P, V=P, O=P, LSE=P, Hkv=2, stream=None)
    a.update(kw)
    return fa.fa_fwd_fp8(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["Hkv"], a["N"],
                         a["d"], a["causal"], a["softmax_scale"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), "FA_ERR_INVALID_ARG"), (dict(K=P + 2), "FA_ERR_INVALID_ARG"),
    (dict(V=None), "FA_ERR_INVALID_ARG"), (dict(O=P + 8), "FA_ERR_INVALID_ARG"),
    (dict(LSE=P + 2), "FA_ERR_INVALID_ARG"), (dict(Hkv=3), "FA_ERR_INVALID_ARG"),
    (dict(N=0), "FA_ERR_INVALID_ARG"), (dict(causal=5), "FA_ERR_INVALID_ARG"),
    (dict(softmax_scale=-1.0), "FA_ERR_INVALID_ARG"), (dict(d=32), "FA_ERR_UNSUPPORTED"),
])
def test_fwd_fp8_validates(kw, status):
    assert fwd8(**kw) == getattr(fa, status)


def quant_mx(**kw):
    a = dict(X=P, codes=P, scales=P + 1, R=2, N=16, d=128, dtype=0, stream=None)
    a.update(kw)
    return fa.fa_quantize_mx_e4m3(a["X"], a["codes"], a["scales"], a["R"], a["N"], a["d"],
                                  a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), "FA_ERR_INVALID_ARG"), (dict(X=P + 2), "FA_ERR_INVALID_ARG"),
    (dict(codes=None), "FA_ERR_INVALID_ARG"), (dict(codes=P + 4), "FA_ERR_INVALID_ARG"),
    (dict(scales=None), "FA_ERR_INVALID_ARG"),
    (dict(R=0), "FA_ERR_INVALID_ARG"), (dict(N=0), "FA_ERR_INVALID_ARG"),
    (dict(R=1 << 14, N=1 << 22, d=64), "FA_ERR_INVALID_ARG"),
    (dict(d=96), "FA_ERR_UNSUPPORTED"), (dict(dtype=3), "FA_ERR_UNSUPPORTED"),
])
def test_quantize_mx_validates(kw, status):
    assert quant_mx(**kw) == getattr(fa, status)


def fwd_mx(**kw):
    a = dict(GOOD, Q=P, K=P, V=P, O=P, LSE=P, Hkv=2, stream=None)
    a.update(kw)
    return fa.fa_fwd_mxfp8(a["Q"], a["K"], a["V"], a["O"], a["LSE"], a["B"], a["H"], a["Hkv"],
                           a["N"], a["d"], a["causal"], a["softmax_scale"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(Q=None), "FA_ERR_INVALID_ARG"), (dict(K=P + 2), "FA_ERR_INVALID_ARG"),
    (dict(V=None), "FA_ERR_INVALID_ARG"), (dict(O=P + 8), "FA_ERR_INVALID_ARG"),
    (dict(LSE=P + 2), "FA_ERR_INVALID_ARG"), (dict(Hkv=3), "FA_ERR_INVALID_ARG"),
    (dict(N=0), "FA_ERR_INVALID_ARG"), (dict(causal=5), "FA_ERR_INVALID_ARG"),
    (dict(softmax_scale=-1.0), "FA_ERR_INVALID_ARG"), (dict(d=32), "FA_ERR_UNSUPPORTED"),
])
def test_fwd_mxfp8_validates(kw, status):
    assert fwd_mx(**kw) == getattr(fa, status)


def test_torch_fp8_wrappers_check_before_calling():
    import torch
    q = torch.zeros(1, 2, 4, 64, dtype=torch.float16)
    with pytest.raises(TypeError):    # the FP8 forward takes bf16 only
        fa.forward_fp8(q, q, q)
    with pytest.raises(TypeError):
        fa.quantize_e4m3(q.float())
    with pytest.raises(TypeError):
        fa.forward_mxfp8(q, q, q)
    with pytest.raises(TypeError):
        fa.quantize_mx_e4m3(q.float())


@pytest.mark.parametrize("dtype", [fa.FA_DTYPE_BF16, fa.FA_DTYPE_F16])
def test_noalloc_validates_like_bwd_ex(dtype):
    """fa_bwd_noalloc rejects what fa_bwd_ex rejects, before any HIP call."""
    def call(B=1, H=2, Hkv=2, N=16, d=128, causal=0, scale=0.125, LSE=P, dt=dtype, Q=P):
        return fa.fa_bwd_noalloc(Q, P, P, P, LSE, P, P, P, P, B, H, Hkv, N, d, causal, scale, dt, None)
    assert call(dt=7) == fa.FA_ERR_UNSUPPORTED
    assert call(d=96) == fa.FA_ERR_UNSUPPORTED
    assert call(B=0) == fa.FA_ERR_INVALID_ARG
    assert call(Hkv=3) == fa.FA_ERR_INVALID_ARG
    assert call(causal=2) == fa.FA_ERR_INVALID_ARG
    assert call(scale=float("nan")) == fa.FA_ERR_INVALID_ARG
    assert call(LSE=None) == fa.FA_ERR_INVALID_ARG
    assert call(Q=P + 8) == fa.FA_ERR_INVALID_ARG


def test_noalloc_rejects_problems_beyond_its_workspace():
    """B * H * N above FA_NOALLOC_MAX_ROWS is FA_ERR_TOO_LARGE, decided on the host."""
    M = fa.FA_NOALLOC_MAX_ROWS
    assert M == 2 ** 21
    # one row over: 1 x 1 x (M + 1) with d = 64 (N * d < 2^31)
    assert fa.fa_bwd_noalloc(P, P, P, P, P, P, P, P, P, 1, 1, 1, M + 1, 64, 1, 0.125,
                             fa.FA_DTYPE_BF16, None) == fa.FA_ERR_TOO_LARGE
    assert fa.fa_bwd_noalloc(P, P, P, P, P, P, P, P, P, 8, 64, 8, 4097, 128, 1, 0.125,
                             fa.FA_DTYPE_BF16, None) == fa.FA_ERR_TOO_LARGE
