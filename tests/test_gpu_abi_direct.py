"""The contract's own entry points on the GPU: fa_fwd and fa_bwd called through
ctypes with raw device pointers from torch allocations and the current stream
(no torch-level convenience in between), compared with the oracle.

"RTX Flash Attention Implementation COMPLETE", Usage Examples: forward(q, k, v,
causal, scale) gives the output and the LSE; backward(dout, q, k, v, out, lse,
causal, scale) gives dq, dk, dv; tensors are [batch, heads, seq_len,
head_dim].
"""
import ctypes
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import GRAD_RTOL, LSE_ATOL, O_ATOL, announce, max_abs, rel_to_max, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _call_direct(fa, x, B, H, N, d, causal, scale):
    """fa_fwd then fa_bwd through the raw ctypes handles of libfa.so."""
    import torch
    lib = fa.load()
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    B, H, N, d, int(causal), ctypes.c_float(scale), stream)
    assert rc == 0, lib.fa_status_string(rc)
    rc = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                    B, H, N, d, int(causal), ctypes.c_float(scale), stream)
    assert rc == 0, lib.fa_status_string(rc)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv


def _compare(x, outs, causal, scale):
    o, lse, dq, dk, dv = outs
    f = {n: oracle.bf16_bits_to_f64(b) for n, b in x.items()}
    o_ref, lse_ref = oracle.attention_forward(f["q"], f["k"], f["v"], causal, scale)
    assert max_abs(to_f64(o), o_ref) <= O_ATOL
    assert max_abs(to_f64(lse), lse_ref) <= LSE_ATOL
    grads = oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], causal, scale)
    for name, g, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), grads):
        err = rel_to_max(to_f64(g), ref)
        assert err <= GRAD_RTOL, (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_direct_calls_ragged(fa, causal):
    B, H, N, d = 2, 3, 777, 128
    seed = 4242 + int(causal)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    announce(f"abi direct ragged B={B} H={H} N={N} d={d} causal={causal} seed={seed}")
    x = ai.make_qkv(B, H, N, d, seed, with_do=True)
    _compare(x, _call_direct(fa, x, B, H, N, d, causal, scale), causal, scale)


def test_direct_calls_medium_workload(fa):
    """The 4x32x1024x128 causal workload (its own Q, K, V bits; dO drawn after them)."""
    w = ai.WORKLOADS["c2"]
    announce(f"abi direct workload c2 {w.label}")
    x = ai.make_qkv(w.B, w.H, w.N, w.d, w.seed, sigma_qk=w.sigma_qk, sigma_v=w.sigma_v, with_do=True)
    _compare(x, _call_direct(fa, x, w.B, w.H, w.N, w.d, True, w.scale), True, w.scale)


def test_direct_errors_enqueue_nothing(fa):
    """Calls that fail validation return their status (with its string) and leave
    the outputs untouched: nothing was enqueued."""
    import torch
    lib = fa.load()
    B, H, N, d = 1, 2, 64, 128
    x = ai.make_qkv(B, H, N, d, 17, with_do=True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o = torch.full_like(q, 7.0)
    lse = torch.full((B, H, N), 7.0, dtype=torch.float32, device="cuda")
    dq = torch.full_like(q, 7.0)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cases = [  # (d, scale, causal, expected status)
        (96, 0.1, 1, 2),           # unsupported head dimension
        (d, float("nan"), 1, 1),   # scale not finite
        (d, -1.0, 0, 1),           # scale not positive
        (d, 0.1, 2, 1),            # causal flag not 0/1
    ]
    for dd, sc, cz, want in cases:
        rc = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        B, H, N, dd, cz, ctypes.c_float(sc), stream)
        assert rc == want, (dd, sc, cz, rc)
        rc = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        do.data_ptr(), dq.data_ptr(), dq.data_ptr(), dq.data_ptr(),
                        B, H, N, dd, cz, ctypes.c_float(sc), stream)
        assert rc == want, (dd, sc, cz, rc)
        assert lib.fa_status_string(rc).decode().startswith(
            "FA_ERR_UNSUPPORTED" if want == 2 else "FA_ERR_INVALID_ARG")
    # a misaligned pointer (2 bytes into q: not 16-byte aligned)
    rc = lib.fa_fwd(q.data_ptr() + 2, k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    B, H, N, d, 1, ctypes.c_float(0.1), stream)
    assert rc == 1
    torch.cuda.synchronize()
    assert bool((o.float() == 7.0).all()) and bool((lse == 7.0).all()) and bool((dq.float() == 7.0).all())
