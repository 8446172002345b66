"""fa_bwd_noalloc (the backward for callers that cannot allocate: its row
statistics live in the library's static per-device workspace) against
fa_bwd_ex, through the C ABI, on two calls in a row, the second smaller.

The first call, at 4 x 64 x 4096 x 128 causal (2^20 query rows, half the
workspace), has one query head per K/V head, so fa_bwd_ex runs the same
kernels with the same dK/dV schedule: the results must be bitwise equal. The
second, smaller call (multi-query, 300 rows) has fa_bwd_ex split the dK/dV
work over query heads while fa_bwd_noalloc does not, so dK and dV are summed
in another order: they must agree within the gradient bar, and both must
match the oracle. The second call also runs over what the first left in the
workspace.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import GRAD_RTOL, announce, rel_to_max, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _both(fa, x, B, H, Hkv, N, d, causal, scale):
    import torch
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal, scale)
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for entry in (fa.fa_bwd_ex, fa.fa_bwd_noalloc):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        rc = entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                   do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, Hkv, N, d,
                   causal, scale, fa.FA_DTYPE_BF16, stream)
        assert rc == fa.FA_OK, fa.fa_status_string(rc)
        outs.append((dq, dk, dv))
    torch.cuda.synchronize()
    return outs


def test_noalloc_matches_bwd_ex_twice(fa):
    import torch
    # call 1: the 4x64x4096x128 causal workload's shape
    w = ai.WORKLOADS["c5"]
    announce(f"no-alloc call 1: {w.label} causal")
    x = ai.make_inputs(w)
    ref, got = _both(fa, x, w.B, w.H, w.H, w.N, w.d, True, w.scale)
    for name, a, b in zip(("dq", "dk", "dv"), ref, got):
        assert torch.equal(a, b), name
    del x, ref, got
    torch.cuda.empty_cache()

    # call 2: smaller, one K/V head for two query heads (fa_bwd_ex splits the dK/dV work)
    B, H, Hkv, N, d, causal = 1, 2, 1, 300, 64, False
    scale = float(np.float32(1.0 / math.sqrt(d)))
    announce(f"no-alloc call 2: B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal}")
    x = ai.make_qkv(B, H, N, d, 515, with_do=True, Hkv=Hkv)
    ref, got = _both(fa, x, B, H, Hkv, N, d, causal, scale)
    f = {n: oracle.bf16_bits_to_f64(b) for n, b in x.items()}
    grads = oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], causal, scale)
    for name, a, b, r in zip(("dq", "dk", "dv"), ref, got, grads):
        assert rel_to_max(to_f64(b), to_f64(a)) <= GRAD_RTOL, name
        assert rel_to_max(to_f64(b), r) <= GRAD_RTOL, name
    assert torch.equal(ref[0], got[0])  # dQ does not depend on the dK/dV split


def test_noalloc_rejects_oversize_on_device(fa):
    """Beyond the workspace: FA_ERR_TOO_LARGE, nothing enqueued (outputs untouched)."""
    import torch
    M = fa.FA_NOALLOC_MAX_ROWS
    t = torch.full((16,), 3.0, dtype=torch.bfloat16, device="cuda")
    p = t.data_ptr()
    rc = fa.fa_bwd_noalloc(p, p, p, p, p, p, p, p, p, 1, 2, 2, M // 2 + 1, 64, 1, 0.125,
                           fa.FA_DTYPE_BF16, torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_ERR_TOO_LARGE
    torch.cuda.synchronize()
    assert bool((t.float() == 3.0).all())
