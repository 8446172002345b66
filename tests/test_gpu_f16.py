"""GPU parity for IEEE binary16 inputs (fa_fwd_ex / fa_bwd_ex with FA_DTYPE_F16,
through the torch wrappers) against the CPU fp64 oracle on the same bits.

The page that describes the method lists FP16 next to BF16 ("RTX Flash
Attention Implementation COMPLETE", Advanced Features, Mixed Precision) and
builds F16 inputs in its Usage Examples. The acceptance bars are the bf16 ones:
binary16 carries more mantissa bits, so they hold with margin.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import GRAD_RTOL, LSE_ATOL, O_ATOL, announce, max_abs, rel_to_max, to_f64

pytestmark = pytest.mark.gpu


def to_dev_f16(bits, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to(device)


def _run(fa, x, causal, scale):
    import torch
    q, k, v, do = (to_dev_f16(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal, scale)
    assert o.dtype == torch.float16
    dq, dk, dv = fa.backward(do, q, k, v, o, lse, causal, scale)
    torch.cuda.synchronize()
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _check_heads(g, f, causal, scale, heads):
    for b, h in heads:
        q, k, v, do = (f[n][b, h] for n in ("q", "k", "v", "do"))
        o_ref, lse_ref = oracle.head_forward(q, k, v, causal, scale)
        grads = oracle.head_backward(q, k, v, do, causal, scale)
        assert max_abs(to_f64(g["o"][b, h]), o_ref) <= O_ATOL, (b, h)
        assert max_abs(to_f64(g["lse"][b, h]), lse_ref) <= LSE_ATOL, (b, h)
        for name, ref in zip(("dq", "dk", "dv"), grads):
            err = rel_to_max(to_f64(g[name][b, h]), ref) if np.max(np.abs(ref)) > 0 \
                else max_abs(to_f64(g[name][b, h]), ref)
            assert err <= GRAD_RTOL, (name, b, h, err)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 129, 300, 513])
def test_f16_small_shapes_every_element(fa, N, causal, d):
    seed = 5000 + N * 4 + 2 * int(causal) + (d == 128)
    x = ai.make_qkv(1, 2, N, d, seed, with_do=True, dtype="f16")
    scale = float(np.float32(1.0 / math.sqrt(d)))
    announce(f"f16 small N={N} d={d} causal={causal} seed={seed}")
    g = _run(fa, x, causal, scale)
    f = {n: oracle.f16_bits_to_f64(b) for n, b in x.items()}
    _check_heads(g, f, causal, scale, [(0, 0), (0, 1)])


@pytest.mark.parametrize("causal", [False, True])
def test_f16_large_logits(fa, causal):
    """Q, K ~ N(0, 3^2), as in the 4x64x4096x128 workload."""
    x = ai.make_qkv(1, 2, 1000, 128, 8123, sigma_qk=3.0, with_do=True, dtype="f16")
    scale = float(np.float32(1.0 / math.sqrt(128)))
    announce(f"f16 large-logit causal={causal}")
    g = _run(fa, x, causal, scale)
    f = {n: oracle.f16_bits_to_f64(b) for n, b in x.items()}
    _check_heads(g, f, causal, scale, [(0, 0), (0, 1)])


def test_f16_medium_workload_sampled_heads(fa):
    """The 4x32x1024x128 causal shape in binary16, fwd + bwd, three heads checked."""
    x = ai.make_qkv(4, 32, 1024, 128, 2, with_do=True, dtype="f16")
    scale = float(np.float32(1.0 / math.sqrt(128)))
    announce("f16 4x32x1024x128 causal")
    g = _run(fa, x, True, scale)
    f = {n: oracle.f16_bits_to_f64(b) for n, b in x.items()}
    _check_heads(g, f, True, scale, [(0, 0), (1, 17), (3, 31)])
