"""Rows past the end of the sequence must read as zeros, never as neighbouring memory.

Every kernel reads its tiles through buffer resources that end at row N, so
the rows of a ragged last tile, the whole tiles the schedules run past the end
(the dQ pass rounds its key tiles up to a multiple of four, the dK/dV pass
pads its query steps to a multiple of three), and the row statistics of those
rows read as zeros and touch no memory. Causal masking and the end-of-sequence
mask of "RTX Flash Attention Implementation COMPLETE" (Advanced Features;
Technical Implementation Details, 2. Memory Tiling Strategy) then exclude
them exactly.

Here each input lives at the start of a larger allocation whose tail (1 MiB)
holds NaN bit patterns. A read past a head's rows into the tail would carry a
NaN through a product (0 x NaN is NaN) into the outputs. Every output of
fa_fwd, fa_bwd, fa_key_mass, fa_fwd_fp8 and fa_fwd_mxfp8 must be finite and within the
oracle bars. With one K/V head the last query heads share it, so K and V end
at the tail too.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import GRAD_RTOL, LSE_ATOL, O_ATOL, announce, max_abs, rel_to_max, to_f64

pytestmark = pytest.mark.gpu

TAIL_BYTES = 1 << 20
BF16_NAN = 0x7FC0
MASS_RTOL = 2.0 ** -8   # the pipeline bar of the key-mass tests (GPU forward's LSE)


def _nan_tailed_bf16(bits: np.ndarray):
    """A bf16 device tensor holding `bits`, followed in its allocation by TAIL_BYTES of NaN."""
    import torch
    n = bits.size
    flat = torch.full((n + TAIL_BYTES // 2,), BF16_NAN, dtype=torch.int16, device="cuda")
    flat[:n] = torch.from_numpy(np.ascontiguousarray(bits).reshape(-1).view(np.int16)).cuda()
    return flat[:n].view(bits.shape).view(torch.bfloat16)


def _nan_tailed_like(t):
    """A copy of device tensor t followed in its allocation by TAIL_BYTES of NaN."""
    import torch
    n = t.numel()
    flat = torch.full((n + TAIL_BYTES // t.element_size(),), float("nan"), dtype=t.dtype,
                      device=t.device)
    flat[:n] = t.reshape(-1)
    return flat[:n].view(t.shape)


def _finite(name, t):
    import torch
    assert bool(torch.isfinite(t.float()).all().item()), f"{name} holds non-finite values"


CASES = [  # B, H, Hkv, N, d, causal
    (1, 2, 2, 65, 128, False),
    (1, 2, 2, 65, 128, True),
    (1, 2, 2, 300, 64, False),
    (1, 2, 2, 300, 64, True),
    (1, 2, 1, 1000, 128, True),    # one K/V head: split dK/dV partial sums
    (1, 3, 3, 1000, 128, False),
    (1, 1, 1, 4096, 128, True),    # dK/dV padding steps past N; dQ round-up past N
]


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", CASES)
def test_nan_tails_stay_out(fa, B, H, Hkv, N, d, causal):
    import torch
    seed = 9100 + N + 7 * H + Hkv + int(causal)
    announce(f"oob B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} seed={seed}")
    x = ai.make_qkv(B, H, N, d, seed, with_do=True, Hkv=Hkv)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q, k, v, do = (_nan_tailed_bf16(x[n]) for n in ("q", "k", "v", "do"))

    o, lse = fa.forward(q, k, v, causal, scale)
    o_t, lse_t = _nan_tailed_like(o), _nan_tailed_like(lse)
    dq, dk, dv = fa.backward(do, q, k, v, o_t, lse_t, causal, scale)
    mass = fa.key_mass(q, k, lse_t, causal, scale)
    o8, lse8 = fa.forward_fp8(q, k, v, causal, scale)
    om, lsem = fa.forward_mxfp8(q, k, v, causal, scale)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv), ("mass", mass),
                    ("O fp8", o8), ("LSE fp8", lse8), ("O mxfp8", om), ("LSE mxfp8", lsem)):
        _finite(name, t)

    f = {n: oracle.bf16_bits_to_f64(b) for n, b in x.items()}
    o_ref, lse_ref = oracle.attention_forward(f["q"], f["k"], f["v"], causal, scale)
    assert max_abs(to_f64(o), o_ref) <= O_ATOL
    assert max_abs(to_f64(lse), lse_ref) <= LSE_ATOL
    grads = oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], causal, scale)
    for name, g, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), grads):
        err = rel_to_max(to_f64(g), ref)
        assert err <= GRAD_RTOL, (name, err)
    assert rel_to_max(to_f64(mass), oracle.key_mass(f["q"], f["k"], causal, scale)) <= MASS_RTOL
    o8_ref, lse8_ref = oracle.fp8_attention_forward(f["q"], f["k"], f["v"], causal, scale)
    assert max_abs(to_f64(o8), o8_ref) <= O_ATOL
    assert max_abs(to_f64(lse8), lse8_ref) <= LSE_ATOL
    om_ref, lsem_ref = oracle.mx_fp8_attention_forward(f["q"], f["k"], f["v"], causal, scale)
    assert max_abs(to_f64(om), om_ref) <= O_ATOL
    assert max_abs(to_f64(lsem), lsem_ref) <= LSE_ATOL
