"""GPU parity for the FP8 (E4M3) path: fa_quantize_e4m3 and fa_fwd_fp8 (through
the torch wrappers) against the CPU fp64 oracle on the same bits.

"GPU Performance Optimization Batch 1 - Design Spec", Item 3, Design, optional
FP8 path: every 16 x 16 block of Q and K is quantised to E4M3 with a scale of
its own before S = Q K^T. The codes are integer decisions taken from float
values, so both sides take them in the same precision (the inputs are exact in
float32 and the scaling by a power of two is exact): codes and scales must be
bit-identical. The forward is then exact attention on the dequantised Q and K
and is held to the bf16 path's bars.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import LSE_ATOL, O_ATOL, announce, max_abs, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _dev16(bits, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda")
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16)


def _decode(bits, dtype):
    return oracle.bf16_bits_to_f64(bits) if dtype == "bf16" else oracle.f16_bits_to_f64(bits)


def _bits(values, dtype):
    """16-bit patterns of values exactly representable in the type."""
    v32 = np.asarray(values, dtype=np.float32)
    bits = ai.f32_to_bf16_bits(v32) if dtype == "bf16" else ai.f32_to_f16_bits(v32)
    assert np.array_equal(_decode(bits, dtype), v32.astype(np.float64)), "not exact in the type"
    return bits


def _check_quant(fa, bits, dtype, label):
    import torch
    announce(f"fp8 quantise {label} {dtype} shape={bits.shape}")
    codes, scales = fa.quantize_e4m3(_dev16(bits, dtype))
    torch.cuda.synchronize()
    R = int(np.prod(bits.shape[:-2]))
    N, d = bits.shape[-2:]
    rc, re, _ = oracle.quantize_e4m3_blocks(_decode(bits, dtype).reshape(R, N, d))
    gc = codes.cpu().numpy().reshape(R, N, d)
    gs = scales.cpu().numpy().astype(np.float64).reshape(re.shape)
    bad = np.argwhere(gc != rc)
    assert len(bad) == 0, (label, bad[:5].tolist(), gc[tuple(bad[0])], rc[tuple(bad[0])])
    assert np.array_equal(gs, np.ldexp(1.0, re)), label


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 15, 16, 17, 100, 257])
def test_quantise_random_bit_exact(fa, N, d, dtype):
    rng = np.random.default_rng(9000 + N + d)
    R = 3
    # per-matrix magnitudes from 2^-12 to 2^12 (f16: within its range)
    mags = 2.0 ** rng.uniform(-12, 12, (R, 1, 1)) if dtype == "bf16" else 2.0 ** rng.uniform(-6, 6, (R, 1, 1))
    x = (rng.standard_normal((R, N, d)) * mags).astype(np.float32)
    bits = ai.f32_to_bf16_bits(x) if dtype == "bf16" else ai.f32_to_f16_bits(x)
    _check_quant(fa, bits, dtype, f"random N={N} d={d}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_quantise_edge_values_bit_exact(fa, dtype):
    """Blocks built to hit every branch: ties between E4M3 neighbours (to even),
    the top value exactly 448 * 2^e and just above it, E4M3 subnormals and
    values that round to zero (negative ones included, encoded +0), an all-zero
    block, and (bf16) a tiny block whose scale stops at 2^-100."""
    rng = np.random.default_rng(9100)
    grid = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))  # 0 .. 448
    mids = (grid[1:] + grid[:-1]) / 2                                # all ties
    blocks = []
    for e in (-4, 0, 3):
        b = rng.choice(np.concatenate([mids, -mids]), size=(16, 16))
        b[0, 0] = 448.0                         # top exactly 448 * 2^e: scale 2^e
        blocks.append(b * 2.0 ** e)
        b2 = b.copy()
        b2[0, 0] = 448.0 + 32.0                 # just above: scale 2^(e+1), ties move
        blocks.append(b2 * 2.0 ** e)
    sub = rng.choice(np.concatenate([grid[:9], -grid[:9], [2.0 ** -10, -2.0 ** -10, 3 * 2.0 ** -11]]),
                     size=(16, 16))
    sub[0, 0] = 448.0
    blocks.append(sub)                          # E4M3 subnormals and values rounding to 0
    blocks.append(np.zeros((16, 16)))           # all zero
    if dtype == "bf16":
        tiny = ai.f32_to_bf16_bits((rng.standard_normal((16, 16)) * 2.0 ** -110).astype(np.float32))
        blocks.append(oracle.bf16_bits_to_f64(tiny))                  # scale stops at 2^-100
    # f16 holds 11 significant bits and exponents down to 2^-24: keep e >= -4 there
    # four 16-column blocks per row block (d = 64): the block, mirrored, negated, flipped
    x = np.concatenate([np.concatenate([b, np.flip(b, 1), -b, np.flip(b, 0)], axis=1)
                        for b in blocks], axis=0)
    bits = _bits(x[None], dtype)
    _check_quant(fa, bits, dtype, "edges")


def test_quantise_workload_shape(fa):
    """The benchmark's Q at 4 x 64 x 4096 x 128 (N(0, 3^2) entries)."""
    w = ai.WORKLOADS["c5"]
    x = ai.make_qkv(w.B, w.H, w.N, w.d, w.seed, sigma_qk=w.sigma_qk, sigma_v=w.sigma_v)
    _check_quant(fa, x["q"][:1, :8], "bf16", "c5 q, 8 heads")
    import torch
    codes, scales = fa.quantize_e4m3(to_dev(x["q"]))
    torch.cuda.synchronize()
    assert tuple(codes.shape) == (w.B, w.H, w.N, w.d) and tuple(scales.shape) == (w.B, w.H, 256, 8)
    # every head: the top scaled magnitude of each block lies in (224, 448]
    q = to_dev(x["q"]).float().view(w.B, w.H, 256, 16, 8, 16).abs().amax(dim=(3, 5))
    top = (q / scales).cpu().numpy()
    assert np.all((top > 224) & (top <= 448))


def _run8(fa, x, causal, scale):
    import torch
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    o, lse = fa.forward_fp8(q, k, v, causal, scale)
    torch.cuda.synchronize()
    return q, k, v, o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 65, 129, 300])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 1)])
def test_fwd_fp8_small_every_element(fa, H, Hkv, N, causal, d):
    B = 1
    seed = 9200 + 8 * N + 2 * H + Hkv + 2 * int(causal) + (d == 128)
    x = ai.make_qkv(B, H, N, d, seed, Hkv=Hkv, sigma_qk=2.0)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    announce(f"fp8 fwd small H={H} Hkv={Hkv} N={N} d={d} causal={causal} seed={seed}")
    _, _, _, o, lse = _run8(fa, x, causal, scale)
    f = {n: oracle.bf16_bits_to_f64(b) for n, b in x.items()}
    o_ref, lse_ref = oracle.fp8_attention_forward(f["q"], f["k"], f["v"], causal, scale)
    assert max_abs(to_f64(o), o_ref) <= O_ATOL
    assert max_abs(to_f64(lse), lse_ref) <= LSE_ATOL


def test_fwd_fp8_equals_plain_forward_on_dequantised(fa):
    """fa_fwd_fp8(q, k, v) is fa_fwd on decode(codes) * scales, bit for bit."""
    import torch
    B, H, Hkv, N, d = 2, 4, 2, 333, 128
    x = ai.make_qkv(B, H, N, d, 9300, Hkv=Hkv, sigma_qk=3.0)
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    for causal in (False, True):
        o8, l8 = fa.forward_fp8(q, k, v, causal, 0.09)

        def deq(t):
            c, s = fa.quantize_e4m3(t)
            vals = c.view(torch.float8_e4m3fn).float()
            sc = s.repeat_interleave(16, dim=-2)[..., :N, :].repeat_interleave(16, dim=-1)
            return (vals * sc).to(torch.bfloat16)

        o, lse = fa.forward(deq(q), deq(k), v, causal, 0.09)
        torch.cuda.synchronize()
        assert torch.equal(o8, o) and torch.equal(l8, lse)


@pytest.mark.parametrize("causal", [True, False])
def test_fwd_fp8_full_size(fa, causal):
    """4 x 64 x 4096 x 128 (the benchmark's inputs): 8 whole heads and sampled
    rows of 24 more against the oracle."""
    import torch
    w = ai.WORKLOADS["c5"]
    x = ai.make_qkv(w.B, w.H, w.N, w.d, w.seed, sigma_qk=w.sigma_qk, sigma_v=w.sigma_v)
    announce(f"fp8 fwd full size {w.label} causal={causal} on GPU")
    _, _, _, o, lse = _run8(fa, x, causal, w.scale)
    o, lse = to_f64(o), to_f64(lse)
    torch.cuda.empty_cache()
    rng = np.random.default_rng(9400 + int(causal))
    heads = [(0, 0), (w.B - 1, w.H - 1)] + [(int(rng.integers(w.B)), int(rng.integers(w.H)))
                                            for _ in range(30)]
    for n, (b, h) in enumerate(heads):
        qd = oracle.quantize_e4m3_blocks(oracle.bf16_bits_to_f64(x["q"][b, h])[None])[2][0]
        kd = oracle.quantize_e4m3_blocks(oracle.bf16_bits_to_f64(x["k"][b, h])[None])[2][0]
        vv = oracle.bf16_bits_to_f64(x["v"][b, h])
        if n < 8:
            ro, rl = oracle.head_forward(qd, kd, vv, causal, w.scale)
            assert max_abs(o[b, h], ro) <= O_ATOL and max_abs(lse[b, h], rl) <= LSE_ATOL, (b, h)
        else:
            rows = np.unique(np.concatenate([[0, w.N - 1], rng.integers(0, w.N, 6)]))
            ro, rl = oracle.rows_forward(qd[rows], kd, vv, rows, causal, w.scale)
            assert max_abs(o[b, h, rows], ro) <= O_ATOL and max_abs(lse[b, h, rows], rl) <= LSE_ATOL
