"""GPU parity for the FP8 (E4M3) path under the 1 x 32 block reading:
fa_quantize_mx_e4m3 and fa_fwd_mxfp8 (through the torch wrappers) against the
CPU fp64 oracle on the same bits.

"GPU Performance Optimization Batch 1 - Design Spec", Item 3, Design,
optional FP8 path, read with the MX block-wise quantisation of the same
spec's Item 2 (Current state): each block of one row by 32 consecutive
columns of Q and K is quantised to E4M3 with a power-of-two scale of its own
before S = Q K^T. Codes and scale bytes are integer decisions taken from
float values that are exact in float32 and scaled by powers of two, so they
must be bit-identical. The forward is exact attention on the dequantised Q
and K, with S from the scaled FP8 matrix instruction (float32 sums of exact
FP8 products), held to the bf16 path's bars.
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
    announce(f"mx quantise {label} {dtype} shape={bits.shape}")
    codes, scales = fa.quantize_mx_e4m3(_dev16(bits, dtype))
    torch.cuda.synchronize()
    R = int(np.prod(bits.shape[:-2]))
    N, d = bits.shape[-2:]
    rc, re, _ = oracle.quantize_e4m3_rows32(_decode(bits, dtype).reshape(R, N, d))
    gc = codes.cpu().numpy().reshape(R, N, d)
    gs = scales.cpu().numpy().astype(np.int64).reshape(R, N, d // 32)
    bad = np.argwhere(gc != rc)
    assert len(bad) == 0, (label, bad[:5].tolist(), gc[tuple(bad[0])], rc[tuple(bad[0])])
    assert np.array_equal(gs - 127, re), label


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 31, 100, 257])
def test_quantise_random_bit_exact(fa, N, d, dtype):
    rng = np.random.default_rng(9500 + N + d)
    R = 3
    # per-row magnitudes from 2^-12 to 2^12 (f16: within its range)
    lim = 12 if dtype == "bf16" else 6
    x = (rng.standard_normal((R, N, d)) * 2.0 ** rng.uniform(-lim, lim, (R, N, 1))).astype(np.float32)
    bits = ai.f32_to_bf16_bits(x) if dtype == "bf16" else ai.f32_to_f16_bits(x)
    _check_quant(fa, bits, dtype, f"random N={N} d={d}")


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_quantise_edge_values_bit_exact(fa, dtype):
    """Rows built to hit every branch: ties between E4M3 neighbours (to even),
    a block's top exactly 448 * 2^e and just above it, E4M3 subnormals and
    values that round to zero (negative ones included, encoded +0), an
    all-zero block, and (bf16) a tiny block whose scale stops at 2^-100."""
    rng = np.random.default_rng(9600)
    grid = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (grid[1:] + grid[:-1]) / 2
    rows = []
    for e in (-4, 0, 3):
        b = rng.choice(np.concatenate([mids, -mids]), size=64)
        b[0] = 448.0
        b[32] = -448.0
        rows.append(b * 2.0 ** e)
        b2 = b.copy()
        b2[5] = 448.0 + 32.0
        rows.append(b2 * 2.0 ** e)
    sub = rng.choice(np.concatenate([grid[:9], -grid[:9], [2.0 ** -10, -2.0 ** -10, 3 * 2.0 ** -11]]), size=64)
    sub[0] = sub[32] = 448.0
    rows.append(sub)
    rows.append(np.zeros(64))
    if dtype == "bf16":
        tiny = ai.f32_to_bf16_bits((rng.standard_normal(64) * 2.0 ** -110).astype(np.float32))
        rows.append(oracle.bf16_bits_to_f64(tiny))
    x = np.stack(rows)                                              # [rows, 64]
    x = np.concatenate([x, np.flip(-x, 1)], axis=1)                 # d = 128
    _check_quant(fa, _bits(x[None], dtype), dtype, "edges")


def _run(fa, x, causal, scale):
    import torch
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    o, lse = fa.forward_mxfp8(q, k, v, causal, scale)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 65, 129, 300, 513])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 1)])
def test_fwd_mxfp8_small_every_element(fa, H, Hkv, N, causal, d):
    B = 1
    seed = 9700 + 8 * N + 2 * H + Hkv + 2 * int(causal) + (d == 128)
    x = ai.make_qkv(B, H, N, d, seed, Hkv=Hkv, sigma_qk=2.0)
    # rows of different magnitudes (factors 1/2, 1, 2: the rows' 1 x 32 scales
    # differ, and the logits stay in the range the bars are written for)
    rng = np.random.default_rng(seed)
    for name in ("q", "k"):
        f = oracle.bf16_bits_to_f64(x[name]) * 2.0 ** rng.integers(-1, 2, x[name].shape[:-1] + (1,))
        x[name] = ai.f32_to_bf16_bits(f.astype(np.float32))
    scale = float(np.float32(1.0 / math.sqrt(d)))
    announce(f"mx fwd small H={H} Hkv={Hkv} N={N} d={d} causal={causal} seed={seed}")
    o, lse = _run(fa, x, causal, scale)
    f = {n: oracle.bf16_bits_to_f64(b) for n, b in x.items()}
    o_ref, lse_ref = oracle.mx_fp8_attention_forward(f["q"], f["k"], f["v"], causal, scale)
    assert max_abs(to_f64(o), o_ref) <= O_ATOL
    assert max_abs(to_f64(lse), lse_ref) <= LSE_ATOL


@pytest.mark.parametrize("causal", [True, False])
def test_fwd_mxfp8_full_size(fa, causal):
    """4 x 64 x 4096 x 128 (the benchmark's inputs): 8 whole heads and sampled
    rows of 24 more against the oracle."""
    import torch
    w = ai.WORKLOADS["c5"]
    x = ai.make_qkv(w.B, w.H, w.N, w.d, w.seed, sigma_qk=w.sigma_qk, sigma_v=w.sigma_v)
    announce(f"mx fwd full size {w.label} causal={causal} on GPU")
    o, lse = _run(fa, x, causal, w.scale)
    o, lse = to_f64(o), to_f64(lse)
    torch.cuda.empty_cache()
    rng = np.random.default_rng(9800 + int(causal))
    heads = [(0, 0), (w.B - 1, w.H - 1)] + [(int(rng.integers(w.B)), int(rng.integers(w.H)))
                                            for _ in range(30)]
    for n, (b, h) in enumerate(heads):
        qd = oracle.quantize_e4m3_rows32(oracle.bf16_bits_to_f64(x["q"][b, h])[None])[2][0]
        kd = oracle.quantize_e4m3_rows32(oracle.bf16_bits_to_f64(x["k"][b, h])[None])[2][0]
        vv = oracle.bf16_bits_to_f64(x["v"][b, h])
        if n < 8:
            ro, rl = oracle.head_forward(qd, kd, vv, causal, w.scale)
            assert max_abs(o[b, h], ro) <= O_ATOL and max_abs(lse[b, h], rl) <= LSE_ATOL, (b, h)
        else:
            rows = np.unique(np.concatenate([[0, w.N - 1], rng.integers(0, w.N, 6)]))
            ro, rl = oracle.rows_forward(qd[rows], kd, vv, rows, causal, w.scale)
            assert max_abs(o[b, h, rows], ro) <= O_ATOL and max_abs(lse[b, h, rows], rl) <= LSE_ATOL
