"""GPU parity for the per-key attention mass (fa_key_mass, through the torch
wrapper) against the CPU fp64 oracle on the same bits.

"GPU Performance Optimization Batch 1 - Design Spec", Item 4 (SnapKV), Design:
the attention weights each key position receives are summed and reduced over
the heads. mass[b, j] = sum_h sum_i P[b, h, i, j].

Tolerance. The kernel recomputes S exactly up to float32 accumulation, takes
P = exp2(c S - LSE2) with the forward's float32 LSE, and sums in float32, so a
mass carries the relative error of its P entries: |dS| c + |dLSE| plus float32
summation over up to H N terms, about 1e-5 in practice. The bar is
max |mass_gpu - mass_ref| <= 1e-3 max |mass_ref| with the oracle's own LSE fed
in (the kernel alone). With the GPU forward's LSE (the pipeline) the bar is
2^-8: that LSE normalises by the sum of the bf16-rounded P (the weights of the
forward's P V product), so a row's recomputed probabilities sum to 1 within a
factor 1 +- 2^-8.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import announce, max_abs, rel_to_max, to_dev, to_f64

pytestmark = pytest.mark.gpu

MASS_RTOL = 1e-3
PIPE_RTOL = 2.0 ** -8


def _dec(x):
    return {k: oracle.bf16_bits_to_f64(v) for k, v in x.items()}


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 65, 129, 300, 513])
@pytest.mark.parametrize("H,Hkv", [(2, 2), (4, 1), (6, 3)])
def test_mass_small_every_key(fa, H, Hkv, N, causal, d):
    import torch
    B = 2
    seed = 8000 + 16 * N + 4 * H + Hkv + 2 * int(causal) + (d == 128)
    x = ai.make_qkv(B, H, N, d, seed, Hkv=Hkv)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    announce(f"mass small B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} seed={seed}")
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    f = _dec(x)
    ref = oracle.key_mass(f["q"], f["k"], causal, scale)
    _, lse_ref = oracle.attention_forward(f["q"], f["k"], f["v"], causal, scale)
    # the kernel alone: the oracle's LSE as input
    m1 = fa.key_mass(q, k, torch.from_numpy(lse_ref.astype(np.float32)).cuda(), causal, scale)
    # the pipeline: the GPU forward's LSE
    _, lse = fa.forward(q, k, v, causal, scale)
    m2 = fa.key_mass(q, k, lse, causal, scale)
    torch.cuda.synchronize()
    for m, tol in ((m1, MASS_RTOL), (m2, PIPE_RTOL)):
        assert tuple(m.shape) == (B, N)
        assert rel_to_max(to_f64(m), ref) <= tol
    # each query row's probabilities sum to 1
    assert np.allclose(to_f64(m1).sum(1), H * N, rtol=1e-4)
    assert np.allclose(to_f64(m2).sum(1), H * N, rtol=PIPE_RTOL)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [33, 300])
def test_mass_f16(fa, N, causal):
    """IEEE binary16 inputs, grouped K/V heads, the oracle's LSE fed in."""
    import torch
    B, H, Hkv, d = 2, 4, 2, 128
    seed = 8600 + N + int(causal)
    x = ai.make_qkv(B, H, N, d, seed, Hkv=Hkv, dtype="f16")
    scale = float(np.float32(1.0 / math.sqrt(d)))
    announce(f"mass f16 N={N} causal={causal} seed={seed}")
    f = {n: oracle.f16_bits_to_f64(b) for n, b in x.items()}
    ref = oracle.key_mass(f["q"], f["k"], causal, scale)
    _, lse_ref = oracle.attention_forward(f["q"], f["k"], f["v"], causal, scale)
    q, k = (torch.from_numpy(np.ascontiguousarray(x[n]).view(np.int16)).cuda().view(torch.float16)
            for n in ("q", "k"))
    m = fa.key_mass(q, k, torch.from_numpy(lse_ref.astype(np.float32)).cuda(), causal, scale)
    torch.cuda.synchronize()
    assert rel_to_max(to_f64(m), ref) <= MASS_RTOL
    assert np.allclose(to_f64(m).sum(1), H * N, rtol=1e-4)


def test_mass_identical_keys_closed_form(fa):
    """All keys equal: P is uniform over the visible keys, so key j gets mass
    H (non-causal) or H sum_{i >= j} 1 / (i + 1) (causal)."""
    import torch
    B, H, N, d = 2, 4, 700, 128
    x = ai.make_qkv(B, H, N, d, 8500)
    kbits = np.repeat(x["k"][:, :, :1], N, axis=2)
    q, k, v = to_dev(x["q"]), to_dev(kbits), to_dev(x["v"])
    scale = float(np.float32(1.0 / math.sqrt(d)))
    for causal in (False, True):
        _, lse = fa.forward(q, k, v, causal, scale)
        m = to_f64(fa.key_mass(q, k, lse, causal, scale))
        torch.cuda.synchronize()
        if causal:
            tail = np.cumsum(1.0 / np.arange(N, 0, -1))[::-1]  # sum_{i >= j} 1 / (i + 1)
            ref = H * tail
        else:
            ref = np.full(N, float(H))
        assert rel_to_max(m, np.broadcast_to(ref, m.shape)) <= PIPE_RTOL, causal


@pytest.mark.parametrize("causal", [True, False])
def test_mass_full_size(fa, causal):
    """4 x 64 x 4096 x 128 (the benchmark's shape): every batch's masses sum to
    H N, and one whole batch against the oracle (all 64 heads)."""
    import torch
    w = ai.WORKLOADS["c5"]
    B, H, N, d = w.B, w.H, w.N, w.d
    x = ai.make_qkv(B, H, N, d, w.seed, sigma_qk=w.sigma_qk, sigma_v=w.sigma_v)
    announce(f"mass full size {w.label} causal={causal} on GPU")
    q, k, v = to_dev(x["q"]), to_dev(x["k"]), to_dev(x["v"])
    _, lse = fa.forward(q, k, v, causal, w.scale)
    m = to_f64(fa.key_mass(q, k, lse, causal, w.scale))
    torch.cuda.synchronize()
    assert np.all(m >= 0)
    assert np.allclose(m.sum(1), H * N, rtol=PIPE_RTOL)
    b = B - 1
    announce("mass full size: oracle for one batch")
    ref = np.zeros(N)
    for h in range(H):
        p, _ = oracle.head_probs(oracle.bf16_bits_to_f64(x["q"][b, h]),
                                 oracle.bf16_bits_to_f64(x["k"][b, h]), causal, w.scale)
        ref += p.sum(axis=0)
        del p
    assert rel_to_max(m[b], ref) <= PIPE_RTOL
