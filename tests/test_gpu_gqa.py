"""GPU parity for grouped K/V heads (multi-query and grouped-query attention)
through fa_fwd_ex / fa_bwd_ex, against the CPU fp64 oracle on the same bits.

The dK/dV kernel has two paths: one workgroup per key block sums the whole
group of G = H / Hkv query heads and writes dK, dV; or, when B * Hkv *
ceil(N / 128) < 1024, the group is split over S workgroups (S the smallest
divisor of G reaching 1024 workgroups) whose float32 partial sums a reduction
kernel adds. The shapes below cover both (noted per case).

"RTX Flash Attention Implementation COMPLETE", Next Steps & Future
Enhancements, Advanced Features, names multi-query / grouped-query attention.
Reading: Hkv divides H, query head h attends with K/V head h // (H / Hkv), and
dK, dV of a K/V head are summed over the query heads of its group. The bars are
the multi-head ones; dK and dV are judged relative to the group sums.
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import (GRAD_RTOL, LSE_ATOL, O_ATOL, announce, max_abs, rel_to_max, to_dev,
                            to_f64)

pytestmark = pytest.mark.gpu


def to_dev_dt(bits, dtype):
    import torch
    if dtype == "bf16":
        return to_dev(bits)
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.float16).to("cuda")


def _decode(bits, dtype):
    return oracle.bf16_bits_to_f64(bits) if dtype == "bf16" else oracle.f16_bits_to_f64(bits)


def _run(fa, x, causal, scale, dtype="bf16"):
    import torch
    q, k, v, do = (to_dev_dt(x[n], dtype) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal, scale)
    dq, dk, dv = fa.backward(do, q, k, v, o, lse, causal, scale)
    torch.cuda.synchronize()
    assert tuple(dk.shape) == tuple(k.shape) and tuple(dv.shape) == tuple(v.shape)
    return {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}


def _grad_err(mine, ref):
    return rel_to_max(mine, ref) if np.max(np.abs(ref)) > 0 else max_abs(mine, ref)


def _check_group(g, head, b, j, H, Hkv, causal, scale):
    """Every output of K/V head j of batch b and of the query heads it serves;
    head(name, b, h) gives one head of an input in float64."""
    G = H // Hkv
    k, v = head("k", b, j), head("v", b, j)
    dk_ref = np.zeros_like(k)
    dv_ref = np.zeros_like(v)
    for h in range(j * G, (j + 1) * G):
        assert oracle.kv_head(h, H, Hkv) == j
        q, do = head("q", b, h), head("do", b, h)
        o_ref, lse_ref = oracle.head_forward(q, k, v, causal, scale)
        dq_ref, dk_h, dv_h = oracle.head_backward(q, k, v, do, causal, scale)
        dk_ref += dk_h
        dv_ref += dv_h
        assert max_abs(to_f64(g["o"][b, h]), o_ref) <= O_ATOL, (b, h)
        assert max_abs(to_f64(g["lse"][b, h]), lse_ref) <= LSE_ATOL, (b, h)
        err = _grad_err(to_f64(g["dq"][b, h]), dq_ref)
        assert err <= GRAD_RTOL, ("dq", b, h, err)
    for name, ref in (("dk", dk_ref), ("dv", dv_ref)):
        err = _grad_err(to_f64(g[name][b, j]), ref)
        assert err <= GRAD_RTOL, (name, b, j, err)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 65, 129, 300])
@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 3)])
def test_grouped_small_every_element(fa, H, Hkv, N, causal, d):
    B = 2
    seed = 7000 + 16 * N + 4 * H + Hkv + 2 * int(causal) + (d == 128)
    x = ai.make_qkv(B, H, N, d, seed, with_do=True, Hkv=Hkv)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    announce(f"gqa small B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} seed={seed}")
    g = _run(fa, x, causal, scale)
    f = {n: oracle.bf16_bits_to_f64(bits) for n, bits in x.items()}
    # the whole-tensor oracle as well, so its own grouping is exercised
    o_ref, lse_ref = oracle.attention_forward(f["q"], f["k"], f["v"], causal, scale)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(f["q"], f["k"], f["v"], f["do"], causal, scale)
    assert max_abs(to_f64(g["o"]), o_ref) <= O_ATOL
    assert max_abs(to_f64(g["lse"]), lse_ref) <= LSE_ATOL
    for name, ref in (("dq", dq_ref), ("dk", dk_ref), ("dv", dv_ref)):
        err = _grad_err(to_f64(g[name]), ref)
        assert err <= GRAD_RTOL, (name, err)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [65, 300])
def test_grouped_f16(fa, N, causal):
    B, H, Hkv, d = 1, 4, 2, 128
    seed = 7500 + N + int(causal)
    x = ai.make_qkv(B, H, N, d, seed, with_do=True, dtype="f16", Hkv=Hkv)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    announce(f"gqa f16 H={H} Hkv={Hkv} N={N} causal={causal} seed={seed}")
    g = _run(fa, x, causal, scale, dtype="f16")
    for j in range(Hkv):
        _check_group(g, lambda n, b, h: oracle.f16_bits_to_f64(x[n][b, h]), 0, j, H, Hkv, causal,
                     scale)


def test_grouped_identical_query_heads(fa):
    """All query heads of a group equal (and their dO equal): O matches the
    single-head result on every query head, dK and dV are G times it."""
    import torch
    B, H, Hkv, N, d = 1, 8, 1, 257, 64
    x = ai.make_qkv(B, 1, N, d, 7700, with_do=True)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q1, k, v, do1 = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    for causal in (False, True):
        announce(f"gqa identical heads causal={causal}")
        o1, l1 = fa.forward(q1, k, v, causal, scale)
        dq1, dk1, dv1 = fa.backward(do1, q1, k, v, o1, l1, causal, scale)
        q8, do8 = q1.expand(B, H, N, d).contiguous(), do1.expand(B, H, N, d).contiguous()
        o8, l8 = fa.forward(q8, k, v, causal, scale)
        dq8, dk8, dv8 = fa.backward(do8, q8, k, v, o8, l8, causal, scale)
        torch.cuda.synchronize()
        for h in range(H):
            assert torch.equal(o8[:, h], o1[:, 0]) and torch.equal(l8[:, h], l1[:, 0])
            assert torch.equal(dq8[:, h], dq1[:, 0])
        for g8, g1 in ((dk8, dk1), (dv8, dv1)):
            ref = to_f64(g1) * H
            assert rel_to_max(to_f64(g8), ref) <= 1e-2


@pytest.mark.parametrize("B,H,Hkv,N,causal,groups", [
    (4, 64, 8, 4096, True, ((0, 0), (3, 7))),      # G = 8, one workgroup per key block
    (4, 64, 8, 4096, False, ((0, 0), (3, 7))),
    (4, 16, 1, 4096, True, ((3, 0),)),             # multi-query: G = 16, split 8 ways
    (4, 32, 1, 2048, False, ((2, 0),)),            # multi-query: G = 32, split 16 ways
    (16, 32, 16, 1000, True, ((0, 0), (15, 15))),  # G = 2, one workgroup, ragged N
    (16, 32, 16, 1000, False, ((0, 0), (15, 15))),
    (2, 8, 2, 1000, True, ((0, 1), (1, 0))),       # G = 4, split 4 ways, ragged N
])
def test_grouped_large(fa, B, H, Hkv, N, causal, groups):
    """B x H query heads x N x 128 over Hkv K/V heads (the multi-head
    benchmark's full size among them), in the launch configuration the
    benchmark uses: every query head at sampled rows, whole groups, and the
    group identities over every K/V head."""
    import torch
    d = 128
    G = H // Hkv
    x = ai.make_qkv(B, H, N, d, 7800 + 2 * Hkv + int(causal), with_do=True, Hkv=Hkv)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    announce(f"gqa large {B}x{H}/{Hkv}x{N}x{d} causal={causal} on GPU")
    g = _run(fa, x, causal, scale)
    o, lse = to_f64(g["o"]), to_f64(g["lse"])
    rng = np.random.default_rng(7900 + 2 * Hkv + int(causal))
    for b in range(B):
        for h in range(H):
            j = h // G
            rows = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 4)]))
            ro, rl = oracle.rows_forward(oracle.bf16_bits_to_f64(x["q"][b, h, rows]),
                                         oracle.bf16_bits_to_f64(x["k"][b, j]),
                                         oracle.bf16_bits_to_f64(x["v"][b, j]), rows, causal, scale)
            assert max_abs(o[b, h, rows], ro) <= O_ATOL, (b, h)
            assert max_abs(lse[b, h, rows], rl) <= LSE_ATOL, (b, h)
    for b, j in groups:
        announce(f"gqa large: oracle group b={b} kv head {j}")
        _check_group(g, lambda n, bb, h: oracle.bf16_bits_to_f64(x[n][bb, h]), b, j, H, Hkv, causal,
                     scale)
    # identities over every K/V head, float64 on the device:
    #   sum_j dV_j = sum over the group's query heads of sum_i dO_i
    #   sum over the group of <dQ_h, Q_h> = <dK, K>
    do = to_dev(x["do"]).double().view(B, Hkv, G, N, d)
    dv_sum = g["dv"].double().sum(2)
    do_sum = do.sum((2, 3))
    r1 = ((dv_sum - do_sum).abs().amax(-1) / do_sum.abs().amax(-1)).max().item()
    q = to_dev(x["q"]).double().view(B, Hkv, G, N, d)
    k = to_dev(x["k"]).double()
    dq = g["dq"].double().view(B, Hkv, G, N, d)
    a = (dq * q).sum((2, 3, 4))
    bb = (g["dk"].double() * k).sum((2, 3))
    den = torch.maximum((dq.abs() * q.abs()).sum((2, 3, 4)), (g["dk"].double().abs() * k.abs()).sum((2, 3)))
    r2 = ((a - bb).abs() / den).max().item()
    announce(f"gqa identities: sum dV {r1:.2e}, <dQ,Q>-<dK,K> {r2:.2e}")
    assert r1 <= 2e-2 and r2 <= 1e-2
    del g
    torch.cuda.empty_cache()
