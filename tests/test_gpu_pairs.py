"""GPU parity for the kernels that give each workgroup a pair of tiles.

The causal forward (and dQ pass) pair query tile nq - 1 - w with tile w in
one workgroup when that leaves at least 256 workgroups: the workgroup runs
the two tiles' sweeps one after the other, and every pair has the same
number of key tiles. When the pairs of key blocks (block p with block nkb - 1 - p; the middle
block of an odd count alone) number at least 1024 over all heads, the dK/dV
pass gives each workgroup one or more pairs and runs its step pipeline from
one block straight into the next: it loads the next block's K or V rows in
the slot where the steps change blocks, writes and clears the finished
block's dK or dV at the end of that slot, and writes the last block's after
the sweep. The shapes below all take that path (block counts
noted per case), with odd and even block counts, a ragged last block, d = 64
and 128, both masks, and grouped K/V heads.

fa_fwd_ex / fa_bwd_ex are called through ctypes on outputs filled with NaN
first, so a row that no workgroup writes stays NaN: every element of every
output must be finite, and sampled heads (the first, the last, one in the
middle) must match the oracle within the multi-head bars. The backward
follows "GPU Performance Optimization Batch 1 - Design Spec", Item 3, Design
(recomputation from the stored log-sum-exp); grouped heads sum dK, dV over
the query heads of a group ("RTX Flash Attention Implementation COMPLETE",
Advanced Features).
"""
import ctypes
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import GRAD_RTOL, LSE_ATOL, O_ATOL, announce, max_abs, rel_to_max, to_dev, to_f64

pytestmark = pytest.mark.gpu

CASES = [  # B, H, Hkv, N, d, causal   (key blocks = B * Hkv * nkb, nkb = ceil(N / 128))
    (2, 72, 72, 1920, 128, True),     # 2160 blocks, 15 per head (odd: a middle block alone)
    (2, 72, 72, 1920, 128, False),
    (1, 128, 128, 2113, 128, True),   # 2176 blocks, 17 per head, last block 65 keys
    (4, 32, 32, 2048, 64, True),      # 2048 blocks (the smallest count that pairs), d = 64
    (4, 64, 32, 2048, 128, True),     # 2048 blocks of 32 K/V heads, two query heads each
]


def _head(x, name, b, h):
    return oracle.bf16_bits_to_f64(x[name][b, h])


def _grad_err(mine, ref):
    return rel_to_max(mine, ref) if np.max(np.abs(ref)) > 0 else max_abs(mine, ref)


@pytest.mark.parametrize("B,H,Hkv,N,d,causal", CASES)
def test_paired_tiles(fa, B, H, Hkv, N, d, causal):
    import torch
    nkb = (N + 127) // 128
    assert B * Hkv * ((nkb + 1) // 2) >= 1024  # the shapes must take the paired path
    seed = 7700 + N + 3 * H + Hkv + d + int(causal)
    announce(f"pairs B={B} H={H} Hkv={Hkv} N={N} d={d} causal={causal} seed={seed}")
    x = ai.make_qkv(B, H, N, d, seed, with_do=True, Hkv=Hkv)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    nan = float("nan")
    o = torch.full_like(q, nan)
    lse = torch.full((B, H, N), nan, dtype=torch.float32, device="cuda")
    dq = torch.full_like(q, nan)
    dk = torch.full_like(k, nan)
    dv = torch.full_like(v, nan)
    lib = fa.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = lib.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, H, Hkv, N, d, int(causal), ctypes.c_float(scale), 0, stream)
    assert rc == 0, lib.fa_status_string(rc)
    rc = lib.fa_bwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                       B, H, Hkv, N, d, int(causal), ctypes.c_float(scale), 0, stream)
    assert rc == 0, lib.fa_status_string(rc)
    torch.cuda.synchronize()
    for name, t in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv)):
        assert bool(torch.isfinite(t.float()).all().item()), f"{name} has elements never written"

    G = H // Hkv
    for b, j in sorted({(0, 0), (B // 2, Hkv // 2), (B - 1, Hkv - 1)}):
        kh, vh = _head(x, "k", b, j), _head(x, "v", b, j)
        dk_ref = np.zeros_like(kh)
        dv_ref = np.zeros_like(vh)
        for h in range(j * G, (j + 1) * G):
            qh, doh = _head(x, "q", b, h), _head(x, "do", b, h)
            o_ref, lse_ref = oracle.head_forward(qh, kh, vh, causal, scale)
            dq_ref, dk_h, dv_h = oracle.head_backward(qh, kh, vh, doh, causal, scale)
            dk_ref += dk_h
            dv_ref += dv_h
            assert max_abs(to_f64(o[b, h]), o_ref) <= O_ATOL, (b, h)
            assert max_abs(to_f64(lse[b, h]), lse_ref) <= LSE_ATOL, (b, h)
            assert _grad_err(to_f64(dq[b, h]), dq_ref) <= GRAD_RTOL, ("dq", b, h)
        for name, got, ref in (("dk", dk, dk_ref), ("dv", dv, dv_ref)):
            err = _grad_err(to_f64(got[b, j]), ref)
            assert err <= GRAD_RTOL, (name, b, j, err)


MASS_CASES = [  # B, H, Hkv, N, d   (causal; key-block pairs = B * H * ceil(nkb / 2) >= 1024)
    (1, 128, 128, 2048, 128),   # 16 key blocks per head
    (1, 136, 136, 1920, 64),    # 15: the middle block alone, d = 64
]


@pytest.mark.parametrize("B,H,Hkv,N,d", MASS_CASES)
def test_paired_key_mass(fa, B, H, Hkv, N, d):
    """The causal key-mass pass pairs key block w with block nkb - 1 - w in one
    workgroup ("GPU Performance Optimization Batch 1 - Design Spec", Item 4,
    Design: the mass each key receives, summed over rows and heads). With the
    oracle's LSE as input, every key's mass must match the oracle's, and no
    element may stay as the NaN the output was filled with."""
    import torch
    nkb = (N + 127) // 128
    assert B * H * ((nkb + 1) // 2) >= 1024  # the shape must take the paired path
    seed = 7900 + N + H + d
    announce(f"pairs key mass B={B} H={H} N={N} d={d} seed={seed}")
    x = ai.make_qkv(B, H, N, d, seed, Hkv=Hkv)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    f = {n: oracle.bf16_bits_to_f64(b) for n, b in x.items()}
    ref = oracle.key_mass(f["q"], f["k"], True, scale)
    _, lse_ref = oracle.attention_forward(f["q"], f["k"], f["v"], True, scale)
    q, k = to_dev(x["q"]), to_dev(x["k"])
    out = torch.full((B, N), float("nan"), dtype=torch.float32, device="cuda")
    fa.key_mass(q, k, torch.from_numpy(lse_ref.astype(np.float32)).cuda(), True, scale, out=out)
    torch.cuda.synchronize()
    m = to_f64(out)
    assert np.isfinite(m).all()
    assert max_abs(m, ref) / np.max(np.abs(ref)) <= 1e-3
