"""GPU parity on a long, ragged sequence: N = 100003 (1563 key tiles of 64, no
size a multiple of any tile), two heads, d = 128.

The forward is checked against the oracle at sampled rows: the first and last
rows, rows on both sides of 64- and 256-row tile boundaries, and random rows.
The causal case draws Q and K from N(0, 3^2), so each row's running maximum
keeps moving over the whole sweep of keys. At this length the backward is
checked through identities that hold for any inputs, in float64 on the
device:
  * sum_j dK_j = 0 per head (each row of dS sums to zero, since D_i equals
    sum_j P_ij dP_ij);
  * sum_j dV_j = sum_i dO_i per head (each row of P sums to one);
  * <dQ, Q> = <dK, K> per head (both equal scale * sum_ij dS_ij q_i . k_j).
The key masses of the same inputs must add up to H N per batch (every query
row's probabilities sum to one). Tolerances: O and LSE as everywhere; the
identities within 2e-2 of the size of their terms, as in the full-size
workload tests (bf16 rounding of P and of the stored gradients, 2^-9
relative each).
"""
import math

import numpy as np
import pytest

import attn_inputs as ai
import oracle
from tests.gpu_util import LSE_ATOL, O_ATOL, announce, max_abs, to_dev, to_f64

pytestmark = pytest.mark.gpu

N_LONG = 100003


def _rows(N, rng):
    edges = []
    for step in (64, 256):
        for m in (1, 2, N // step // 2, N // step - 1, N // step):
            edges += [m * step - 1, m * step]
    rows = np.concatenate([[0, 1, N - 2, N - 1], edges, rng.integers(0, N, 8)])
    return np.unique(rows[(rows >= 0) & (rows < N)])


@pytest.mark.parametrize("causal,sigma_qk,seed", [(True, 3.0, 31), (False, 1.0, 32)])
def test_long_ragged_sequence(fa, causal, sigma_qk, seed):
    import torch
    B, H, N, d = 1, 2, N_LONG, 128
    scale = float(np.float32(1.0 / math.sqrt(d)))
    announce(f"long sequence N={N} causal={causal} sigma_qk={sigma_qk}")
    x = ai.make_qkv(B, H, N, d, seed, sigma_qk=sigma_qk, with_do=True)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    o, lse = fa.forward(q, k, v, causal, scale)
    dq, dk, dv = fa.backward(do, q, k, v, o, lse, causal, scale)
    mass = fa.key_mass(q, k, lse, causal, scale)
    torch.cuda.synchronize()

    # forward at sampled rows of every head
    rng = np.random.default_rng(seed)
    of, lf = to_f64(o), to_f64(lse)
    for h in range(H):
        rows = _rows(N, rng)
        qb = oracle.bf16_bits_to_f64(x["q"][0, h, rows])
        kb = oracle.bf16_bits_to_f64(x["k"][0, h])
        vb = oracle.bf16_bits_to_f64(x["v"][0, h])
        ro, rl = oracle.rows_forward(qb, kb, vb, rows, causal, scale)
        e_o, e_l = max_abs(of[0, h, rows], ro), max_abs(lf[0, h, rows], rl)
        announce(f"  head {h}: {len(rows)} rows, max|dO| {e_o:.2e}, max|dLSE| {e_l:.2e}")
        assert e_o <= O_ATOL and e_l <= LSE_ATOL, (h, e_o, e_l)

    # backward identities per head, float64 on the device
    qd, kd, dod = q.double(), k.double(), do.double()
    dqd, dkd, dvd = dq.double(), dk.double(), dv.double()
    r_dk = ((dkd.sum(2).abs().amax(-1)) / dkd.abs().sum(2).amax(-1)).max().item()
    do_sum = dod.sum(2)
    r_dv = ((dvd.sum(2) - do_sum).abs().amax(-1) / do_sum.abs().amax(-1)).max().item()
    a = (dqd * qd).sum((2, 3))
    b = (dkd * kd).sum((2, 3))
    den = torch.maximum((dqd.abs() * qd.abs()).sum((2, 3)), (dkd.abs() * kd.abs()).sum((2, 3)))
    r_qk = ((a - b).abs() / den).max().item()
    announce(f"  identities: sum dK {r_dk:.2e}, sum dV - sum dO {r_dv:.2e}, "
             f"<dQ,Q>-<dK,K> {r_qk:.2e}")
    assert r_dk <= 2e-2 and r_dv <= 2e-2 and r_qk <= 2e-2
    assert torch.isfinite(dqd).all() and torch.isfinite(dkd).all() and torch.isfinite(dvd).all()

    # key masses add up to H N
    tot = mass.double().sum().item()
    announce(f"  key mass total {tot:.6f} (expected {H * N})")
    assert abs(tot - H * N) <= 1e-3 * H * N
