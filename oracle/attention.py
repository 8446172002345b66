"""CPU fp64 oracle for exact scaled-dot-product attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg do. It shares no code with the GPU library.

What it computes is the plain definition of softmax attention, materialised in
full (the N x N score matrix is built per head), in float64:

  * "RTX Flash Attention Implementation COMPLETE", Executive Summary: the tiled
    method is exact, so its result is that of ordinary softmax attention;
    Usage Examples: tensors are [batch, heads, seq_len, head_dim], forward
    takes (q, k, v, causal, scale) and returns the output and the LSE, backward
    takes (dout, q, k, v, out, lse, causal, scale) and returns dq, dk, dv.
  * Same page, Advanced Features: causal (autoregressive) masking.
  * "GPU Performance Optimization Batch 1 - Design Spec", Item 3, Verification:
    correctness is judged against naive O(N^2) attention; Item 3, Design
    (backward file): the backward works from the stored log-sum-exp.

Readings where the pages are silent (each one is listed in the design notes):
  * LSE_i = ln sum_{j visible} exp(scale * q_i . k_j), natural log.
  * causal: key j is visible to query i iff j <= i; masked entries are
    excluded exactly (probability 0), not given a large negative logit.
  * scale multiplies Q K^T before the softmax; the float32 value the library
    receives is used exactly (widened to float64).
  * the backward gets the gradient through O only (no gradient w.r.t. LSE).
  * grouped K/V heads (same page, Next Steps & Future Enhancements, Advanced
    Features: multi-query / grouped-query attention): H / Hkv consecutive
    query heads share one K/V head; its dK, dV sum over them.

Every function takes float64 arrays; ``bf16_bits_to_f64`` and
``f16_bits_to_f64`` turn the uint16 bit patterns the GPU receives (bfloat16 or
IEEE binary16: the Mixed Precision item of the same page's Advanced Features
names both) into exactly the same values.
"""
from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float64.

    A bfloat16 value is the top half of a float32, so shifting the bits into
    the high 16 bits of a uint32 gives the float32 with the same value.
    """
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    # signalling-NaN patterns raise the invalid flag when widened; they stay NaN
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of IEEE binary16 bit patterns (uint16) to float64.

    Every binary16 value (normal, subnormal, zero, infinity) is exactly
    representable in float64; numpy's float16 type reads the bits as such.
    """
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def exact_scale(scale: float) -> float:
    """The softmax scale as the library sees it: a float32, widened exactly."""
    return float(np.float64(np.float32(scale)))


def causal_visible(n: int) -> np.ndarray:
    """Boolean [n, n] matrix: True where key j is visible to query i (j <= i)."""
    return np.tril(np.ones((n, n), dtype=bool))


def head_probs(q: np.ndarray, k: np.ndarray, causal: bool, scale: float):
    """Softmax probabilities of one head, from the definition.

    q, k: [N, d] float64. Returns (P [N, N], LSE [N]) where
    S = scale * q k^T, masked entries are excluded, m_i = max_j S_ij,
    P_ij = exp(S_ij - m_i) / sum_j exp(S_ij - m_i), LSE_i = m_i + ln(sum_j ...).
    """
    sc = exact_scale(scale)
    n = q.shape[0]
    s = sc * (q @ k.T)
    if causal:
        vis = causal_visible(n)
        s = np.where(vis, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)          # exp(-inf) = 0: masked keys contribute nothing
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    lse = m[:, 0] + np.log(l[:, 0])
    return p, lse


def head_forward(q, k, v, causal: bool, scale: float):
    """O = P V and LSE for one head ([N, d] float64 inputs)."""
    p, lse = head_probs(q, k, causal, scale)
    return p @ v, lse


def head_backward(q, k, v, do, causal: bool, scale: float):
    """dQ, dK, dV of L = <dO, O> for one head, recomputing P from the inputs.

    With P = softmax(S), S = sc q k^T and O = P V:
      dV = P^T dO;   dP = dO V^T;   D_i = sum_j P_ij dP_ij;
      dS = P * (dP - D);   dQ = sc dS K;   dK = sc dS^T Q.
    """
    sc = exact_scale(scale)
    p, _ = head_probs(q, k, causal, scale)
    dv = p.T @ do
    dp = do @ v.T
    dvec = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - dvec)
    dq = sc * (ds @ k)
    dk = sc * (ds.T @ q)
    return dq, dk, dv


def kv_head(h: int, H: int, Hkv: int) -> int:
    """The K/V head that query head h attends with, H query heads sharing Hkv.

    "RTX Flash Attention Implementation COMPLETE", Next Steps & Future
    Enhancements, Advanced Features, names multi-query and grouped-query
    attention without fixing the grouping. Reading: Hkv divides H, and the
    query heads form Hkv consecutive groups of H / Hkv, group g sharing K/V
    head g (Hkv = H: one K/V head per query head; Hkv = 1: one for all).
    """
    if Hkv < 1 or H % Hkv:
        raise ValueError(f"{Hkv} K/V heads cannot serve {H} query heads")
    return h // (H // Hkv)


def attention_forward(q, k, v, causal: bool, scale: float):
    """O [B,H,N,d] and LSE [B,H,N] (float64) over every (batch, query head).

    q is [B,H,N,d]; k, v are [B,Hkv,N,d], query head h reading K/V head
    kv_head(h, H, Hkv) (Hkv = H is plain multi-head attention).
    """
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            o[b, h], lse[b, h] = head_forward(q[b, h], k[b, g], v[b, g], causal, scale)
    return o, lse


def attention_backward(q, k, v, do, causal: bool, scale: float):
    """dQ [B,H,N,d] and dK, dV [B,Hkv,N,d] (float64).

    A K/V head shared by several query heads enters the loss once per query
    head, so its gradients are the sums of the per-query-head gradients.
    """
    B, H = q.shape[:2]
    Hkv = k.shape[1]
    dq = np.empty_like(q, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for h in range(H):
            g = kv_head(h, H, Hkv)
            dq[b, h], dk_h, dv_h = head_backward(q[b, h], k[b, g], v[b, g], do[b, h], causal, scale)
            dk[b, g] += dk_h
            dv[b, g] += dv_h
    return dq, dk, dv


def key_mass(q, k, causal: bool, scale: float):
    """Attention mass per key position: mass[b, j] = sum_h sum_i P[b, h, i, j].

    "GPU Performance Optimization Batch 1 - Design Spec", Item 4 (SnapKV +
    Prefix Caching), Design: during prefill the attention kernel sums the
    attention weights each key position receives, and a reduction over the
    heads turns them into one score per key, the importance used to evict
    keys. Reading: the sum runs over every query row and every query head (a
    key shared by grouped query heads collects the mass of all of them), P
    being the forward's exact, masked softmax. q: [B,H,N,d], k: [B,Hkv,N,d];
    returns [B,N] float64.
    """
    B, H, N, _ = q.shape
    Hkv = k.shape[1]
    mass = np.zeros((B, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            p, _ = head_probs(q[b, h], k[b, kv_head(h, H, Hkv)], causal, scale)
            mass[b] += p.sum(axis=0)
    return mass


def rows_forward(q_rows, k, v, rows, causal: bool, scale: float):
    """O and LSE for selected query rows of one head.

    q_rows: [R, d] (the queries at positions ``rows``), k, v: [N, d].
    Row i sees keys 0..N-1, or 0..rows[i] when causal. This is the same
    definition restricted to a few rows, for spot checks at full size.
    """
    sc = exact_scale(scale)
    s = sc * (q_rows @ k.T)
    if causal:
        j = np.arange(k.shape[0])[None, :]
        s = np.where(j <= np.asarray(rows)[:, None], s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    return (e / l) @ v, m[:, 0] + np.log(l[:, 0])


def online_softmax_stats(x: np.ndarray, bounds):
    """Running max m and running sum l of exp(x), folded in tile by tile.

    Follows the update of "RTX Flash Attention Implementation COMPLETE",
    Technical Implementation Details, 1. Online Softmax Algorithm, applied to a
    whole tile at a time: for a tile t, m' = max(m, max t) and
    l' = l * exp(m - m') + sum exp(t - m'). Initial state m = -inf, l = 0
    (the page does not give one; the first tile's terms then make l exact).
    ``bounds`` are the tile edges over x (a sorted list of split points, in
    any processing order given as a list of (start, stop) pairs).
    Returns (m, l) with ln(sum exp x) = m + ln l.
    """
    m, l = -np.inf, 0.0
    for lo, hi in bounds:
        t = x[lo:hi]
        if t.size == 0:
            continue
        m_new = max(m, float(t.max()))
        alpha = 0.0 if m == -np.inf else np.exp(m - m_new)
        l = l * alpha + float(np.exp(t - m_new).sum())
        m = m_new
    return m, l
