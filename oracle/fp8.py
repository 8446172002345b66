"""CPU fp64 oracle for the FP8 (E4M3) attention path.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: nothing in the product
path may import, call or execute it. It shares no code with the GPU library.

"GPU Performance Optimization Batch 1 - Design Spec", Item 3 (FlashAttention-3),
Design, optional FP8 path: before the matrix product, every 16 x 16 block of Q
and of K is quantised to E4M3 with a scale factor of its own. Item 2, Design,
Step 1 fixes the cast: a saturating clamp to [-448, 448] before encoding E4M3
(448 being E4M3's largest finite value).

Two block shapes are provided. The 16 x 16 blocks follow the FP8 path's own
words. The 1 x 32 blocks (one token row by 32 consecutive head-dim columns,
a power-of-two scale per block: the OCP MX block layout) are an alternative
reading: the same spec names MX block-wise quantisation among its existing
FP8 pieces (Item 2, Current state), and the FP8 path is there for roughly
twice the matrix throughput, which FP8 matrix units that scale per 32
values along the contraction only give to blocks of that width.

Readings where the pages are silent (each listed in the design notes):
  * a block is 16 consecutive token rows x 16 consecutive head-dim columns of
    one head's [N, d] matrix; the last row block of a head may be shorter;
  * the scale of a block is the power of two 2^e with the smallest e for which
    the block's largest magnitude amax is at most 448 * 2^e (so nothing
    saturates and the dequantised values stay exact in bf16), with e clamped
    to at least -100 (dequantised values stay normal floats) and e = 0 for an
    all-zero block;
  * a value x is encoded as the E4M3 value nearest to x / 2^e, ties to even
    (OCP E4M3: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormal step 2^-9, largest finite 448), zero always as +0 (code 0x00);
  * only S = Q K^T sees the quantised operands: the forward is exact attention
    on Q~ = decode(code) * 2^e and K~ likewise, with V, P and O as in the
    bf16 path.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_forward

E4M3_MAX = 448.0
BLOCK = 16
MX_BLOCK = 32
E_MIN = -100


def e4m3_round(y: np.ndarray) -> np.ndarray:
    """Nearest E4M3 value to each y (float64, |y| <= 448), ties to even.

    Normal E4M3 values 1.m * 2^E (E = -6..8) are spaced 2^(E - 3); below 2^-6
    the subnormals are spaced 2^-9. Dividing by the spacing (a power of two,
    exact) and rounding half to even gives the nearest multiple.
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if np.any(a > E4M3_MAX):
        raise ValueError("e4m3_round expects |y| <= 448")
    _, ex = np.frexp(a)                    # a = m 2^ex, m in [0.5, 1): floor(log2 a) = ex - 1
    expo = np.maximum(ex - 1, -6)          # binade, subnormals share the -6 spacing
    step = np.ldexp(1.0, expo - 3)
    r = np.round(a / step) * step          # numpy rounds halves to even
    return np.where(r == 0.0, 0.0, np.copysign(r, y))


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Byte codes of E4M3 values v (already representable); 0 -> 0x00."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sign = (v < 0).astype(np.uint8) << 7
    _, ex = np.frexp(a)
    expo = ex - 1
    normal = a >= 2.0 ** -6
    e_field = np.where(normal, expo + 7, 0)
    mant = np.where(normal, np.ldexp(a, -expo) - 1.0, np.ldexp(a, 9)) * np.where(normal, 8.0, 1.0)
    code = (e_field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(a == 0.0, 0, code)
    return (code.astype(np.uint8) | np.where(a == 0.0, 0, sign).astype(np.uint8)).astype(np.uint8)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    """Values of E4M3 byte codes (OCP E4M3: 0x7F / 0xFF are NaN)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, np.ldexp(m.astype(np.float64), -9),
                   np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def block_exponent(amax: np.ndarray) -> np.ndarray:
    """Smallest e with amax <= 448 * 2^e (448 = 0.875 * 2^9), at least E_MIN;
    0 where amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(amax)                 # amax = m 2^ex, m in [0.5, 1)
    e = np.where(m <= 0.875, ex - 9, ex - 8)
    e = np.maximum(e, E_MIN)
    return np.where(amax == 0.0, 0, e).astype(np.int64)


def quantize_e4m3_blocks(x: np.ndarray):
    """Quantise [R, N, d] (float64; R heads of N rows) per 16 x 16 block.

    Returns (codes uint8 [R, N, d], exponents int64 [R, ceil(N/16), d/16],
    dequantised float64 [R, N, d] = decode(codes) * 2^e).
    """
    x = np.asarray(x, dtype=np.float64)
    R, N, d = x.shape
    if d % BLOCK:
        raise ValueError("d must be a multiple of 16")
    nrb = -(-N // BLOCK)
    codes = np.zeros((R, N, d), dtype=np.uint8)
    deq = np.zeros((R, N, d), dtype=np.float64)
    expo = np.zeros((R, nrb, d // BLOCK), dtype=np.int64)
    for rb in range(nrb):
        rows = slice(rb * BLOCK, min(N, (rb + 1) * BLOCK))
        for cb in range(d // BLOCK):
            cols = slice(cb * BLOCK, (cb + 1) * BLOCK)
            blk = x[:, rows, cols]                               # [R, <=16, 16]
            e = block_exponent(np.abs(blk).max(axis=(1, 2)))     # [R]
            y = np.ldexp(blk, -e[:, None, None])
            v = e4m3_round(y)
            codes[:, rows, cols] = e4m3_encode(v)
            deq[:, rows, cols] = np.ldexp(v, e[:, None, None])
            expo[:, rb, cb] = e
    return codes, expo, deq


def fp8_attention_forward(q, k, v, causal: bool, scale: float):
    """O and LSE of the FP8 path: exact attention on the block-quantised Q, K.

    q: [B,H,N,d], k, v: [B,Hkv,N,d] float64 (the decoded 16-bit inputs).
    """
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    _, _, qd = quantize_e4m3_blocks(q.reshape(B * H, N, d))
    _, _, kd = quantize_e4m3_blocks(k.reshape(B * Hkv, N, d))
    return attention_forward(qd.reshape(q.shape), kd.reshape(k.shape), v, causal, scale)


def quantize_e4m3_rows32(x: np.ndarray):
    """Quantise [R, N, d] (float64) per 1 x 32 block: one row, columns
    32 c .. 32 c + 31, with the same scale rule and rounding as the 16 x 16
    blocks.

    Returns (codes uint8 [R, N, d], exponents int64 [R, N, d/32],
    dequantised float64 [R, N, d] = decode(codes) * 2^e).
    """
    x = np.asarray(x, dtype=np.float64)
    R, N, d = x.shape
    if d % MX_BLOCK:
        raise ValueError("d must be a multiple of 32")
    nb = d // MX_BLOCK
    blk = x.reshape(R, N, nb, MX_BLOCK)
    e = block_exponent(np.abs(blk).max(axis=3))            # [R, N, nb]
    v = e4m3_round(np.ldexp(blk, -e[..., None]))
    codes = e4m3_encode(v).reshape(R, N, d)
    deq = np.ldexp(v, e[..., None]).reshape(R, N, d)
    return codes, e.astype(np.int64), deq


def mx_fp8_attention_forward(q, k, v, causal: bool, scale: float):
    """O and LSE of the FP8 path under the 1 x 32 block reading: exact
    attention on Q, K quantised per row and 32 columns.

    q: [B,H,N,d], k, v: [B,Hkv,N,d] float64 (the decoded 16-bit inputs).
    """
    B, H, N, d = q.shape
    Hkv = k.shape[1]
    qd = quantize_e4m3_rows32(q.reshape(B * H, N, d))[2].reshape(q.shape)
    kd = quantize_e4m3_rows32(k.reshape(B * Hkv, N, d))[2].reshape(k.shape)
    return attention_forward(qd, kd, v, causal, scale)
