/*
 * fa.h - exact tiled attention for AMD Instinct MI355X (gfx950), C ABI.
 *
 * The operation is exact scaled-dot-product attention computed tile by tile
 * with an online softmax, as described on "RTX Flash Attention Implementation
 * COMPLETE" (Executive Summary; Technical Implementation Details, 1. Online
 * Softmax Algorithm and 2. Memory Tiling Strategy; Usage Examples) and, for
 * the backward that recomputes the probabilities from the stored log-sum-exp,
 * "GPU Performance Optimization Batch 1 - Design Spec", Item 3 (Design).
 *
 * For one (batch b, head h), with q_i, k_j, v_j the rows of Q, K, V:
 *   s_ij   = softmax_scale * q_i . k_j
 *   vis(i) = { j : j <= i } if causal, else all j     (key j visible to query i)
 *   LSE_i  = ln sum_{j in vis(i)} exp(s_ij)            (natural log)
 *   P_ij   = exp(s_ij - LSE_i) for j in vis(i), else 0
 *   O_i    = sum_j P_ij v_j
 * and, given dO (the gradient of the loss with respect to O):
 *   dV_j = sum_i P_ij dO_i
 *   dS_ij = P_ij (dO_i . v_j - dO_i . O_i)
 *   dQ_i = softmax_scale * sum_j dS_ij k_j,   dK_j = softmax_scale * sum_i dS_ij q_i
 * With grouped K/V heads (fa_fwd_ex / fa_bwd_ex, Hkv < H; "RTX Flash
 * Attention Implementation COMPLETE", Next Steps & Future Enhancements,
 * Advanced Features: multi-query and grouped-query attention), query head h
 * attends with K/V head h / (H / Hkv) (integer division), and dK, dV of a K/V
 * head are the sums of the above over the H / Hkv query heads that share it.
 *
 * Layout. Every tensor is dense and contiguous in row-major order:
 *   Q, K, V, O, dO, dQ, dK, dV : [B, H, N, d] 16-bit floats (raw 16-bit storage):
 *                                bfloat16 for fa_fwd / fa_bwd, bfloat16 or IEEE
 *                                binary16 (fa_dtype) for fa_fwd_ex / fa_bwd_ex
 *   LSE                        : [B, H, N]    float32
 * except that for fa_fwd_ex / fa_bwd_ex K, V, dK, dV are [B, Hkv, N, d].
 * Pointers are device pointers on the current HIP device. 16-bit tensors must
 * be 16-byte aligned, LSE 4-byte aligned. Outputs are overwritten, never
 * accumulated into; they must not alias the inputs.
 *
 * Limits: d in {64, 128}; N >= 1; B, H >= 1; Hkv >= 1 dividing H; N * d < 2^31 and
 * B * H * ceil(N / 32) < 2^31; softmax_scale finite and > 0; causal in {0, 1}.
 *
 * Precision. Inputs are read in their element type; both contractions run on
 * matrix cores of that type (bf16 or f16) with float32 accumulation; the
 * softmax runs in float32, and P and dS enter the products in the element
 * type. The row sum that normalises O adds P as rounded to the element type,
 * the weights the P V product uses, so O is a convex combination of V rows up
 * to float32 sums; LSE is taken from the same sum, which puts it within
 * ln(1 + 2^-8) (bf16; ln(1 + 2^-11) for f16) of the exact log-sum-exp. O, dQ,
 * dK, dV are rounded to the element type with round-to-nearest-even; LSE is
 * float32.
 *
 * Errors and threading. Every entry point validates its arguments on the host
 * before any HIP call and returns an fa_status. FA_ERR_HIP means a HIP call or
 * kernel launch failed at enqueue time; faults inside a kernel surface at the
 * caller's next synchronisation. Calls only enqueue work on `stream` (a
 * hipStream_t; NULL is the default stream) and return; results are valid once
 * the stream has reached them. Apart from fa_bwd_noalloc's per-device
 * workspace, the library holds no global mutable state (only a per-thread
 * record of the last HIP error), so calls from several threads on different
 * streams are safe.
 */
#ifndef FA_H_
#define FA_H_

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad shape, bad scale or flag */
  FA_ERR_UNSUPPORTED = 2,   /* head dimension other than 64 or 128, or unknown fa_dtype */
  FA_ERR_HIP = 3,           /* a HIP runtime call or a kernel launch failed */
  FA_ERR_OUT_OF_MEMORY = 4, /* fa_bwd, fa_key_mass, fa_fwd_fp8 or fa_fwd_mxfp8 could not get its scratch */
  FA_ERR_TOO_LARGE = 5      /* fa_bwd_noalloc: B * H * N exceeds FA_NOALLOC_MAX_ROWS */
} fa_status;

/*
 * Forward pass ("RTX Flash Attention Implementation COMPLETE", Usage Examples:
 * forward(q, k, v, causal, scale) returning the output and the LSE).
 *
 *   Q, K, V  in : [B,H,N,d] bf16
 *   O        out: [B,H,N,d] bf16
 *   LSE      out: [B,H,N] float32, natural-log log-sum-exp of the scaled,
 *                 masked logits of each query row; may be NULL (not written).
 *
 * Allocates nothing. Returns FA_OK or an error status (nothing is enqueued on
 * error).
 */
int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE,
           int B, int H, int N, int d, int causal, float softmax_scale,
           void* stream);

/*
 * Backward pass (same page, Usage Examples: backward(dout, q, k, v, out, lse,
 * causal, scale) returning dq, dk, dv; "GPU Performance Optimization Batch 1 -
 * Design Spec", Item 3, Design: the probabilities are recomputed from the
 * stored LSE instead of keeping the N x N matrix).
 *
 *   Q, K, V, O, dO  in : [B,H,N,d] bf16 (O and LSE as produced by fa_fwd with
 *                        the same causal flag and scale)
 *   LSE             in : [B,H,N] float32, must not be NULL
 *   dQ, dK, dV      out: [B,H,N,d] bf16
 *
 * Needs float32 scratch of 8*B*H*N bytes (rounded up to 256), taken stream-ordered with
 * hipMallocAsync on `stream` and released with hipFreeAsync on the same
 * stream (no host synchronisation). Returns FA_ERR_OUT_OF_MEMORY if it cannot
 * be had.
 */
int fa_bwd(const void* Q, const void* K, const void* V, const void* O,
           const float* LSE, const void* dO, void* dQ, void* dK, void* dV,
           int B, int H, int N, int d, int causal, float softmax_scale,
           void* stream);

/*
 * Element types of the 16-bit tensors. "RTX Flash Attention Implementation
 * COMPLETE" lists FP16 and BF16 among its Advanced Features (Mixed Precision)
 * and its Usage Examples build F16 inputs.
 */
typedef enum {
  FA_DTYPE_BF16 = 0, /* bfloat16: 8 exponent bits, 7 mantissa bits */
  FA_DTYPE_F16 = 1   /* IEEE 754 binary16: 5 exponent bits, 10 mantissa bits */
} fa_dtype;

/*
 * fa_fwd with Hkv K/V heads and the element type of Q, K, V and O given by
 * `dtype` (an fa_dtype); fa_fwd(..., H, N, ...) is fa_fwd_ex(..., H, H, N,
 * ..., FA_DTYPE_BF16, stream).
 *
 *   Q        in : [B,H,N,d]     dtype
 *   K, V     in : [B,Hkv,N,d]   dtype; query head h reads K/V head h / (H / Hkv)
 *   O        out: [B,H,N,d]     dtype
 *   LSE      out: [B,H,N] float32, or NULL
 *
 * Hkv == H is multi-head attention, Hkv == 1 multi-query attention, anything
 * between grouped-query attention. Otherwise the same layout, ownership and
 * errors as fa_fwd: FA_ERR_INVALID_ARG if Hkv < 1 or Hkv does not divide H,
 * FA_ERR_UNSUPPORTED for an unknown dtype value. For f16 the inputs must be
 * finite binary16 values.
 */
int fa_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* LSE,
              int B, int H, int Hkv, int N, int d, int causal,
              float softmax_scale, int dtype, void* stream);

/*
 * fa_bwd with Hkv K/V heads and the element type of Q, K, V, O, dO, dQ, dK
 * and dV given by `dtype`; fa_bwd(..., H, N, ...) is fa_bwd_ex(..., H, H, N,
 * ..., FA_DTYPE_BF16, stream).
 *
 *   Q, O, dO  in : [B,H,N,d]    dtype;  LSE in: [B,H,N] float32, not NULL
 *   K, V      in : [B,Hkv,N,d]  dtype
 *   dQ        out: [B,H,N,d]    dtype
 *   dK, dV    out: [B,Hkv,N,d]  dtype, each summed over the H / Hkv query
 *                               heads that share the K/V head
 *
 * Scratch as in fa_bwd (stream-ordered hipMallocAsync / hipFreeAsync), of
 * 8*B*H*N bytes (rounded up to 256) plus, when B * Hkv * ceil(N / 128) is
 * under 1024, 8*S*B*Hkv*N*d bytes of float32 partial sums of dK and dV, where
 * S > 1 is the smallest divisor of H / Hkv that brings S * B * Hkv *
 * ceil(N / 128) to 1024, or the largest one whose partial sums stay within
 * 1 GiB. Same ownership and errors
 * as fa_bwd, plus FA_ERR_INVALID_ARG if Hkv < 1 or Hkv does not divide H and
 * FA_ERR_UNSUPPORTED for an unknown dtype value.
 */
int fa_bwd_ex(const void* Q, const void* K, const void* V, const void* O,
              const float* LSE, const void* dO, void* dQ, void* dK, void* dV,
              int B, int H, int Hkv, int N, int d, int causal,
              float softmax_scale, int dtype, void* stream);

/* Query rows (B * H * N) that fa_bwd_noalloc's static workspace holds. */
#define FA_NOALLOC_MAX_ROWS 2097152

/*
 * fa_bwd_ex for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same
 * arguments, layout, results and validation as fa_bwd_ex; it calls no
 * allocating routine.
 *
 * The backward's scratch (two float32 planes of row statistics, 8 bytes per
 * query row) lives in a workspace the library keeps in device memory of each
 * GPU it runs on: 8 * FA_NOALLOC_MAX_ROWS bytes = 16 MiB, held until the
 * process ends; its address is looked up on the first call on each device.
 * B * H * N must not exceed FA_NOALLOC_MAX_ROWS (FA_ERR_TOO_LARGE otherwise;
 * 4 x 64 x 4096 is 2^20 rows). Nothing in it needs clearing: every row the
 * call reads is written earlier in the same call. The dK/dV work is never
 * split over the query heads of a K/V head (no partial sums), so with few K/V
 * heads (B * Hkv * ceil(N / 128) < 1024) it runs on fewer workgroups than
 * fa_bwd_ex and sums dK, dV in another order; otherwise its results are
 * bitwise those of fa_bwd_ex.
 *
 * Every call on one GPU shares that GPU's workspace: calls that overlap in
 * time on one GPU (on two streams, or from two threads) race and give wrong
 * results; order them on one stream. FA_ERR_HIP if the workspace's device
 * address cannot be obtained.
 */
int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O,
                   const float* LSE, const void* dO, void* dQ, void* dK, void* dV,
                   int B, int H, int Hkv, int N, int d, int causal,
                   float softmax_scale, int dtype, void* stream);

/*
 * Attention mass per key position ("GPU Performance Optimization Batch 1 -
 * Design Spec", Item 4, SnapKV + Prefix Caching, Design: the attention weights
 * each key position receives during prefill are summed and reduced over the
 * heads, giving the importance score that decides which keys to evict):
 *
 *   mass[b, j] = sum over query heads h and query rows i of P[b, h, i, j]
 *
 * with P the softmax probabilities of fa_fwd_ex (same causal flag, scale and
 * K/V grouping), recomputed from Q, K and the forward's LSE.
 *
 *   Q     in : [B,H,N,d]    dtype
 *   K     in : [B,Hkv,N,d]  dtype; query head h reads K head h / (H / Hkv)
 *   LSE   in : [B,H,N] float32 as written by fa_fwd_ex for these Q, K; not NULL
 *   mass  out: [B,N] float32, 4-byte aligned, overwritten
 *
 * Every query row's probabilities sum to 1, so each batch's masses sum to
 * H * N (within a factor 1 +- 2^-8 with the LSE of fa_fwd_ex on bf16, whose
 * row sums add the rounded P). P is computed in float32 from the float32 S of the matrix cores and
 * summed in float32, per head in a fixed order, then over the heads in order
 * 0 .. H-1: the result is deterministic. Needs B*H*N*4 bytes of scratch,
 * taken and released stream-ordered on `stream` like fa_bwd's. Limits and
 * errors as fa_fwd_ex; FA_ERR_OUT_OF_MEMORY if the scratch cannot be had.
 */
int fa_key_mass(const void* Q, const void* K, const float* LSE, float* mass,
                int B, int H, int Hkv, int N, int d, int causal,
                float softmax_scale, int dtype, void* stream);

/*
 * FP8 (E4M3) quantisation of 16 x 16 blocks ("GPU Performance Optimization
 * Batch 1 - Design Spec", Item 3, Design, optional FP8 path: each 16 x 16
 * block of Q and K is quantised to E4M3 with a per-block scale factor; Item 2,
 * Design, Step 1: the E4M3 cast saturates at +-448).
 *
 *   X       in : [R, N, d] 16-bit (dtype), R matrices (heads) of N rows
 *   codes   out: [R, N, d] uint8 E4M3 codes (OCP E4M3: sign, 4 exponent bits
 *                with bias 7, 3 mantissa bits), 16-byte aligned
 *   scales  out: [R, ceil(N/16), d/16] float32, one per block, 4-byte aligned
 *
 * A block is 16 consecutive rows (fewer in the last row block) x 16
 * consecutive columns of one matrix. Its scale is 2^e for the smallest integer
 * e with amax <= 448 * 2^e (amax: the block's largest magnitude), but at
 * least 2^-100, and 1 for an all-zero block. codes = the E4M3 value nearest to
 * x / 2^e (ties to even; zero encoded as 0x00), so x ~ decode(code) * scale
 * and no value saturates. Inputs must be finite. Allocates nothing. Errors:
 * FA_ERR_INVALID_ARG (null or misaligned pointer, R or N < 1, N*d >= 2^31),
 * FA_ERR_UNSUPPORTED (d not 64 or 128, unknown dtype).
 */
int fa_quantize_e4m3(const void* X, void* codes, float* scales, int R, int N,
                     int d, int dtype, void* stream);

/*
 * Forward pass of the FP8 path (same page, Item 3, Design, optional FP8
 * path): Q and K are quantised per 16 x 16 block as fa_quantize_e4m3 does,
 * and O, LSE are exact attention on the dequantised decode(code) * scale
 * values of Q and K, with V, P and O as in fa_fwd_ex. Arguments, layout and
 * errors as fa_fwd_ex with dtype bf16 (the only element type of this path;
 * there is no FP8 backward). The dequantised values have at most 4
 * significant bits, so the bf16 matrix products use them exactly. Inputs must
 * be finite with magnitudes below 2^120. Takes 2*B*Hkv*N*d bytes of scratch
 * (the dequantised K; Q is quantised as the forward loads it), stream-ordered
 * like fa_bwd's; FA_ERR_OUT_OF_MEMORY if it cannot be had.
 * Speed: the products run on the bf16 matrix cores, so this call costs about
 * as much as fa_fwd_ex plus the quantisation of K; it exists for its numerics.
 * gfx950's only FP8 matrix instruction faster than bf16 (the 32x32x64 one,
 * about twice the rate) scales per 32 values along the contraction, which a
 * 16-wide block cannot use without re-encoding its codes; the 16-deep FP8
 * instruction runs at the bf16 rate. fa_fwd_mxfp8 (1 x 32 blocks) is the FP8
 * forward that uses the faster instruction.
 */
int fa_fwd_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE,
               int B, int H, int Hkv, int N, int d, int causal,
               float softmax_scale, void* stream);

/*
 * FP8 (E4M3) quantisation of 1 x 32 blocks: the alternative reading of the
 * FP8 path ("GPU Performance Optimization Batch 1 - Design Spec", Item 3,
 * Design, optional FP8 path, read with Item 2's MX block-wise quantisation:
 * a block is one row by 32 consecutive columns, the OCP MX block size, which
 * gfx950's scaled FP8 matrix instruction applies at twice the bf16 rate).
 *
 *   X       in : [R, N, d] 16-bit (dtype), R matrices (heads) of N rows
 *   codes   out: [R, N, d] uint8 E4M3 codes, 16-byte aligned
 *   scales  out: [R, N, d/32] uint8 E8M0 scales: byte s means 2^(s - 127)
 *
 * Block c of row n covers columns 32c .. 32c + 31. Its exponent e, the codes
 * and the saturation rule are those of fa_quantize_e4m3 (smallest e with
 * amax <= 448 * 2^e, at least -100, 0 for a zero block; nearest E4M3 value
 * of x / 2^e, ties to even, zero as 0x00); the scale byte is 127 + e. Inputs
 * must be finite. Allocates nothing. Errors: FA_ERR_INVALID_ARG (null or
 * misaligned pointer, R or N < 1, R*N*d >= 2^40), FA_ERR_UNSUPPORTED (d not
 * 64 or 128, unknown dtype).
 */
int fa_quantize_mx_e4m3(const void* X, void* codes, void* scales, int R, int N, int d, int dtype,
                        void* stream);

/*
 * Forward pass of the FP8 path under the 1 x 32 block reading (see
 * fa_quantize_mx_e4m3): Q and K are quantised per row and 32 columns, and O,
 * LSE are exact attention on the dequantised decode(code) * 2^e values of Q
 * and K, with V, P and O as in fa_fwd_ex. The S = Q K^T products run on the
 * scaled 32x32x64 FP8 matrix instruction (E4M3 codes with their E8M0 block
 * scales), the P V products on bf16 matrix cores. Arguments, layout and
 * errors as fa_fwd_ex with dtype bf16 (no FP8 backward). Inputs must be
 * finite. Takes B*Hkv*N*(d + 4) bytes of scratch (K's codes and a 4-byte
 * scale word per key; Q is quantised as the forward loads it), stream-ordered
 * like fa_bwd's; FA_ERR_OUT_OF_MEMORY if it cannot be had.
 */
int fa_fwd_mxfp8(const void* Q, const void* K, const void* V, void* O, float* LSE,
                 int B, int H, int Hkv, int N, int d, int causal,
                 float softmax_scale, void* stream);

/* A static, human-readable description of a status code (never NULL). */
const char* fa_status_string(int status);

/*
 * Diagnostics: the name of the HIP error behind the most recent FA_ERR_HIP or
 * FA_ERR_OUT_OF_MEMORY returned on the calling thread ("hipSuccess" if none).
 * The string is static; the value is per thread.
 */
const char* fa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
