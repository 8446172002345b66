// FP8 (E4M3) path: Q and K quantised per 16 x 16 block before S = Q K^T
// ("GPU Performance Optimization Batch 1 - Design Spec", Item 3, Design,
// optional FP8 path; Item 2, Design, Step 1 for the saturating E4M3 cast).
// This file holds the quantisation kernels (fa_quantize_e4m3, and K for
// fa_fwd_fp8; fa_quantize_mx_e4m3, and K for fa_fwd_mxfp8, the 1 x 32 block
// reading); the forward quantises Q itself as it loads it (fa_fwd.hip).
//
// A block is 16 token rows x 16 head-dim columns of one head. Its scale is
// the power of two 2^e with the smallest e such that the block's largest
// magnitude amax is at most 448 * 2^e (e >= -100; e = 0 for a zero block);
// every value is encoded as the E4M3 value nearest to x / 2^e, ties to even,
// zero as +0. With power-of-two scales the dequantised values
// decode(code) * 2^e have at most 4 significant bits and stay exact in bf16,
// so the forward runs its bf16 matrix products on them unchanged. (gfx950's
// FP8 matrix instructions contract 64 values per row and scale them, if at
// all, per 32 along the contraction in powers of two: a 16-wide block with a
// scale of its own cannot ride them at their full rate.)

#include <stdint.h>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// One wave per (matrix, 16-row block). The block's rows are consecutive in
// memory (16 D 2 bytes), so instruction v of the wave moves bytes
// [1024 v, 1024 v + 1024) of it: lane l takes the 16-byte chunk l % CPR of
// row v RPI + l / CPR (CPR = D / 8 chunks per row, RPI = 64 / CPR rows per
// instruction). Every load and store instruction is one contiguous span. A
// lane's chunks all lie in 16-column block (l % CPR) / 2, and the lanes of one
// block differ in bit 0 and in the bits from CPR up: a 3- or 4-step XOR
// shuffle gives the block's amax.
template <int D, bool F16>
__global__ __launch_bounds__(256) void quant_e4m3_kernel(const __bf16* __restrict__ X,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ scales,
                                                         __bf16* __restrict__ deq, int N,
                                                         long long nblk) {
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;   // rows per instruction
  constexpr int NI = 16 / RPI;    // instructions per block
  constexpr int EL = 8 * NI;      // elements per lane
  const long long wb = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wb >= nblk) return;         // whole waves only
  const int lane = threadIdx.x & 63;
  const int nrb = (N + 15) / 16;
  const long long r = wb / nrb;
  const int rb = (int)(wb - r * nrb);
  const int rows = min(16, N - 16 * rb);  // rows of this block (the last may be short)
  const int c = lane % CPR;               // chunk of the row
  const size_t blk0 = ((size_t)r * N + 16 * rb) * D;  // first element of the block

  float x[EL];
#pragma unroll
  for (int v = 0; v < NI; ++v) {
    const int rr = v * RPI + lane / CPR;
    const u32x4 w = rr < rows ? ld_global16(X + blk0 + (size_t)rr * D + 8 * c) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      x[8 * v + 2 * m] = lo16<F16>(w[m]);
      x[8 * v + 2 * m + 1] = hi16<F16>(w[m]);
    }
  }

  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < EL; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
#pragma unroll
  for (int sh = CPR; sh < 64; sh <<= 1) amax = fmaxf(amax, __shfl_xor(amax, sh));
  const int e = e4m3_block_exp(amax);

  uint32_t cw[EL / 4];  // codes, 4 per dword
#pragma unroll
  for (int j = 0; j < EL / 4; ++j) cw[j] = e4m3_codes4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3], e);

#pragma unroll
  for (int v = 0; v < NI; ++v) {
    const int rr = v * RPI + lane / CPR;
    if (rr >= rows) continue;
    const size_t off = blk0 + (size_t)rr * D + 8 * c;
    if (codes != nullptr) *reinterpret_cast<u32x2*>(codes + off) = u32x2{cw[2 * v], cw[2 * v + 1]};
    if (deq != nullptr) {
      // decode(code) * 2^e has at most 4 significant bits and a normal
      // exponent: exact in bf16, so its top 16 bits are the bf16 value
      u32x4 o;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int i = 8 * v + 2 * m;  // elements i, i + 1: dword i / 4, bytes i % 4, i % 4 + 1
        o[m] = e4m3_deq2_bf16(cw[i / 4], i % 4, e);
      }
      *reinterpret_cast<u32x4*>(deq + off) = o;
    }
  }
  if (scales != nullptr && lane < CPR && (lane & 1) == 0)
    scales[((size_t)r * nrb + rb) * (D / 16) + lane / 2] = __builtin_amdgcn_ldexpf(1.f, e);
}

// 1 x 32 blocks (one row, 32 aligned columns; the same scale rule and
// rounding): thread g quantises block g, which is elements [32 g, 32 g + 32)
// of the [R, N, d] input (64 contiguous bytes), and writes its 32 codes and
// its scale byte 127 + e (E8M0: 2^(byte - 127)) at byte c of its row's
// scale_stride bytes (c = the block's index in the row, of bpr = d / 32). No
// shuffles: a block is one thread's.
template <bool F16>
__global__ __launch_bounds__(256) void quant_mx_kernel(const __bf16* __restrict__ X,
                                                       uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, long long nblk,
                                                       int bpr, int scale_stride) {
  const long long g = (long long)blockIdx.x * 256 + threadIdx.x;
  if (g >= nblk) return;
  const __bf16* src = X + g * 32;
  float x[32];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const u32x4 w = ld_global16(src + 8 * v);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      x[8 * v + 2 * m] = lo16<F16>(w[m]);
      x[8 * v + 2 * m + 1] = hi16<F16>(w[m]);
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const int e = e4m3_block_exp(amax);
  u32x4 c0, c1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    c0[j] = e4m3_codes4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3], e);
    c1[j] = e4m3_codes4(x[16 + 4 * j], x[17 + 4 * j], x[18 + 4 * j], x[19 + 4 * j], e);
  }
  *reinterpret_cast<u32x4*>(codes + g * 32) = c0;
  *reinterpret_cast<u32x4*>(codes + g * 32 + 16) = c1;
  const long long row = g / bpr;
  scales[row * scale_stride + (g - row * bpr)] = (uint8_t)(127 + e);
}

hipError_t launch_quant_mx(const QuantMxArgs& a) {
  const long long nblk = (long long)a.R * a.N * (a.d / 32);
  const dim3 grid((unsigned)((nblk + 255) / 256));
  if (a.f16)
    return launch_kernel(quant_mx_kernel<true>, grid, dim3(256), a.stream, (const __bf16*)a.X, a.codes,
                         a.scales, nblk, a.d / 32, a.scale_stride);
  return launch_kernel(quant_mx_kernel<false>, grid, dim3(256), a.stream, (const __bf16*)a.X, a.codes,
                       a.scales, nblk, a.d / 32, a.scale_stride);
}

template <int D, bool F16>
static hipError_t launch_quant_t(const QuantArgs& a) {
  const long long nblk = (long long)a.R * ((a.N + 15) / 16);
  return launch_kernel(quant_e4m3_kernel<D, F16>, dim3((unsigned)((nblk + 3) / 4)), dim3(256), a.stream,
                       (const __bf16*)a.X, a.codes, a.scales, (__bf16*)a.deq, a.N, nblk);
}

hipError_t launch_quant(const QuantArgs& a) {
  if (a.d == 128) return a.f16 ? launch_quant_t<128, true>(a) : launch_quant_t<128, false>(a);
  return a.f16 ? launch_quant_t<64, true>(a) : launch_quant_t<64, false>(a);
}

}  // namespace fa
