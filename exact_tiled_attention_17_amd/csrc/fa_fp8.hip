// FP8 (E4M3) path: Q and K quantised per 16 x 16 block before S = Q K^T
// ("GPU Performance Optimization Batch 1 - Design Spec", Item 3, Design,
// optional FP8 path; Item 2, Design, Step 1 for the saturating E4M3 cast).
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

// Byte b (0..3) of w decoded from E4M3 (the byte selector must be a constant).
__device__ __forceinline__ float e4m3_byte(uint32_t w, int b) {
  switch (b) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}

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
  // amax = m 2^E, m in [0.5, 1); 448 = 0.875 2^9
  const float mant = __builtin_amdgcn_frexp_mantf(amax);
  const int E = __builtin_amdgcn_frexp_expf(amax);
  int e = mant <= 0.875f ? E - 9 : E - 8;
  e = e < -100 ? -100 : e;
  e = amax == 0.f ? 0 : e;

  uint32_t cw[EL / 4];  // codes, 4 per dword
#pragma unroll
  for (int j = 0; j < EL / 4; ++j) {
    const float* y4 = &x[4 * j];
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(y4[0], -e),
                                            __builtin_amdgcn_ldexpf(y4[1], -e), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(y4[2], -e),
                                        __builtin_amdgcn_ldexpf(y4[3], -e), w, true);
    uint32_t u = (uint32_t)w;
    // zero is +0: clear the sign of every byte whose magnitude bits are 0
#pragma unroll
    for (int b = 0; b < 4; ++b)
      if (((u >> (8 * b)) & 0x7Fu) == 0u) u &= ~(0xFFu << (8 * b));
    cw[j] = u;
  }

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
        const float a = __builtin_amdgcn_ldexpf(e4m3_byte(cw[i / 4], i % 4), e);
        const float b = __builtin_amdgcn_ldexpf(e4m3_byte(cw[i / 4], i % 4 + 1), e);
        o[m] = (__builtin_bit_cast(uint32_t, a) >> 16) | (__builtin_bit_cast(uint32_t, b) & 0xFFFF0000u);
      }
      *reinterpret_cast<u32x4*>(deq + off) = o;
    }
  }
  if (scales != nullptr && lane < CPR && (lane & 1) == 0)
    scales[((size_t)r * nrb + rb) * (D / 16) + lane / 2] = __builtin_amdgcn_ldexpf(1.f, e);
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
