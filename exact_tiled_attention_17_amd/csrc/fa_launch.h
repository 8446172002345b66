// Host-side launch interface between the C ABI (fa_abi.hip) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* LSE;
  int B, H, N, d;
  bool causal;
  float softmax_scale;
  hipStream_t stream;
  bool f16;  // element type of Q, K, V, O: IEEE binary16 (true) or bf16
  int Hkv;   // K/V heads; divides H (query head h reads K/V head h / (H / Hkv))
  // FP8 paths (bf16 only): 0 none; 1: 16 x 16 blocks, Q quantised on load, K
  // given dequantised (bf16); 2: 1 x 32 blocks, Q quantised on load, K given
  // as E4M3 codes ([B,Hkv,N,d] bytes) with E8M0 scale bytes in k_scales
  // ([B,Hkv,N,d/32]), the S products on the scaled FP8 matrix instruction
  int fp8 = 0;
  const uint8_t* k_scales = nullptr;
};

struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const float* LSE;
  const void* dO;
  void* dQ;
  void* dK;
  void* dV;
  int B, H, N, d;
  bool causal;
  float softmax_scale;
  hipStream_t stream;
  float* rowstat; // scratch of bwd_scratch_bytes: 2 x [B,H,N] float32 (LSE in base 2 for
                  // every row, then -D = -dO . O), then the dK/dV partial sums if split
  bool f16;       // element type of the 16-bit tensors: IEEE binary16 (true) or bf16
  int Hkv;        // K/V heads (K, V, dK, dV are [B,Hkv,N,d]); divides H
  bool no_split = false;  // never split the dK/dV work (scratch holds the row statistics only)
};

struct MassArgs {
  const void* Q;
  const void* K;
  const float* LSE;
  float* mass;   // [B, N] float32 output
  float* part;   // [B*H, N] float32 scratch: per-head column sums
  int B, H, Hkv, N, d;
  bool causal;
  float softmax_scale;
  hipStream_t stream;
  bool f16;
};

struct QuantArgs {
  const void* X;    // [R, N, d] 16-bit input
  uint8_t* codes;   // [R, N, d] E4M3 codes, or nullptr
  float* scales;    // [R, ceil(N / 16), d / 16] block scales (powers of two), or nullptr
  void* deq;        // [R, N, d] bf16 dequantised values, or nullptr
  int R, N, d;
  hipStream_t stream;
  bool f16;
};

// 1 x 32 blocks: codes [R, N, d] and E8M0 scale bytes (2^(byte - 127)),
// scale_stride bytes per row (d / 32 of them written), both required
struct QuantMxArgs {
  const void* X;
  uint8_t* codes;
  uint8_t* scales;
  int R, N, d;
  hipStream_t stream;
  bool f16;
  int scale_stride;
};

// Enqueues `kernel` and returns the status of this launch alone (not the
// runtime's sticky last error, which other libraries in the process may have
// left behind).
template <class T>
struct same_type {
  using type = T;
};
template <typename... KArgs>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                                typename same_type<KArgs>::type... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, argv, 0, stream);
}

hipError_t launch_fwd(const FwdArgs& a);
hipError_t launch_bwd(const BwdArgs& a);
hipError_t launch_mass(const MassArgs& a);
hipError_t launch_quant(const QuantArgs& a);
hipError_t launch_quant_mx(const QuantMxArgs& a);

// float32 row statistics of the backward: LSE in base 2, then -D, per query row
// (padded to a multiple of 64 floats so that what follows stays 256-byte aligned).
inline size_t rowstat_floats(int B, int H, int N) {
  return ((size_t)B * H * N * 2 + 63) / 64 * 64;
}

// Workgroups that share the query heads of one K/V head in the dK/dV kernel
// (a divisor S of G = H / Hkv). With few K/V heads, one workgroup per key
// block would leave most of the 256 compute units idle (multi-query
// attention: B * ceil(N / 128) workgroups), so the group is split until the
// grid has 1024 workgroups (four per compute unit), each split writing
// float32 partial sums (8 * S * B * Hkv * N * d bytes in all, kept under 1 GiB).
// The causal forward and dQ pass pair query tiles (tile nq - 1 - w with tile
// w in one workgroup) when at least this many workgroups remain.
constexpr long long kFwdPairMinWorkgroups = 256;

// The causal key-mass pass pairs key blocks when at least this many
// workgroups (four per CU run at once) remain.
constexpr long long kMassPairMinWorkgroups = 1024;

// The dK/dV pass can give a workgroup pairs of key blocks (block p with
// block nkb - 1 - p: equally long workgroups under the causal mask, fewer of
// them). Pairs per workgroup: the largest of 4, 2, 1 that leaves at least
// kDkdvMinWorkgroups workgroups for `blocks` key blocks (nkb per head), or 0
// (one block per workgroup) if even single pairs would leave fewer.
// More than one pair per workgroup measured no faster (two) or slower (four)
// at 4x64x4096x128 and 8x64x2048x128 causal.
constexpr long long kDkdvMinWorkgroups = 1024;
constexpr int kDkdvMaxPairsPerWorkgroup = 1;

inline int dkdv_pairs_per_workgroup(long long blocks, int nkb) {
  const long long heads = blocks / nkb;  // (batch, K/V head, split) triples
  const int npb = (nkb + 1) / 2;
  for (int m = kDkdvMaxPairsPerWorkgroup; m >= 1; m /= 2)
    if (heads * ((npb + m - 1) / m) >= kDkdvMinWorkgroups && 2 * m <= nkb) return m;
  return 0;
}

inline int dkdv_splits(int B, int H, int Hkv, int N, int d) {
  const int G = H / Hkv;
  const long long blocks = (long long)B * Hkv * ((N + 127) / 128);
  const long long part_per_split = 8LL * B * Hkv * N * d;
  int best = 1;
  for (int S = 2; S <= G; ++S) {
    if (G % S) continue;
    if (blocks * best >= 1024 || part_per_split * S > (1LL << 30)) break;
    best = S;
  }
  return best;
}

// Scratch bytes fa_bwd needs for a problem of this size.
inline size_t bwd_scratch_bytes(int B, int H, int Hkv, int N, int d) {
  const int S = dkdv_splits(B, H, Hkv, N, d);
  size_t bytes = rowstat_floats(B, H, N) * 4;
  if (S > 1) bytes += (size_t)S * 8 * B * Hkv * N * d;
  return bytes;
}

}  // namespace fa
