// Host-side launch interface between the C ABI (fa_abi.hip) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>

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
  float* rowstat; // 2 x [B,H,N] float32 scratch: LSE in base 2 for every row, then D = dO . O
  bool f16;       // element type of the 16-bit tensors: IEEE binary16 (true) or bf16
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

// Scratch bytes fa_bwd needs for a problem of this size.
inline size_t bwd_scratch_bytes(int B, int H, int N, int d) {
  (void)d;
  return (size_t)B * H * N * 8;
}

}  // namespace fa
