// C ABI of the exact tiled attention library (declared in include/fa.h).
// Validation is pure host code and happens before any HIP call; a call that
// fails validation enqueues nothing.

#include <stdint.h>

#include <cmath>
#include <mutex>

#include "../../include/fa.h"
#include "fa_launch.h"

// fa_bwd_noalloc's workspace: the backward's two float32 planes of row
// statistics for up to FA_NOALLOC_MAX_ROWS query rows (16 MiB), one copy in
// the memory of each GPU the library runs on, kept until the process ends.
// In host code `scratch` is only a host-side stand-in: kernels get the device
// address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) float scratch[2 * (size_t)FA_NOALLOC_MAX_ROWS];

namespace {

thread_local hipError_t g_last_hip_error = hipSuccess;

// Device address of `scratch` on each device, looked up on the first
// fa_bwd_noalloc call made with that device current.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_on_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

int hip_status(hipError_t e, int status_on_error) {
  if (e == hipSuccess) return FA_OK;
  g_last_hip_error = e;
  return status_on_error;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_common(int B, int H, int Hkv, int N, int d, int causal, float scale) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (Hkv < 1 || H % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)N * d >= (1LL << 31)) return FA_ERR_INVALID_ARG;
  // grid sizes: at most ceil(N/32) workgroups per head, one head per (b, h)
  const long long tiles = ((long long)N + 31) / 32;
  if ((long long)B * H > (1LL << 31) / tiles) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

int check_tensor(const void* p) {
  if (p == nullptr || !aligned(p, 16)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
              int Hkv, int N, int d, int causal, float softmax_scale, int dtype, void* stream) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_UNSUPPORTED;
  int st = check_common(B, H, Hkv, N, d, causal, softmax_scale);
  if (st != FA_OK) return st;
  for (const void* p : {Q, K, V, (const void*)O})
    if ((st = check_tensor(p)) != FA_OK) return st;
  if (LSE != nullptr && !aligned(LSE, 4)) return FA_ERR_INVALID_ARG;

  fa::FwdArgs a{Q, K, V, O, LSE, B, H, N, d, causal != 0, softmax_scale,
                reinterpret_cast<hipStream_t>(stream), dtype == FA_DTYPE_F16, Hkv};
  return hip_status(fa::launch_fwd(a), FA_ERR_HIP);
}

int fa_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int N,
           int d, int causal, float softmax_scale, void* stream) {
  return fa_fwd_ex(Q, K, V, O, LSE, B, H, H, N, d, causal, softmax_scale, FA_DTYPE_BF16, stream);
}

int fa_bwd_ex(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
              const void* dO, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N, int d,
              int causal, float softmax_scale, int dtype, void* stream) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_UNSUPPORTED;
  int st = check_common(B, H, Hkv, N, d, causal, softmax_scale);
  if (st != FA_OK) return st;
  for (const void* p : {Q, K, V, O, dO, (const void*)dQ, (const void*)dK, (const void*)dV})
    if ((st = check_tensor(p)) != FA_OK) return st;
  if (LSE == nullptr || !aligned(LSE, 4)) return FA_ERR_INVALID_ARG;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  const hipError_t m = hipMallocAsync(&scratch, fa::bwd_scratch_bytes(B, H, Hkv, N, d), s);
  if (m != hipSuccess || scratch == nullptr)
    return hip_status(m == hipSuccess ? hipErrorOutOfMemory : m, FA_ERR_OUT_OF_MEMORY);
  fa::BwdArgs a{Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, N, d, causal != 0, softmax_scale, s,
                static_cast<float*>(scratch), dtype == FA_DTYPE_F16, Hkv};
  const hipError_t e = fa::launch_bwd(a);
  const hipError_t f = hipFreeAsync(scratch, s);
  return hip_status(e != hipSuccess ? e : f, FA_ERR_HIP);
}

int fa_bwd_noalloc(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
                   const void* dO, void* dQ, void* dK, void* dV, int B, int H, int Hkv, int N,
                   int d, int causal, float softmax_scale, int dtype, void* stream) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_UNSUPPORTED;
  int st = check_common(B, H, Hkv, N, d, causal, softmax_scale);
  if (st != FA_OK) return st;
  for (const void* p : {Q, K, V, O, dO, (const void*)dQ, (const void*)dK, (const void*)dV})
    if ((st = check_tensor(p)) != FA_OK) return st;
  if (LSE == nullptr || !aligned(LSE, 4)) return FA_ERR_INVALID_ARG;
  if ((long long)B * H * N > FA_NOALLOC_MAX_ROWS) return FA_ERR_TOO_LARGE;

  float* ws = nullptr;
  const hipError_t w = scratch_on_current_device(&ws);
  if (w != hipSuccess) return hip_status(w, FA_ERR_HIP);
  fa::BwdArgs a{Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, N, d, causal != 0, softmax_scale,
                reinterpret_cast<hipStream_t>(stream), ws, dtype == FA_DTYPE_F16, Hkv};
  a.no_split = true;
  return hip_status(fa::launch_bwd(a), FA_ERR_HIP);
}

int fa_bwd(const void* Q, const void* K, const void* V, const void* O, const float* LSE,
           const void* dO, void* dQ, void* dK, void* dV, int B, int H, int N, int d, int causal,
           float softmax_scale, void* stream) {
  return fa_bwd_ex(Q, K, V, O, LSE, dO, dQ, dK, dV, B, H, H, N, d, causal, softmax_scale,
                   FA_DTYPE_BF16, stream);
}

int fa_key_mass(const void* Q, const void* K, const float* LSE, float* mass, int B, int H, int Hkv,
                int N, int d, int causal, float softmax_scale, int dtype, void* stream) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_UNSUPPORTED;
  int st = check_common(B, H, Hkv, N, d, causal, softmax_scale);
  if (st != FA_OK) return st;
  for (const void* p : {Q, K})
    if ((st = check_tensor(p)) != FA_OK) return st;
  if (LSE == nullptr || !aligned(LSE, 4) || mass == nullptr || !aligned(mass, 4))
    return FA_ERR_INVALID_ARG;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* part = nullptr;
  const hipError_t m = hipMallocAsync(&part, (size_t)B * H * N * 4, s);
  if (m != hipSuccess || part == nullptr)
    return hip_status(m == hipSuccess ? hipErrorOutOfMemory : m, FA_ERR_OUT_OF_MEMORY);
  fa::MassArgs a{Q, K, LSE, mass, static_cast<float*>(part), B, H, Hkv, N, d, causal != 0,
                 softmax_scale, s, dtype == FA_DTYPE_F16};
  const hipError_t e = fa::launch_mass(a);
  const hipError_t f = hipFreeAsync(part, s);
  return hip_status(e != hipSuccess ? e : f, FA_ERR_HIP);
}

int fa_quantize_e4m3(const void* X, void* codes, float* scales, int R, int N, int d, int dtype,
                     void* stream) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_UNSUPPORTED;
  if (R < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)N * d >= (1LL << 31)) return FA_ERR_INVALID_ARG;
  if ((long long)R * ((N + 15) / 16) >= (1LL << 31)) return FA_ERR_INVALID_ARG;
  int st = check_tensor(X);
  if (st != FA_OK) return st;
  if (codes == nullptr || !aligned(codes, 16) || scales == nullptr || !aligned(scales, 4))
    return FA_ERR_INVALID_ARG;
  fa::QuantArgs a{X, static_cast<uint8_t*>(codes), scales, nullptr, R, N, d,
                  reinterpret_cast<hipStream_t>(stream), dtype == FA_DTYPE_F16};
  return hip_status(fa::launch_quant(a), FA_ERR_HIP);
}

int fa_fwd_fp8(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
               int Hkv, int N, int d, int causal, float softmax_scale, void* stream) {
  int st = check_common(B, H, Hkv, N, d, causal, softmax_scale);
  if (st != FA_OK) return st;
  for (const void* p : {Q, K, V, (const void*)O})
    if ((st = check_tensor(p)) != FA_OK) return st;
  if (LSE != nullptr && !aligned(LSE, 4)) return FA_ERR_INVALID_ARG;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // K is quantised into scratch (it reaches the forward's LDS tiles by direct
  // loads); Q is quantised by the forward itself as it loads its operands
  const size_t k_bytes = (size_t)B * Hkv * N * d * 2;
  void* scratch = nullptr;  // dequantised K (bf16)
  const hipError_t m = hipMallocAsync(&scratch, k_bytes, s);
  if (m != hipSuccess || scratch == nullptr)
    return hip_status(m == hipSuccess ? hipErrorOutOfMemory : m, FA_ERR_OUT_OF_MEMORY);
  char* kd = static_cast<char*>(scratch);
  hipError_t e = fa::launch_quant(fa::QuantArgs{K, nullptr, nullptr, kd, B * Hkv, N, d, s, false});
  if (e == hipSuccess) {
    fa::FwdArgs fa_args{Q, kd, V, O, LSE, B, H, N, d, causal != 0, softmax_scale, s, false, Hkv};
    fa_args.fp8 = 1;
    e = fa::launch_fwd(fa_args);
  }
  const hipError_t f = hipFreeAsync(scratch, s);
  return hip_status(e != hipSuccess ? e : f, FA_ERR_HIP);
}

int fa_quantize_mx_e4m3(const void* X, void* codes, void* scales, int R, int N, int d, int dtype,
                        void* stream) {
  if (dtype != FA_DTYPE_BF16 && dtype != FA_DTYPE_F16) return FA_ERR_UNSUPPORTED;
  if (R < 1 || N < 1) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if ((long long)R * N * d >= (1LL << 40)) return FA_ERR_INVALID_ARG;
  int st = check_tensor(X);
  if (st != FA_OK) return st;
  if (codes == nullptr || !aligned(codes, 16) || scales == nullptr) return FA_ERR_INVALID_ARG;
  fa::QuantMxArgs a{X, static_cast<uint8_t*>(codes), static_cast<uint8_t*>(scales), R, N, d,
                    reinterpret_cast<hipStream_t>(stream), dtype == FA_DTYPE_F16, d / 32};
  return hip_status(fa::launch_quant_mx(a), FA_ERR_HIP);
}

int fa_fwd_mxfp8(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                 int Hkv, int N, int d, int causal, float softmax_scale, void* stream) {
  int st = check_common(B, H, Hkv, N, d, causal, softmax_scale);
  if (st != FA_OK) return st;
  for (const void* p : {Q, K, V, (const void*)O})
    if ((st = check_tensor(p)) != FA_OK) return st;
  if (LSE != nullptr && !aligned(LSE, 4)) return FA_ERR_INVALID_ARG;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // K is quantised into scratch: its codes, then a 4-byte word of scale bytes
  // per key (d / 32 of them used); Q is quantised by the forward as it loads it
  const size_t code_bytes = (size_t)B * Hkv * N * d;
  const size_t scale_bytes = (size_t)B * Hkv * N * 4;
  void* scratch = nullptr;
  const hipError_t m = hipMallocAsync(&scratch, code_bytes + scale_bytes, s);
  if (m != hipSuccess || scratch == nullptr)
    return hip_status(m == hipSuccess ? hipErrorOutOfMemory : m, FA_ERR_OUT_OF_MEMORY);
  uint8_t* kc = static_cast<uint8_t*>(scratch);
  uint8_t* ks = kc + code_bytes;
  hipError_t e = fa::launch_quant_mx(fa::QuantMxArgs{K, kc, ks, B * Hkv, N, d, s, false, 4});
  if (e == hipSuccess) {
    fa::FwdArgs fa_args{Q, kc, V, O, LSE, B, H, N, d, causal != 0, softmax_scale, s, false, Hkv};
    fa_args.fp8 = 2;
    fa_args.k_scales = ks;
    e = fa::launch_fwd(fa_args);
  }
  const hipError_t f = hipFreeAsync(scratch, s);
  return hip_status(e != hipSuccess ? e : f, FA_ERR_HIP);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARG:
      return "FA_ERR_INVALID_ARG: null or misaligned pointer, bad shape (K/V heads must divide "
             "query heads), scale or causal flag";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: head dimension must be 64 or 128, element type bf16 or f16";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP call or kernel launch failed";
    case FA_ERR_OUT_OF_MEMORY: return "FA_ERR_OUT_OF_MEMORY: scratch allocation failed";
    case FA_ERR_TOO_LARGE:
      return "FA_ERR_TOO_LARGE: B * H * N exceeds the static workspace of fa_bwd_noalloc "
             "(FA_NOALLOC_MAX_ROWS = 2097152 query rows)";
    default: return "unknown fa_status";
  }
}

const char* fa_last_hip_error(void) { return hipGetErrorName(g_last_hip_error); }

}  // extern "C"
