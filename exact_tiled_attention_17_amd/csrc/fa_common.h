// Device-side building blocks shared by the forward and backward kernels:
// vector types for bf16 MFMA operands, 128-bit memory moves, cross-lane
// reductions within a 64-wide wavefront, and the launch plumbing that maps
// workgroups onto the eight XCDs of an MI355X.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ u32x4 as_u32x4(bf16x8 v) { return __builtin_bit_cast(u32x4, v); }

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// One 32x32x16 bf16 matrix-core product with float32 accumulation.
// Operand layout for a 64-lane wave (lane l, half h = l / 32):
//   A (32 x 16): lane l holds row l % 32, k = 8h .. 8h+7
//   B (16 x 32): lane l holds column l % 32, k = 8h .. 8h+7
//   C (32 x 32): lane l holds column l % 32, rows 8*(r/4) + 4h + r%4, r = 0..15
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// The same product on 16-bit operands held as raw bits: bf16 (F16 = false)
// or IEEE binary16 (F16 = true), float32 accumulation either way.
template <bool F16>
__device__ __forceinline__ f32x16 mfma32x(bf16x8 a, bf16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- E4M3 (OCP FP8: bias 7, largest finite 448) block quantisation ---------
// The scale of a block with largest magnitude amax is 2^e with the smallest e
// for which amax <= 448 2^e, e >= -100, and e = 0 for a zero block. Then
// nothing saturates and every dequantised value decode(code) 2^e has at most
// 4 significant bits and a normal exponent, so it is exact in bf16.
__device__ __forceinline__ int e4m3_block_exp(float amax) {
  // amax = m 2^E, m in [0.5, 1); 448 = 0.875 2^9
  const float mant = __builtin_amdgcn_frexp_mantf(amax);
  const int E = __builtin_amdgcn_frexp_expf(amax);
  int e = mant <= 0.875f ? E - 9 : E - 8;
  e = e < -100 ? -100 : e;
  return amax == 0.f ? 0 : e;
}
// Codes of x0..x3 / 2^e (the E4M3 value nearest, ties to even), byte i for
// x_i; a code of magnitude zero is +0.
__device__ __forceinline__ uint32_t e4m3_codes4(float x0, float x1, float x2, float x3, int e) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(x0, -e),
                                          __builtin_amdgcn_ldexpf(x1, -e), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(__builtin_amdgcn_ldexpf(x2, -e),
                                      __builtin_amdgcn_ldexpf(x3, -e), w, true);
  uint32_t u = (uint32_t)w;
#pragma unroll
  for (int b = 0; b < 4; ++b)
    if (((u >> (8 * b)) & 0x7Fu) == 0u) u &= ~(0xFFu << (8 * b));
  return u;
}
// Byte b (0..3) of w decoded from E4M3 (the byte selector must be a constant).
__device__ __forceinline__ float e4m3_byte(uint32_t w, int b) {
  switch (b) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)w, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)w, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  }
}
// Bytes b, b + 1 of codes w dequantised at scale 2^e, as a packed bf16 pair
// (exact: the top halves of the float32 values).
__device__ __forceinline__ uint32_t e4m3_deq2_bf16(uint32_t w, int b, int e) {
  const float a = __builtin_amdgcn_ldexpf(e4m3_byte(w, b), e);
  const float c = __builtin_amdgcn_ldexpf(e4m3_byte(w, b + 1), e);
  return (__builtin_bit_cast(uint32_t, a) >> 16) | (__builtin_bit_cast(uint32_t, c) & 0xFFFF0000u);
}

// S^T += A B on the scaled 32x32x64 FP8 matrix instruction, both operands
// E4M3 codes. Lane layout (gfx950, measured by an in-bounds probe): lane l
// holds row (A) or column (B) l % 32; its bytes 0..15 are k = 16 (l / 32) +
// 0..15 and bytes 16..31 are k = 32 + 16 (l / 32) + 0..15. The products of
// k-block kb (k = 32 kb .. 32 kb + 31) of row i (column j) are scaled by the
// E8M0 byte OP of lane i + 32 kb's scale word (j + 32 kb's for B): 2^(byte -
// 127). C starts at zero when FIRST.
template <int OP, bool FIRST>
__device__ __forceinline__ f32x16 mfma_mx(i32x8 a, i32x8 b, f32x16 c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, FIRST ? f32x16{} : c, 0, 0, OP, (int)sa,
                                                         OP, (int)sb);
}

// Lanes l and l ^ 32 exchange values; returns (own, partner) in some order,
// so symmetric reductions (max, sum) over the pair are exact either way.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// s_waitcnt vmcnt(0): every outstanding vector-memory load has landed. Placed
// where that is already true in effect, it tells the compiler's wait-count
// analysis so, and later uses of those registers need no wait.
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// float32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}

// float32 pair -> packed 16-bit pair of the element type, round to nearest
// even (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32); low half = lo.
template <bool F16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 f = {lo, hi};
  if constexpr (F16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
// the low / high 16-bit element of a packed pair, widened exactly to float32
template <bool F16>
__device__ __forceinline__ float lo16(uint32_t w) {
  if constexpr (F16) return (float)__builtin_bit_cast(f16x2, w)[0];
  else return __uint_as_float(w << 16);
}
template <bool F16>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (F16) return (float)__builtin_bit_cast(f16x2, w)[1];
  else return __uint_as_float(w & 0xFFFF0000u);
}
// float32 -> one 16-bit element (bits), round to nearest even
template <bool F16>
__device__ __forceinline__ uint16_t to16(float v) {
  if constexpr (F16) return __builtin_bit_cast(uint16_t, (_Float16)v);
  else return __builtin_bit_cast(uint16_t, (__bf16)v);
}

// Buffer resource over `bytes` bytes at `base` (raw addressing, no stride).
// The range check of a raw buffer access (CDNA3 / CDNA4 ISA reference guides,
// buffer addressing, range checking) compares the instruction's immediate
// offset plus its per-lane offset with the record count; the scalar offset
// is not part of it. A load whose immediate + per-lane offset is at or past
// `bytes` returns zeros (into registers or LDS) and touches no memory. The
// kernels therefore never put a row offset in the scalar operand: each tile
// gets a resource of its own (rows_rsrc), and only offsets inside the tile
// go in the per-lane operand.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Resource over rows row0 .. nrows - 1 of an array of `row_bytes`-byte rows at
// `base` (wave-uniform arguments, so it lives in scalar registers): per-lane
// offset o reads byte o of row row0, and offsets that reach row nrows or
// beyond read as zeros. A tile that starts at or past nrows gets an empty
// resource at `base` itself, so no address past the array is ever formed.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, int row0, int nrows,
                                                            uint32_t row_bytes) {
  const bool inside = row0 < nrows;
  const char* p = static_cast<const char*>(base) + (inside ? (size_t)row0 * row_bytes : 0);
  const uint32_t bytes = inside ? (uint32_t)(nrows - row0) * row_bytes : 0u;
  return make_rsrc(p, bytes);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

// 16 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds_base + 16 l (lds_base is wave-uniform); the source is byte voff (per
// lane, range-checked) of the buffer. Completion is tracked by vmcnt, like
// any vector-memory load. The scalar offset is always 0 (see make_rsrc).
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, __bf16* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16,
                                           voff, 0, 0, 0);
}

// 4 bytes per lane from a buffer straight into LDS: lane l's bytes land at
// lds_base + 4 l.
__device__ __forceinline__ void buf_load4_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 4,
                                           voff, 0, 0, 0);
}

// 2 or 4 bytes per lane through a buffer resource: a store whose per-lane
// offset (plus the immediate) is past the resource's end writes nothing.
__device__ __forceinline__ void buf_store2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, voff, 0, 0);
}
__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, voff, 0, 0);
}

__device__ __forceinline__ f32x4 buf_load16f(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_global8(void* p, u32x2 v) {
  *reinterpret_cast<u32x2*>(p) = v;
}
__device__ __forceinline__ bf16x8 ld_lds16(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ void st_lds16(__bf16* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ void st_lds8(__bf16* p, u32x2 v) {
  *reinterpret_cast<u32x2*>(p) = v;
}

// Writes a wave's 32 x D tile, held transposed in D / 32 accumulators (lane
// l: row l % 32; register r of block b: column 32 b + 8 (r / 4) + 4 (l / 32)
// + r % 4), each row scaled by the lane's `mul` and rounded to the 16-bit
// type, to rows row0 .. row0 + 31 of a row-major [*, D] tensor `dst` (rows
// >= nrows are skipped). The tile goes through `stage`, 32 * D elements of
// LDS owned by this wave, so that each global store instruction writes
// 64 x 16 consecutive bytes (whole rows) instead of 64 scattered 8-byte
// pieces. In `stage`, 16-byte chunk c of row r sits at c ^ (r mod CPR), CPR
// the chunks per row, which spreads both the writes and the reads over the
// banks. Every lane of the wave must run it (rows past the end included).
template <int D, bool F16>
__device__ __forceinline__ void store_rows_via_lds(const f32x16 (&acc)[D / 32], float mul, __bf16* stage,
                                                   __bf16* dst, int row0, int nrows) {
  constexpr int CPR = D / 8;       // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;    // rows per store instruction
  // (the lane index is made opaque so that the addresses below are formed
  // here, not hoisted out of the caller's loops and kept live across them)
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack2<F16>(acc[b][4 * g] * mul, acc[b][4 * g + 1] * mul);
      w[1] = pack2<F16>(acc[b][4 * g + 2] * mul, acc[b][4 * g + 3] * mul);
      const int c = (4 * b + g) ^ (l32 & (CPR - 1));
      st_lds8(stage + l32 * D + 8 * c + 4 * hh, w);
    }
#pragma unroll
  for (int k = 0; k < 32 / RPI; ++k) {
    const int r = k * RPI + lane / CPR, c = lane % CPR;
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + r * D + 8 * (c ^ (r & (CPR - 1))));
    if (row0 + r < nrows) *reinterpret_cast<u32x4*>(dst + (size_t)(row0 + r) * D + 8 * c) = v;
  }
}

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16). Within each group of 16 lanes,
// lane 16g+i reads 4 bf16 at its own address; lane 16g+t then receives element
// (t & 3) of the reads of lanes 16g + (t >> 2) + 4e, for e = 0..3. So to give
// lane l the values X[row(e)][col0 + l % 16] of a row-major tile X, lane 16g+i
// passes the address of X[row(i >> 2)][col0 + 4 (i & 3)].
__device__ __forceinline__ bf16x4 ld_lds_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((__attribute__((address_space(3))) bf16x4*)p);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Row-major tiles of d-wide rows keep 16-byte chunk c of row r at chunk
// position c ^ swz(r). For d = 128 the swizzle makes both access patterns
// conflict-free: 16 consecutive rows at one chunk (operand rows), and 4
// consecutive rows x 4 consecutive chunks (transposing reads).
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (r >> 1) & 7;
}
template <int D>
__device__ __forceinline__ int tile_off(int r, int col) {  // element offset of (r, col), col % 4 == 0
  return r * D + (((col >> 3) ^ swz<D>(r)) << 3) + (col & 4);
}
// Maps a linear workgroup id to (head, tile) so that the workgroups that land
// on one XCD (the hardware deals ids round-robin over the 8 XCDs) cover whole
// heads, which then share that XCD's L2; within an XCD, heads go one after the
// other, each head's tiles in increasing order.
__device__ __forceinline__ void xcd_remap(int bid, int total, int tiles, int& head, int& tile) {
  int v = bid;
  if (total % kXcds == 0) {
    const int per = total / kXcds;
    v = (bid % kXcds) * per + bid / kXcds;
  }
  head = v / tiles;
  tile = v % tiles;
}

}  // namespace fa
