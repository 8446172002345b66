// Attention mass per key position for SnapKV-style key eviction
// ("GPU Performance Optimization Batch 1 - Design Spec", Item 4, Design: the
// attention weights each key receives during prefill are summed, then reduced
// over the heads):
//   mass[b, j] = sum over query heads h and query rows i of P[b, h, i, j].
// P needs the final log-sum-exp of its row, so this is a second, key-major
// pass after the forward: for each block of keys the workgroup recomputes
// S = Q K^T over the query tiles that see the block and sums
// P = exp2(c S - LSE2) down each key's column (the dK/dV kernel's P step
// without the products that follow). Per-head column sums go to a float32
// [B*H, N] scratch; a second kernel adds the heads in a fixed order, so the
// result does not depend on scheduling.

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct MassCfg {
  static constexpr int NW = 4;              // waves per workgroup, 32 keys each
  static constexpr int THREADS = 64 * NW;
  static constexpr int BCB = 32 * NW;       // keys per workgroup
  static constexpr int QB = 2;              // 32-query blocks per step
  static constexpr int BRB = 32 * QB;       // queries per step
  static constexpr int CH = D / 8;          // 16-byte chunks per row
  static constexpr int TI = BRB * CH / 64;  // direct-to-LDS instructions per Q tile
  static_assert(TI % NW == 0, "tile loads split evenly over the waves");
};

// Four waves per SIMD (128 registers): the exponentials of one wave hide under
// the products of the others. (At 132 registers the compiler's choice gives
// three; capping at 128 costs a few spills outside the step loop and measured
// 0.79 -> 0.75 ms at 4 x 64 x 4096 x 128.)
template <int D, bool CAUSAL, bool F16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4)))
void key_mass_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const float* __restrict__ LSE, float* __restrict__ part, int N, int BH, int G,
                     float c_log2, int pairs) {
  // BH query heads; query head bh reads K head bh / G
  using C = MassCfg<D>;
  constexpr int BRB = C::BRB, QB = C::QB, CH = C::CH, LM = C::TI / C::NW;
  // Q tiles row-major, 16-byte chunk c of row r at c ^ swz(r) (operand-row
  // reads conflict-free); two buffers, as separate arrays so that every access
  // names its buffer statically
  __shared__ __attribute__((aligned(16))) __bf16 qs0[BRB * D];
  __shared__ __attribute__((aligned(16))) __bf16 qs1[BRB * D];
  __shared__ __attribute__((aligned(16))) float ls0[BRB];  // LSE (natural log) of the step's queries
  __shared__ __attribute__((aligned(16))) float ls1[BRB];

  // With `pairs` (causal only) the workgroup runs key block w, then block
  // nkb - 1 - w: every pair has the same number of query steps.
  const int nkb = (N + C::BCB - 1) / C::BCB;
  const int nwb = pairs ? (nkb + 1) / 2 : nkb;
  int bh, wb;
  xcd_remap(blockIdx.x, nwb * BH, nwb, bh, wb);
  const int nit = pairs && wb != nkb - 1 - wb ? 2 : 1;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const __bf16* const Qh = Q + (size_t)bh * N * D;
  const float* const Lh = LSE + (size_t)bh * N;
  const auto rK = make_rsrc(K + (size_t)(bh / G) * N * D, head_bytes);

  // ---- step loads, straight from HBM into LDS: instruction n fills chunk
  // positions [64 n, 64 n + 64) of the Q tile (dealt round-robin over the
  // waves); wave 0 also loads the 64 LSE values. Both go through resources
  // that start at the step's first query and end at query N, so the rows past
  // N of a ragged last step read as zeros --------------------------------------
  uint32_t src_w[LM];
#pragma unroll
  for (int m = 0; m < LM; ++m) {
    const int p = 64 * (wave + C::NW * m) + lane;
    const int r = p / CH, pc = p % CH;
    src_w[m] = (uint32_t)(r * (D * 2) + ((pc ^ swz<D>(r)) * 16));
  }
  const int nqt = (N + BRB - 1) / BRB;
  int rw = tile_off<D>(l32, 8 * hh);  // operand row l32, chunk hh; k-step st at rw ^ 16 st
  asm volatile("" : "+v"(rw));
  auto barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // one key block: its sweep over the query steps and its column sums
  auto run_item = [&](const int kb) __attribute__((always_inline)) {
    const int k0 = kb * C::BCB;
    const int kw0 = k0 + 32 * wave;  // this wave's first key
    const int key = kw0 + l32;       // this lane's key (column of S); rows past N read as 0

    bf16x8 frag[D / 16];  // the lane's K row as B operands
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      frag[s] = as_bf16x8(buf_load16(rK, (uint32_t)key * (D * 2) + (16 * s + 8 * hh) * 2));

    const int i0 = CAUSAL ? k0 / BRB : 0;  // first query tile that sees the block's keys
    const int nsteps = nqt - i0;
    auto load_step = [&](int s, __bf16* qd, float* ld) __attribute__((always_inline)) {
      const int q0 = (i0 + s) * BRB;
      const auto rQ = rows_rsrc(Qh, q0, N, D * 2);
#pragma unroll
      for (int m = 0; m < LM; ++m) buf_load16_lds(rQ, src_w[m], qd + 64 * (wave + C::NW * m) * 8);
      if (wave == 0) buf_load4_lds(rows_rsrc(Lh, q0, N, 4), 4u * lane, ld);
    };

    float colsum = 0.f;  // this lane's share of its key's mass (half the rows of each block)
    auto step = [&](int s, const __bf16* tile, const float* lse) __attribute__((always_inline)) {
      // S for 64 queries x this wave's 32 keys: lane = one key, 16 queries per block
      f32x16 sd[QB];
      constexpr int NP = (D / 16) * QB;  // product i: k-step i / QB, query block i % QB
      constexpr int R = 2;
      auto rd = [&](int i) { return ld_lds16(tile + (rw ^ (16 * (i / QB))) + 32 * (i % QB) * D); };
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sd[qb] = f32x16{};
      bf16x8 ar[R];
#pragma unroll
      for (int j = 0; j < R; ++j) ar[j] = rd(j);
#pragma unroll
      for (int i = 0; i < NP; ++i) {
        sd[i % QB] = mfma32x<F16>(ar[i % R], frag[i / QB], sd[i % QB]);
        if (i + R < NP) ar[i % R] = rd(i + R);
      }
      // P = exp2(c S - LSE2), masked: query q0 + m (m = 32 qb + 8 g + 4 hh + e)
      // counts iff (unsigned)(m + mbase) < mbound (it exists and, if causal,
      // is at or after the key); a key past the end collects nothing
      const int q0 = (i0 + s) * BRB;
      const bool need_mask = (CAUSAL && q0 < kw0 + 31) || (kw0 + 32 > N) || (q0 + BRB > N);
      const int qlo = CAUSAL ? key : 0;
      const int mbase = q0 - qlo;
      const unsigned mbound = key < N ? (unsigned)(N - qlo) : 0u;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int m0 = 32 * qb + 8 * g + 4 * hh;
          const f32x4 l4 = *reinterpret_cast<const f32x4*>(&lse[m0]);
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            p[e] = fast_exp2(__builtin_fmaf(sd[qb][4 * g + e], c_log2, -l4[e] * kLog2e));
          if (need_mask) {  // selects under one wave-uniform branch
#pragma unroll
            for (int e = 0; e < 4; ++e) p[e] = (unsigned)(m0 + e + mbase) >= mbound ? 0.f : p[e];
          }
          colsum += (p[0] + p[1]) + (p[2] + p[3]);
        }
    };
    barrier();  // the previous block's last step is read by every wave
    load_step(0, qs0, ls0);
    wait_vmem_all();
    barrier();
    int s = 0;
    for (; s + 1 < nsteps; s += 2) {
      load_step(s + 1, qs1, ls1);
      step(s, qs0, ls0);
      wait_vmem_all();  // step s + 1 has landed (every wave, after the barrier)
      barrier();        // ... and nobody reads buffer 0 any more
      if (s + 2 < nsteps) load_step(s + 2, qs0, ls0);
      step(s + 1, qs1, ls1);
      wait_vmem_all();
      barrier();
    }
    if (s < nsteps) step(s, qs0, ls0);

    // the two half-waves hold the other rows of the same keys
    colsum += __shfl_xor(colsum, 32);
    if (hh == 0 && key < N) part[(size_t)bh * N + key] = colsum;
  };
  if constexpr (CAUSAL) {
    for (int it = 0; it < nit; ++it) run_item(it == 0 ? wb : nkb - 1 - wb);
  } else {
    run_item(wb);
  }
}

// mass[b, j] = sum_h part[b, h, j], heads added in order 0 .. H-1
__global__ __launch_bounds__(256) void key_mass_reduce_kernel(const float* __restrict__ part,
                                                              float* __restrict__ mass, int H,
                                                              int N, long long total) {
  const long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const long long b = t / N;
  const int j = (int)(t - b * N);
  const float* src = part + (size_t)b * H * N + j;
  float acc = 0.f;
  for (int h = 0; h < H; ++h) acc += src[(size_t)h * N];
  mass[t] = acc;
}

template <int D, bool CAUSAL, bool F16>
static hipError_t launch_mass_t(const MassArgs& a) {
  using C = MassCfg<D>;
  const int nkb = (a.N + C::BCB - 1) / C::BCB;
  const long long heads = (long long)a.B * a.H;
  const int pairs = CAUSAL && nkb >= 2 && heads * ((nkb + 1) / 2) >= kMassPairMinWorkgroups ? 1 : 0;
  const long long grid = (pairs ? (nkb + 1) / 2 : nkb) * heads;
  hipError_t e = launch_kernel(key_mass_kernel<D, CAUSAL, F16>, dim3((unsigned)grid), dim3(C::THREADS),
                               a.stream, (const __bf16*)a.Q, (const __bf16*)a.K, a.LSE, a.part, a.N,
                               a.B * a.H, a.H / a.Hkv, a.softmax_scale * kLog2e, pairs);
  if (e != hipSuccess) return e;
  const long long total = (long long)a.B * a.N;
  return launch_kernel(key_mass_reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256),
                       a.stream, (const float*)a.part, a.mass, a.H, a.N, total);
}

template <bool F16>
static hipError_t launch_mass_dt(const MassArgs& a) {
  if (a.d == 128) return a.causal ? launch_mass_t<128, true, F16>(a) : launch_mass_t<128, false, F16>(a);
  return a.causal ? launch_mass_t<64, true, F16>(a) : launch_mass_t<64, false, F16>(a);
}

hipError_t launch_mass(const MassArgs& a) {
  return a.f16 ? launch_mass_dt<true>(a) : launch_mass_dt<false>(a);
}

}  // namespace fa
