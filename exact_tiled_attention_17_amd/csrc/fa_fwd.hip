// Forward pass of exact tiled attention on gfx950.
//
// The method is the tiled attention with an online softmax of "RTX Flash
// Attention Implementation COMPLETE" (Technical Implementation Details: the
// running max m and running sum l, and the Q-block / KV-block tiling), with the
// causal masking of that page's Advanced Features. What this kernel does on
// MI355X:
//
//  * One workgroup owns BR = 32 * NW query rows of one (batch, head); each of
//    its NW waves owns 32 of them for the whole sweep over the keys.
//  * Both products are computed transposed, S^T = K Q^T and O^T = V^T P^T,
//    on 32x32x16 bf16 matrix cores. In the accumulator layout of S^T every lane
//    then holds 16 scores of a single query row (its partner lane l ^ 32 holds
//    the other 16), so the row max needs one cross-lane swap, the row sum none
//    until the end, and the rescale factor of a lane's O^T accumulators is the
//    lane's own. P^T goes from the S^T registers straight into the B operand of
//    the second product (no LDS round trip); the V^T operand comes from the
//    row-major V tile through gfx950's transposing LDS read, rows taken in the
//    key order of the P^T operand.
//  * K/V tiles of BC = 64 keys are staged in LDS, double buffered: the global
//    loads of tile j+1 are issued before tile j is computed and written to LDS
//    after it, one barrier per tile. Both tiles are row-major with an XOR
//    swizzle on 16-byte chunks that keeps operand-row reads and transposing
//    reads free of bank conflicts.
//  * Causal: tiles entirely above the diagonal are never loaded; a wave skips
//    tiles fully masked for its own rows; masks are applied only to tiles that
//    cross the diagonal or the end of the sequence.
//  * The softmax runs in base 2 in float32: c = scale * log2(e) is folded into
//    one FMA per score; P is rounded to bf16 for the matrix core and the row
//    sum l is accumulated from those same rounded values (dot2 with 1s). The
//    reference max only moves when the row max outgrows it by 2^8, so the
//    O^T rescale runs on few tiles.
//  * Global reads go through buffer resources: rows past the end of the
//    sequence read as zeros, with no branches around the loads.
//  * The two waves sharing a SIMD raise their priority in their matrix-core
//    phases, so one wave's softmax overlaps the other's products.

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

template <int D, int NW>
struct FwdCfg {
  static constexpr int BR = 32 * NW;  // query rows per workgroup
  static constexpr int BC = 64;       // keys per K/V tile
  static constexpr int CH = D / 8;    // 16-byte chunks per row
  static constexpr int THREADS = 64 * NW;
  static constexpr int LOADERS = THREADS / 2;  // half the threads load K, half V
  static constexpr int TPT = BC * CH / LOADERS;  // 16-byte chunks per loader thread
  static_assert(TPT >= 1 && BC * CH % LOADERS == 0, "loader split");
};

template <int D, int NW, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW)))
void fwd_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                const __bf16* __restrict__ V, __bf16* __restrict__ O,
                float* __restrict__ LSE, int N, int BH, float c_log2) {
  using C = FwdCfg<D, NW>;
  constexpr int BR = C::BR, BC = C::BC, CH = C::CH;
  // Lazy rescaling: the running max used for P only moves when the true row
  // max exceeds it by more than TAU (base-2 units), so P <= 2^TAU and the
  // O^T rescale is skipped on most tiles. The result is exact either way:
  // O = sum_j 2^(c s_j - m) v_j / sum_j 2^(c s_j - m) for any common m.
  constexpr float TAU = 8.f;
  __shared__ __attribute__((aligned(16))) __bf16 ks[2][BC * D];  // K tiles, row-major
  __shared__ __attribute__((aligned(16))) __bf16 vs[2][BC * D];  // V tiles, row-major

  const int nq = (N + BR - 1) / BR;
  int bh, qt;
  xcd_remap(blockIdx.x, nq * BH, nq, bh, qt);
  if (CAUSAL) qt = nq - 1 - qt;  // longest rows first

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int tr_grp = lane >> 4, tr_i = lane & 15;         // transposing-read addressing
  const int tr_e = tr_i >> 2;
  const int tr_col = 16 * (tr_grp & 1) + 4 * (tr_i & 3);

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rQ = make_rsrc(Q + head, head_bytes);
  const auto rK = make_rsrc(K + head, head_bytes);
  const auto rV = make_rsrc(V + head, head_bytes);

  const int q0 = qt * BR;
  const int wrow0 = q0 + 32 * wave;  // first query row of this wave
  const int row = wrow0 + l32;       // this lane's query row
  const int nkv_all = (N + BC - 1) / BC;
  const int last_row_wg = min(q0 + BR, N) - 1;
  const int nkv = CAUSAL ? min(nkv_all, last_row_wg / BC + 1) : nkv_all;
  const bool wave_active = wrow0 < N;
  const int jw_last = CAUSAL ? min(wrow0 + 31, N - 1) / BC : nkv - 1;

  // ---- Q^T operand: lane holds row `row`, d = 16 s + 8 hh .. +7 (0 past N) --
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s)
    qf[s] = as_bf16x8(buf_load16(rQ, (uint32_t)row * (D * 2) + (16 * s + 8 * hh) * 2));

  // ---- K/V tile staging: waves 0..NW/2-1 load K, the rest V (wave-uniform);
  // both tiles row-major with the chunk swizzle of tile_off ---------------------
  const bool k_loader = wave < NW / 2;
  const int lt = tid % C::LOADERS;
  const auto rT = k_loader ? rK : rV;
  u32x4 stg[C::TPT];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int r = 0; r < C::TPT; ++r) {
      const int i = lt + r * C::LOADERS;
      stg[r] = buf_load16(rT, (uint32_t)(j * BC + i / CH) * (D * 2) + (i % CH) * 16);
    }
  };
  auto store_tile = [&](int buf) {
    __bf16* t = k_loader ? ks[buf] : vs[buf];
#pragma unroll
    for (int r = 0; r < C::TPT; ++r) {
      const int i = lt + r * C::LOADERS;
      st_lds16(&t[tile_off<D>(i / CH, 8 * (i % CH))], stg[r]);
    }
  };

  // ---- running state ----------------------------------------------------------
  f32x16 o[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b) o[b] = f32x16{};
  float m_run = -INFINITY;  // reference max of c * s for this row (base-2 units)
  float l_run = 0.f;        // this lane's share of the running sum
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

  load_tile(0);
  store_tile(0);
  wait_vmem_all();
  __syncthreads();

  for (int j = 0; j < nkv; ++j) {
    const int buf = j & 1;
    if (j + 1 < nkv) load_tile(j + 1);

    if (wave_active && j <= jw_last) {
      // S^T = K_j Q^T : two 32-key blocks, interleaved accumulation chains
      // K fragments stream through a register ring PF k-steps deep, so each
      // product's LDS read was issued several products earlier.
      constexpr int PF = D / 16 < 4 ? D / 16 : 4;
      __builtin_amdgcn_s_setprio(1);
      f32x16 s[BC / 32];
      bf16x8 kr[PF][BC / 32];
#pragma unroll
      for (int st = 0; st < PF; ++st)
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
          kr[st][kb] = ld_lds16(&ks[buf][tile_off<D>(32 * kb + l32, 16 * st + 8 * hh)]);
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb) s[kb] = f32x16{};
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch reads ahead of their use
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb) {
          s[kb] = mfma32(kr[st % PF][kb], qf[st], s[kb]);
          if (st + PF < D / 16)
            kr[st % PF][kb] = ld_lds16(&ks[buf][tile_off<D>(32 * kb + l32, 16 * (st + PF) + 8 * hh)]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
      // masks: causal (key > row) and sequence end (key >= N), only where needed
      const int kv0 = j * BC;
      const bool need_mask = (CAUSAL && kv0 + BC - 1 > wrow0) || (kv0 + BC > N);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (key >= N || (CAUSAL && key > row)) s[kb][r] = -INFINITY;
          }
      }
      // online softmax (base 2) with lazy rescaling
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = pair_max(mx) * c_log2;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);  // 0 on the first tile
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int b = 0; b < D / 32; ++b) o[b] *= alpha;
      }
      const float neg_m = -m_run;

      u32x4 pf[BC / 16];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(__builtin_fmaf(s[kb][8 * t + 2 * e], c_log2, neg_m));
            const float p1 = fast_exp2(__builtin_fmaf(s[kb][8 * t + 2 * e + 1], c_log2, neg_m));
            const uint32_t pk = pack_bf16(p0, p1);
            pf[2 * kb + t][e] = pk;
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pk), ones, lsum, false);
          }
      l_run += lsum;

      // O^T += V^T P^T; V^T by transposing reads, keys in the P^T slot order
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < BC / 16; ++t) {
        const int r_lo = 16 * t + 4 * hh + tr_e;  // slots 8hh + 0..3
        const int r_hi = r_lo + 8;                // slots 8hh + 4..7
#pragma unroll
        for (int b = 0; b < D / 32; ++b) {
          const int col = 32 * b + tr_col;
          const bf16x8 a = cat8(ld_lds_tr(&vs[buf][tile_off<D>(r_lo, col)]),
                                ld_lds_tr(&vs[buf][tile_off<D>(r_hi, col)]));
          o[b] = mfma32(a, as_bf16x8(pf[t]), o[b]);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    }

    if (j + 1 < nkv) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, LSE = ln 2 * (m + log2 l) ------------------------
  if (!wave_active) return;
  const float l_tot = pair_sum(l_run);
  if (row >= N) return;
  const float inv = 1.f / l_tot;
  __bf16* Orow = O + head + (size_t)row * D;
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u32x2 w;
      w[0] = pack_bf16(o[b][4 * g] * inv, o[b][4 * g + 1] * inv);
      w[1] = pack_bf16(o[b][4 * g + 2] * inv, o[b][4 * g + 3] * inv);
      st_global8(Orow + 32 * b + 8 * g + 4 * hh, w);
    }
  if (LSE != nullptr && hh == 0)
    LSE[(size_t)bh * N + row] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
}

template <int D, int NW, bool CAUSAL>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  using C = FwdCfg<D, NW>;
  const int nq = (a.N + C::BR - 1) / C::BR;
  const long long total = (long long)nq * a.B * a.H;
  return launch_kernel(fwd_kernel<D, NW, CAUSAL>, dim3((unsigned)total), dim3(C::THREADS), a.stream,
                       (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V, (__bf16*)a.O,
                       a.LSE, a.N, a.B * a.H, a.softmax_scale * kLog2e);
}

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.d == 128) return a.causal ? launch_fwd_t<128, 8, true>(a) : launch_fwd_t<128, 8, false>(a);
  return a.causal ? launch_fwd_t<64, 4, true>(a) : launch_fwd_t<64, 4, false>(a);
}

}  // namespace fa
