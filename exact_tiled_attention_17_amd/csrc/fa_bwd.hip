// Backward pass of exact tiled attention on gfx950.
//
// The probabilities are recomputed from the stored log-sum-exp rather than
// kept ("GPU Performance Optimization Batch 1 - Design Spec", Item 3, Design,
// backward file). Two launches on one stream (three with the dK/dV split):
//
//  1. bwd_dq_kernel: one workgroup per (batch, head, query tile), sweeping key
//     tiles like the forward (and with its two-group schedule): S and dP are
//     recomputed and dQ += dS K is summed in registers, so dQ needs no atomics
//     and no float32 scratch. It first forms its rows' statistics, D_i =
//     dO_i . O_i (float32) and the LSE in base 2, and stores them (the LSE in
//     base 2 and -D) as two planes for the next pass.
//  2. bwd_dkdv_kernel: one workgroup per (batch, head, block of 128 keys); each
//     32-key block has a P-wave (dV) and a dS-wave (dK) on one SIMD, holding
//     float32 accumulators for the whole sweep over query tiles of 64 rows,
//     pipelined one query step apart. The Q, dO tiles sit row-major in LDS;
//     operands that need them transposed use gfx950's transposing LDS read
//     instead of a second, transposed copy. Per query tile, on 32x32x16 bf16
//     matrix cores:
//        S = Q K^T, dP - D = dO V^T - D (lane = one key, 16 queries; the
//                                       accumulator starts at -D)
//        P = exp2(c S - LSE2), dS = P (dP - D)
//        dV += P^T dO, dK += dS^T Q    (P^T, dS^T straight from registers)
//     Causal: query tiles that see none of the block's keys are skipped, and
//     a workgroup takes key blocks kb and nkb - 1 - kb in turn (equal work per
//     workgroup), its step pipeline running from one block into the other.
//     The dQ pass likewise pairs query tiles nq - 1 - w and w.
//  (3. bwd_reduce_kernel, only when the dK/dV work of few K/V heads is split
//     over several workgroups: sums their float32 partials.)
//
// The pages' backward gathers dQ with atomic updates ("RTX Flash Attention
// Implementation COMPLETE", CUDA Kernel Design, backward kernel); on MI355X the
// float32 atomics cost more than recomputing S and dP in a second pass, so
// this backward recomputes instead.
//
// Global reads go through buffer resources whose range check ends at row N,
// so rows past the end of the sequence read as zeros without branches (the
// rule is at make_rsrc in fa_common.h).

#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// ---------------------------------------------------------------------------
// dK/dV kernel
// ---------------------------------------------------------------------------
template <int D>
struct BwdCfg {
  static constexpr int KBLK = 4;            // 32-key blocks per workgroup
  static constexpr int NW = 2 * KBLK;       // a P-wave and a dS-wave per key block
  static constexpr int THREADS = 64 * NW;
  static constexpr int BCB = 32 * KBLK;     // keys per workgroup
  static constexpr int QB = 2;              // 32-query blocks per step
  static constexpr int BRB = 32 * QB;       // queries per step
  static constexpr int CH = D / 8;          // 16-byte chunks per row
  static constexpr int TI = BRB * CH / 64;  // direct-to-LDS instructions per Q or dO tile
  static_assert(BRB * CH % 64 == 0, "tile loads");
};

// Each 32-key block of the workgroup is served by two waves on one SIMD:
//   P-wave:  S = Q K^T, P = exp2(c S - LSE2), dV += P^T dO;
//   dS-wave: dP = dO V^T, dS = P (dP - D) with P from its partner through
//            LDS (as bf16, the precision the products use), dK += dS^T Q.
// Splitting the dK and dV accumulators keeps each wave under 256 registers.
// The two are pipelined one query step apart, one barrier per slot: in slot s
//   P-wave:  dV += P_{s-1}^T dO_{s-1}; S_s; P_s (vector ALUs) -> LDS
//   dS-wave: dS_{s-1} (vector ALUs); dK += dS_{s-1}^T Q_{s-1}; dP_s
// so on each SIMD the products of one wave overlap the vector work of the
// other. Q, dO tiles and row statistics of three steps are resident (s - 1,
// s, and s + 1 being loaded straight from HBM into LDS).
// With G query heads per K/V head the workgroup owns a key block of one K/V
// head and its steps run over the query tiles of each of GS query heads of
// the group in turn, so dK and dV are summed over them inside the
// accumulators. When GS < G (few K/V heads: too few workgroups otherwise),
// the G / GS workgroups of a key block write float32 partial sums to `part`
// and bwd_reduce_kernel adds them up; with GS == G (part == nullptr) the
// workgroup writes dK, dV directly.
template <int D, bool CAUSAL, bool F16, bool PAIRS>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                     const float* __restrict__ rowstat, __bf16* __restrict__ dK,
                     __bf16* __restrict__ dV, int N, int BH, int G, int GS, float c_log2,
                     float scale, float* __restrict__ part, int ppw) {
  // BH query heads, BH / G K/V heads; K/V head j serves query heads G j .. G j + G - 1
  using C = BwdCfg<D>;
  constexpr int BCB = C::BCB, BRB = C::BRB, QB = C::QB, CH = C::CH, TI = C::TI;
  // three buffers of each kind, as separate arrays so that every access
  // names its buffer statically; Q and dO tiles row-major, chunk c of row r at
  // c ^ swz(r) (operand-row and transposing reads both conflict-free)
  __shared__ __attribute__((aligned(16))) __bf16 qs0[BRB * D];
  __shared__ __attribute__((aligned(16))) __bf16 qs1[BRB * D];
  __shared__ __attribute__((aligned(16))) __bf16 qs2[BRB * D];
  __shared__ __attribute__((aligned(16))) __bf16 os0[BRB * D];
  __shared__ __attribute__((aligned(16))) __bf16 os1[BRB * D];
  __shared__ __attribute__((aligned(16))) __bf16 os2[BRB * D];
  __shared__ __attribute__((aligned(16))) u32x4 ps0[C::KBLK][2 * QB][64];  // P^T operands, lane-major
  __shared__ __attribute__((aligned(16))) u32x4 ps1[C::KBLK][2 * QB][64];
  __shared__ __attribute__((aligned(16))) u32x4 ps2[C::KBLK][2 * QB][64];
  __shared__ __attribute__((aligned(16))) float rs0[2 * BRB];  // LSE2 of the step's queries, then -D
  __shared__ __attribute__((aligned(16))) float rs1[2 * BRB];
  __shared__ __attribute__((aligned(16))) float rs2[2 * BRB];

  const int nkb = (N + BCB - 1) / BCB;
  const int BKV = BH / G;  // K/V heads
  const int S = G / GS;    // workgroups per key block
  // With PAIRS, key block p is paired with block nkb - 1 - p (the middle
  // block of an odd count stands alone), workgroup w owns the ppw pairs
  // starting at pair w * ppw, and its step pipeline runs through their
  // blocks in turn (p, nkb - 1 - p, p + 1, ...). Under the causal mask every
  // pair has the same number of steps, and the workgroup's fixed costs
  // (prologue, pipeline fill and drain) are paid once for all its blocks.
  const int npb = (nkb + 1) / 2;                           // pairs per (K/V head, split)
  const int nwb = PAIRS ? (npb + ppw - 1) / ppw : nkb;      // workgroups per (K/V head, split)
  int hs, wb;
  xcd_remap(blockIdx.x, nwb * BKV * S, nwb, hs, wb);  // causal: low key blocks (most work) first
  const int p0 = wb * ppw;                        // first pair (PAIRS)
  const int npw = PAIRS ? min(ppw, npb - p0) : 1;  // pairs of this workgroup (PAIRS)
  // items (key blocks) of this workgroup
  const int nit = PAIRS ? 2 * npw - ((nkb & 1) && p0 + npw == npb ? 1 : 0) : 1;
  const int bkv = hs / S;
  const int split = hs - bkv * S;
  const int qh0 = bkv * G + split * GS;  // first query head this workgroup serves

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const bool pwave = wave < C::KBLK;           // role (wave-uniform)
  const int kblk = pwave ? wave : wave - C::KBLK;
  const int tr_i = lane & 15;
  const int tr_e = tr_i >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (tr_i & 3);

  const size_t kvhead = (size_t)bkv * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rK = make_rsrc(K + kvhead, head_bytes);
  const auto rV = make_rsrc(V + kvhead, head_bytes);

  // first key of item it's block, and of this wave's 32 keys in it
  auto blk_k0 = [&](int it) {
    if constexpr (!PAIRS) return wb * BCB;
    const int p = p0 + (it >> 1);
    return ((it & 1) ? nkb - 1 - p : p) * BCB;
  };
  auto wave_k0 = [&](int it) { return blk_k0(it) + 32 * kblk; };

  // K rows (P-wave) or V rows (dS-wave) of this lane's key as B operands (0 past N)
  bf16x8 frag[D / 16];
  const auto rF = pwave ? rK : rV;
  auto load_frag = [&](int it) __attribute__((always_inline)) {
    const int key = wave_k0(it) + l32;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      frag[s] = as_bf16x8(buf_load16(rF, (uint32_t)key * (D * 2) + (16 * s + 8 * hh) * 2));
  };
  load_frag(0);

  // ---- step loads, straight from HBM into LDS: the Q and dO tiles of 64
  // queries (instruction n fills chunk positions [64 n, 64 n + 64), dealt
  // round-robin over the 8 waves) and the 64 row statistics (wave 0) -------
  auto src = [&](int n) -> uint32_t {
    const int p = 64 * n + lane;
    const int r = p / CH, pc = p % CH;
    return (uint32_t)(r * (D * 2) + ((pc ^ swz<D>(r)) * 16));
  };
  constexpr int LM = (TI + 7) / 8;
  uint32_t src_w[LM];
#pragma unroll
  for (int m = 0; m < LM; ++m) src_w[m] = src(wave + 8 * m);
  const int nqt = (N + BRB - 1) / BRB;
  // first query tile that sees item it's keys, and its steps per query head
  auto first_tile = [&](int it) { return CAUSAL ? blk_k0(it) / BRB : 0; };
  auto nsteps = [&](int it) { return nqt - first_tile(it); };
  // A step is (it, g, t): item it, query head qh0 + g, query tile
  // first_tile(it) + t. Steps run over t = 0 .. nsteps(it) - 1 for
  // g = 0 .. GS - 1, for it = 0 .. nit - 1; the padding steps after the last
  // keep it = nit - 1, g = GS - 1 with t >= nsteps(it), so that all their
  // queries are past N.
  struct Step {
    int it, g, t;
  };
  auto advance = [&](Step p) __attribute__((always_inline)) {
    ++p.t;
    if (p.t == nsteps(p.it)) {
      if (p.g + 1 < GS) {
        p.t = 0;
        ++p.g;
      } else if (p.it + 1 < nit) {
        p.t = 0;
        p.g = 0;
        ++p.it;
      }
    }
    return p;
  };
  // Each step's tiles are read through resources that start at its first
  // query and end at query N, so the rows of a ragged last step and every row
  // of a padding step (all past N) read as zeros and touch no memory.
  auto load_step = [&](Step p, __bf16* qd, __bf16* od, float* rsd) __attribute__((always_inline)) {
    const size_t qh = (size_t)(qh0 + p.g);  // query head
    const size_t head = qh * (size_t)N * D;
    const int q0 = (first_tile(p.it) + p.t) * BRB;
    const auto rQ = rows_rsrc(Q + head, q0, N, D * 2);
    const auto rdO = rows_rsrc(dO + head, q0, N, D * 2);
    // row statistics: LSE in base 2 for all rows, then -D = -dO . O for all rows
    const auto rL2 = rows_rsrc(rowstat + qh * N, q0, N, 4);
    const auto rDD = rows_rsrc(rowstat + (size_t)BH * N + qh * N, q0, N, 4);
#pragma unroll
    for (int m = 0; m < LM; ++m) {
      const int n = wave + 8 * m;
      if (n < TI) {
        buf_load16_lds(rQ, src_w[m], qd + 64 * n * 8);
        buf_load16_lds(rdO, src_w[m], od + 64 * n * 8);
      }
    }
    if (wave == 0) {
      buf_load4_lds(rL2, 4u * lane, rsd);
      buf_load4_lds(rDD, 4u * lane, rsd + BRB);
    }
  };

  // ---- LDS read offsets (elements): operand rows (row 32 qb + l32, chunk
  // 2 st + hh) at rw ^ 16 st (+ 32 qb D); transposing reads (rows
  // 32 qb + 16 t + 4 hh + tr_e and that + 8, column 32 b + tr_col) at
  // tw ^ 32 b (+ (32 qb + 16 t) D) -------------------------------------------
  int rw = tile_off<D>(l32, 8 * hh);
  int tw0 = tile_off<D>(4 * hh + tr_e, tr_col);
  int tw1 = tile_off<D>(4 * hh + tr_e + 8, tr_col);
  asm volatile("" : "+v"(rw), "+v"(tw0), "+v"(tw1));

  f32x16 acc_kd[D / 32];  // dV (P-wave) or dK (dS-wave): M = keys, N = d
#pragma unroll
  for (int b = 0; b < D / 32; ++b) acc_kd[b] = f32x16{};
  f32x16 sd[QB];      // S (P-wave) or dP (dS-wave) of a step: lane = one key, 16 queries
  u32x4 opnd[QB][2];  // P^T (P-wave) or dS^T (dS-wave) as A operands, 2 k-steps each

  // sd = (Q or dO tile rows) x frag^T, one product per 32-query block,
  // accumulated onto zeros (S) or onto -D of each query (dP - D: `negd`, the
  // step's -D plane in LDS), so that dS needs no subtraction. In both products
  // the operand reads run R products ahead of their use, fenced so that the
  // scheduler keeps that depth.
  constexpr int R = 2;
  auto first_product = [&](const __bf16* tile, const float* negd) __attribute__((always_inline)) {
    constexpr int NP = (D / 16) * QB;  // product i: k-step i / QB, query block i % QB
    auto rd = [&](int i) { return ld_lds16(tile + (rw ^ (16 * (i / QB))) + 32 * (i % QB) * D); };
    if (negd == nullptr) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) sd[qb] = f32x16{};
    } else {
      // registers 4 g .. 4 g + 3 of block qb hold queries 32 qb + 8 g + 4 hh + 0..3
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(&negd[32 * qb + 8 * g + 4 * hh]);
#pragma unroll
          for (int e = 0; e < 4; ++e) sd[qb][4 * g + e] = v[e];
        }
    }
    bf16x8 ar[R];
#pragma unroll
    for (int j = 0; j < R; ++j) ar[j] = rd(j);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      sd[i % QB] = mfma32x<F16>(ar[i % R], frag[i / QB], sd[i % QB]);
      if (i + R < NP) ar[i % R] = rd(i + R);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // acc_kd += opnd^T (dO or Q tile): M = keys, N = d, k = queries; the B
  // operand is read transposed, rows in the A operand's slot order
  auto second_product = [&](const __bf16* tile) __attribute__((always_inline)) {
    constexpr int NB = D / 32;
    constexpr int NP = QB * 2 * NB;  // product i: k-step i / NB (= 2 qb + t), d block i % NB
    auto rd = [&](int i) {
      const __bf16* base = tile + 16 * (i / NB) * D;
      const int b = i % NB;
      return cat8(ld_lds_tr(base + (tw0 ^ (32 * b))), ld_lds_tr(base + (tw1 ^ (32 * b))));
    };
    bf16x8 br[R];
#pragma unroll
    for (int j = 0; j < R; ++j) br[j] = rd(j);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int ks = i / NB;
      acc_kd[i % NB] = mfma32x<F16>(as_bf16x8(opnd[ks >> 1][ks & 1]), br[i % R], acc_kd[i % NB]);
      if (i + R < NP) br[i % R] = rd(i + R);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // query q0 + m (m = 32 qb + 8 g + 4 hh + e) contributes to this lane's key
  // iff (unsigned)(m + mbase) < mbound: the query exists and, if causal, is at
  // or after the key; a key past the end contributes nothing
  auto mask_bounds = [&](int q0, int key, int& mbase, unsigned& mbound) __attribute__((always_inline)) {
    const int qlo = CAUSAL ? key : 0;
    mbase = q0 - qlo;
    mbound = key < N ? (unsigned)(N - qlo) : 0u;
  };
  // P-wave: P = exp2(c S - LSE2) -> opnd (bf16) and to LDS for the partner
  auto p_phase = [&](Step p, const float* rsb, u32x4 (*psb)[2 * QB][64]) __attribute__((always_inline)) {
    const int q0 = (first_tile(p.it) + p.t) * BRB;
    const int kw0 = wave_k0(p.it);
    const bool need_mask = (CAUSAL && q0 < kw0 + 31) || (kw0 + 32 > N) || (q0 + BRB > N);
    int mbase;
    unsigned mbound;
    mask_bounds(q0, kw0 + l32, mbase, mbound);
    f32x4 l4[QB][4];  // LSE2 of queries 32 qb + 8 g + 4 hh + 0..3, all read up front
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) l4[qb][g] = *reinterpret_cast<const f32x4*>(&rsb[32 * qb + 8 * g + 4 * hh]);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int m0 = 32 * qb + 8 * g + 4 * hh;
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = fast_exp2(__builtin_fmaf(sd[qb][4 * g + e], c_log2, -l4[qb][g][e]));
        if (need_mask) {  // selects under one wave-uniform branch
#pragma unroll
          for (int e = 0; e < 4; ++e) p[e] = (unsigned)(m0 + e + mbase) >= mbound ? 0.f : p[e];
        }
        // registers 4g..4g+3 are elements 4(g%2)..+3 of k-step g/2
        opnd[qb][g >> 1][2 * (g & 1)] = pack2<F16>(p[0], p[1]);
        opnd[qb][g >> 1][2 * (g & 1) + 1] = pack2<F16>(p[2], p[3]);
      }
#pragma unroll
    for (int j = 0; j < 2 * QB; ++j) psb[kblk][j][lane] = opnd[j >> 1][j & 1];
  };
  // dS-wave: dS = P (dP - D) -> opnd (bf16); sd already holds dP - D
  auto ds_phase = [&](const u32x4 (*psb)[2 * QB][64]) __attribute__((always_inline)) {
    u32x4 pp[2 * QB];
#pragma unroll
    for (int j = 0; j < 2 * QB; ++j) pp[j] = psb[kblk][j][lane];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t w0 = pp[2 * qb + (g >> 1)][2 * (g & 1)];
        const uint32_t w1 = pp[2 * qb + (g >> 1)][2 * (g & 1) + 1];
        const float p[4] = {lo16<F16>(w0), hi16<F16>(w0), lo16<F16>(w1), hi16<F16>(w1)};
        float ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ds[e] = p[e] * sd[qb][4 * g + e];
        opnd[qb][g >> 1][2 * (g & 1)] = pack2<F16>(ds[0], ds[1]);
        opnd[qb][g >> 1][2 * (g & 1) + 1] = pack2<F16>(ds[2], ds[3]);
      }
  };

  auto slot_barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- schedule ------------------------------------------------------------------
  // Slot 0 has only step 0's first half, the last slot only the last step's
  // second half. The middle slots run in groups of three (buffer index
  // s mod 3, static in each copy); their count is padded to a multiple of 3
  // with steps past the end of the sequence, whose queries are all masked.
  // `cur` is step s, `nxt` step s + 1 (the one being loaded).
  int total = 0;
  for (int it = 0; it < nit; ++it) total += GS * nsteps(it);
  const int last = 3 * ((total + 1) / 3) + 1;  // >= total, == 1 (mod 3)
  __bf16* const qbuf[3] = {qs0, qs1, qs2};
  __bf16* const obuf[3] = {os0, os1, os2};
  u32x4 (*const pbuf[3])[2 * QB][64] = {ps0, ps1, ps2};
  float* const rbuf[3] = {rs0, rs1, rs2};

  // dV = dV_acc (P-waves) or dK = scale * dK_acc (dS-waves) of item it's keys
  const float osc = pwave ? 1.f : scale;
  auto flush = [&](int it) __attribute__((always_inline)) {
    // Rows kw0 .. kw0 + 31 through a resource that starts at row kw0 and ends
    // at row N: rows past N are dropped by the range check. Lane (l32, hh)
    // writes column 32 b + l32 of rows 8 g + 4 hh + e (g = r / 4, e = r % 4):
    // one offset register per g, the rest in the immediate.
    const int kw0 = wave_k0(it);
    if (part != nullptr) {
      // float32 partial sums, [dV, dK][split][K/V head][N][D]
      float* pout = part + ((size_t)(pwave ? 0 : S) + split) * BKV * (size_t)N * D + kvhead;
      const auto rP = rows_rsrc(pout, kw0, N, D * 4);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t vo = (uint32_t)(((8 * g + 4 * hh) * D + l32) * 4);
        asm volatile("" : "+v"(vo));  // formed here, not kept live across the loop
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int b = 0; b < D / 32; ++b)
            buf_store4(rP, vo + (uint32_t)((e * D + 32 * b) * 4),
                       __builtin_bit_cast(uint32_t, acc_kd[b][4 * g + e] * osc));
      }
    } else {
      const auto rO = rows_rsrc((pwave ? dV : dK) + kvhead, kw0, N, D * 2);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint32_t vo = (uint32_t)(((8 * g + 4 * hh) * D + l32) * 2);
        asm volatile("" : "+v"(vo));  // formed here, not kept live across the loop
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int b = 0; b < D / 32; ++b)
            buf_store2(rO, vo + (uint32_t)((e * D + 32 * b) * 2), to16<F16>(acc_kd[b][4 * g + e] * osc));
      }
    }
  };

  // ROLE: P-wave (true) or dS-wave; each role runs its own straight-line copy
  // of the schedule (same barriers), so neither carries the other's registers.
  // `cur`, `nxt` are steps s and s + 1, `prv_it` the item of step s - 1. In
  // the slot where the first item's last step is s - 1 and the second item's
  // first step is `cur`,
  // the wave loads the second block's K or V rows at the start (their last
  // reader, the first product of step s - 1, ran in the previous slot), and
  // writes and clears its accumulators at the end (the second product of step
  // s - 1 completed them).
  auto slot = [&](auto ROLE, auto B3, auto HAS_PREV, auto HAS_CUR, int s, int& prv_it, Step& cur,
                  Step& nxt) __attribute__((always_inline)) {
    constexpr bool p_role = decltype(ROLE)::value;
    constexpr int b = decltype(B3)::value, bp = (b + 2) % 3, bn = (b + 1) % 3;
    constexpr bool has_prev = decltype(HAS_PREV)::value, has_cur = decltype(HAS_CUR)::value;
    bool item_switch = false;
    if constexpr (PAIRS && has_prev && has_cur) {
      item_switch = prv_it != cur.it;
      if (item_switch) load_frag(cur.it);
    }
    if constexpr (has_cur)
      if (s + 1 < last) load_step(nxt, qbuf[bn], obuf[bn], rbuf[bn]);
    if constexpr (p_role) {
      if constexpr (has_prev) second_product(obuf[bp]);  // dV += P_{s-1}^T dO_{s-1}
    } else {
      if constexpr (has_prev) {
        ds_phase(pbuf[bp]);                               // dS_{s-1}
        second_product(qbuf[bp]);                         // dK += dS_{s-1}^T Q_{s-1}
      }
    }
    if constexpr (has_cur) {
      if constexpr (p_role) {
        first_product(qbuf[b], nullptr);                  // S_s
        p_phase(cur, rbuf[b], pbuf[b]);                   // P_s
      } else {
        first_product(obuf[b], rbuf[b] + BRB);            // dP_s - D
      }
    }
    wait_vmem_all();  // the loads of step s + 1 have landed
    // The finished item's stores go out after that wait, so that they
    // complete during the next slot instead of holding up this one.
    if constexpr (PAIRS && has_prev && has_cur) {
      if (item_switch) {
        flush(prv_it);
#pragma unroll
        for (int bb = 0; bb < D / 32; ++bb) acc_kd[bb] = f32x16{};
      }
    }
    slot_barrier();
    prv_it = cur.it;
    cur = nxt;
    nxt = advance(nxt);
  };
  using c0 = std::integral_constant<int, 0>;
  using c1 = std::integral_constant<int, 1>;
  using c2 = std::integral_constant<int, 2>;
  using yes = std::true_type;
  using no = std::false_type;
  auto run = [&](auto ROLE) __attribute__((always_inline)) {
    int prv_it = 0;
    Step cur{0, 0, 0};
    Step nxt = advance(cur);
    slot(ROLE, c0{}, no{}, yes{}, 0, prv_it, cur, nxt);
    for (int s = 1; s < last; s += 3) {
      slot(ROLE, c1{}, yes{}, yes{}, s, prv_it, cur, nxt);
      slot(ROLE, c2{}, yes{}, yes{}, s + 1, prv_it, cur, nxt);
      slot(ROLE, c0{}, yes{}, yes{}, s + 2, prv_it, cur, nxt);
    }
    slot(ROLE, c1{}, yes{}, no{}, last, prv_it, cur, nxt);
  };

  load_step(Step{0, 0, 0}, qs0, os0, rs0);
  wait_vmem_all();
  __syncthreads();
  if (pwave)
    run(yes{});
  else
    run(no{});

  // ---- epilogue: the last item's dV (P-waves) or dK (dS-waves) ---------------
  flush(nit - 1);
}

// dV and dK from the float32 partial sums of S workgroups: `part` is
// [dV, dK][S][n] with n = K/V heads * N * D; each thread sums 4 consecutive
// elements of one plane and stores them rounded to the 16-bit type.
template <bool F16>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ part, int S,
                                                         long long n, __bf16* __restrict__ dV,
                                                         __bf16* __restrict__ dK) {
  const long long gt = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long quads = n / 4;
  if (gt >= 2 * quads) return;
  const int plane = gt >= quads ? 1 : 0;
  const long long i = 4 * (gt - plane * quads);
  const float* src = part + (size_t)plane * S * n + i;
  f32x4 acc = *reinterpret_cast<const f32x4*>(src);
  for (int s = 1; s < S; ++s) acc += *reinterpret_cast<const f32x4*>(src + (size_t)s * n);
  u32x2 w;
  w[0] = pack2<F16>(acc[0], acc[1]);
  w[1] = pack2<F16>(acc[2], acc[3]);
  st_global8((plane ? dK : dV) + i, w);
}

// ---------------------------------------------------------------------------
// dQ kernel
// ---------------------------------------------------------------------------
// One workgroup per (batch, head, tile of 256 queries); each of its 8 waves
// owns 32 query rows and sweeps the key tiles like the forward kernel, with
// the products transposed so that a lane owns one query:
//   S^T = K_j Q^T, dP^T = V_j dO^T     (lane = one query, 16 keys per block)
//   P^T = exp2(c S^T - LSE2), dS^T = P^T (dP^T - D)   (LSE2, D: the lane's own)
//   dQ^T += K_j^T dS^T                 (dS^T straight from registers; K_j^T
//                                       by transposing reads of the K tile)
// and writes dQ = scale * dQ^T as bf16. No atomics: each dQ row is summed
// over all keys inside one wave. Before the sweep each lane forms its row's
// statistics (D = dO . O from the dO^T operand it holds and the O row, and
// the LSE in base 2), which it uses itself and stores for the dK/dV pass: this
// pass runs first, and no separate statistics pass reads O and dO again.
// The schedule is the forward's two-group ping-pong: a wave alternates
//   M(t): dQ^T += K_t^T dS^T_t, then S^T_{t+1}, dP^T_{t+1}   (matrix cores)
//   V(t): dS^T_t from S^T_t, dP^T_t                          (vector ALUs)
// with the second group one phase behind, so on every SIMD one wave's dS
// overlaps the other's products. K_t is read in M(t) as well as (for S_t) in
// M(t-1), so K tiles are kept in four buffers, V tiles in two; all are loaded
// straight from HBM into LDS.
template <int D>
struct DqCfg {
  static constexpr int NW = 8;          // two groups of 4 waves
  static constexpr int BR = 32 * NW;    // query rows per workgroup
  static constexpr int BC = 64;         // keys per K/V tile
  static constexpr int CH = D / 8;      // 16-byte chunks per row
  static constexpr int THREADS = 64 * NW;
  static constexpr int TI = BC * CH / 64;  // direct-to-LDS instructions per tile
  static_assert(BC * CH % 64 == 0, "tile loads");
};

template <int D, bool CAUSAL, bool F16>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                   const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                   const __bf16* __restrict__ O, const float* __restrict__ LSE,
                   float* __restrict__ rowstat, __bf16* __restrict__ dQ, int N, int BH,
                   int G, float c_log2, float scale, int pairs) {
  // BH query heads; query head bh reads K/V head bh / G
  using C = DqCfg<D>;
  constexpr int BR = C::BR, BC = C::BC, CH = C::CH, TI = C::TI;
  // K tiles in four buffers, V tiles in two; separate arrays so that every
  // access names its buffer statically. Row-major, 16-byte chunk c of row r at
  // c ^ swz(r): conflict-free for operand-row reads and transposing reads.
  __shared__ __attribute__((aligned(16))) __bf16 ks0[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 ks1[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 ks2[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 ks3[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 vs0[BC * D];
  __shared__ __attribute__((aligned(16))) __bf16 vs1[BC * D];

  // With `pairs` (causal only) the workgroup runs query tile nq - 1 - w and
  // then tile w, as the forward does: equally long workgroups, half as many.
  const int nq = (N + BR - 1) / BR;
  const int nwq = pairs ? (nq + 1) / 2 : nq;
  int bh, wq;
  xcd_remap(blockIdx.x, nwq * BH, nwq, bh, wq);
  const int qt_first = CAUSAL ? nq - 1 - wq : wq;  // longest rows first
  const int nit = pairs && wq != nq - 1 - wq ? 2 : 1;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int grp = wave >> 2;              // 0: group A, 1: group B
  const int wl = wave & 3;                // wave index within its group
  const int rblk = 2 * wl + grp;          // this wave's 32-row block
  const int tr_i = lane & 15;
  const int tr_e = tr_i >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (tr_i & 3);

  const size_t head = (size_t)bh * (size_t)N * D;
  const size_t kvhead = (size_t)(bh / G) * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rQ = make_rsrc(Q + head, head_bytes);
  const __bf16* const Kh = K + kvhead;
  const __bf16* const Vh = V + kvhead;
  const auto rdO = make_rsrc(dO + head, head_bytes);
  const auto rO = make_rsrc(O + head, head_bytes);
  const auto rL = make_rsrc(LSE + (size_t)bh * N, (uint32_t)N * 4u);

  // one query tile: its row statistics, its sweep over the key tiles, its dQ
  auto run_item = [&](const int qt) __attribute__((always_inline)) {
    const int q0 = qt * BR;
    const int wrow0 = q0 + 32 * rblk;
    const int row = wrow0 + l32;
    const int nkv_all = (N + BC - 1) / BC;
    const int last_row_wg = min(q0 + BR, N) - 1;
    const int T = CAUSAL ? min(nkv_all, last_row_wg / BC + 1) : nkv_all;  // key tiles
    const bool wave_active = wrow0 < N;
    // last key tile this wave needs (-1: none)
    const int jw_last = !wave_active ? -1 : CAUSAL ? min(wrow0 + 31, N - 1) / BC : T - 1;

    // Q^T and dO^T operands (rows past N read as zeros), and the row statistics:
    // the LSE in base 2, and D = dO . O (the lane's half of the row, then its
    // partner's). This pass runs first and stores both for the dK/dV pass.
    bf16x8 qf[D / 16], of[D / 16];
    float dacc = 0.f;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const uint32_t off = (uint32_t)row * (D * 2) + (16 * s + 8 * hh) * 2;
      qf[s] = as_bf16x8(buf_load16(rQ, off));
      of[s] = as_bf16x8(buf_load16(rdO, off));
      const u32x4 ow = buf_load16(rO, off), dw = as_u32x4(of[s]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        dacc += lo16<F16>(ow[m]) * lo16<F16>(dw[m]);
        dacc += hi16<F16>(ow[m]) * hi16<F16>(dw[m]);
      }
    }
    const float dval = pair_sum(dacc);
    f32x16 negd16;
#pragma unroll
    for (int r = 0; r < 16; ++r) negd16[r] = -dval;
    const float l2 =
        __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rL, (uint32_t)row * 4u, 0, 0)) * kLog2e;
    const float neg_l2 = -l2;
    if (hh == 0 && row < N) {
      rowstat[(size_t)bh * N + row] = l2;                     // LSE in base 2
      rowstat[(size_t)BH * N + (size_t)bh * N + row] = -dval; // -D
    }

    // ---- tile loads, straight from HBM into LDS: instruction n of a tile fills
    // chunk positions [64 n, 64 n + 64); each lane fetches the chunk the layout
    // puts at its position. K and V tiles share the layout, hence the offsets.
    auto src = [&](int n) -> uint32_t {
      const int p = 64 * n + lane;
      const int r = p / CH, pc = p % CH;
      return (uint32_t)(r * (D * 2) + ((pc ^ swz<D>(r)) * 16));
    };
    // This wave's offsets as one of the four in-loop loaders: instructions
    // wl + 4 m lie 256 chunks (4096 bytes, 256 / CH rows, a whole number of
    // swizzle periods) apart. The first is formed at each tile load from a
    // fresh lane index (v_mbcnt), so that no register is held for them
    // across the tile loop (the compiler spilled them, and reloaded and
    // waited for them at every tile).
    static_assert((256 / CH) % 16 == 0, "in-loop loader offsets step by whole swizzle periods");
    // tile j of K or V (src = the head's first row), through a resource that
    // starts at the tile's first key and ends at key N
    auto load_tile = [&](auto NL, const __bf16* src_head, int w, int j, __bf16* t)
        __attribute__((always_inline)) {
      constexpr int nl = decltype(NL)::value;
      const auto r = rows_rsrc(src_head, j * BC, N, D * 2);
      uint32_t o0 = 0;
      if constexpr (nl == 4) {
        uint32_t ln;  // the lane index, formed here (volatile: not merged with the kernel's own)
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        const uint32_t p = 64u * (uint32_t)w + ln;
        const int rr = (int)(p / CH), pc = (int)(p % CH);
        o0 = (uint32_t)(rr * (D * 2) + ((pc ^ swz<D>(rr)) * 16));
        asm volatile("" : "+v"(o0));
      }
#pragma unroll
      for (int m = 0; m * nl < TI; ++m) {
        const int n = m * nl + w;
        if (n < TI) buf_load16_lds(r, nl == 4 ? o0 + 4096u * m : src(n), t + 64 * n * 8);
      }
    };
    using four = std::integral_constant<int, 4>;
    using eight = std::integral_constant<int, 8>;

    // ---- LDS read offsets (elements) -----------------------------------------------
    // With the swizzle, the operand-row read of k-step st (row 32 kb + l32, chunk
    // 2 st + hh) sits at rw ^ 16 st (+ 32 kb D), and the transposing read of d
    // block b (rows 16 t + 4 hh + tr_e, and + 8; column 32 b + tr_col) at
    // tw ^ 32 b (+ 16 t D): one register each, one XOR per read.
    int rw = tile_off<D>(l32, 8 * hh);
    int tw0 = tile_off<D>(4 * hh + tr_e, tr_col);
    int tw1 = tile_off<D>(4 * hh + tr_e + 8, tr_col);
    asm volatile("" : "+v"(rw), "+v"(tw0), "+v"(tw1));

    // ---- running state -----------------------------------------------------------
    f32x16 acc[D / 32];  // dQ^T: M = d, N = this wave's 32 queries
#pragma unroll
    for (int b = 0; b < D / 32; ++b) acc[b] = f32x16{};
    f32x16 s[BC / 32], dp[BC / 32];  // S^T, dP^T of the tile in flight
    u32x4 dsf[BC / 16];              // dS^T as B operands, 4 k-steps of 16 keys

    // V(u): dS^T of key tile u from s, dp (= dP^T - D)
    auto vphase = [&](int u) __attribute__((always_inline)) {
      const int kv0 = u * BC;
      const bool need_mask = (CAUSAL && kv0 + BC - 1 > wrow0) || (kv0 + BC > N);
      if (need_mask) {
        // Key kv0 + 32 kb + 8 (r / 4) + 4 hh + r % 4 is masked iff its offset
        // 32 kb + 8 (r / 4) + r % 4 exceeds lim (one compare with a constant).
        // A masked score becomes -inf, so P = 0 and dS = P (dP - D) = 0 exactly
        // (dP is finite: past the sequence end K and V read as zeros). One
        // branch around the whole tile: per-element branches would be flattened
        // into selects that every tile pays for.
        const int lim = (CAUSAL ? min(row, N - 1) : N - 1) - kv0 - 4 * hh;
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[kb][r] = 32 * kb + 8 * (r >> 2) + (r & 3) > lim ? -INFINITY : s[kb][r];
      }
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          float d2[2];
#pragma unroll
          for (int u2 = 0; u2 < 2; ++u2) {
            const float p = fast_exp2(__builtin_fmaf(s[kb][r + u2], c_log2, neg_l2));
            d2[u2] = p * dp[kb][r + u2];
          }
          dsf[2 * kb + (r >> 3)][(r & 7) >> 1] = pack2<F16>(d2[0], d2[1]);
        }
    };

    // M phase: dQ^T += K_t^T dS^T_t (if DO_DQ), then S^T, dP^T of the next tile
    // from K_n, V_n. Operand reads run two products ahead of their use, fenced
    // so that the scheduler keeps that depth.
    auto mphase = [&](auto DO_DQ, const __bf16* kt, const __bf16* kn, const __bf16* vn)
        __attribute__((always_inline)) {
      constexpr bool do_dq = decltype(DO_DQ)::value;
      constexpr int R = 2;
      __builtin_amdgcn_s_setprio(1);
      if constexpr (do_dq) {
        constexpr int NP = (BC / 16) * (D / 32);
        auto tread = [&](int i) {  // K^T fragment of product i: key step i / (D/32), d block i % (D/32)
          const int t = i / (D / 32), b = i % (D / 32);
          return cat8(ld_lds_tr(kt + (tw0 ^ (32 * b)) + 16 * t * D),
                      ld_lds_tr(kt + (tw1 ^ (32 * b)) + 16 * t * D));
        };
        bf16x8 ar[R];
#pragma unroll
        for (int j = 0; j < R; ++j) ar[j] = tread(j);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int t = i / (D / 32), b = i % (D / 32);
          acc[b] = mfma32x<F16>(ar[i % R], as_bf16x8(dsf[t]), acc[b]);
          if (i + R < NP) ar[i % R] = tread(i + R);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      {
        constexpr int NP = (D / 16) * (BC / 32);
        auto kread = [&](int i) {
          const int st = i / (BC / 32), kb = i % (BC / 32);
          return ld_lds16(kn + (rw ^ (16 * st)) + 32 * kb * D);
        };
        auto vread = [&](int i) {
          const int st = i / (BC / 32), kb = i % (BC / 32);
          return ld_lds16(vn + (rw ^ (16 * st)) + 32 * kb * D);
        };
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb) {
          s[kb] = f32x16{};
          dp[kb] = negd16;  // dP^T - D: every element of a lane is its query's
        }
        bf16x8 kr[R], vr[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
          kr[j] = kread(j);
          vr[j] = vread(j);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          const int st = i / (BC / 32), kb = i % (BC / 32);
          s[kb] = mfma32x<F16>(kr[i % R], qf[st], s[kb]);
          if (i + R < NP) kr[i % R] = kread(i + R);
          dp[kb] = mfma32x<F16>(vr[i % R], of[st], dp[kb]);
          if (i + R < NP) vr[i % R] = vread(i + R);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
    };
    using yes = std::true_type;
    using no = std::false_type;

    // Workgroup barrier without a memory fence (tile loads are waited for
    // explicitly; the LDS reads of a phase are consumed by its own products);
    // the fences keep every instruction on its side.
    auto slot_barrier = [] {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };

    // ---- schedule (as in the forward kernel) ---------------------------------------
    // Group A: S_0/dP_0 in slot 0, V(t) in slot 2t+1, M(t) in slot 2t+2; group B
    // one slot later. K_0, K_1, V_0, V_1 are loaded up front; group B issues
    // K_{t+2} (into the buffer of K_{t-2}, last read in slot 2t-1) and V_{t+2}
    // (into that of V_t, last read in slot 2t+1) at the start of its V(t), slot
    // 2t+2, and waits for them at the end of its M(t), slot 2t+3; the first
    // reader is group A's M(t+1) in slot 2t+4.
    // Every wave runs T4 = T rounded up to 4 tiles (the barriers must match):
    // the full work, in groups of 4, up to its last needed tile rounded up to 4
    // (the extra tiles are fully masked, so they add nothing), then only the
    // loads and barriers. All T4 tiles are loaded, so no product ever reads a
    // buffer that was never filled: a tile past the sequence end gets an empty
    // resource (rows_rsrc) and fills its buffer with zeros without reading memory.
    const int T4 = (T + 3) & ~3;
    const int jw4 = (jw_last + 4) & ~3;
    __syncthreads();  // a previous tile's epilogue may still read its dQ stage in these buffers
    load_tile(eight{}, Kh, wave, 0, ks0);
    load_tile(eight{}, Vh, wave, 0, vs0);
    load_tile(eight{}, Kh, wave, 1, ks1);
    load_tile(eight{}, Vh, wave, 1, vs1);
    wait_vmem_all();
    __syncthreads();
    if (grp == 1) __syncthreads();
    mphase(no{}, ks0, ks0, vs0);  // S_0, dP_0
    slot_barrier();
    // one tile t; P = t & 3 (static in each copy) names the buffers
    auto tile = [&](auto P, int t) __attribute__((always_inline)) {
      constexpr int p = decltype(P)::value;
      __bf16* const kbuf[4] = {ks0, ks1, ks2, ks3};
      __bf16* const vbuf[2] = {vs0, vs1};
      if (grp == 1 && t + 2 < T4) {
        load_tile(four{}, Kh, wl, t + 2, kbuf[(p + 2) & 3]);
        load_tile(four{}, Vh, wl, t + 2, vbuf[p & 1]);
      }
      vphase(t);
      slot_barrier();
      mphase(yes{}, kbuf[p], kbuf[(p + 1) & 3], vbuf[(p + 1) & 1]);
      wait_vmem_all();  // (group A has none in flight)
      slot_barrier();
    };
    using c0 = std::integral_constant<int, 0>;
    using c1 = std::integral_constant<int, 1>;
    using c2 = std::integral_constant<int, 2>;
    using c3 = std::integral_constant<int, 3>;
    int t = 0;
    for (; t < jw4; t += 4) {
      tile(c0{}, t);
      tile(c1{}, t + 1);
      tile(c2{}, t + 2);
      tile(c3{}, t + 3);
    }
    for (; t < T4; ++t) {
      if (grp == 1 && t + 2 < T4) {
        __bf16* kf = ((t + 2) & 3) == 0 ? ks0 : ((t + 2) & 3) == 1 ? ks1 : ((t + 2) & 3) == 2 ? ks2 : ks3;
        load_tile(four{}, Kh, wl, t + 2, kf);
        load_tile(four{}, Vh, wl, t + 2, (t & 1) ? vs1 : vs0);
      }
      slot_barrier();
      wait_vmem_all();
      slot_barrier();
    }
    if (grp == 0) slot_barrier();

    // ---- epilogue: dQ = scale * dQ^T, bf16, through an 8 KB LDS stage per wave
    // in the (now idle) K tile buffers; the next tile's loads wait for a barrier
    if (!wave_active) return;
    __bf16* const stage = (wave < 2 ? ks0 : wave < 4 ? ks1 : wave < 6 ? ks2 : ks3) + (wave & 1) * 32 * D;
    store_rows_via_lds<D, F16>(acc, scale, stage, dQ + head, wrow0, N);
  };
  if constexpr (CAUSAL) {
    for (int it = 0; it < nit; ++it) run_item(it == 0 ? qt_first : wq);
  } else {
    run_item(qt_first);
  }
}

template <int D, bool CAUSAL, bool F16>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  using C = BwdCfg<D>;
  using Cq = DqCfg<D>;
  float* rowstat = a.rowstat;
  const float c_log2 = a.softmax_scale * kLog2e;
  {
    // dQ pass first: it also writes the row statistics the dK/dV pass reads
    const int nq = (a.N + Cq::BR - 1) / Cq::BR;
    const long long heads = (long long)a.B * a.H;
    const int pairs = CAUSAL && nq >= 2 && heads * ((nq + 1) / 2) >= kFwdPairMinWorkgroups ? 1 : 0;
    const long long total = (pairs ? (nq + 1) / 2 : nq) * heads;
    const hipError_t e = launch_kernel(
        bwd_dq_kernel<D, CAUSAL, F16>, dim3((unsigned)total), dim3(Cq::THREADS), a.stream,
        (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V, (const __bf16*)a.dO,
        (const __bf16*)a.O, a.LSE, rowstat, (__bf16*)a.dQ, a.N, a.B * a.H, a.H / a.Hkv, c_log2,
        a.softmax_scale, pairs);
    if (e != hipSuccess) return e;
  }
  {
    const int nkb = (a.N + C::BCB - 1) / C::BCB;
    const int G = a.H / a.Hkv;
    const int S = a.no_split ? 1 : dkdv_splits(a.B, a.H, a.Hkv, a.N, a.d);
    float* part = S > 1 ? a.rowstat + rowstat_floats(a.B, a.H, a.N) : nullptr;
    const long long blocks = (long long)nkb * a.B * a.Hkv * S;
    // two key blocks per workgroup when that still leaves >= 1024 workgroups
    const int ppw = dkdv_pairs_per_workgroup(blocks, nkb);
    const bool pairs = ppw > 0;
    const long long total =
        pairs ? (long long)(((nkb + 1) / 2 + ppw - 1) / ppw) * a.B * a.Hkv * S : blocks;
    const hipError_t e = launch_kernel(
        pairs ? bwd_dkdv_kernel<D, CAUSAL, F16, true> : bwd_dkdv_kernel<D, CAUSAL, F16, false>,
        dim3((unsigned)total), dim3(C::THREADS), a.stream,
        (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V, (const __bf16*)a.dO,
        (const float*)rowstat, (__bf16*)a.dK, (__bf16*)a.dV, a.N, a.B * a.H, G, G / S,
        c_log2, a.softmax_scale, part, pairs ? ppw : 1);
    if (e != hipSuccess) return e;
    if (S > 1) {
      const long long n = (long long)a.B * a.Hkv * a.N * D;
      const long long threads = 2 * (n / 4);
      const hipError_t r = launch_kernel(bwd_reduce_kernel<F16>, dim3((unsigned)((threads + 255) / 256)),
                                         dim3(256), a.stream, (const float*)part, S, n,
                                         (__bf16*)a.dV, (__bf16*)a.dK);
      if (r != hipSuccess) return r;
    }
  }
  return hipSuccess;
}

template <bool F16>
static hipError_t launch_bwd_dt(const BwdArgs& a) {
  if (a.d == 128) return a.causal ? launch_bwd_t<128, true, F16>(a) : launch_bwd_t<128, false, F16>(a);
  return a.causal ? launch_bwd_t<64, true, F16>(a) : launch_bwd_t<64, false, F16>(a);
}

hipError_t launch_bwd(const BwdArgs& a) {
  return a.f16 ? launch_bwd_dt<true>(a) : launch_bwd_dt<false>(a);
}

}  // namespace fa
