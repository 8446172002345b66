// Forward pass of exact tiled attention on gfx950.
//
// The method is the tiled attention with an online softmax of "RTX Flash
// Attention Implementation COMPLETE" (Technical Implementation Details: the
// running max m and running sum l, and the Q-block / KV-block tiling), with the
// causal masking of that page's Advanced Features. What this kernel does on
// MI355X:
//
//  * One workgroup owns BR = 32 * NW query rows of one (batch, head); each of
//    its NW waves owns 32 of them for the whole sweep over the keys. The
//    query tile is staged in LDS (loaded with the first K/V tiles, 1 KB of
//    consecutive bytes per instruction); each wave then keeps its rows in
//    registers, as the B operand of S^T = K Q^T, for the whole sweep.
//  * Both products are computed transposed, S^T = K Q^T and O^T = V^T P^T,
//    on 32x32x16 bf16 matrix cores. In the accumulator layout of S^T every lane
//    then holds 16 scores of a single query row (its partner lane l ^ 32 holds
//    the other 16), so the row max needs one cross-lane swap and the rescale
//    factor of a lane's O^T accumulators is the lane's own. P^T goes from the
//    S^T registers straight into the B operand of the second product (no LDS
//    round trip); the V^T operand comes from the
//    row-major V tile through gfx950's transposing LDS read, rows taken in the
//    key order of the P^T operand.
//  * K/V tiles of BC = 64 keys are staged in LDS, double buffered, and loaded
//    straight from HBM into LDS (buffer loads with the LDS destination), so no
//    registers carry tile data. K rows are padded by 16 bytes; V rows carry an
//    XOR swizzle on 16-byte chunks; both keep the operand reads free of bank
//    conflicts.
//  * The eight waves form two groups that run the same phase sequence one
//    phase apart (a ping-pong): while one wave of a SIMD runs its products,
//    the other runs its softmax. Each phase ends at a workgroup barrier.
//  * Causal: tiles entirely above the diagonal are never loaded; a wave skips
//    the work of tiles fully masked for its own rows; masks are applied only to
//    tiles that cross the diagonal or the end of the sequence. A workgroup
//    runs two query tiles, nq - 1 - w and then w, so that all workgroups do
//    the same number of key tiles (uneven workgroups leave CUs idle while
//    work is still queued).
//  * O leaves through LDS: each wave writes its finished rows into a stage in
//    the idle K/V buffers and stores them as whole rows.
//  * The softmax runs in base 2 in float32: c = scale * log2(e) is folded into
//    one FMA per score; P is rounded to bf16 for the matrix core. The row sum
//    l is a product too: an all-ones A operand against the same P^T operands
//    sums the rounded P per query, so l adds exactly the weights the P V
//    product uses (O is a convex combination of V rows up to float32 sums; with
//    the unrounded P in l, a row dominated by one key would carry that key's
//    rounding error, up to 2^-8 |V|, into O) and costs the vector ALUs
//    nothing. The reference max
//    only moves when the row max outgrows it by 2^15, so the O^T rescale runs on
//    few tiles.
//  * Global reads go through buffer resources whose range check ends at row
//    N: rows past the end of the sequence read as zeros, with no branches
//    around the loads (make_rsrc in fa_common.h gives the rule).

#include <type_traits>

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

template <int D>
struct FwdCfg {
  static constexpr int NW = 8;         // two groups of 4 waves: one wave of each per SIMD
  static constexpr int BR = 32 * NW;   // query rows per workgroup
  static constexpr int BC = 64;        // keys per K/V tile
  static constexpr int CH = D / 8;     // 16-byte chunks per row
  static constexpr int THREADS = 64 * NW;
  static constexpr int KST = D + 8;           // K tile row stride (elements): 16 bytes of padding
  static constexpr int KCH = KST / 8;          // 16-byte chunk positions per K row
  static constexpr int K_INSTR = BC * KCH / 64;  // direct-to-LDS instructions per K tile
  static constexpr int V_INSTR = BC * CH / 64;   // ... per V tile
  static_assert(BC * KCH % 64 == 0 && BC * CH % 64 == 0, "tile loads");
};

// K tiles: row-major with rows padded by 16 bytes. The S^T products read
// operand rows (16 consecutive keys at one chunk), which the padding spreads
// over all banks; every read is one base address plus an immediate.
// V tiles: row-major, 16-byte chunk c of row r at c ^ vswz(r). The transposing
// reads of the V^T operand take 4 consecutive rows x 4 consecutive chunks; the
// swizzle on the row's low bits puts those in distinct banks, and leaves the
// address independent of the key step.
template <int D>
__device__ __forceinline__ int vswz(int r) {
  if constexpr (D == 128) return (r & 3) << 2;
  else return ((r >> 1) & 1) << 2;
}
template <int D>
__device__ __forceinline__ int voff(int r, int col) {  // element offset of (r, col), col % 4 == 0
  return r * D + (((col >> 3) ^ vswz<D>(r)) << 3) + (col & 4);
}

// Each wave alternates two phases per key tile t:
//   M(t): S_{t+1} = K_{t+1} Q^T  and  O^T += V_t P_t^T      (matrix cores)
//   V(t): online softmax of S_{t+1} -> P_{t+1}, rescale O    (vector ALUs)
// (plus S_0 and softmax(S_0) up front). Group B (waves 4..7) runs one phase
// behind group A (waves 0..3); each phase ends at a workgroup barrier, so on
// every SIMD one wave's softmax runs while the other wave's products do.
// QM, the FP8 paths (bf16 only):
//  1: Q quantised to E4M3 per 16 x 16 block (scale rule in fa_common.h) and
//     dequantised in registers as it is loaded; K arrives dequantised.
//  2: the 1 x 32 block reading: Q quantised per row and 32 columns in
//     registers and kept as E4M3 codes; K arrives as codes with E8M0 scale
//     bytes (Ksc: 4 bytes per key, d / 32 of them used); S^T = K Q^T runs on
//     the scaled 32x32x64 FP8 matrix instruction, which applies both block
//     scales, at twice the bf16 rate.
template <int D, bool CAUSAL, bool F16, int QM>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fwd_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                const __bf16* __restrict__ V, __bf16* __restrict__ O,
                float* __restrict__ LSE, int N, int BH, int G, float c_log2,
                const uint8_t* __restrict__ Ksc, int pairs) {
  // BH query heads; query head bh reads K/V head bh / G (G query heads per
  // K/V head: 1 for multi-head attention, H for multi-query attention)
  using C = FwdCfg<D>;
  constexpr int BR = C::BR, BC = C::BC, CH = C::CH;
  // Lazy rescaling: the running max used for P only moves when the true row
  // max exceeds it by more than TAU (base-2 units), so P <= 2^TAU and the
  // O^T rescale is skipped on most tiles. The result is exact either way:
  // O = sum_j 2^(c s_j - m) v_j / sum_j 2^(c s_j - m) for any common m.
  // TAU = 15 keeps P <= 2^15 within binary16 (largest finite 65504) and makes
  // rescales rare even for peaked rows (large logits move the row max often).
  constexpr float TAU = 15.f;
  constexpr int KST = C::KST, KCH = C::KCH;
  constexpr int RING = 2;  // operand reads in flight ahead of their products, per stream
  // Double-buffered tiles as four separate arrays: every access names its
  // buffer statically, so the compiler can tell that the tile loads in flight
  // do not write what the current products read (and waits for none of them).
  __shared__ __attribute__((aligned(16))) __bf16 ks0[BC * KST];  // K tiles, padded rows
  __shared__ __attribute__((aligned(16))) __bf16 ks1[BC * KST];
  __shared__ __attribute__((aligned(16))) __bf16 vs0[BC * D];    // V tiles, swizzled
  __shared__ __attribute__((aligned(16))) __bf16 vs1[BC * D];
  // QM 2: the K tiles' scale words (one per key) beside the code tiles, which
  // use the first BC * (D + 16) bytes of ks0 / ks1
  __shared__ __attribute__((aligned(16))) uint32_t ksc0[QM == 2 ? BC : 1];
  __shared__ __attribute__((aligned(16))) uint32_t ksc1[QM == 2 ? BC : 1];
  // bf16/f16 path: the query tile's rows, loaded straight into LDS with the
  // tile loads; row r's 16-byte chunk c at c ^ (r mod CH)
  __shared__ __attribute__((aligned(16))) __bf16 qst[QM == 0 ? BR * D : 8];

  // With `pairs` (causal only) the workgroup runs query tile nq - 1 - w and
  // then tile w: every pair has the same number of key tiles, so the
  // workgroups are equally long (uneven ones leave CUs idle while work is
  // still queued) and there are half as many.
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
  const int grp = wave >> 2;                        // 0: group A, 1: group B
  // this wave's 32-row block: SIMD s (waves s and s + 4) holds blocks s and
  // 7 - s, so on the tiles that cross the causal diagonal, where the lower
  // blocks run out of keys, every SIMD keeps one wave busy and that wave's
  // phases run without a partner on its SIMD (shorter than shared phases)
  const int rblk = grp == 0 ? (wave & 3) : 7 - (wave & 3);
  const int tr_grp = lane >> 4, tr_i = lane & 15;   // transposing-read addressing
  const int tr_e = tr_i >> 2;
  const int wl = wave & 3;  // wave index within its group
  const int tr_col = 16 * (tr_grp & 1) + 4 * (tr_i & 3);

  const size_t head = (size_t)bh * (size_t)N * D;
  const size_t kvhead = (size_t)(bh / G) * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rQ = make_rsrc(Q + head, head_bytes);
  const __bf16* const Kh = K + kvhead;
  const __bf16* const Vh = V + kvhead;

  // one query tile: its sweep over the key tiles and its epilogue
  auto run_item = [&](const int qt) __attribute__((always_inline)) {
    const int q0 = qt * BR;
    const int wrow0 = q0 + 32 * rblk;  // first query row of this wave
    const int row = wrow0 + l32;       // this lane's query row
    const int nkv_all = (N + BC - 1) / BC;
    const int last_row_wg = min(q0 + BR, N) - 1;
    const int T = CAUSAL ? min(nkv_all, last_row_wg / BC + 1) : nkv_all;  // key tiles
    const bool wave_active = wrow0 < N;
    // last key tile this wave needs (-1: none)
    const int jw_last = !wave_active ? -1 : CAUSAL ? min(wrow0 + 31, N - 1) / BC : T - 1;

    // ---- Q^T operand: lane holds row `row`, d = 16 s + 8 hh .. +7 (0 past N).
    // QM 0 stages the query tile in LDS first (in the prologue below, with the
    // K/V tiles); QM 1 loads it here, as its in-register quantisation needs.
    bf16x8 qf[QM == 2 ? 1 : D / 16];
    if constexpr (QM == 1) {
#pragma unroll
      for (int s = 0; s < D / 16; ++s)
        qf[s] = as_bf16x8(buf_load16(rQ, (uint32_t)row * (D * 2) + (16 * s + 8 * hh) * 2));
    }
    // QM 2: Q^T as E4M3 codes, the B operand of the scaled FP8 product. For the
    // 64-column step st the lane holds columns 64 st + 16 hh .. + 15 (bytes
    // 0..15, block 2 st) and 64 st + 32 + 16 hh .. + 15 (bytes 16..31, block
    // 2 st + 1); each block of the row is split over the lane pair (hh = 0, 1),
    // so its amax takes one swap. The scale word's byte 2 st is the lane's own
    // block exponent for the instruction (block 2 st + hh), plus 127.
    constexpr int NST = D / 64;
    i32x8 qf8[QM == 2 ? NST : 1];
    uint32_t qsw = 0;
    if constexpr (QM == 2) {
      static_assert(!F16, "the FP8 paths take bf16 inputs");
      uint32_t sw = 0;
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const uint32_t off = (uint32_t)row * (D * 2) + (64 * st + 32 * hb + 16 * hh) * 2;
          const u32x4 w0 = buf_load16(rQ, off), w1 = buf_load16(rQ, off + 16);
          float x[16];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            x[2 * m] = lo16<false>(w0[m]);
            x[2 * m + 1] = hi16<false>(w0[m]);
            x[8 + 2 * m] = lo16<false>(w1[m]);
            x[8 + 2 * m + 1] = hi16<false>(w1[m]);
          }
          float amax = 0.f;
#pragma unroll
          for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
          const int e = e4m3_block_exp(pair_max(amax));
#pragma unroll
          for (int j = 0; j < 4; ++j)
            qf8[st][4 * hb + j] = (int)e4m3_codes4(x[4 * j], x[4 * j + 1], x[4 * j + 2], x[4 * j + 3], e);
          sw |= (uint32_t)(127 + e) << (8 * (2 * st + hb));
        }
      qsw = sw >> (8 * hh);
    }
    if constexpr (QM == 1) {
      // A 16 x 16 block of Q is 16 rows (lanes l32 in one half of 0..31; wave
      // rows start at multiples of 32, block rows at multiples of 16) by 16
      // columns (k-step s, both half-waves): its amax takes a 5-step XOR
      // reduction over lane bits 0..3 and 5. Rows past N read as zeros, as in
      // the short last block of the quantisation kernel.
      static_assert(!F16, "the FP8 paths take bf16 inputs");
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        const u32x4 w = as_u32x4(qf[s]);
        float x[8];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          x[2 * m] = lo16<false>(w[m]);
          x[2 * m + 1] = hi16<false>(w[m]);
        }
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(x[i]));
#pragma unroll
        for (int sh = 1; sh < 16; sh <<= 1) amax = fmaxf(amax, __shfl_xor(amax, sh));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const int e = e4m3_block_exp(amax);
        const uint32_t c0 = e4m3_codes4(x[0], x[1], x[2], x[3], e);
        const uint32_t c1 = e4m3_codes4(x[4], x[5], x[6], x[7], e);
        qf[s] = as_bf16x8(u32x4{e4m3_deq2_bf16(c0, 0, e), e4m3_deq2_bf16(c0, 2, e),
                                e4m3_deq2_bf16(c1, 0, e), e4m3_deq2_bf16(c1, 2, e)});
      }
    }

    // ---- K/V tiles, straight from HBM into LDS: instruction n of a tile fills
    // the 64 consecutive 16-byte chunk positions [64 n, 64 n + 64) of the tile's
    // LDS image, each lane fetching the global chunk that the layout puts at its
    // position. The instructions of a tile are dealt round-robin over NL loader
    // waves (w = index among them). Each tile is read through a resource that
    // starts at its first row and ends at row N (rows_rsrc), with per-lane
    // offsets relative to the tile's first row: rows past N read as zeros.
    auto k_src = [&](int n) -> uint32_t {  // padding positions fetch chunk 0 again
      const int i = 64 * n + lane;
      const int kr = i / KCH, pos = i % KCH;
      return (uint32_t)(kr * (D * 2) + (pos < CH ? pos * 16 : 0));
    };
    // V: 64 positions are whole rows (64 / CH of them, a multiple of the swizzle
    // period), so instruction n's offsets are instruction 0's plus 1024 n bytes.
    const uint32_t v_src0 = (uint32_t)((lane / CH) * (D * 2) + (((lane % CH) ^ vswz<D>(lane / CH)) * 16));
    // this wave's K and V offsets as one of the four in-loop loaders (n = wl + 4 m)
    constexpr int KM = (C::K_INSTR + 3) / 4;
    constexpr int VM = (C::V_INSTR + 3) / 4;
    uint32_t k_src_b[KM], v_src_b[VM];
#pragma unroll
    for (int m = 0; m < KM; ++m) k_src_b[m] = k_src(wl + 4 * m);
#pragma unroll
    for (int m = 0; m < VM; ++m) v_src_b[m] = v_src0 + 1024u * (wl + 4 * m);

    // QM 2: K tiles of E4M3 codes, rows padded to D + 16 bytes (the same
    // conflict-free spread as the bf16 rows), and the tile's scale words
    constexpr int KST8 = D + 16, KCH8 = KST8 / 16, K_INSTR8 = BC * KCH8 / 64;
    constexpr int KM8 = (K_INSTR8 + 3) / 4;
    const uint8_t* const K8h = reinterpret_cast<const uint8_t*>(K) + (size_t)(bh / G) * N * D;
    const uint8_t* const Ksch = Ksc + (size_t)(bh / G) * N * 4;
    auto k8_src = [&](int n) -> uint32_t {  // padding positions fetch chunk 0 again
      const int i = 64 * n + lane;
      const int kr = i / KCH8, pos = i % KCH8;
      return (uint32_t)(kr * D + (pos < D / 16 ? pos * 16 : 0));
    };
    uint32_t k8_src_b[QM == 2 ? KM8 : 1];
    if constexpr (QM == 2) {
#pragma unroll
      for (int m = 0; m < KM8; ++m) k8_src_b[m] = k8_src(wl + 4 * m);
    }
    auto load_k = [&](auto NL, int w, int j, __bf16* t, uint32_t* sc) __attribute__((always_inline)) {
      constexpr int nl = decltype(NL)::value;
      if constexpr (QM == 2) {
        const auto r = rows_rsrc(K8h, j * BC, N, D);
#pragma unroll
        for (int m = 0; m * nl < K_INSTR8; ++m) {
          const int n = m * nl + w;
          if (n < K_INSTR8)
            buf_load16_lds(r, nl == 4 ? k8_src_b[m] : k8_src(n),
                           reinterpret_cast<__bf16*>(reinterpret_cast<uint8_t*>(t) + 1024 * n));
        }
        if (w == 0) buf_load4_lds(rows_rsrc(Ksch, j * BC, N, 4), 4u * lane, sc);
      } else {
        const auto r = rows_rsrc(Kh, j * BC, N, D * 2);
#pragma unroll
        for (int m = 0; m * nl < C::K_INSTR; ++m) {
          const int n = m * nl + w;
          if (n < C::K_INSTR) buf_load16_lds(r, nl == 4 ? k_src_b[m] : k_src(n), t + 64 * n * 8);
        }
      }
    };
    auto load_v = [&](auto NL, int w, int j, __bf16* t) __attribute__((always_inline)) {
      constexpr int nl = decltype(NL)::value;
      const auto r = rows_rsrc(Vh, j * BC, N, D * 2);
#pragma unroll
      for (int m = 0; m * nl < C::V_INSTR; ++m) {
        const int n = m * nl + w;
        if (n < C::V_INSTR) buf_load16_lds(r, nl == 4 ? v_src_b[m] : v_src0 + 1024u * n, t + 64 * n * 8);
      }
    };
    using four = std::integral_constant<int, 4>;
    using eight = std::integral_constant<int, 8>;

    // ---- running state ----------------------------------------------------------
    f32x16 o[D / 32];
#pragma unroll
    for (int b = 0; b < D / 32; ++b) o[b] = f32x16{};
    f32x16 sacc[BC / 32];     // S^T of the tile being processed
    u32x4 pf[BC / 16];        // P^T of the previous tile, bf16, as B operands
    float m_run = -INFINITY;  // reference max of c * s for this row (base-2 units)
    // running sum of the row's rounded P, from the matrix cores: every element
    // holds it (the A operand is all ones); only element 0 is rescaled and read
    f32x16 lacc = f32x16{};

    // online softmax of sacc (key tile u) -> pf; rescales o, l
    auto softmax = [&](int u) __attribute__((always_inline)) {
      const int kv0 = u * BC;
      const bool need_mask = (CAUSAL && kv0 + BC - 1 > wrow0) || (kv0 + BC > N);
      if (need_mask) {
        // key kv0 + 32 kb + 8 (r / 4) + 4 hh + r % 4 is masked iff its offset
        // 32 kb + 8 (r / 4) + r % 4 exceeds lim (one compare with a constant)
        const int lim = (CAUSAL ? min(row, N - 1) : N - 1) - kv0 - 4 * hh;
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            sacc[kb][r] = 32 * kb + 8 * (r >> 2) + (r & 3) > lim ? -INFINITY : sacc[kb][r];
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = pair_max(mx) * c_log2;
      if (__builtin_amdgcn_ballot_w64(mx > m_run + TAU) != 0) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = fast_exp2(m_run - m_new);  // 0 on the first tile
        m_run = m_new;
        lacc[0] *= alpha;
#pragma unroll
        for (int b = 0; b < D / 32; ++b) o[b] *= alpha;
      }
      const float neg_m = -m_run;
#pragma unroll
      for (int kb = 0; kb < BC / 32; ++kb)
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(__builtin_fmaf(sacc[kb][8 * t + 2 * e], c_log2, neg_m));
            const float p1 = fast_exp2(__builtin_fmaf(sacc[kb][8 * t + 2 * e + 1], c_log2, neg_m));
            const uint32_t pk = pack2<F16>(p0, p1);
            pf[2 * kb + t][e] = pk;

          }
    };

    // Per-lane element offsets of the transposing V^T reads, one per d block:
    // the swizzle of row 16 tk + 4 hh + tr_e (and of that row + 8) depends only on
    // tr_e, so the key step tk adds a constant. Kept live across the loop (the
    // asm stops the compiler from recomputing them in every product phase).
    int vrow[D / 32];
#pragma unroll
    for (int b = 0; b < D / 32; ++b) {
      vrow[b] = voff<D>(4 * hh + tr_e, 32 * b + tr_col);
      asm volatile("" : "+v"(vrow[b]));
    }

    // M phase: S_u = K_u Q^T into sacc (if DO_S) and O^T += V_t P_t^T with
    // l += 1 P_t^T (if DO_PV), the product streams interleaved. Operands stream through register rings
    // two products deep (fenced so the scheduler keeps that depth instead of
    // hoisting every read, which would not fit the register budget).
    auto mphase = [&](auto DO_S, auto DO_PV, const __bf16* kt, const __bf16* vt, const uint32_t* sct)
        __attribute__((always_inline)) {
      constexpr bool do_s = decltype(DO_S)::value, do_pv = decltype(DO_PV)::value;
      constexpr int NM = (D / 16) * (BC / 32);  // = (BC / 16) * (D / 32): products per stream

      auto kread = [&](int i) {  // K fragment of S product i (k-step i / 2, key block i % 2)
        const int st = i / (BC / 32), kb = i % (BC / 32);
        return ld_lds16(&kt[(32 * kb + l32) * KST + 16 * st + 8 * hh]);
      };
      auto vread = [&](int i) {  // V^T fragment of PV product i (key step i / 4, d block i % 4)
        const int tk = i / (D / 32), b = i % (D / 32);
        const __bf16* p = vt + vrow[b] + 16 * tk * D;  // rows 16 tk + 4 hh + tr_e: slots 8hh + 0..3
        return cat8(ld_lds_tr(p), ld_lds_tr(p + 8 * D));  // rows + 8: slots 8hh + 4..7
      };
      if constexpr (QM == 2) {
        // S^T on the scaled FP8 instruction: product j takes k-step j / 2 (64
        // columns) of key block j % 2, one per four P V products; the K code
        // operands stream through a two-deep ring, the keys' scale words (the
        // instruction's block 2 st + hh in byte 2 st) are read once per tile
        constexpr int NS = 2 * NST, SEV = NM / NS;
        static_assert(NM % NS == 0, "S products interleave evenly");
        const uint8_t* const k8 = reinterpret_cast<const uint8_t*>(kt);
        auto kread8 = [&](int j) {
          const uint8_t* p = k8 + (32 * (j & 1) + l32) * KST8 + 64 * (j >> 1) + 16 * hh;
          const u32x4 a = as_u32x4(ld_lds16(reinterpret_cast<const __bf16*>(p)));
          const u32x4 b = as_u32x4(ld_lds16(reinterpret_cast<const __bf16*>(p + 32)));
          return i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3], (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
        };
        const uint32_t ksw[2] = {sct[l32] >> (8 * hh), sct[32 + l32] >> (8 * hh)};
        i32x8 kr8[2] = {kread8(0), kread8(1)};
        constexpr int R = RING;
        bf16x8 vr[R];
        const uint32_t one2 = 0x3F803F80u;
        const bf16x8 ones = as_bf16x8(u32x4{one2, one2, one2, one2});
        if constexpr (do_pv) {
#pragma unroll
          for (int j = 0; j < R; ++j) vr[j] = vread(j);
        }
        __builtin_amdgcn_s_setprio(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < (do_pv ? NM : NS * SEV); ++i) {
          if (i % SEV == 0) {
            const int j = i / SEV, st = j >> 1, kb = j & 1;
            if (st == 0)
              sacc[kb] = mfma_mx<0, true>(kr8[j & 1], qf8[0], sacc[kb], ksw[kb], qsw);
            else
              sacc[kb] = mfma_mx<2, false>(kr8[j & 1], qf8[NST - 1], sacc[kb], ksw[kb], qsw);
            if (j + 2 < NS) kr8[j & 1] = kread8(j + 2);
          }
          if constexpr (do_pv) {
            const int tk = i / (D / 32), b = i % (D / 32);
            o[b] = mfma32x<F16>(vr[i % R], as_bf16x8(pf[tk]), o[b]);
            if (i + R < NM) vr[i % R] = vread(i + R);
            if (b == D / 32 - 1) lacc = mfma32x<F16>(ones, as_bf16x8(pf[tk]), lacc);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        return;
      }
      constexpr int R = RING;
      bf16x8 kr[R], vr[R];
      const uint32_t one2 = F16 ? 0x3C003C00u : 0x3F803F80u;
      const bf16x8 ones = as_bf16x8(u32x4{one2, one2, one2, one2});
      if constexpr (do_s) {
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb) sacc[kb] = f32x16{};
#pragma unroll
        for (int j = 0; j < R; ++j) kr[j] = kread(j);
      }
      if constexpr (do_pv) {
#pragma unroll
        for (int j = 0; j < R; ++j) vr[j] = vread(j);
      }
      __builtin_amdgcn_s_setprio(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        if constexpr (do_s) {
          const int st = i / (BC / 32), kb = i % (BC / 32);
          sacc[kb] = mfma32x<F16>(kr[i % R], qf[st], sacc[kb]);
          if (i + R < NM) kr[i % R] = kread(i + R);
        }
        if constexpr (do_pv) {
          const int tk = i / (D / 32), b = i % (D / 32);
          o[b] = mfma32x<F16>(vr[i % R], as_bf16x8(pf[tk]), o[b]);
          if (i + R < NM) vr[i % R] = vread(i + R);
          // l += sum over this key step of the rounded P, per query
          if (b == D / 32 - 1) lacc = mfma32x<F16>(ones, as_bf16x8(pf[tk]), lacc);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    using yes = std::true_type;
    using no = std::false_type;

    // Workgroup barrier without a memory fence: the LDS reads of a phase are all
    // consumed by its own products before it ends, and tile loads are waited for
    // explicitly (a fenced barrier would also wait for the loads still meant to
    // be in flight). The asm keeps the compiler from moving memory accesses
    // across it, the scheduling fences keep all other instructions on their side
    // (leftover softmax work moved into a product phase would delay its products).
    auto slot_barrier = [] {
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };

    // ---- schedule ----------------------------------------------------------------
    // Barrier-delimited slots. Group A runs S_0 in slot 0, then softmax(t) in
    // slot 2t+1 and M(t) in slot 2t+2; group B runs the same sequence one slot
    // later (it waits out slot 0, group A waits out the last slot), so in every
    // slot from 1 on one group's products overlap the other's softmax. Both
    // groups run straight-line code: no phase is conditional, which keeps the
    // accumulators in place across the loop.
    // Tiles: K_0, K_1 and V_0 are loaded up front. Group B issues K_{t+2} (into
    // the buffer of K_t) and V_{t+1} (into that of V_{t-1}) at the start of its
    // softmax(t), slot 2t+2, after the last reads of those buffers (slot 2t+1),
    // and waits for them at the end of its M(t), slot 2t+3; their first reader is
    // group A's M(t+1) in slot 2t+4.
    __syncthreads();  // a previous tile's epilogue may still read its O stage in these buffers
    if constexpr (QM == 0) {
      // the query tile into the stage: instruction n = wave + 8 m fills rows
      // RPI n .. RPI n + RPI - 1 (whole rows, 1 KB of consecutive bytes); the
      // rows of m and m + 1 lie 8 RPI (a multiple of CH) apart, so the
      // swizzle and the offsets within them repeat, 8192 bytes further on
      constexpr int RPI = 64 / CH, QI = BR * D * 2 / 1024 / 8;
      const auto r = rows_rsrc(Q + head, q0, N, D * 2);
      const int rl = RPI * wave + lane / CH, sl = lane % CH;
      const uint32_t base = (uint32_t)(rl * (D * 2) + ((sl ^ (rl & (CH - 1))) * 16));
#pragma unroll
      for (int m = 0; m < QI; ++m) buf_load16_lds(r, base + 8192u * m, qst + 64 * (wave + 8 * m) * 8);
    }
    load_k(eight{}, wave, 0, ks0, ksc0);
    if (T > 1) load_k(eight{}, wave, 1, ks1, ksc1);
    load_v(eight{}, wave, 0, vs0);
    wait_vmem_all();
    __syncthreads();
    if constexpr (QM == 0) {
      const __bf16* const qrow = qst + (32 * rblk + l32) * D;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qf[s] = ld_lds16(qrow + 8 * ((2 * s + hh) ^ (l32 & (CH - 1))));
    }
    if (grp == 1) __syncthreads();
    mphase(yes{}, no{}, ks0, vs0, ksc0);  // S_0
    slot_barrier();
    // one tile, t: buffers of parity P = t & 1 (static in each copy)
    auto tile = [&](auto P, int t) __attribute__((always_inline)) {
      constexpr bool odd = decltype(P)::value;
      __bf16* k_this = odd ? ks1 : ks0;  // K_t, refilled with K_{t+2}
      __bf16* k_next = odd ? ks0 : ks1;  // K_{t+1}
      __bf16* v_this = odd ? vs1 : vs0;  // V_t
      __bf16* v_next = odd ? vs0 : vs1;  // V_{t+1}, loaded now
      uint32_t* sc_this = odd ? ksc1 : ksc0;  // scale words of K_t, then K_{t+2}
      uint32_t* sc_next = odd ? ksc0 : ksc1;
      if (grp == 1) {
        if (t + 2 < T) load_k(four{}, wl, t + 2, k_this, sc_this);
        if (t + 1 < T) load_v(four{}, wl, t + 1, v_next);
      }
      softmax(t);
      slot_barrier();
      mphase(yes{}, yes{}, k_next, v_this, sc_next);
      wait_vmem_all();  // (group A has none in flight; waiting on every wave keeps the
      slot_barrier();   //  compiler's view of pending loads exact)
    };
    using even_t = std::false_type;
    using odd_t = std::true_type;
    int t = 0;
    // tiles with unmasked keys for this wave's rows (M(t) of the last one also
    // computes an unused S_{t+1}, from whatever its buffer holds)
    for (; t + 1 <= jw_last; t += 2) {
      tile(even_t{}, t);
      tile(odd_t{}, t + 1);
    }
    if (t <= jw_last) tile(even_t{}, t++);
    // tiles whose keys are all masked for this wave's rows: keep to the schedule
    for (; t < T; ++t) {
      if (grp == 1) {
        if (t & 1) {
          if (t + 2 < T) load_k(four{}, wl, t + 2, ks1, ksc1);
          if (t + 1 < T) load_v(four{}, wl, t + 1, vs0);
        } else {
          if (t + 2 < T) load_k(four{}, wl, t + 2, ks0, ksc0);
          if (t + 1 < T) load_v(four{}, wl, t + 1, vs1);
        }
      }
      slot_barrier();
      wait_vmem_all();
      slot_barrier();
    }
    if (grp == 0) slot_barrier();

    // ---- epilogue: O = O^T / l, LSE = ln 2 * (m + log2 l) ------------------------
    // O goes out through an 8 KB LDS stage per wave in the (now idle) K/V tile
    // buffers; the next tile's loads wait for a barrier first
    if (!wave_active) return;
    const float l_tot = lacc[0];
    __bf16* const stage = (wave < 2 ? ks0 : wave < 4 ? ks1 : wave < 6 ? vs0 : vs1) + (wave & 1) * 32 * D;
    store_rows_via_lds<D, F16>(o, 1.f / l_tot, stage, O + head, wrow0, N);
    if (LSE != nullptr && hh == 0 && row < N)
      LSE[(size_t)bh * N + row] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  };
  if constexpr (CAUSAL) {
    for (int it = 0; it < nit; ++it) run_item(it == 0 ? qt_first : wq);
  } else {
    run_item(qt_first);
  }
}

template <int D, bool CAUSAL, bool F16, int QM>
static hipError_t launch_fwd_t(const FwdArgs& a) {
  using C = FwdCfg<D>;
  const int nq = (a.N + C::BR - 1) / C::BR;
  // causal: pair query tiles while that leaves at least one workgroup per CU
  const long long heads = (long long)a.B * a.H;
  const int pairs = CAUSAL && nq >= 2 && heads * ((nq + 1) / 2) >= kFwdPairMinWorkgroups ? 1 : 0;
  const long long total = (pairs ? (nq + 1) / 2 : nq) * heads;
  return launch_kernel(fwd_kernel<D, CAUSAL, F16, QM>, dim3((unsigned)total), dim3(C::THREADS), a.stream,
                       (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V, (__bf16*)a.O,
                       a.LSE, a.N, a.B * a.H, a.H / a.Hkv, a.softmax_scale * kLog2e, a.k_scales, pairs);
}

template <bool F16, int QM>
static hipError_t launch_fwd_dt(const FwdArgs& a) {
  if (a.d == 128)
    return a.causal ? launch_fwd_t<128, true, F16, QM>(a) : launch_fwd_t<128, false, F16, QM>(a);
  return a.causal ? launch_fwd_t<64, true, F16, QM>(a) : launch_fwd_t<64, false, F16, QM>(a);
}

hipError_t launch_fwd(const FwdArgs& a) {
  if (a.fp8 == 1) return a.f16 ? hipErrorInvalidValue : launch_fwd_dt<false, 1>(a);
  if (a.fp8 == 2) return a.f16 || a.k_scales == nullptr ? hipErrorInvalidValue : launch_fwd_dt<false, 2>(a);
  return a.f16 ? launch_fwd_dt<true, 0>(a) : launch_fwd_dt<false, 0>(a);
}

}  // namespace fa
