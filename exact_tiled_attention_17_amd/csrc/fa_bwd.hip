// Backward pass of exact tiled attention on gfx950.
//
// The probabilities are recomputed from the stored log-sum-exp rather than
// kept ("GPU Performance Optimization Batch 1 - Design Spec", Item 3, Design,
// backward file), and dQ is gathered with atomic updates ("RTX Flash Attention
// Implementation COMPLETE", CUDA Kernel Design, backward kernel: gradient
// recomputation and atomic memory operations). Three launches on one stream:
//
//  1. bwd_pre_kernel: per query row, D_i = dO_i . O_i (float32) and the LSE in
//     base 2; zeroes the float32 dQ accumulator.
//  2. bwd_kernel: one workgroup per (batch, head, block of 128 keys); each of
//     its 4 waves keeps 32 keys' K and V rows in registers and their dK, dV
//     accumulators in float32 for the whole sweep over query tiles of BRB rows.
//     Per query tile, on 32x32x16 bf16 matrix cores:
//        S = Q K^T, dP = dO V^T        (lane = one key, 16 queries per block)
//        P = exp2(c S - LSE2), dS = P (dP - D)
//        dV += P^T dO, dK += dS^T Q    (P^T, dS^T straight from registers)
//        dQ += dS K                    (dS through LDS, float32 atomics)
//     Causal: query tiles that see none of the block's keys are skipped.
//  3. bwd_dq_kernel: dQ = bf16(scale * dQ_acc).
//
// Global reads and the dQ atomics go through buffer resources, so rows past
// the end of the sequence read as zeros / are dropped without branches.

#include "fa_common.h"
#include "fa_launch.h"

namespace fa {

// ---------------------------------------------------------------------------
// 1. Row statistics and dQ accumulator reset
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const __bf16* __restrict__ O,
                                                     const __bf16* __restrict__ dO,
                                                     const float* __restrict__ LSE,
                                                     float* __restrict__ dq_acc,
                                                     f32x2* __restrict__ rowstat, long long rows) {
  constexpr int CH = D / 8;  // lanes per row
  const long long gt = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long row = gt / CH;
  const int c = (int)(gt % CH);
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = ld_global16(O + row * D + 8 * c);
    const u32x4 b = ld_global16(dO + row * D + 8 * c);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc += __uint_as_float(a[m] << 16) * __uint_as_float(b[m] << 16);
      acc += __uint_as_float(a[m] & 0xFFFF0000u) * __uint_as_float(b[m] & 0xFFFF0000u);
    }
    f32x4* z = reinterpret_cast<f32x4*>(dq_acc + row * D + 8 * c);
    z[0] = f32x4{};
    z[1] = f32x4{};
  }
#pragma unroll
  for (int off = CH / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, CH);
  if (row < rows && c == 0) rowstat[row] = f32x2{LSE[row] * kLog2e, acc};
}

// ---------------------------------------------------------------------------
// 2. Main backward kernel
// ---------------------------------------------------------------------------
template <int D, int BRB_>
struct BwdCfg {
  static constexpr int NW = 4;
  static constexpr int BCB = 32 * NW;  // keys per workgroup
  static constexpr int BRB = BRB_;     // queries per step
  static constexpr int QB = BRB / 32;  // 32-query blocks per step
  static constexpr int CH = D / 8;
  static constexpr int KTS = BCB + 8;  // padded row length of K^T in LDS
  static constexpr int QTS = BRB + 8;  // padded row length of Q^T, dO^T in LDS
  static constexpr int DSS = BCB + 8;  // padded row length of dS in LDS
  static constexpr int NDB = D / 32;   // 32-wide column blocks of d
  static constexpr int KSPLIT = NW / NDB;       // waves sharing one dQ column block
  static constexpr int DQ_KEYS = BCB / KSPLIT;  // keys each wave sums for dQ
  // Query-tile loading: per tensor (Q, dO), (BRB/4) row groups x CH chunks;
  // half of the loader waves take Q, the other half dO.
  static constexpr int TG = (BRB / 4) * CH;                 // groups per tensor
  static constexpr int LWT = TG >= 64 * (NW / 2) ? NW / 2 : (TG + 63) / 64;  // waves per tensor
  static constexpr int GPT = TG / (64 * LWT);               // groups per loader thread
  static_assert(GPT >= 1 && GPT * 64 * LWT == TG, "tile loaders");
};

template <int D, int BRB_, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(1, 1)))
void bwd_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                const f32x2* __restrict__ rowstat, float* __restrict__ dq_acc,
                __bf16* __restrict__ dK, __bf16* __restrict__ dV, int N, int BH,
                float c_log2, float scale) {
  using C = BwdCfg<D, BRB_>;
  constexpr int BCB = C::BCB, BRB = C::BRB, QB = C::QB, CH = C::CH;
  constexpr int KTS = C::KTS, QTS = C::QTS, DSS = C::DSS;
  __shared__ __attribute__((aligned(16))) __bf16 kt[D * KTS];
  // Query tiles are single-buffered: the next tile is written after the
  // mid-step barrier, when every wave has finished reading the current one.
  __shared__ __attribute__((aligned(16))) __bf16 qs[BRB * D];
  __shared__ __attribute__((aligned(16))) __bf16 dos[BRB * D];
  __shared__ __attribute__((aligned(16))) __bf16 qtr[D * QTS];
  __shared__ __attribute__((aligned(16))) __bf16 dotr[D * QTS];
  __shared__ __attribute__((aligned(16))) __bf16 dss[BRB * DSS];
  __shared__ __attribute__((aligned(16))) f32x2 rs[BRB];

  const int nkb = (N + BCB - 1) / BCB;
  int bh, kb;
  xcd_remap(blockIdx.x, nkb * BH, nkb, bh, kb);  // causal: low key blocks (most work) first

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const size_t head = (size_t)bh * (size_t)N * D;
  const uint32_t head_bytes = (uint32_t)N * D * 2u;
  const auto rQ = make_rsrc(Q + head, head_bytes);
  const auto rK = make_rsrc(K + head, head_bytes);
  const auto rV = make_rsrc(V + head, head_bytes);
  const auto rdO = make_rsrc(dO + head, head_bytes);
  const auto rdQ = make_rsrc(dq_acc + head, head_bytes * 2u);
  const auto rRS = make_rsrc(rowstat + (size_t)bh * N, (uint32_t)N * 8u);

  const int k0 = kb * BCB;
  const int kw0 = k0 + 32 * wave;  // this wave's first key
  const int key = kw0 + l32;       // this lane's key (column of S)

  // K and V rows of this lane's key as B operands: d = 16 s + 8 hh .. +7 (0 past N)
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const uint32_t off = (uint32_t)key * (D * 2) + (16 * s + 8 * hh) * 2;
    kf[s] = as_bf16x8(buf_load16(rK, off));
    vf[s] = as_bf16x8(buf_load16(rV, off));
  }
  // K^T of the whole block in LDS (natural key order), for dQ = dS K
  for (int g = tid; g < (BCB / 4) * CH; g += 256) {
    const int kg = g / CH, dc = g % CH;
    u32x4 r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = buf_load16(rK, (uint32_t)(k0 + 4 * kg + i) * (D * 2) + dc * 16);
    u32x2 col[8];
    transpose4x8(r[0], r[1], r[2], r[3], col);
#pragma unroll
    for (int e = 0; e < 8; ++e) st_lds8(&kt[(8 * dc + e) * KTS + 4 * kg], col[e]);
  }

  // Query-tile loaders (wave-uniform roles)
  const bool tile_loader = wave < 2 * C::LWT;
  const bool loads_q = wave < C::LWT;
  const int tbase = (wave % C::LWT) * 64 + lane;
  const auto rT = loads_q ? rQ : rdO;
  u32x4 stg[4 * C::GPT];
  f32x2 rstg = {INFINITY, 0.f};
  const bool rs_loader = wave == C::NW - 1 && lane < BRB;

  auto load_q = [&](int i) {
    const int q0 = i * BRB;
    if (tile_loader) {
#pragma unroll
      for (int gi = 0; gi < C::GPT; ++gi) {
        const int g = tbase + gi * 64 * C::LWT;
        const int qg = g / CH, dc = g % CH;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          stg[4 * gi + r] = buf_load16(rT, (uint32_t)(q0 + 4 * qg + r) * (D * 2) + dc * 16);
      }
    }
    if (wave == C::NW - 1) {
      // one row per lane; rows past the end get LSE2 = +inf, D = 0, so P = dS = 0
      const int q = q0 + lane;
      const u32x2 v = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(rRS, (uint32_t)q * 8u, 0, 0));
      rstg = q < N ? __builtin_bit_cast(f32x2, v) : f32x2{INFINITY, 0.f};
    }
  };
  auto store_q = [&]() {
    if (tile_loader) {
      __bf16* rm = loads_q ? qs : dos;
      __bf16* tr = loads_q ? qtr : dotr;
#pragma unroll
      for (int gi = 0; gi < C::GPT; ++gi) {
        const int g = tbase + gi * 64 * C::LWT;
        const int qg = g / CH, dc = g % CH;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int q = 4 * qg + r;
          st_lds16(&rm[q * D + ((dc ^ (q & (CH - 1))) * 8)], stg[4 * gi + r]);
        }
        u32x2 col[8];
        transpose4x8(stg[4 * gi], stg[4 * gi + 1], stg[4 * gi + 2], stg[4 * gi + 3], col);
        const int pos = kperm(4 * qg);
#pragma unroll
        for (int e = 0; e < 8; ++e) st_lds8(&tr[(8 * dc + e) * QTS + pos], col[e]);
      }
    }
    if (rs_loader) rs[lane] = rstg;
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int b = 0; b < D / 32; ++b) {
    dk[b] = f32x16{};
    dv[b] = f32x16{};
  }

  const int nqt = (N + BRB - 1) / BRB;
  const int i0 = CAUSAL ? k0 / BRB : 0;
  const int nsteps = nqt - i0;
  // dQ work split of this wave: column block and key range
  const int db = wave % C::NDB;
  const int dq_k0 = (wave / C::NDB) * C::DQ_KEYS;

  load_q(i0);
  store_q();
  wait_vmem_all();
  __syncthreads();

  for (int it = 0; it < nsteps; ++it) {
    const int i = i0 + it;
    const int q0 = i * BRB;
    if (it + 1 < nsteps) load_q(i + 1);

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qb0 = q0 + 32 * qb;  // first query of this 32-query block
      const bool idle = (CAUSAL && qb0 + 31 < kw0) || kw0 >= N;
      if (idle) {
        // every score of this wave's keys is masked here: dS = 0 for its columns
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
          dss[m * DSS + 32 * wave + l32] = (__bf16)0.f;
        }
        continue;
      }
      f32x16 s = f32x16{}, dp = f32x16{};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const int c = 2 * st + hh;
        const int qr = 32 * qb + l32;
        const bf16x8 aq = ld_lds16(&qs[qr * D + ((c ^ (qr & (CH - 1))) * 8)]);
        s = mfma32(aq, kf[st], s);
        const bf16x8 ao = ld_lds16(&dos[qr * D + ((c ^ (qr & (CH - 1))) * 8)]);
        dp = mfma32(ao, vf[st], dp);
      }
      __builtin_amdgcn_s_setprio(0);
      const bool need_mask = (CAUSAL && qb0 < kw0 + 31) || (kw0 + 32 > N);
      u32x4 pt[2], dst[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // queries 8g + 4hh + 0..3 of this block: two (LSE2, D) pairs per 16 bytes
        const int m0 = 32 * qb + 8 * g + 4 * hh;
        const f32x4 st01 = *reinterpret_cast<const f32x4*>(&rs[m0]);
        const f32x4 st23 = *reinterpret_cast<const f32x4*>(&rs[m0 + 2]);
        const float l2v[4] = {st01[0], st01[2], st23[0], st23[2]};
        const float dvv[4] = {st01[1], st01[3], st23[1], st23[3]};
        float p[4], ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          float pv = fast_exp2(__builtin_fmaf(s[r], c_log2, -l2v[e]));
          if (need_mask) {
            const int q = qb0 + 8 * g + 4 * hh + e;
            if (key >= N || (CAUSAL && key > q)) pv = 0.f;
          }
          p[e] = pv;
          ds[e] = pv * (dp[r] - dvv[e]);
        }
        // registers 4g..4g+3 are elements 4(g%2)..+3 of k-step g/2
        pt[g >> 1][2 * (g & 1)] = pack_bf16(p[0], p[1]);
        pt[g >> 1][2 * (g & 1) + 1] = pack_bf16(p[2], p[3]);
        const uint32_t d01 = pack_bf16(ds[0], ds[1]);
        const uint32_t d23 = pack_bf16(ds[2], ds[3]);
        dst[g >> 1][2 * (g & 1)] = d01;
        dst[g >> 1][2 * (g & 1) + 1] = d23;
        __bf16* col = &dss[m0 * DSS + 32 * wave + l32];
        col[0] = __builtin_bit_cast(bf16x2, d01)[0];
        col[DSS] = __builtin_bit_cast(bf16x2, d01)[1];
        col[2 * DSS] = __builtin_bit_cast(bf16x2, d23)[0];
        col[3 * DSS] = __builtin_bit_cast(bf16x2, d23)[1];
      }
      // dV += P^T dO, dK += dS^T Q   (M = keys, N = d, k = queries of this block)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int b = 0; b < D / 32; ++b) {
          const int qoff = 32 * qb + 16 * t + 8 * hh;
          const bf16x8 bo = ld_lds16(&dotr[(32 * b + l32) * QTS + qoff]);
          dv[b] = mfma32(as_bf16x8(pt[t]), bo, dv[b]);
          const bf16x8 bq = ld_lds16(&qtr[(32 * b + l32) * QTS + qoff]);
          dk[b] = mfma32(as_bf16x8(dst[t]), bq, dk[b]);
        }
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();

    // dQ[q0.., 32 db ..] += dS[:, keys] K[keys, 32 db ..]   (M = queries, N = d)
    {
      f32x16 acc[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) acc[qb] = f32x16{};
#pragma unroll
      for (int t = 0; t < C::DQ_KEYS / 16; ++t) {
        const int kk = dq_k0 + 16 * t + 8 * hh;
        const bf16x8 b = ld_lds16(&kt[(32 * db + l32) * KTS + kk]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const bf16x8 a = ld_lds16(&dss[(32 * qb + l32) * DSS + kk]);
          acc[qb] = mfma32(a, b, acc[qb]);
        }
      }
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = q0 + 32 * qb + 8 * (r >> 2) + 4 * hh + (r & 3);
          buf_atomic_add(rdQ, ((uint32_t)q * D + 32 * db + l32) * 4u, acc[qb][r]);
        }
    }
    if (it + 1 < nsteps) store_q();
    __syncthreads();
  }

  // ---- epilogue: dK = scale * dK_acc, dV = dV_acc, bf16 ----------------------
#pragma unroll
  for (int b = 0; b < D / 32; ++b)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kk = kw0 + 8 * (r >> 2) + 4 * hh + (r & 3);
      if (kk < N) {
        const size_t off = head + (size_t)kk * D + 32 * b + l32;
        dK[off] = (__bf16)(dk[b][r] * scale);
        dV[off] = (__bf16)dv[b][r];
      }
    }
}

// ---------------------------------------------------------------------------
// 3. dQ = bf16(scale * dQ_acc)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_dq_kernel(const float* __restrict__ acc,
                                                    __bf16* __restrict__ dQ, float scale,
                                                    long long n8) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  const f32x4 a = reinterpret_cast<const f32x4*>(acc)[2 * i];
  const f32x4 b = reinterpret_cast<const f32x4*>(acc)[2 * i + 1];
  u32x4 w;
  w[0] = pack_bf16(a[0] * scale, a[1] * scale);
  w[1] = pack_bf16(a[2] * scale, a[3] * scale);
  w[2] = pack_bf16(b[0] * scale, b[1] * scale);
  w[3] = pack_bf16(b[2] * scale, b[3] * scale);
  reinterpret_cast<u32x4*>(dQ)[i] = w;
}

#ifndef FA_BWD_BRB
#define FA_BWD_BRB 64
#endif

template <int D, bool CAUSAL>
static hipError_t launch_bwd_t(const BwdArgs& a) {
  using C = BwdCfg<D, FA_BWD_BRB>;
  const long long rows = (long long)a.B * a.H * a.N;
  f32x2* rowstat = reinterpret_cast<f32x2*>(a.rowstat);
  {
    const long long threads = rows * (D / 8);
    const hipError_t e = launch_kernel(bwd_pre_kernel<D>, dim3((unsigned)((threads + 255) / 256)),
                                       dim3(256), a.stream, (const __bf16*)a.O, (const __bf16*)a.dO,
                                       a.LSE, a.dq_acc, rowstat, rows);
    if (e != hipSuccess) return e;
  }
  {
    const int nkb = (a.N + C::BCB - 1) / C::BCB;
    const long long total = (long long)nkb * a.B * a.H;
    const hipError_t e = launch_kernel(
        bwd_kernel<D, FA_BWD_BRB, CAUSAL>, dim3((unsigned)total), dim3(256), a.stream,
        (const __bf16*)a.Q, (const __bf16*)a.K, (const __bf16*)a.V, (const __bf16*)a.dO,
        (const f32x2*)rowstat, a.dq_acc, (__bf16*)a.dK, (__bf16*)a.dV, a.N, a.B * a.H,
        a.softmax_scale * kLog2e, a.softmax_scale);
    if (e != hipSuccess) return e;
  }
  {
    const long long n8 = rows * D / 8;
    return launch_kernel(bwd_dq_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), a.stream,
                         (const float*)a.dq_acc, (__bf16*)a.dQ, a.softmax_scale, n8);
  }
}

hipError_t launch_bwd(const BwdArgs& a) {
  if (a.d == 128) return a.causal ? launch_bwd_t<128, true>(a) : launch_bwd_t<128, false>(a);
  return a.causal ? launch_bwd_t<64, true>(a) : launch_bwd_t<64, false>(a);
}

}  // namespace fa
