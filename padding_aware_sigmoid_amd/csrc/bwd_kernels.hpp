// Backward kernels (bf16, MFMA) of padding-aware sigmoid attention, and of
// softmax attention with the same padding design.
//
// Method (rainbus.top summary of arXiv:2604.27124, section "方法步骤详情", steps 4-5):
//  - P = sigma(S) is recomputed from Q and K.
//  - dS = P (1 - P) (dO V^T).
//  - The backward is split into a dQ kernel and a dK/dV kernel. The dK/dV
//    kernel takes the same product in the transposed view.
//  - Neither kernel needs atomics.
// The chain rule gives:
//    dQ = alpha dS K,   dK = alpha dS^T Q,   dV = P^T dO.
//
// Padding: padded rows of K, V (keys >= n_k) and of Q, dO (queries >= n_q) are
// never read. Their LDS rows are zeros. A zero V row gives dP = 0, so dS = 0,
// and a zero dO row gives dP = 0 and adds P * 0 to dV. Padding therefore adds
// exactly nothing to any valid gradient row. Tiles wholly in padding are skipped
// and their output rows written as zeros.
#pragma once

#include "common.hpp"

namespace sigattn {

template <int D>
struct BwdCfg {
  static constexpr int W = 64;          // rows a wave owns: queries (dQ kernel) or keys (dK/dV kernel)
  static constexpr int NWAVE = 4;       // one wave per SIMD
  static constexpr int BQ_DQ = 256;     // dQ kernel: query rows per workgroup
  static constexpr int BK_DQ = 64;      // dQ kernel: keys per LDS tile
  static constexpr int BK_KV = 256;     // dK/dV kernel: key rows per tile_counts entry (1 or 2 workgroups)
  static constexpr int BQ_KV = 64;      // dK/dV kernel: queries per LDS tile
  static constexpr int KS = D / 16;     // MFMA k-steps over the head dim
  static constexpr int NB = D / 32;     // 32-wide column blocks of the gradients
  static constexpr int TILE = 64 * D;   // elements of one 64-row LDS tile (swizzled, unpadded)
};

// Which attention the backward differentiates.
//   ACT_SIGMOID: P = sigma(S) (the pages' method), dS = P (1 - P) dP.
//   ACT_SOFTMAX: P = softmax over keys, recomputed from the forward's row
//                log-sum-exp as e^(alpha s - LSE) = 2^(c1 (s - LSE / alpha));
//                dS = P (dP - D) with D_i = dO_i . O_i. Both row statistics
//                come as float2 {LSE / alpha, D} per query row and head.
enum Act { ACT_SIGMOID = 0, ACT_SOFTMAX = 1 };

// ------------------------------------------------------------------------------------------ dQ
// Wave w owns 64 query rows (two 32-row blocks). It holds Q and dO as B
// operands, for:
//   S^T  = K Q^T   (A = K from LDS)
//   dP^T = V dO^T  (A = V from LDS)
// dS^T = P (1 - P) dP^T is built in registers and fed as the A operand of
// dQ += dS K. That product takes K from LDS through transposed reads.
// Key tiles of 64 rows stream through a 3-slot LDS ring by DMA. Per 32-key
// block, the previous block's dQ MFMAs run beside this block's sigma and dS.
// At D = 128 each tile runs as one explicit stream of steps that reads every
// LDS operand two steps ahead.
// Tile t-2 is last read in iteration t-1 (the dQ of its second block), so the
// DMA of tile t+1 into its slot starts only after iteration t's barrier.
// Each slot is its own LDS variable and the key loop is unrolled by three, so
// every LDS access names its slot at compile time. The compiler can then tell
// the in-flight DMA apart from the reads of the other two slots and does not
// wait for it before them.
template <int D, int ACT>
__global__ __launch_bounds__(256, kWavesPerSimd<D>) void dq_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                      const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                                                      __bf16* __restrict__ dQ, const float2* __restrict__ stats,
                                                      SeqLayout sl, int Z, int H, float alpha, float c1,
                                                      float c0_base, int32_t* __restrict__ tile_counts) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 sK0[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sK1[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sK2[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV2[C::TILE];
  __shared__ RankLds rank_lds;
  const int n_qt = (sl.L + C::BQ_DQ - 1) / C::BQ_DQ;
  const TileCoord tcd = schedule_tile(blockIdx.x, Z, H, n_qt, sl, rank_lds);
  const int z = tcd.z, h = tcd.h, m = tcd.m;
  const int nq = sl.nq(z);
  const int nk = sl.nk(z);
  const float c0 = sl.c0_for(c0_base, nk);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)H * D;
  const size_t base = (sl.row0_q(z) * H + h) * D;    // Q, dO and dQ
  const size_t base_k = (sl.row0_k(z) * H + h) * D;  // K and V
  const int rows = sl.rows(nq);                       // rows of this sample in dQ
  const int q0 = m * C::BQ_DQ;
  __bf16* dQb = dQ + base;

  if (q0 >= nq) {
    const int rows_here = min(C::BQ_DQ, rows - q0);
    const bf16x8 zz = zero_bf16x8();
    for (int c = tid; c < rows_here * (D / 8); c += 256)
      *(bf16x8*)(dQb + (size_t)(q0 + c / (D / 8)) * rs + (c % (D / 8)) * 8) = zz;
    if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = 0;
    return;
  }

  bf16x8 qf[2][C::KS], dof[2][C::KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qr = q0 + 64 * w + 32 * qb + l32;
    const bool ok = qr < nq;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      qf[qb][s] = ok ? *(const bf16x8*)(Q + base + (size_t)qr * rs + 16 * s + 8 * half) : zero_bf16x8();
      dof[qb][s] = ok ? *(const bf16x8*)(dO + base + (size_t)qr * rs + 16 * s + 8 * half) : zero_bf16x8();
    }
  }
  f32x16 acc[2][C::NB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < C::NB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][db][r] = 0.0f;
  // softmax: this lane's query rows' {c1 LSE / alpha = LSE log2 e, D}
  float2 st[2] = {make_float2(0.0f, 0.0f), make_float2(0.0f, 0.0f)};
  if constexpr (ACT == ACT_SOFTMAX) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qr = q0 + 64 * w + 32 * qb + l32;
      if (qr < nq) st[qb] = stats[(sl.row0_q(z) + qr) * H + h];
      st[qb].x *= c1;
    }
  }

  const int nkt = (nk + C::BK_DQ - 1) / C::BK_DQ;  // live key tiles; no other tile is computed
  int executed = 0;                                 // key tiles whose scores this workgroup computed
  if (nkt > 0) {
    const uint32_t row_bytes = (uint32_t)(rs * 2);
    const __bf16* Kb = K + base_k;
    const __bf16* Vb = V + base_k;
    auto fetch = [&](__bf16* sk, __bf16* sv, int tile) {
      const int k0 = tile * C::BK_DQ;
      const size_t off = (size_t)(k0 < nk ? k0 : 0) * rs;  // no row is read past n_k
      dma_tile<D, 64, 256>(sk, Kb + off, row_bytes, nk - k0, tid);
      dma_tile<D, 64, 256>(sv, Vb + off, row_bytes, nk - k0, tid);
    };
    // The dQ of the previous 32-key block, beside this block's sigma and dS.
    auto dq_mfmas = [&](const __bf16* kt, int kbp, const bf16x8 (&dsp)[2][2]) {
#pragma unroll
      for (int db = 0; db < C::NB; ++db)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 b = lds_tr<D>(kt, kbp * 32 + ks * 16, db * 32, lane);
          acc[0][db] = mfma32(dsp[0][ks], b, acc[0][db]);
          acc[1][db] = mfma32(dsp[1][ks], b, acc[1][db]);
        }
    };
    // dS of the previous 32-key block (block 1 of the previous tile), waiting
    // for its dQ MFMAs; dS of block 0 of the current tile, for block 1's.
    bf16x8 ds_prev[2][2], ds_mid[2][2];
    // Each key tile is two 32-key blocks. Block 0 of tile t: S^T, dP^T, then
    // the dQ MFMAs of block 1 of tile t-1 beside sigma and dS. Block 1: S^T,
    // dP^T, then the dQ of block 0 of the same tile. The key loop runs block 1
    // of tile t and block 0 of tile t+1 per body, so each body adds exactly
    // one key tile (t+1). The prologue is block 0 of tile 0 (there is no
    // tile -1 to take dQ from) and the epilogue block 1 of the last tile plus
    // its dQ.
    //
    // At D = 128 a block runs as one explicit stream of steps, each one LDS
    // read and two MFMAs (one per query block):
    //   block steps 0 .. KS - 1: S^T of this block (K read by rows);
    //   block steps KS .. 2 KS - 1: dP^T of this block (V read by rows), beside
    //     P = sigma(S), written over the scores;
    //   block steps 2 KS .. 2 KS + 2 NB - 1: dQ += dS K of the previous block
    //     (K read transposed), beside dS of this block.
    // Each step's operand is read two steps ahead, from block 0 into block 1;
    // block 0's first two reads follow the barrier that publishes its tile.
    // Splitting sigma from dS this way spreads the VALU work over two thirds of
    // the steps instead of one third: 1% faster than all of it beside dQ.
    // sk, sv: this block's tile; skq: the tile whose block (1 - BLK) the dQ
    // MFMAs read (the previous tile for block 0, the same tile for block 1).
    constexpr int NA = 2 * C::KS, NSB = NA + 2 * C::NB, NT = 2 * NSB;
    constexpr int NE = 32;  // scores per lane and block: two query blocks of 16
    bf16x8 ops[3];
    auto block_stream = [&](auto blk_c, auto nodq_c, const __bf16* sk, const __bf16* sv,
                            const __bf16* skq) __attribute__((always_inline)) {
      constexpr int BLK = decltype(blk_c)::value;
      constexpr bool NO_DQ = decltype(nodq_c)::value;
      auto read = [&](auto gc) -> bf16x8 {
        constexpr int g = decltype(gc)::value, blk = g / NSB, j = g % NSB;
        if constexpr (j < NA) {
          return lds_nat<D>(j >= C::KS ? sv : sk, blk * 32 + l32, 2 * (j % C::KS) + half);
        } else {
          constexpr int i = j - NA, db = i >> 1, ks = i & 1;
          return lds_tr<D>(skq, (1 - blk) * 32 + ks * 16, db * 32, lane);
        }
      };
      f32x16 sacc[2], pacc[2];
      if constexpr (BLK == 0) {
        ops[0] = read(std::integral_constant<int, 0>{});
        ops[1] = read(std::integral_constant<int, 1>{});
      }
      static_for<BLK * NSB, BLK * NSB + NSB>([&](auto gc) {
        constexpr int g = decltype(gc)::value, blk = g / NSB, j = g % NSB;
        // the read two steps ahead: none into the dQ steps of a block without
        // them, none past the tile (block 0 of the next tile follows a barrier)
        constexpr int ga = g + 2;
        constexpr bool skip_ahead = ga >= NT || (NO_DQ && ga / NSB == BLK && ga % NSB >= NA);
        if constexpr (!skip_ahead) ops[ga % 3] = read(std::integral_constant<int, ga>{});
        const bf16x8 op = ops[g % 3];
        if constexpr (j == 0) {
#pragma unroll
          for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r) sacc[qb][r] = pacc[qb][r] = 0.0f;
        }
        if constexpr (j < NA) {
          constexpr int s = j % C::KS;
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            if constexpr (j >= C::KS)
              pacc[qb] = mfma32(op, dof[qb][s], pacc[qb]);
            else
              sacc[qb] = mfma32(op, qf[qb][s], sacc[qb]);
          }
        } else if constexpr (!NO_DQ) {
          constexpr int i = j - NA, db = i >> 1, ks = i & 1;
          const bf16x8 (&dsB)[2][2] = blk == 0 ? ds_prev : ds_mid;
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) acc[qb][db] = mfma32(dsB[qb][ks], op, acc[qb][db]);
        }
        // P = sigma(S) in place beside the dP^T MFMAs (from the second of them,
        // once the last S^T MFMA has landed), dS beside the dQ MFMAs.
        constexpr int NP = C::KS - 1;
        constexpr bool PST = j > C::KS && j < NA, DST = j >= NA;
        constexpr int p0 = PST ? (j - C::KS - 1) * NE / NP : 0, p1 = PST ? (j - C::KS) * NE / NP : 0;
        constexpr int d0 = DST ? (j - NA) * NE / (NSB - NA) : 0, d1 = DST ? (j - NA + 1) * NE / (NSB - NA) : 0;
        bf16x8 (&dsV)[2][2] = blk == 0 ? ds_mid : ds_prev;
        static_for<p0, p1>([&](auto ec) {
          constexpr int e = decltype(ec)::value, qb = e >> 4, r = e & 15;
          if constexpr (ACT == ACT_SIGMOID)
            sacc[qb][r] = sigmoid_dot(sacc[qb][r], c1, c0);
          else
            sacc[qb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][r], c1, -st[qb].x));
        });
        static_for<d0, d1>([&](auto ec) {
          constexpr int e = decltype(ec)::value, qb = e >> 4, r = e & 15;
          const float p = sacc[qb][r];
          if constexpr (ACT == ACT_SIGMOID)
            dsV[qb][r >> 3][r & 7] = (__bf16)(__builtin_fmaf(-p, p, p) * pacc[qb][r]);
          else
            dsV[qb][r >> 3][r & 7] = (__bf16)(p * (pacc[qb][r] - st[qb].y));
        });
        constexpr int nds = skip_ahead ? 0 : ((ga % NSB) < NA ? 1 : 2);
        constexpr int nvalu = (p1 - p0) * (ACT == ACT_SIGMOID ? 4 : 2) + (d1 - d0) * 3;
        sched_step<g, nds, (NO_DQ && j >= NA) ? 0 : 2, nvalu, 1>();
      });
    };
    // The same block in plain loops (D = 64): S^T and dP^T, then the dQ
    // MFMAs of the previous block beside this block's sigma and dS, scheduled
    // by the compiler.
    auto block_plain = [&](auto blk_c, auto nodq_c, const __bf16* sk, const __bf16* sv,
                           const __bf16* skq) __attribute__((always_inline)) {
      constexpr int BLK = decltype(blk_c)::value;
      constexpr bool NO_DQ = decltype(nodq_c)::value;
      f32x16 sacc[2], pacc[2];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qb][r] = pacc[qb][r] = 0.0f;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const bf16x8 ak = lds_nat<D>(sk, BLK * 32 + l32, 2 * s + half);
        const bf16x8 av = lds_nat<D>(sv, BLK * 32 + l32, 2 * s + half);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          sacc[qb] = mfma32(ak, qf[qb][s], sacc[qb]);
          pacc[qb] = mfma32(av, dof[qb][s], pacc[qb]);
        }
      }
      if constexpr (!NO_DQ) dq_mfmas(skq, 1 - BLK, BLK == 0 ? ds_prev : ds_mid);
      bf16x8 (&dsV)[2][2] = BLK == 0 ? ds_mid : ds_prev;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (ACT == ACT_SIGMOID) {
            const float p = sigmoid_dot(sacc[qb][r], c1, c0);
            dsV[qb][r >> 3][r & 7] = (__bf16)(__builtin_fmaf(-p, p, p) * pacc[qb][r]);
          } else {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][r], c1, -st[qb].x));
            dsV[qb][r >> 3][r & 7] = (__bf16)(p * (pacc[qb][r] - st[qb].y));
          }
        }
      interleave_mfma_valu<4 * C::KS + (NO_DQ ? 0 : 2 * C::NB * 2), 6>();
    };
    // At D = 128 the explicit step stream keeps each LDS read four MFMAs ahead
    // of its use; in plain loops the compiler leaves a third of the reads right
    // before their MFMA. Measured at L = 16K, H = 16: 2.85 ms against 3.13 (a
    // fence every step or every second step: the same). At D = 64 (softmax dQ;
    // sigmoid takes the swapped dK/dV kernel) the stream spills 47 registers
    // and the softmax backward ran 16% slower on cellbatch8k, so it keeps the
    // plain loops.
    auto block = [&](auto blk_c, auto nodq_c, const __bf16* sk, const __bf16* sv,
                     const __bf16* skq) __attribute__((always_inline)) {
      if constexpr (D == 128)
        block_stream(blk_c, nodq_c, sk, sv, skq);
      else
        block_plain(blk_c, nodq_c, sk, sv, skq);
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using DQ = std::false_type;
    using NODQ = std::true_type;
    // Tile t sits in slot t mod 3. Tile 0, then tile 1 behind block 0 of tile 0.
    fetch(sK0, sV0, 0);
    dma_wait();
    __syncthreads();
    if (nkt > 1) fetch(lds_opaque(sK1), lds_opaque(sV1), 1);  // waited for at the first body's barrier
    block(B0{}, NODQ{}, sK0, sV0, sK0);
    executed = 1;
    // Body for tile t in slot T (tile t+1 in slot N; slot P held tile t-1 and
    // receives tile t+2): block 1 of tile t, the barrier (tile t+1 is in LDS,
    // every wave is done with slot P), then block 0 of tile t+1.
    auto body = [&](const __bf16* kT, const __bf16* vT, __bf16* kN, __bf16* vN, __bf16* kP, __bf16* vP,
                    int t) __attribute__((always_inline)) {
      block(B1{}, DQ{}, kT, vT, kT);
      dma_wait();
      __syncthreads();
      if (t + 2 < nkt) fetch(kP, vP, t + 2);
      block(B0{}, DQ{}, kN, vN, kT);
      ++executed;
    };
    // Whole rounds of three bodies, then the one or two left over, with their
    // slots through lds_opaque: named at compile time they made the compiler
    // rebuild the loop's LDS addresses; opaque, it also leaves their DMA to
    // the explicit dma_wait and barrier of the next body.
    const int nb = nkt - 1, nb3 = nb / 3 * 3;
    for (int t = 0; t < nb3; t += 3) {
      body(sK0, sV0, sK1, sV1, sK2, sV2, t);
      body(sK1, sV1, sK2, sV2, sK0, sV0, t + 1);
      body(sK2, sV2, sK0, sV0, sK1, sV1, t + 2);
    }
    if (nb3 < nb)
      body(lds_opaque(sK0), lds_opaque(sV0), lds_opaque(sK1), lds_opaque(sV1), lds_opaque(sK2), lds_opaque(sV2), nb3);
    if (nb3 + 1 < nb)
      body(lds_opaque(sK1), lds_opaque(sV1), lds_opaque(sK2), lds_opaque(sV2), lds_opaque(sK0), lds_opaque(sV0),
           nb3 + 1);
    // Epilogue: block 1 of the last tile (slot nb mod 3), then its dQ.
    const int last = nb - nb3;
    const __bf16* kL = lds_opaque(last == 0 ? sK0 : (last == 1 ? sK1 : sK2));
    const __bf16* vL = lds_opaque(last == 0 ? sV0 : (last == 1 ? sV1 : sV2));
    block(B1{}, DQ{}, kL, vL, kL);
    dq_mfmas(kL, 1, ds_prev);
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < C::NB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = q0 + 64 * w + 32 * qb + acc_row(r, half);
        if (row < rows) dQb[(size_t)row * rs + db * 32 + l32] = (__bf16)(row < nq ? alpha * acc[qb][db][r] : 0.0f);
      }
  if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = executed;
}

// ---------------------------------------------------------------------------------------- dK/dV
// Wave w owns KB 32-row key blocks (KB = 2, 64 keys, in the separate dK and dV
// kernels; KB = 1 in the fused form). It holds K and V as B operands, for:
//   S  = Q K^T   (A = Q from LDS)
//   dP = dO V^T  (A = dO from LDS)
// P^T and dS^T come straight from those accumulators as A operands, for:
//   dV += P^T dO   (B = dO through transposed LDS reads)
//   dK += dS^T Q   (B = Q through transposed LDS reads)
// The query axis runs in blocks of 32, pipelined three deep as in the dQ
// kernel:
//   A: S (and dP) of block i
//   B: dV (and dK) += ... of block i-2
//   V: P (and dS) of block i-1
// Query tiles of 64 rows reach a 3-slot LDS ring by DMA.
//
// MODE selects what one launch computes:
//   KV_BOTH (dK and dV together) shares S between them: 8*D MFMA FLOP per pair.
//   KV_DK (S, dP, dK: 6*D) and KV_DV (S, dV: 4*D) split the work over two
//   launches.
// The fused form gives each wave 32 keys (KB = 1), so a workgroup covers 128
// keys (kKeysPerWg) and streams all query tiles once for them. At D = 128 the K
// and V operands plus both accumulators for 64 keys do not fit one wave's
// registers; at D = 64 they do, but at the register limit, where no
// scheduling fence fits, and the one-block form measured 13-14% faster
// (cellbatch8k and stress8k). The split forms keep KB = 2.
enum KvMode { KV_BOTH = 0, KV_DK = 1, KV_DV = 2 };

// Key blocks of 32 rows per wave.
template <int D, int MODE>
constexpr int kKB = MODE == KV_BOTH ? 1 : 2;

// stA (softmax only): the row statistics {LSE / alpha, D} of the tile whose
// query block qba the A stage processes. The A stage starts its accumulators
// at -LSE / alpha and -D instead of 0, so its MFMAs leave s' = s - LSE / alpha
// and dP' = dP - D, and the V stage needs no statistics: P = 2^(c1 s') and
// dS = P dP'.
template <int D, int MODE, int ACT, bool DO_A, bool DO_B, bool DO_V, int KB = kKB<D, MODE>>
__device__ __forceinline__ void kv_step(const __bf16* sQa, const __bf16* sGa, int qba, const __bf16* sQb,
                                        const __bf16* sGb, int qbb, f32x16 (&sN)[KB], f32x16 (&pN)[KB],
                                        f32x16 (&dkacc)[KB][BwdCfg<D>::NB], f32x16 (&dvacc)[KB][BwdCfg<D>::NB],
                                        const bf16x8 (&ptB)[KB][2], const bf16x8 (&dsB)[KB][2], bf16x8 (&ptV)[KB][2],
                                        bf16x8 (&dsV)[KB][2], const f32x16 (&sV)[KB], const f32x16 (&pV)[KB],
                                        const bf16x8 (&kf)[KB][BwdCfg<D>::KS], const bf16x8 (&vf)[KB][BwdCfg<D>::KS],
                                        float c1, float c0, const float2* stA, int l32, int half, int lane) {
  using C = BwdCfg<D>;
  constexpr bool DK = MODE != KV_DV, DV = MODE != KV_DK;
  constexpr int PA = DK ? 2 : 1;                // A operands per k-step: Q (and dO)
  constexpr int PB = (DK ? 1 : 0) + (DV ? 1 : 0);  // B operands per (db, ks): dO tr (dV), Q tr (dK)
  constexpr int NA = DO_A ? PA * C::KS : 0;
  constexpr int NSTEP = NA + (DO_B ? PB * 2 * C::NB : 0);
  constexpr int NV = DO_V ? 16 * KB : 0;
  // which job operand j belongs to: 0 = Q nat, 1 = dO nat, 2 = dO tr, 3 = Q tr
  auto kind = [](int j) constexpr -> int {
    if (j < NA) return (PA == 2 && (j & 1)) ? 1 : 0;
    const int i = j - NA;
    if (PB == 2) return (i & 1) ? 3 : 2;
    return DV ? 2 : 3;
  };
  auto read = [&](auto jc) -> bf16x8 {
    constexpr int j = decltype(jc)::value;
    constexpr int k = kind(j);
    if constexpr (k <= 1) {
      return lds_nat<D>(k == 1 ? sGa : sQa, qba * 32 + l32, 2 * (j / PA) + half);
    } else {
      constexpr int i = (j - NA) / PB, db = i >> 1, ks = i & 1;
      return lds_tr<D>(k == 2 ? sGb : sQb, qbb * 32 + ks * 16, db * 32, lane);
    }
  };
  if constexpr (DO_A && ACT == ACT_SIGMOID) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sN[kb][r] = 0.0f;
        if constexpr (DK) pN[kb][r] = 0.0f;
      }
  } else if constexpr (DO_A) {
    // Register r holds row (r/4)*8 + 4*half + r%4 of the block: 4 groups of 4 rows.
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4* src = (const float4*)(stA + qba * 32 + g * 8 + 4 * half);
      const float4 a = src[0], b = src[1];
      const float l[4] = {a.x, a.z, b.x, b.z}, d[4] = {a.y, a.w, b.y, b.w};
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          sN[kb][4 * g + rr] = -l[rr];
          if constexpr (DK) pN[kb][4 * g + rr] = -d[rr];
        }
    }
  }
  bf16x8 ops[3];
  ops[0] = read(std::integral_constant<int, 0>{});
  ops[1] = read(std::integral_constant<int, 1>{});
  float den[NV > 0 ? NV : 1];  // 1 + 2^(c1 s + c0) between the two halves of sigma
  static_for<0, NSTEP>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    constexpr int k = kind(j);
    if constexpr (j + 2 < NSTEP) ops[(j + 2) % 3] = read(std::integral_constant<int, j + 2>{});
    const bf16x8 op = ops[j % 3];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      if constexpr (k == 0) {
        sN[kb] = mfma32(op, kf[kb][j / PA], sN[kb]);
      } else if constexpr (k == 1) {
        pN[kb] = mfma32(op, vf[kb][j / PA], pN[kb]);
      } else {
        constexpr int i = (j - NA) / PB, db = i >> 1, ks = i & 1;
        if constexpr (k == 2)
          dvacc[kb][db] = mfma32(ptB[kb][ks], op, dvacc[kb][db]);
        else
          dkacc[kb][db] = mfma32(dsB[kb][ks], op, dkacc[kb][db]);
      }
    }
    constexpr int e0 = j * NV / NSTEP, e1 = (j + 1) * NV / NSTEP;
    // Sigmoid at D = 64: each score's chain (FMA, exp, add, rcp, then dS and
    // the bf16 packs) is split over two consecutive steps, 1 + 2^(c1 s + c0)
    // in one and the rest in the next, so that no step waits on one long
    // dependent chain between its MFMAs: 3% faster there (stress8k dK/dV and
    // dQ). At D = 128 the fused kernel is bound by its LDS reads (the
    // transposed ones run at half rate) and the split measured 1% slower.
    // Softmax's chain is short and stays in one step.
    constexpr bool SPLIT = ACT == ACT_SIGMOID && NV > 0 && D == 64;
    constexpr int f0 = (SPLIT && j > 0) ? (j - 1) * NV / (NSTEP - 1) : 0;  // second halves
    constexpr int f1 = (SPLIT && j > 0) ? j * NV / (NSTEP - 1) : 0;
    constexpr int g0 = (SPLIT && j + 1 < NSTEP) ? j * NV / (NSTEP - 1) : 0;  // first halves
    constexpr int g1 = (SPLIT && j + 1 < NSTEP) ? (j + 1) * NV / (NSTEP - 1) : 0;
    if constexpr (SPLIT) {
      static_for<f0, f1>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        constexpr int kb = e >> 4, r = e & 15;
        const float p = __builtin_amdgcn_rcpf(den[e]);
        if constexpr (DV) ptV[kb][r >> 3][r & 7] = (__bf16)p;
        if constexpr (DK) dsV[kb][r >> 3][r & 7] = (__bf16)(__builtin_fmaf(-p, p, p) * pV[kb][r]);
      });
      static_for<g0, g1>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        constexpr int kb = e >> 4, r = e & 15;
        den[e] = 1.0f + __builtin_amdgcn_exp2f(__builtin_fmaf(sV[kb][r], c1, c0));
      });
    } else {
      static_for<e0, e1>([&](auto ec) {
        constexpr int e = decltype(ec)::value;
        constexpr int kb = e >> 4, r = e & 15;
        if constexpr (ACT == ACT_SIGMOID) {
          const float p = sigmoid_dot(sV[kb][r], c1, c0);
          if constexpr (DV) ptV[kb][r >> 3][r & 7] = (__bf16)p;
          if constexpr (DK) dsV[kb][r >> 3][r & 7] = (__bf16)(__builtin_fmaf(-p, p, p) * pV[kb][r]);
        } else {
          const float p = __builtin_amdgcn_exp2f(sV[kb][r] * c1);
          if constexpr (DV) ptV[kb][r >> 3][r & 7] = (__bf16)p;
          if constexpr (DK) dsV[kb][r >> 3][r & 7] = (__bf16)(p * pV[kb][r]);
        }
      });
    }
    constexpr int nvalu = SPLIT ? (g1 - g0) * 3 + (f1 - f0) * (DK ? 4 : 2) : (e1 - e0) * (DK ? 7 : 5);
    constexpr int nds = (j + 2 < NSTEP) ? (kind(j + 2) <= 1 ? 1 : 2) : 0;
    // A hard fence every step (the fused form) or every second step (the dV
    // kernel) keeps the LDS reads two steps ahead of their MFMAs. Measured on
    // the fused form at D = 128: fences every 1, 2, 4 steps and none, 4.05,
    // 4.08, 4.44, 4.49 ms (L = 16K, H = 16). In the separate dK kernel a fence
    // makes the compiler spill or fail, so it schedules each kv_step as one
    // region. With the tiles' LDS addresses folded into immediates, the
    // sigmoid fused form at D = 128 runs best with the fences alone and the
    // compiler's order within each step (3.93 -> 3.84 ms); softmax and
    // D = 64 keep the groups (the softmax backward 1.5% slower without them).
    constexpr int FENCE = KB == 1 ? 1 : (MODE == KV_DV ? 2 : kNoFence);
    if constexpr (D == 128 && ACT == ACT_SIGMOID && MODE == KV_BOTH)
      sched_fence<j, FENCE>();
    else
      sched_step<j, nds, KB, nvalu, FENCE>();
  });
}

// Whether the dK/dV query loop is unrolled over the three ring slots. Unrolled,
// every LDS access names its slot at compile time, and the compiler does not
// wait for the DMA into one slot before reading the others. The separate dK
// kernel at D = 128 is at the register limit and spills heavily when
// unrolled. It keeps a runtime slot index into one array, with the DMA
// destinations hidden from the compiler (lds_opaque), which then does not
// wait for a DMA before its next LDS read either.
template <int D, int MODE>
constexpr bool kUnrolledRing = !(MODE == KV_DK && D == 128);

// Keys per workgroup: 4 waves of 32 KB keys, 128 in the one-block form
// (KB = 1: the fused kernel and the exchanged dQ), 256 in the split kernels.
// A tile of BK_KV keys (the unit of tile_counts) is then one or two
// workgroups; the first of them writes its count. Workgroups of 128 keys
// make a launch's last round shorter when sample lengths differ (a padded
// batch finishes with its shortest samples' workgroups), and measured
// registers below the earlier form of two passes of 128 keys per workgroup
// (459 against 476 at D = 128).
template <int D, int MODE, bool SWAP>
constexpr int kKeysPerWg = BwdCfg<D>::NWAVE * 32 * (SWAP ? 1 : kKB<D, MODE>);

// One launch computes what MODE selects (KV_BOTH, KV_DK or KV_DV), for the
// attention ACT selects. With softmax each query tile's row statistics
// {LSE / alpha, D} (64 float2) ride the LDS ring beside its Q and dO.
template <int D, int MODE, int ACT, bool SWAP = false>
__global__ __launch_bounds__(256, MODE == KV_BOTH ? kWavesPerSimd<D> : 1) void dkdv_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                        const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                                                        __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                                                        const float2* __restrict__ stats, SeqLayout sl, int Z, int H,
                                                        float alpha, float c1, float c0_base,
                                                        int32_t* __restrict__ tile_counts) {
  using C = BwdCfg<D>;
  constexpr bool DO_DK = MODE != KV_DV, DO_DV = MODE != KV_DK;
  constexpr bool SM = ACT == ACT_SOFTMAX;
  constexpr bool UR = SWAP || kUnrolledRing<D, MODE>;
  constexpr int TS = UR ? C::TILE : 8;  // the runtime-indexed ring lives in sRing instead
  __shared__ __attribute__((aligned(1024))) __bf16 sQ0[TS];
  __shared__ __attribute__((aligned(1024))) __bf16 sQ1[TS];
  __shared__ __attribute__((aligned(1024))) __bf16 sQ2[TS];
  __shared__ __attribute__((aligned(1024))) __bf16 sG0[TS];
  __shared__ __attribute__((aligned(1024))) __bf16 sG1[TS];
  __shared__ __attribute__((aligned(1024))) __bf16 sG2[TS];
  __shared__ __attribute__((aligned(64))) float2 sS0[SM && UR ? 64 : 1];
  __shared__ __attribute__((aligned(64))) float2 sS1[SM && UR ? 64 : 1];
  __shared__ __attribute__((aligned(64))) float2 sS2[SM && UR ? 64 : 1];
  __shared__ __attribute__((aligned(1024))) __bf16 sRing[UR ? 8 : 6 * C::TILE];
  __shared__ __attribute__((aligned(64))) float2 sSRing[SM && !UR ? 3 * 64 : 1];
  __shared__ RankLds rank_lds;
  constexpr int KT = kKeysPerWg<D, MODE, SWAP>;
  constexpr int WPT = C::BK_KV / KT;  // workgroups per tile of tile_counts
  const int n_kt = (sl.L + C::BK_KV - 1) / C::BK_KV;
  const int n_wt = (sl.L + KT - 1) / KT;
  const TileCoord tcd = schedule_tile(blockIdx.x, Z, H, n_wt, sl, rank_lds);
  const int z = tcd.z, h = tcd.h, t = tcd.m;
  // With SWAP the roles of queries and keys are exchanged (the sigmoid dQ
  // kernel at D = 64): "keys" here are the query rows the workgroup owns,
  // "queries" the key rows it streams, K and V arrive as Q and dO, dO and Q
  // as V and K, and the dK written is dQ. The per-sample bias still follows
  // the true key count.
  const int nq = SWAP ? sl.nk(z) : sl.nq(z);
  const int nk = SWAP ? sl.nq(z) : sl.nk(z);
  const float c0 = sl.c0_for(c0_base, sl.nk(z));
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)H * D;
  const size_t base = ((SWAP ? sl.row0_q(z) : sl.row0_k(z)) * H + h) * D;    // K, V, dK and dV
  const size_t base_q = ((SWAP ? sl.row0_k(z) : sl.row0_q(z)) * H + h) * D;  // Q and dO
  const int rows = sl.rows(nk);                                              // rows of this sample in dK, dV
  const int k0 = t * KT;
  __bf16* dKb = dK + base;
  __bf16* dVb = dV + base;

  if (k0 >= nk) {
    const int rows_here = min(KT, rows - k0);
    const bf16x8 zz = zero_bf16x8();
    for (int c = tid; c < rows_here * (D / 8); c += 256) {
      const size_t off = (size_t)(k0 + c / (D / 8)) * rs + (c % (D / 8)) * 8;
      if (DO_DK) *(bf16x8*)(dKb + off) = zz;
      if (DO_DV) *(bf16x8*)(dVb + off) = zz;
    }
    if (tile_counts != nullptr && tid == 0 && t % WPT == 0) tile_counts[((size_t)z * H + h) * n_kt + t / WPT] = 0;
    return;
  }

  constexpr int KB = SWAP ? 1 : kKB<D, MODE>;
  constexpr int WK = 32 * KB;           // keys per wave
  static_assert(C::NWAVE * WK == KT, "the workgroup's waves cover its keys");
  const int nqt = (nq + C::BQ_KV - 1) / C::BQ_KV;  // live query tiles; no other tile is computed
  int executed = 0;                                 // query tiles whose A stage ran (the prologue and each iteration)
  // One pass over the query tiles for the workgroup's keys kh .. kh + KT - 1.
  // The loop runs once. Written as a plain block instead, the same code
  // compiled to 502 registers instead of 459 (fused kernel, D = 128), 56
  // spilled registers instead of 13 (D = 64), and the exchanged dQ to 258
  // (one wave per SIMD) instead of 240.
  for (int pass = 0; pass < 1; ++pass) {
    const int kh = k0;
    bf16x8 kf[KB][C::KS], vf[KB][C::KS];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int kr = kh + WK * w + 32 * kb + l32;
      const bool ok = kr < nk;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        kf[kb][s] = ok ? *(const bf16x8*)(K + base + (size_t)kr * rs + 16 * s + 8 * half) : zero_bf16x8();
        if (DO_DK) vf[kb][s] = ok ? *(const bf16x8*)(V + base + (size_t)kr * rs + 16 * s + 8 * half) : zero_bf16x8();
      }
    }
    f32x16 dkacc[KB][C::NB], dvacc[KB][C::NB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int db = 0; db < C::NB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) dkacc[kb][db][r] = dvacc[kb][db][r] = 0.0f;

    if (nqt > 0) {
      const uint32_t row_bytes = (uint32_t)(rs * 2);
      const __bf16* Qb = Q + base_q;
      const __bf16* dOb = dO + base_q;
      const float2* Sb = SM ? stats + sl.row0_q(z) * H + h : nullptr;
      auto fetch = [&](__bf16* sq, __bf16* sg, float2* ss, int tile) {
        const int r0 = tile * C::BQ_KV;
        const size_t off = (size_t)(r0 < nq ? r0 : 0) * rs;  // no row is read past n_q
        dma_tile<D, 64, 256>(sq, Qb + off, row_bytes, nq - r0, tid);
        dma_tile<D, 64, 256>(sg, dOb + off, row_bytes, nq - r0, tid);
        if constexpr (SM) dma_stats64(ss, Sb + (size_t)(r0 < nq ? r0 : 0) * H, (uint32_t)(H * 8), nq - r0, tid);
      };
      f32x16 sX[KB], pX[KB], sY[KB], pY[KB];
      bf16x8 ptX[KB][2], ptY[KB][2], dsX[KB][2], dsY[KB][2];
      // Query tile u: its slot (q_cur, g_cur), tile u-1's slot (q_prev, g_prev)
      // and the slot that receives tile u+1 (it held tile u-2).
      // The V stage of each step turns the previous A stage's block into P (and
      // dS). The A stage reads the row statistics of its own tile (s_cur).
      auto iteration = [&](__bf16* q_cur, __bf16* g_cur, float2* s_cur, __bf16* q_prev, __bf16* g_prev,
                           __bf16* q_next, __bf16* g_next, float2* s_next, int u, int n_tiles) {
        dma_wait();
        __syncthreads();
        if (u + 1 < n_tiles) fetch(q_next, g_next, s_next, u + 1);
        kv_step<D, MODE, ACT, true, true, true, KB>(q_cur, g_cur, 0, q_prev, g_prev, 0, sX, pX, dkacc, dvacc, ptX, dsX,
                                                ptY, dsY, sY, pY, kf, vf, c1, c0, s_cur, l32, half, lane);
        kv_step<D, MODE, ACT, true, true, true, KB>(q_cur, g_cur, 1, q_prev, g_prev, 1, sY, pY, dkacc, dvacc, ptY, dsY,
                                                ptX, dsX, sX, pX, kf, vf, c1, c0, s_cur, l32, half, lane);
        ++executed;
      };
      // Tile 0 into slot 0, then tile 1 into slot 1 (q1, g1, s1: its DMA
      // destinations) behind the first A stages.
      auto prologue = [&](__bf16* q0, __bf16* g0, float2* s0, __bf16* q1, __bf16* g1, float2* s1, int n_tiles) {
        fetch(q0, g0, s0, 0);
        dma_wait();
        __syncthreads();
        if (n_tiles > 1) fetch(q1, g1, s1, 1);  // no DMA may be left in flight when the kernel ends
        kv_step<D, MODE, ACT, true, false, false, KB>(q0, g0, 0, q0, g0, 0, sX, pX, dkacc, dvacc, ptX, dsX, ptY, dsY, sY,
                                                  pY, kf, vf, c1, c0, s0, l32, half, lane);
        kv_step<D, MODE, ACT, true, false, true, KB>(q0, g0, 1, q0, g0, 0, sY, pY, dkacc, dvacc, ptY, dsY, ptX, dsX, sX,
                                                 pX, kf, vf, c1, c0, s0, l32, half, lane);
        executed = 1;
      };
      auto epilogue = [&](__bf16* q_last, __bf16* g_last, float2* s_last) {
        kv_step<D, MODE, ACT, false, true, true, KB>(q_last, g_last, 0, q_last, g_last, 0, sX, pX, dkacc, dvacc, ptX,
                                                 dsX, ptY, dsY, sY, pY, kf, vf, c1, c0, s_last, l32, half, lane);
        kv_step<D, MODE, ACT, false, true, false, KB>(q_last, g_last, 0, q_last, g_last, 1, sY, pY, dkacc, dvacc, ptY,
                                                  dsY, ptX, dsX, sX, pX, kf, vf, c1, c0, s_last, l32, half, lane);
      };
      if constexpr (UR) {
        // Query tile u sits in slot u mod 3. Exactly the nqt live tiles run:
        // tile 0 in the prologue, tiles 1 .. nqt-1 in the iterations (whole
        // rounds of three, then the one or two left over), and the last
        // tile's B and V stages in the epilogue. A loop entered or left in the
        // middle of a round makes the compiler spill heavily, so the leftover
        // iterations sit after it.
        prologue(sQ0, sG0, sS0, sQ1, sG1, sS1, nqt);
        const int ni = nqt - 1, ni3 = ni / 3 * 3;
        for (int u = 1; u <= ni3; u += 3) {
          iteration(sQ1, sG1, sS1, sQ0, sG0, sQ2, sG2, sS2, u, nqt);
          iteration(sQ2, sG2, sS2, sQ1, sG1, sQ0, sG0, sS0, u + 1, nqt);
          iteration(sQ0, sG0, sS0, sQ2, sG2, sQ1, sG1, sS1, u + 2, nqt);
        }
        // At D = 128 the leftover iterations take their slots through
        // lds_opaque: the compiler then neither shares their LDS addresses
        // with the loop's (sharing them cost the loop 40 address adds per
        // round) nor waits for their DMA on its own; each iteration waits for
        // it itself (dma_wait and the barrier at its top). At D = 64 the
        // opaque form left 8 more spill accesses in the loop (cellbatch8k
        // dK/dV 4% slower), and named slots leave the loop as it was.
        auto o = [](auto* x) {
          if constexpr (D == 128)
            return lds_opaque(x);
          else
            return x;
        };
        if (ni3 < ni) iteration(o(sQ1), o(sG1), o(sS1), o(sQ0), o(sG0), o(sQ2), o(sG2), o(sS2), ni3 + 1, nqt);
        if (ni3 + 1 < ni) iteration(o(sQ2), o(sG2), o(sS2), o(sQ1), o(sG1), o(sQ0), o(sG0), o(sS0), ni3 + 2, nqt);
        // The last tile's B and V stages, in its slot (nqt - 1) mod 3, named at
        // compile time: with a runtime-selected slot the compiler also
        // rebuilt the loop's LDS addresses (40 more address adds per round).
        const int last = ni % 3;  // the slot of tile nqt - 1
        epilogue(last == 0 ? sQ0 : (last == 1 ? sQ1 : sQ2), last == 0 ? sG0 : (last == 1 ? sG1 : sG2),
                 last == 0 ? sS0 : (last == 1 ? sS1 : sS2));
      } else {
        // The three slots are parts of one array, indexed at run time. Every
        // read names that array, so the compiler can match it against DMAs.
        // The DMA destinations are passed through lds_opaque: the compiler does
        // not match the reads against them and inserts no wait for the DMA in
        // flight. The DMA of a tile is waited for explicitly (dma_wait and the
        // barrier at the top of the next iteration) before any read of it.
        auto q_at = [&](int i) { return sRing + (2 * i) * C::TILE; };
        auto g_at = [&](int i) { return sRing + (2 * i + 1) * C::TILE; };
        auto s_at = [&](int i) { return SM ? sSRing + 64 * i : sSRing; };
        prologue(q_at(0), g_at(0), s_at(0), lds_opaque(q_at(1)), lds_opaque(g_at(1)), lds_opaque(s_at(1)), nqt);
        int cur = 0;
        for (int u = 1; u < nqt; ++u) {
          const int prev = cur;
          cur = (cur == 2) ? 0 : cur + 1;
          const int next = (cur == 2) ? 0 : cur + 1;
          iteration(q_at(cur), g_at(cur), s_at(cur), q_at(prev), g_at(prev), lds_opaque(q_at(next)),
                    lds_opaque(g_at(next)), lds_opaque(s_at(next)), u, nqt);
        }
        epilogue(q_at(cur), g_at(cur), s_at(cur));
      }
    }
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int db = 0; db < C::NB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = kh + WK * w + 32 * kb + acc_row(r, half);
          if (row < rows) {
            const bool ok = row < nk;
            if (DO_DK) dKb[(size_t)row * rs + db * 32 + l32] = (__bf16)(ok ? alpha * dkacc[kb][db][r] : 0.0f);
            if (DO_DV) dVb[(size_t)row * rs + db * 32 + l32] = (__bf16)(ok ? dvacc[kb][db][r] : 0.0f);
          }
        }
  }
  if (tile_counts != nullptr && tid == 0 && t % WPT == 0) tile_counts[((size_t)z * H + h) * n_kt + t / WPT] = executed;
}

// The softmax dK kernel at D = 128 lives in its own translation unit, built
// without the VGPR form of MFMA results: at this register count the compiler
// cannot build it in that form.
hipError_t launch_dk_bf16_softmax_d128(const void* q, const void* k, const void* v, const void* dout, void* dk,
                                       const void* stats, SeqLayout sl, int Z, int H, float alpha, float c1,
                                       int32_t* tc, hipStream_t st);

}  // namespace sigattn
