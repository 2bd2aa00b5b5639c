// Forward kernels: O = sigma(alpha Q K^T + b) V with padding-aware tile skipping.
//
// Method: rainbus.top summary of arXiv:2604.27124, section "方法步骤详情",
// steps 1-3 (blocking of [Z,L,H,D] tensors, skipping of query blocks wholly in
// padding, -inf at padded keys, sigma accumulated into O); gist.science summary
// section 2.A (forward formula).
//
// CDNA4 design (bf16):
//  - One workgroup computes one query tile of BQ = 256 rows for one (z, h).
//    It has 4 waves (one per SIMD) of 64 query rows each. A wave's two 32-row
//    blocks share every K and V operand read from LDS, which halves LDS
//    traffic per MFMA compared with 32-row waves.
//  - A query tile at or past n_q writes zeros and exits.
//  - Only key tiles below n_k are visited, so wholly padded key tiles are
//    skipped.
//  - K and V tiles reach LDS by DMA (16 bytes per lane, coalesced), into an
//    XOR-swizzled layout.
//  - A padded key row is never read: its lanes fetch out of range, so its LDS
//    row holds zeros. Its score is then b, and its weight is multiplied by
//    V = 0. Its contribution is therefore exactly 0, whatever the padding
//    holds.
//  - Scores are computed transposed, S^T = K Q^T, so the accumulator already
//    has the layout of the A operand of P V. P never leaves registers.
//  - V reaches the MFMA through ds_read_b64_tr_b16.
//  - sigma takes one v_exp_f32 and one FMA per score, t - t^2 with t = e^S,
//    on every 32 x 32 block of weights whose scores all lie at or below -3.47
//    (relative error t^2, at most 2^-10; the bias b = -ln n puts nearly all scores
//    there), and the exact 1 / (1 + e^-S) (v_exp_f32, v_rcp_f32) on the
//    others: a ballot after each block tells the wave to recompute it. A
//    workgroup whose first block of scores already leaves that range (large
//    score norms) runs the exact form throughout.
#include "common.hpp"

namespace sigattn {

template <int D>
struct FwdCfg {
  static constexpr int WQ = 64;           // query rows per wave (two 32-row MFMA blocks)
  static constexpr int NWAVE = 4;         // one wave per SIMD
  static constexpr int BQ = WQ * NWAVE;   // 256 query rows per workgroup
  static constexpr int BK = 64;           // keys per LDS tile (two 32-key MFMA blocks)
  static constexpr int NBUF = 3;          // LDS ring depth (tiles t-1, t, t+1 live at once)
  static constexpr int KS = D / 16;       // MFMA k-steps over the head dim
  static constexpr int NB = D / 32;       // 32-wide column blocks of O
  static constexpr int TILE = BK * D;     // elements of one K (or V) tile in LDS (swizzled, unpadded)
};

// S^T for one 32-key block kb of a K tile and the wave's two 32-query blocks.
template <int D>
__device__ __forceinline__ void scores_t(f32x16 (&sacc)[2], const __bf16* sK, int kb,
                                         const bf16x8 (&qf)[2][FwdCfg<D>::KS], int l32, int half) {
  using C = FwdCfg<D>;
#pragma unroll
  for (int r = 0; r < 16; ++r) sacc[0][r] = sacc[1][r] = 0.0f;
#pragma unroll
  for (int s = 0; s < C::KS; ++s) {
    const bf16x8 a = lds_nat<D>(sK, kb * 32 + l32, 2 * s + half);
    sacc[0] = mfma32(a, qf[0][s], sacc[0]);
    sacc[1] = mfma32(a, qf[1][s], sacc[1]);
  }
}

// O += P V for one 32-key block kb of a V tile.
template <int D>
__device__ __forceinline__ void accumulate_pv(f32x16 (&oacc)[2][FwdCfg<D>::NB], const bf16x8 (&p)[2][2],
                                              const __bf16* sV, int kb, int lane) {
  using C = FwdCfg<D>;
#pragma unroll
  for (int db = 0; db < C::NB; ++db)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 b = lds_tr<D>(sV, kb * 32 + ks * 16, db * 32, lane);
      oacc[0][db] = mfma32(p[0][ks], b, oacc[0][db]);
      oacc[1][db] = mfma32(p[1][ks], b, oacc[1][db]);
    }
}

// P for the wave's two 32-query blocks and one 32-key block, with the exact
// sigma (the fallback of the one-transcendental form).
__device__ __forceinline__ void sigmoid_exact_block(bf16x8 (&p)[2][2], const f32x16 (&s)[2], float c1, float c0) {
#pragma unroll
  for (int e = 0; e < 32; ++e) p[e >> 4][(e & 15) >> 3][e & 7] = (__bf16)sigmoid_dot(s[e >> 4][e & 15], c1, c0);
}

// The forward of one wave, written as a fixed step schedule. With one wave per
// SIMD, latency can only be hidden inside the wave's own instruction stream.
// Key tile t is two phases of NSTEP steps, 2 MFMAs each:
//   phase A: S(t, 2nd half) = K Q^T (KS steps), then O += P(t-1, 2nd half) V
//            (2*NB steps)                          || P(t, 1st half) = sigma(S)
//   barrier (at_barrier: the DMA of tile t+1 has landed; the next one starts)
//   phase B: O += P(t, 1st half) V (2*NB steps), then S(t+1, 1st half)
//            (KS steps)                            || P(t, 2nd half) = sigma(S)
// fwd_steps runs steps [G0, G1) of that stream for one tile. The key loop runs
// phase B of tile t followed by phase A of tile t+1, so each loop body adds
// exactly one key tile (t+1); the first tile's phase A (which has no tile -1)
// and the last tile's phase B (which has no tile t+1) are written out apart
// from the loop. The LDS operand of step g+3 is requested at step g, through
// the barrier and on into the next phase. Reads that precede the barrier touch
// only V of tile t, which landed a tile earlier; tile t+1's K is read only
// after the barrier. Since S of phase B is finished by its last steps, phase
// A's sigma starts one step late. ops[0..3] is a ring indexed by step mod 4
// (2 * NSTEP is a multiple of 4).
// Slots: kT, vT hold tile t; vP holds tile t-1 (phase A's P V); kN holds tile
// t+1 (phase B's S, and the reads ahead into the next phase A).
template <int D, int G0, int G1, bool SMALL, typename AtBarrier, typename DmaChunk>
__device__ __forceinline__ void fwd_steps(const __bf16* kT, const __bf16* vP, const __bf16* vT, const __bf16* kN,
                                          f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2],
                                          f32x16 (&oacc)[2][FwdCfg<D>::NB], bf16x8 (&p0)[2][2], bf16x8 (&p1)[2][2],
                                          bf16x8 (&ops)[4], const bf16x8 (&qf)[2][FwdCfg<D>::KS], float c1, float c0,
                                          uint32_t& tmax, int l32, int half, int lane, AtBarrier&& at_barrier,
                                          DmaChunk&& dma_chunk) {
  using C = FwdCfg<D>;
  constexpr int KS = C::KS, NB2 = 2 * C::NB;
  constexpr int NSTEP = KS + NB2;  // steps per phase: 16 at D = 128, 8 at D = 64
  constexpr int G = 2 * NSTEP;     // steps per tile
  static_assert(G % 4 == 0 && KS >= 3 && NB2 >= 3, "ring of four operands, three steps ahead");
  static_assert(0 <= G0 && G0 < G1 && G1 <= G, "a step range of one tile");
  // The next DMA is NDMA instructions per thread (K and V), spread one per
  // DSTRIDE steps over phase B: issued in one burst they stall the wave.
  constexpr int NDMA = 2 * kDmaChunks<D, C::BK, 256>;
  constexpr int DSTRIDE = NSTEP / NDMA > 0 ? NSTEP / NDMA : 1;
  static_assert(NDMA <= NSTEP, "one DMA instruction per step at most");
  // The operand of step g; g >= G are the next tile's first steps (K of tile t+1, 2nd half).
  auto read = [&](auto gc) -> bf16x8 {
    constexpr int g = decltype(gc)::value;
    if constexpr (g < KS) {
      return lds_nat<D>(kT, 32 + l32, 2 * g + half);
    } else if constexpr (g < NSTEP) {
      constexpr int i = g - KS;
      return lds_tr<D>(vP, 32 + (i & 1) * 16, (i >> 1) * 32, lane);
    } else if constexpr (g < NSTEP + NB2) {
      constexpr int i = g - NSTEP;
      return lds_tr<D>(vT, (i & 1) * 16, (i >> 1) * 32, lane);
    } else if constexpr (g < G) {
      return lds_nat<D>(kN, l32, 2 * (g - NSTEP - NB2) + half);
    } else {
      return lds_nat<D>(kN, 32 + l32, 2 * (g - G) + half);
    }
  };
  auto reads_of = [](int g) constexpr -> int {  // LDS instructions behind step g's operand
    const int h = g % G;
    return (h < KS || h >= NSTEP + NB2) ? 1 : 2;
  };
  static_for<G0, G1>([&](auto gc) {
    constexpr int g = decltype(gc)::value;
    if constexpr (g == 0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s_nxt[0][r] = s_nxt[1][r] = 0.0f;
    }
    if constexpr (g == NSTEP) {
      pin_before_barrier(p0);
      at_barrier();
      // With the one-transcendental sigma: P(t, 1st half) is complete here and
      // unused so far, and its scores are intact until the next line. If one
      // of them left the form's range, the wave recomputes the block exactly.
      if constexpr (SMALL) {
        if (small_sigma_out_of_range(tmax)) sigmoid_exact_block(p0, s_cur, c1, c0);
        tmax = 0;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) s_cur[0][r] = s_cur[1][r] = 0.0f;
    }
    ops[(g + 3) % 4] = read(std::integral_constant<int, g + 3>{});
    const bf16x8 op = ops[g % 4];
    if constexpr (g < KS) {
      s_nxt[0] = mfma32(op, qf[0][g], s_nxt[0]);
      s_nxt[1] = mfma32(op, qf[1][g], s_nxt[1]);
    } else if constexpr (g < NSTEP) {
      constexpr int i = g - KS, db = i >> 1, ks = i & 1;
      oacc[0][db] = mfma32(p1[0][ks], op, oacc[0][db]);
      oacc[1][db] = mfma32(p1[1][ks], op, oacc[1][db]);
    } else if constexpr (g < NSTEP + NB2) {
      constexpr int i = g - NSTEP, db = i >> 1, ks = i & 1;
      oacc[0][db] = mfma32(p0[0][ks], op, oacc[0][db]);
      oacc[1][db] = mfma32(p0[1][ks], op, oacc[1][db]);
    } else {
      constexpr int s = g - NSTEP - NB2;
      s_cur[0] = mfma32(op, qf[0][s], s_cur[0]);
      s_cur[1] = mfma32(op, qf[1][s], s_cur[1]);
    }
    // sigma: phase A turns S(t, 1st half) into p0 over steps 1..NSTEP-1,
    // phase B turns S(t, 2nd half) into p1 over steps 0..NSTEP-1.
    constexpr int e0 = g < NSTEP ? (g == 0 ? 0 : (g - 1) * 32 / (NSTEP - 1)) : (g - NSTEP) * 32 / NSTEP;
    constexpr int e1 = g < NSTEP ? (g == 0 ? 0 : g * 32 / (NSTEP - 1)) : (g - NSTEP + 1) * 32 / NSTEP;
    static_for<e0, e1>([&](auto ec) {
      constexpr int e = decltype(ec)::value, qb = e >> 4, r = e & 15;
      if constexpr (g < NSTEP)
        p0[qb][r >> 3][r & 7] = (__bf16)sigmoid_pass<SMALL>(s_cur[qb][r], c1, c0, tmax);
      else
        p1[qb][r >> 3][r & 7] = (__bf16)sigmoid_pass<SMALL>(s_nxt[qb][r], c1, c0, tmax);
    });
    // P(t, 2nd half) is complete at the last step of phase B, and its scores
    // are intact until the next phase starts: the same check and recomputation.
    if constexpr (SMALL && g == G - 1) {
      if (small_sigma_out_of_range(tmax)) sigmoid_exact_block(p1, s_nxt, c1, c0);
      tmax = 0;
    }
    constexpr bool dma_here = g >= NSTEP && (g - NSTEP) % DSTRIDE == 0 && (g - NSTEP) / DSTRIDE < NDMA;
    if constexpr (dma_here) {
      dma_chunk((g - NSTEP) / DSTRIDE);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // the DMA first in its step
    }
    // At D = 128 the compiler's own order beats the step groups and fences
    // now that every LDS operand address is a base register plus an
    // immediate: without them 1.91 -> 1.82 ms (nopad16k). At D = 64 they
    // stay (within 1% either way).
    if constexpr (D != 128) sched_step<g, reads_of(g + 3), 2, (SMALL ? 4 : 5) * (e1 - e0), 2>();
  });
}

// Forward. Each wave owns 64 query rows. The key loop is software-pipelined in
// half-tiles (32 keys) so that the MFMAs of one half-tile run beside the sigma
// of another (fwd_steps). The LDS ring holds tiles t-1, t and t+1, and there is
// one barrier per key tile. K and V come straight from global memory into LDS
// by DMA, with padded key rows replaced by zeros on the way. Each ring slot is
// its own LDS variable and the key loop is unrolled by three, so every access
// names its slot at compile time; the compiler then sees that the reads after
// the barrier cannot touch the slot the DMA is filling and does not wait for
// the DMA before them.
//
// Exactly the key tiles below n_k are computed, each once: the prologue takes
// tile 0's scores, each loop body one more tile, and the epilogue finishes the
// last tile's P V. Tile t sits in slot t mod 3. tile_counts receives the
// number of key tiles whose scores this workgroup computed.
template <int D, bool SMALL>
__global__ __launch_bounds__(256, kWavesPerSimd<D>) void fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                       const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                                       SeqLayout sl, int Z, int H, float c1, float c0_base,
                                                       int32_t* __restrict__ tile_counts) {
  using C = FwdCfg<D>;
  static_assert(C::NBUF == 3, "the key loop is unrolled over a ring of three slots");
  __shared__ __attribute__((aligned(1024))) __bf16 sK0[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sK1[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sK2[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV2[C::TILE];

  __shared__ RankLds rank_lds;
  __shared__ int vote;  // a wave's first block left the one-transcendental range
  const int n_qt = (sl.L + C::BQ - 1) / C::BQ;
  const TileCoord tc = schedule_tile(blockIdx.x, Z, H, n_qt, sl, rank_lds);
  const int z = tc.z, h = tc.h, m = tc.m;
  const int nq = sl.nq(z);
  const int nk = sl.nk(z);
  const float c0 = sl.c0_for(c0_base, nk);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)H * D;
  const size_t base = (sl.row0_q(z) * H + h) * D;    // Q and O
  const size_t base_k = (sl.row0_k(z) * H + h) * D;  // K and V
  const int rows = sl.rows(nq);                       // rows of this sample in O
  __bf16* Ob = O + base;
  const int q0 = m * C::BQ;

  if (q0 >= nq) {  // wholly padded query tile: write zeros, skip all work
    const int rows_here = min(C::BQ, rows - q0);
    const bf16x8 zz = zero_bf16x8();
    for (int c = tid; c < rows_here * (D / 8); c += 256)
      *(bf16x8*)(Ob + (size_t)(q0 + c / (D / 8)) * rs + (c % (D / 8)) * 8) = zz;
    if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = 0;
    return;
  }

  // Q as the B operand of S^T = K Q^T: query row q0 + 64w + 32qb + l32, d = 16s + 8*half + 0..7.
  bf16x8 qf[2][C::KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qr = q0 + 64 * w + 32 * qb + l32;
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      qf[qb][s] = (qr < nq) ? *(const bf16x8*)(Q + base + (size_t)qr * rs + 16 * s + 8 * half) : zero_bf16x8();
  }
  f32x16 oacc[2][C::NB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < C::NB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.0f;

  const int nkt = (nk + C::BK - 1) / C::BK;  // live key tiles; no other tile is computed
  int executed = 0;                          // key tiles whose scores this workgroup computed
  if (nkt > 0) {
    const uint32_t row_bytes = (uint32_t)(rs * 2);
    const __bf16* Kb = K + base_k;
    const __bf16* Vb = V + base_k;
    auto fetch = [&](__bf16* sk, __bf16* sv, int tile) {  // DMA key tile `tile` into one slot
      const int k0 = tile * C::BK;
      const size_t off = (size_t)(k0 < nk ? k0 : 0) * rs;  // no row is read past n_k
      dma_tile<D, C::BK, 256>(sk, Kb + off, row_bytes, nk - k0, tid);
      dma_tile<D, C::BK, 256>(sv, Vb + off, row_bytes, nk - k0, tid);
    };
    // A launch allowed the one-transcendental form (SMALL) takes it in a
    // workgroup only if the scores of every wave's 64 queries against keys
    // 0 .. 31 lie well inside the form's range (t <= 2^-6), tested on K tile
    // 0 before the key loop. Inputs whose scores leave the range (large norms) show it at
    // once, and the workgroup then runs the exact form throughout instead of
    // computing most blocks twice. Either way each block is checked before
    // use. The decision is the workgroup's (a vote in LDS), so all waves run
    // the same loop.
    bool small_wg = false;
    if constexpr (SMALL) {
      if (tid == 0) vote = 0;
      dma_tile<D, C::BK, 256>(sK0, Kb, row_bytes, nk, tid);
      dma_wait();
      __syncthreads();
      f32x16 probe[2];
      scores_t<D>(probe, sK0, 0, qf, l32, half);
      float ymax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 32; ++e) ymax = fmaxf(ymax, __builtin_fmaf(probe[e >> 4][e & 15], -c1, -c0));
      if (!(ymax <= -6.0f)) vote = 1;
      __syncthreads();
      small_wg = __builtin_amdgcn_readfirstlane(vote) == 0;
    }
    // The key loop, with one form of sigma or the other.
    auto run = [&](auto sm_c) {
      constexpr bool SM = decltype(sm_c)::value;
      // Tile t sits in slot t mod 3. (Tile 0's K may be in slot 0 already,
      // read by the test above before the last barrier; it is written again
      // with the same bytes.)
      fetch(sK0, sV0, 0);
      if (nkt > 1) fetch(sK1, sV1, 1);
      dma_wait();
      __syncthreads();

      f32x16 s_cur[2], s_nxt[2];
      bf16x8 p0[2][2], p1[2][2], ops[4];
      uint32_t tmax = 0;  // the largest t = e^S of the current half-tile (one-transcendental form)
      // Prologue: S(0, 1st half), then S(0, 2nd half) beside P(0, 1st half) = sigma(S).
      scores_t<D>(s_cur, sK0, 0, qf, l32, half);
      scores_t<D>(s_nxt, sK0, 1, qf, l32, half);
#pragma unroll
      for (int e = 0; e < 32; ++e)
        p0[e >> 4][(e & 15) >> 3][e & 7] = (__bf16)sigmoid_pass<SM>(s_cur[e >> 4][e & 15], c1, c0, tmax);
      interleave_mfma_valu<2 * C::KS, 10>();
      // the operands of phase B's first three steps: V of tile 0, 1st half
#pragma unroll
      for (int i = 0; i < 3; ++i) ops[(2 * C::KS + 2 * C::NB + i) % 4] = lds_tr<D>(sV0, (i & 1) * 16, (i >> 1) * 32, lane);
      executed = 1;

      // Loop body for tile t in slot T (tile t-1 in slot P, tile t+1 in slot N):
      // phase B of tile t, then phase A of tile t+1. Phase B starts tile t+2's
      // DMA into slot P (every wave has finished with tile t-1 at the barrier).
      // The DMA of a tile past n_k (t + 2 = nkt) has no row in range and fills
      // its slot with zeros, which nothing reads.
      auto body = [&](auto t_c, auto p_c, auto n_c, int t) {
        constexpr int T = decltype(t_c)::value, P = decltype(p_c)::value, N = decltype(n_c)::value;
        constexpr int KS = C::KS, NSTEP = KS + 2 * C::NB, G = 2 * NSTEP;
        auto dma_chunk = [&](int i) {
          constexpr int NC = kDmaChunks<D, C::BK, 256>;
          const int k0 = (t + 2) * C::BK;
          const size_t off = (size_t)(k0 < nk ? k0 : 0) * rs;  // no row is read past n_k
          if (i < NC)
            dma_tile_chunk<D, C::BK, 256>(ring<P>(sK0, sK1, sK2), Kb + off, row_bytes, nk - k0, tid, i);
          else
            dma_tile_chunk<D, C::BK, 256>(ring<P>(sV0, sV1, sV2), Vb + off, row_bytes, nk - k0, tid, i - NC);
        };
        auto at_barrier = [&] {
          dma_wait();       // this wave's DMA of tile t+1 has landed
          __syncthreads();  // ... everyone's has, and every wave is done with slot P
        };
        auto none = [](int) {};
        auto no_barrier = [] {};
        fwd_steps<D, NSTEP, G, SM>(ring<T>(sK0, sK1, sK2), ring<P>(sV0, sV1, sV2), ring<T>(sV0, sV1, sV2),
                                      ring<N>(sK0, sK1, sK2), s_cur, s_nxt, oacc, p0, p1, ops, qf, c1, c0, tmax, l32,
                                      half, lane, at_barrier, dma_chunk);
        fwd_steps<D, 0, NSTEP, SM>(ring<N>(sK0, sK1, sK2), ring<T>(sV0, sV1, sV2), ring<N>(sV0, sV1, sV2),
                                      ring<P>(sK0, sK1, sK2), s_cur, s_nxt, oacc, p0, p1, ops, qf, c1, c0, tmax, l32,
                                      half, lane, no_barrier, none);
        ++executed;
      };
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      // Bodies for tiles 0 .. nkt-2: whole rounds of three (slots 0, 1, 2), then
      // the one or two left over. The compiler keeps the three-body loop as free
      // of spills as the earlier form (a loop entered or left in the middle of a
      // round spilled up to 388 registers); the leftover bodies and the epilogue
      // sit after it.
      const int nb = nkt - 1, nb3 = nb / 3 * 3;
      for (int t = 0; t < nb3; t += 3) {
        body(I0{}, I2{}, I1{}, t);
        body(I1{}, I0{}, I2{}, t + 1);
        body(I2{}, I1{}, I0{}, t + 2);
      }
      if (nb3 < nb) body(I0{}, I2{}, I1{}, nb3);
      if (nb3 + 1 < nb) body(I1{}, I0{}, I2{}, nb3 + 1);
      // Epilogue, the last tile (slot nb mod 3): P(1st half) V beside
      // P(2nd half) = sigma(S), then P(2nd half) V.
      const int last = nb - nb3;
      const __bf16* vL = last == 0 ? sV0 : (last == 1 ? sV1 : sV2);
      // P(last, 1st half) meets no barrier before its use: the check here.
      if constexpr (SM) {
        if (small_sigma_out_of_range(tmax)) sigmoid_exact_block(p0, s_cur, c1, c0);
        tmax = 0;
      }
      accumulate_pv<D>(oacc, p0, vL, 0, lane);
#pragma unroll
      for (int e = 0; e < 32; ++e)
        p1[e >> 4][(e & 15) >> 3][e & 7] = (__bf16)sigmoid_pass<SM>(s_nxt[e >> 4][e & 15], c1, c0, tmax);
      interleave_mfma_valu<2 * C::NB * 2, 10>();
      if constexpr (SM) {
        if (small_sigma_out_of_range(tmax)) sigmoid_exact_block(p1, s_nxt, c1, c0);
      }
      accumulate_pv<D>(oacc, p1, vL, 1, lane);
      dma_wait();  // the last body's DMA (all zeros) must not outlive the kernel
    };
    if constexpr (SMALL) {
      if (small_wg) run(std::true_type{});
      else run(std::false_type{});
    } else {
      run(std::false_type{});
    }
  }

  // Epilogue. Register r of oacc[qb][db] holds query row 64w + 32qb + acc_row(r, half), column 32db + l%32.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < C::NB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = q0 + 64 * w + 32 * qb + acc_row(r, half);
        if (row < rows) Ob[(size_t)row * rs + db * 32 + l32] = (__bf16)(row < nq ? oacc[qb][db][r] : 0.0f);
      }
  if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = executed;
}

// ---------------------------------------------------------------------------------------------
// fp32 validation forward: scalar fp32 arithmetic, one thread per query row.
// The tile logic is the same (BQ = 64 rows per workgroup, BK = 32 keys per LDS tile).
template <int D>
__global__ __launch_bounds__(64) void fwd_fp32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      SeqLayout sl, int H, float c1, float c0_base,
                                                      int32_t* __restrict__ tile_counts) {
  constexpr int BQ = 64, BK = 32;
  __shared__ float sK[BK][D];
  __shared__ float sV[BK][D];
  const int n_qt = (sl.L + BQ - 1) / BQ;
  int bid = blockIdx.x;
  const int m = bid % n_qt;
  bid /= n_qt;
  const int h = bid % H;
  const int z = bid / H;
  const int nq = sl.nq(z);
  const int nk = sl.nk(z);
  const float c0 = sl.c0_for(c0_base, nk);
  const size_t rs = (size_t)H * D;
  const size_t base = (sl.row0_q(z) * H + h) * D;
  const size_t base_k = (sl.row0_k(z) * H + h) * D;
  const int rows = sl.rows(nq);
  const int tid = threadIdx.x;
  const int q0 = m * BQ;
  const int row = q0 + tid;
  if (q0 >= nq) {
    if (row < rows)
      for (int d = 0; d < D; ++d) O[base + (size_t)row * rs + d] = 0.0f;
    if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = 0;
    return;
  }
  float q[D], o[D];
  const bool live = row < nq;
  for (int d = 0; d < D; ++d) {
    q[d] = live ? Q[base + (size_t)row * rs + d] : 0.0f;
    o[d] = 0.0f;
  }
  const int nkt = (nk + BK - 1) / BK;
  for (int t = 0; t < nkt; ++t) {
    for (int c = tid; c < BK * D; c += 64) {
      const int r = c / D, d = c % D, kr = t * BK + r;
      sK[r][d] = kr < nk ? K[base_k + (size_t)kr * rs + d] : 0.0f;
      sV[r][d] = kr < nk ? V[base_k + (size_t)kr * rs + d] : 0.0f;
    }
    __syncthreads();
    for (int j = 0; j < BK; ++j) {
      float s = 0.0f;
      for (int d = 0; d < D; ++d) s = __builtin_fmaf(q[d], sK[j][d], s);
      const float p = sigmoid_dot(s, c1, c0);
      for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, sV[j][d], o[d]);
    }
    __syncthreads();
  }
  if (row < rows)
    for (int d = 0; d < D; ++d) O[base + (size_t)row * rs + d] = live ? o[d] : 0.0f;
  if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = nkt;
}

// Launchers (called from api.hip). They return the hipError_t of the launch.
template <int D>
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, SeqLayout sl, int Z, int H,
                           float c1, float c0, int32_t* tc, hipStream_t st) {
  using C = FwdCfg<D>;
  const long long blocks = (long long)Z * H * ((sl.L + C::BQ - 1) / C::BQ);
  if (use_small_sigma(c0, sl.bias_per_sample))
    hipLaunchKernelGGL((fwd_bf16_kernel<D, true>), dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (__bf16*)o, sl, Z, H, c1, c0, tc);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, false>), dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (__bf16*)o, sl, Z, H, c1, c0, tc);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_fp32(const void* q, const void* k, const void* v, void* o, SeqLayout sl, int Z, int H,
                           float c1, float c0, int32_t* tc, hipStream_t st) {
  const long long blocks = (long long)Z * H * ((sl.L + 63) / 64);
  hipLaunchKernelGGL(fwd_fp32_kernel<D>, dim3((unsigned)blocks), dim3(64), 0, st, (const float*)q, (const float*)k,
                     (const float*)v, (float*)o, sl, H, c1, c0, tc);
  return hipGetLastError();
}

#define SIGATTN_INST_FWD(NAME, D) \
  template hipError_t NAME<D>(const void*, const void*, const void*, void*, SeqLayout, int, int, float, float, \
                              int32_t*, hipStream_t);
SIGATTN_INST_FWD(launch_fwd_bf16, 64)
SIGATTN_INST_FWD(launch_fwd_bf16, 128)
SIGATTN_INST_FWD(launch_fwd_fp32, 64)
SIGATTN_INST_FWD(launch_fwd_fp32, 128)

}  // namespace sigattn
