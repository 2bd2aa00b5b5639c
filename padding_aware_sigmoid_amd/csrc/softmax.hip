// Padding-aware softmax attention: the forward, and the row sums the backward
// needs. The backward's dQ and dK/dV kernels are the sigmoid path's, with the
// softmax element function (bwd.hip).
//
// Method: attention weights are the softmax over keys of the scaled scores,
// softmax(a)_i = e^{a_i} / sum_j e^{a_j} (rainbus.top summary of
// arXiv:2604.27124, section "前置知识", entries "自注意力机制" and
// "Softmax 归一化"), with the padding-aware kernel design carried over from
// sigmoid attention (same summary, "未来方向"): keys j >= n_k take no part,
// query rows i >= n_q are written 0, wholly padded tiles are skipped.
//
// Outputs: O, and the row log-sum-exp LSE_i = log sum_j e^{alpha q_i.k_j}
// (natural log, fp32, one value per query row and head, laid out like Q
// without D). A row with no key has O = 0 and LSE = 0.
//
// CDNA4 design (bf16 forward):
//  - The sigmoid forward's tiles, waves, LDS ring, DMA and step schedule.
//  - Scores S^T = K Q^T as there, so each lane holds 16 keys of one query:
//    the row maximum and the row sum are lane-local, plus one exchange with
//    the lane 32 apart that holds the other 16 keys.
//  - O is accumulated transposed, O^T += V^T P^T (A = V through the
//    transposed LDS read, B = P from registers), so each lane also holds O^T
//    values of its own query only: rescaling O needs no exchange.
//  - Running maxima are lazy: P = 2^(c s - m) with m the row's reference
//    maximum; only when a lane sees a score above m + 8 (log2 units) does
//    the wave rescale O^T and the row sum and move m. So P <= 2^8 always,
//    and after the first tiles rescales are rare.
//  - The row sum adds the bf16 P values that enter the MFMA (v_dot2 against
//    (1, 1)), so the weights are normalised exactly as they are applied.
//  - Keys at or past n_k are masked to -1e30 before the maximum.
#include <algorithm>

#include "common.hpp"

namespace sigattn {

constexpr float kRescaleLog2 = 8.0f;  // lazy rescale threshold, log2 units
constexpr float kMasked = -1e30f;     // score of a key at or past n_k

// -------------------------------------------------------------------------------------- bf16 forward
// The forward's tiles: 4 waves of 64 query rows, 64-key LDS tiles in a ring of three.
template <int D>
struct SmCfg {
  static constexpr int BQ = 256;         // query rows per workgroup
  static constexpr int BK = 64;          // keys per LDS tile
  static constexpr int KS = D / 16;      // MFMA k-steps over the head dim
  static constexpr int NB = D / 32;      // 32-wide blocks of the head dim
  static constexpr int TILE = BK * D;    // elements of one K (or V) tile in LDS
};

// Softmax of one 32-key block for one 32-query block (16 keys per lane):
// mask, lane-local maximum, lazy rescale of (oT, lsum, m) when needed, then
// P = 2^(c1 s - m) packed as the B operand of the P V MFMA and added into lsum.
template <int D>
__device__ __forceinline__ void softmax_block_max(const f32x16& s, float& mx) {
  float a = fmaxf(fmaxf(s[0], s[1]), s[2]);
  float b = fmaxf(fmaxf(s[3], s[4]), s[5]);
  float c = fmaxf(fmaxf(s[6], s[7]), s[8]);
  float d = fmaxf(fmaxf(s[9], s[10]), s[11]);
  float e = fmaxf(fmaxf(s[12], s[13]), s[14]);
  mx = fmaxf(fmaxf(fmaxf(a, b), fmaxf(c, d)), fmaxf(e, s[15]));
}

// Lazy rescale before a block's exponentials. The reference maximum m is an
// integer (log2 units), so the rescale factor f = 2^(m_old - m_new) is a power
// of two and scales O^T, the row sum and the pending P block exactly. The
// pending block (HAS_PENDING) is the previous block's P, already added into
// lsum but not yet into O^T (its P V MFMAs run after this point in the
// schedule): it is brought to the new m with the rest. Without that, a block
// whose maximum rises more than kRescaleLog2 above m would add the previous
// block's P V at the old scale.
template <int D, bool HAS_PENDING>
__device__ __forceinline__ void softmax_rescale_if_needed(f32x16 (&s)[2], f32x16 (&oT)[2][SmCfg<D>::NB],
                                                          float (&m)[2], float (&lsum)[2], bf16x8 (&pending)[2][2],
                                                          float c1, int key0, int nk, int half) {
  // mask keys >= n_k. Register r of lane l holds key key0 + (r/4)*8 + 4*half + r%4.
  if (key0 + 32 > nk) {
    const int lim = nk - key0 - 4 * half;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool ok = ((r >> 2) * 8 + (r & 3)) < lim;
      s[0][r] = ok ? s[0][r] : kMasked;
      s[1][r] = ok ? s[1][r] : kMasked;
    }
  }
  float mc[2];
  bool need = false;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    softmax_block_max<D>(s[qb], mc[qb]);
    mc[qb] *= c1;
    need |= mc[qb] > m[qb] + kRescaleLog2;
  }
  if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mp = fmaxf(mc[qb], __shfl_xor(mc[qb], 32));
      const float mn = fmaxf(m[qb], __builtin_ceilf(mp));
      const float f = __builtin_amdgcn_exp2f(m[qb] - mn);  // 0 when m was -inf; else 2^-k, k a whole number
      lsum[qb] *= f;
#pragma unroll
      for (int db = 0; db < SmCfg<D>::NB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oT[qb][db][r] *= f;
      if constexpr (HAS_PENDING) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int j = 0; j < 8; ++j) pending[qb][ks][j] = (__bf16)((float)pending[qb][ks][j] * f);
      }
      m[qb] = mn;
    }
  }
}

// P = 2^(c1 s - m) for element e (0..31: qb = e/16, r = e%16), packed into p and summed into lsum.
__device__ __forceinline__ void softmax_elem(bf16x8 (&p)[2][2], float (&lsum)[2], const f32x16 (&s)[2],
                                             const float (&m)[2], float c1, int e) {
  const int qb = e >> 4, r = e & 15;
  p[qb][r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(__builtin_fmaf(s[qb][r], c1, -m[qb]));
  if (e & 1) {  // every second element: add the bf16 pair just formed
    const bf16x2 pr = {p[qb][r >> 3][(r & 7) - 1], p[qb][r >> 3][r & 7]};
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    lsum[qb] = __builtin_amdgcn_fdot2_f32_bf16(pr, one, lsum[qb], false);
  }
}

// The forward of one wave, in the sigmoid forward's step schedule. Key tile t
// is two phases:
//   phase A: S(t, 2nd half) (KS steps), then O^T += V(t-1, 2nd half)^T P (2*NB steps)
//            || P(t, 1st half) = softmax part of S(t, 1st half)
//   barrier
//   phase B: O^T += V(t, 1st half)^T P (2*NB steps), then S(t+1, 1st half) (KS steps)
//            || P(t, 2nd half) = softmax part of S(t, 2nd half)
// Each phase first takes its block's maximum (and rescales if needed, the
// other phase's pending P included); the exponentials are then spread over
// the steps. sm_steps runs steps [G0, G1) of one tile's stream; the key loop
// runs phase B of tile t, then phase A of tile t+1. key_t is tile t's first key.
template <int D, int G0, int G1, typename AtBarrier, typename DmaChunk>
__device__ __forceinline__ void sm_steps(const __bf16* kT, const __bf16* vP, const __bf16* vT, const __bf16* kN,
                                         f32x16 (&s_cur)[2], f32x16 (&s_nxt)[2], f32x16 (&oT)[2][SmCfg<D>::NB],
                                         bf16x8 (&p0)[2][2], bf16x8 (&p1)[2][2], float (&m)[2], float (&lsum)[2],
                                         bf16x8 (&ops)[4], const bf16x8 (&qf)[2][SmCfg<D>::KS], float c1, int key_t,
                                         int nk, int l32, int half, int lane, AtBarrier&& at_barrier,
                                         DmaChunk&& dma_chunk) {
  using C = SmCfg<D>;
  constexpr int KS = C::KS, NB2 = 2 * C::NB;
  constexpr int NSTEP = KS + NB2;
  constexpr int G = 2 * NSTEP;
  static_assert(0 <= G0 && G0 < G1 && G1 <= G, "a step range of one tile");
  constexpr int NDMA = 2 * kDmaChunks<D, C::BK, 256>;
  constexpr int DSTRIDE = NSTEP / NDMA > 0 ? NSTEP / NDMA : 1;
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
  auto reads_of = [](int g) constexpr -> int {
    const int h = g % G;
    return (h < KS || h >= NSTEP + NB2) ? 1 : 2;
  };
  static_for<G0, G1>([&](auto gc) {
    constexpr int g = decltype(gc)::value;
    if constexpr (g == 0) {
      // phase A's block: S(t, 1st half), keys key_t .. key_t + 31; p1 (tile
      // t-1, 2nd half) is still to be added into O^T
      softmax_rescale_if_needed<D, true>(s_cur, oT, m, lsum, p1, c1, key_t, nk, half);
#pragma unroll
      for (int r = 0; r < 16; ++r) s_nxt[0][r] = s_nxt[1][r] = 0.0f;
    }
    if constexpr (g == NSTEP) {
      pin_before_barrier(p0);
      at_barrier();
      // phase B's block: S(t, 2nd half), keys key_t + 32 .. key_t + 63; p0 is pending
      softmax_rescale_if_needed<D, true>(s_nxt, oT, m, lsum, p0, c1, key_t + 32, nk, half);
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
      oT[0][db] = mfma32(op, p1[0][ks], oT[0][db]);
      oT[1][db] = mfma32(op, p1[1][ks], oT[1][db]);
    } else if constexpr (g < NSTEP + NB2) {
      constexpr int i = g - NSTEP, db = i >> 1, ks = i & 1;
      oT[0][db] = mfma32(op, p0[0][ks], oT[0][db]);
      oT[1][db] = mfma32(op, p0[1][ks], oT[1][db]);
    } else {
      constexpr int s = g - NSTEP - NB2;
      s_cur[0] = mfma32(op, qf[0][s], s_cur[0]);
      s_cur[1] = mfma32(op, qf[1][s], s_cur[1]);
    }
    constexpr int e0 = (g % NSTEP) * 32 / NSTEP, e1 = (g % NSTEP + 1) * 32 / NSTEP;
    static_for<e0, e1>([&](auto ec) {
      constexpr int e = decltype(ec)::value;
      if constexpr (g < NSTEP)
        softmax_elem(p0, lsum, s_cur, m, c1, e);
      else
        softmax_elem(p1, lsum, s_nxt, m, c1, e);
    });
    constexpr bool dma_here = g >= NSTEP && (g - NSTEP) % DSTRIDE == 0 && (g - NSTEP) / DSTRIDE < NDMA;
    if constexpr (dma_here) {
      dma_chunk((g - NSTEP) / DSTRIDE);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    sched_step<g, reads_of(g + 3), 2, 4 * (e1 - e0), 2>();
  });
}

// O^T += V(kb)^T P for the last half tile.
template <int D>
__device__ __forceinline__ void sm_accumulate_pv(f32x16 (&oT)[2][SmCfg<D>::NB], const bf16x8 (&p)[2][2],
                                                 const __bf16* sV, int kb, int lane) {
#pragma unroll
  for (int db = 0; db < SmCfg<D>::NB; ++db)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8 a = lds_tr<D>(sV, kb * 32 + ks * 16, db * 32, lane);
      oT[0][db] = mfma32(a, p[0][ks], oT[0][db]);
      oT[1][db] = mfma32(a, p[1][ks], oT[1][db]);
    }
}

template <int D>
__global__ __launch_bounds__(256, kWavesPerSimd<D>) void sm_fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                          const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                                          float* __restrict__ LSE, SeqLayout sl, int Z, int H,
                                                          float c1) {
  using C = SmCfg<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 sK0[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sK1[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sK2[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV2[C::TILE];
  __shared__ RankLds rank_lds;
  const int n_qt = (sl.L + C::BQ - 1) / C::BQ;
  const TileCoord tc = schedule_tile(blockIdx.x, Z, H, n_qt, sl, rank_lds);
  const int z = tc.z, h = tc.h, m0 = tc.m;
  const int nq = sl.nq(z), nk = sl.nk(z);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)H * D;
  const size_t base = (sl.row0_q(z) * H + h) * D;
  const size_t base_k = (sl.row0_k(z) * H + h) * D;
  const size_t lbase = sl.row0_q(z) * H + h;  // LSE[row * H + h]
  const int rows = sl.rows(nq);
  __bf16* Ob = O + base;
  const int q0 = m0 * C::BQ;

  if (q0 >= nq) {
    const int rows_here = min(C::BQ, rows - q0);
    const bf16x8 zz = zero_bf16x8();
    for (int c = tid; c < rows_here * (D / 8); c += 256)
      *(bf16x8*)(Ob + (size_t)(q0 + c / (D / 8)) * rs + (c % (D / 8)) * 8) = zz;
    for (int r = tid; r < rows_here; r += 256) LSE[lbase + (size_t)(q0 + r) * H] = 0.0f;
    return;
  }

  bf16x8 qf[2][C::KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qr = q0 + 64 * w + 32 * qb + l32;
#pragma unroll
    for (int s = 0; s < C::KS; ++s)
      qf[qb][s] = (qr < nq) ? *(const bf16x8*)(Q + base + (size_t)qr * rs + 16 * s + 8 * half) : zero_bf16x8();
  }
  f32x16 oT[2][C::NB];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < C::NB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oT[qb][db][r] = 0.0f;
  float m[2] = {-__builtin_inff(), -__builtin_inff()}, lsum[2] = {0.0f, 0.0f};

  // Exactly the key tiles below n_k are computed, each once, as in the
  // sigmoid forward: tile 0's scores in the prologue, one more tile per loop
  // body (phase B of tile t, phase A of tile t+1), the last tile's P V in the
  // epilogue. Tile t sits in slot t mod 3.
  const int nkt = (nk + C::BK - 1) / C::BK;
  if (nkt > 0) {
    const uint32_t row_bytes = (uint32_t)(rs * 2);
    const __bf16* Kb = K + base_k;
    const __bf16* Vb = V + base_k;
    auto fetch = [&](__bf16* sk, __bf16* sv, int tile) {
      const int k0 = tile * C::BK;
      const size_t off = (size_t)(k0 < nk ? k0 : 0) * rs;
      dma_tile<D, C::BK, 256>(sk, Kb + off, row_bytes, nk - k0, tid);
      dma_tile<D, C::BK, 256>(sv, Vb + off, row_bytes, nk - k0, tid);
    };
    fetch(sK0, sV0, 0);
    if (nkt > 1) fetch(sK1, sV1, 1);
    dma_wait();
    __syncthreads();

    f32x16 s_cur[2], s_nxt[2];
    bf16x8 p0[2][2], p1[2][2], ops[4];
    // Prologue: S(0, 1st half) and S(0, 2nd half) = K Q^T, then P(0, 1st half).
#pragma unroll
    for (int r = 0; r < 16; ++r) s_cur[0][r] = s_cur[1][r] = s_nxt[0][r] = s_nxt[1][r] = 0.0f;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const bf16x8 a = lds_nat<D>(sK0, l32, 2 * s + half);
      s_cur[0] = mfma32(a, qf[0][s], s_cur[0]);
      s_cur[1] = mfma32(a, qf[1][s], s_cur[1]);
    }
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const bf16x8 a = lds_nat<D>(sK0, 32 + l32, 2 * s + half);
      s_nxt[0] = mfma32(a, qf[0][s], s_nxt[0]);
      s_nxt[1] = mfma32(a, qf[1][s], s_nxt[1]);
    }
    softmax_rescale_if_needed<D, false>(s_cur, oT, m, lsum, p1, c1, 0, nk, half);
#pragma unroll
    for (int e = 0; e < 32; ++e) softmax_elem(p0, lsum, s_cur, m, c1, e);
    // the operands of phase B's first three steps: V of tile 0, 1st half
#pragma unroll
    for (int i = 0; i < 3; ++i) ops[(2 * C::KS + 2 * C::NB + i) % 4] = lds_tr<D>(sV0, (i & 1) * 16, (i >> 1) * 32, lane);

    // Body for tile t in slot T (tile t-1 in slot P, which receives tile t+2;
    // tile t+1 in slot N). The DMA of a tile past n_k fills its slot with
    // zeros, which nothing reads.
    auto body = [&](auto t_c, auto p_c, auto n_c, int t) __attribute__((always_inline)) {
      constexpr int T = decltype(t_c)::value, P = decltype(p_c)::value, N = decltype(n_c)::value;
      constexpr int NSTEP = C::KS + 2 * C::NB, G = 2 * NSTEP;
      auto dma_chunk = [&](int i) {
        constexpr int NC = kDmaChunks<D, C::BK, 256>;
        const int k0 = (t + 2) * C::BK;
        const size_t off = (size_t)(k0 < nk ? k0 : 0) * rs;
        if (i < NC)
          dma_tile_chunk<D, C::BK, 256>(ring<P>(sK0, sK1, sK2), Kb + off, row_bytes, nk - k0, tid, i);
        else
          dma_tile_chunk<D, C::BK, 256>(ring<P>(sV0, sV1, sV2), Vb + off, row_bytes, nk - k0, tid, i - NC);
      };
      auto at_barrier = [&] {
        dma_wait();
        __syncthreads();
      };
      sm_steps<D, NSTEP, G>(ring<T>(sK0, sK1, sK2), ring<P>(sV0, sV1, sV2), ring<T>(sV0, sV1, sV2),
                            ring<N>(sK0, sK1, sK2), s_cur, s_nxt, oT, p0, p1, m, lsum, ops, qf, c1, t * C::BK, nk,
                            l32, half, lane, at_barrier, dma_chunk);
      sm_steps<D, 0, NSTEP>(ring<N>(sK0, sK1, sK2), ring<T>(sV0, sV1, sV2), ring<N>(sV0, sV1, sV2),
                            ring<P>(sK0, sK1, sK2), s_cur, s_nxt, oT, p0, p1, m, lsum, ops, qf, c1, (t + 1) * C::BK,
                            nk, l32, half, lane, [] {}, [](int) {});
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    // Whole rounds of three bodies, then the one or two left over (a loop
    // entered or left in the middle of a round spills heavily).
    const int nb = nkt - 1, nb3 = nb / 3 * 3;
    for (int t = 0; t < nb3; t += 3) {
      body(I0{}, I2{}, I1{}, t);
      body(I1{}, I0{}, I2{}, t + 1);
      body(I2{}, I1{}, I0{}, t + 2);
    }
    if (nb3 < nb) body(I0{}, I2{}, I1{}, nb3);
    if (nb3 + 1 < nb) body(I1{}, I0{}, I2{}, nb3 + 1);
    // Epilogue, the last tile (slot nb mod 3): phase B without the next
    // tile's scores, then the P V of its second half.
    const int last = nb - nb3;
    const __bf16* vL = last == 0 ? sV0 : (last == 1 ? sV1 : sV2);
    softmax_rescale_if_needed<D, true>(s_nxt, oT, m, lsum, p0, c1, nb * C::BK + 32, nk, half);
    sm_accumulate_pv<D>(oT, p0, vL, 0, lane);
#pragma unroll
    for (int e = 0; e < 32; ++e) softmax_elem(p1, lsum, s_nxt, m, c1, e);
    interleave_mfma_valu<2 * C::NB * 2, 8>();
    sm_accumulate_pv<D>(oT, p1, vL, 1, lane);
    dma_wait();  // the last body's DMA (all zeros) must not outlive the kernel
  }

  // Epilogue: combine the two half-lanes' row sums, normalise, store O and LSE.
  // oT[qb][db] register r holds d = 32 db + (r/4)*8 + 4 half + r%4 of query l32.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float ltot = lsum[qb] + __shfl_xor(lsum[qb], 32);
    const int row = q0 + 64 * w + 32 * qb + l32;
    const bool live = row < nq && ltot > 0.0f;
    const float inv = live ? __builtin_amdgcn_rcpf(ltot) : 0.0f;
    if (row < rows) {
#pragma unroll
      for (int db = 0; db < C::NB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bf16x4 v;
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = (__bf16)(oT[qb][db][4 * g4 + j] * inv);
          *(bf16x4*)(Ob + (size_t)row * rs + db * 32 + g4 * 8 + 4 * half) = v;
        }
      if (half == 0)
        LSE[lbase + (size_t)row * H] = live ? (m[qb] + __builtin_amdgcn_logf(ltot)) * 0.69314718055994531f : 0.0f;
    }
  }
}

// ------------------------------------------------------------------------------- backward row stats
// Per valid query row and head, the pair {LSE_i / alpha, D_i} with
// D_i = sum_d dO_id O_id (fp32). The backward kernels recompute
// P_ij = e^(alpha s_ij - LSE_i) = 2^(c1 (s_ij - LSE_i / alpha)) and form
// dS = P (dP - D). Padded rows get {0, 0}: their (zero) score rows give P = 1
// against dP = D = 0, so dS = 0.
// A group of D / VEC lanes takes one (row, head): each lane one 16-byte piece
// of O and of dO, so every load is coalesced; shuffles sum the group. The grid
// strides over the rows.
template <typename T, int D>
__global__ __launch_bounds__(256) void sm_rowstats_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                          const float* __restrict__ LSE, float2* __restrict__ stats,
                                                          SeqLayout sl, int Z, int H, float alpha) {
  constexpr int VEC = 16 / (int)sizeof(T), LP = D / VEC, PER_BLOCK = 256 / LP;
  const int sub = threadIdx.x % LP;
  const long long items = (long long)Z * sl.L * H;
  // Every lane of a group sees the same item, so whole groups skip together and
  // a shuffle partner (lane ^ m, m < LP) is always live.
  for (long long item = (long long)blockIdx.x * PER_BLOCK + threadIdx.x / LP; item < items;
       item += (long long)gridDim.x * PER_BLOCK) {
    const int h = (int)(item % H);
    const long long zi = item / H;
    const int z = (int)(zi / sl.L), i = (int)(zi % sl.L);
    const int nq = sl.nq(z);
    if (i >= sl.rows(nq)) continue;
    const size_t row = sl.row0_q(z) + i;
    float acc = 0.0f;
    if (i < nq) {
      const size_t off = (row * H + h) * D + (size_t)sub * VEC;
      if constexpr (sizeof(T) == 2) {
        const bf16x8 o = *(const bf16x8*)(O + off), g = *(const bf16x8*)(dO + off);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = __builtin_fmaf((float)o[j], (float)g[j], acc);
      } else {
        const float4 o = *(const float4*)(O + off), g = *(const float4*)(dO + off);
        acc = __builtin_fmaf(o.x, g.x, __builtin_fmaf(o.y, g.y, __builtin_fmaf(o.z, g.z, o.w * g.w)));
      }
    }
#pragma unroll
    for (int m = LP / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (sub == 0) stats[row * H + h] = make_float2(i < nq ? LSE[row * H + h] / alpha : 0.0f, acc);
  }
}

// -------------------------------------------------------------------------------------- fp32 backward
// Validation build. dQ: one thread per query row; dK/dV: one thread per key row.
// Both read the row stats {LSE log2 e, D} of every query they touch.
template <int D>
__global__ __launch_bounds__(64) void sm_dq_fp32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                        const float* __restrict__ V, const float* __restrict__ dO,
                                                        const float2* __restrict__ stats, float* __restrict__ dQ,
                                                        SeqLayout sl, int H, float alpha, float c1) {
  constexpr int BQ = 64, BK = 32;
  __shared__ float sK[BK][D];
  __shared__ float sV[BK][D];
  const int n_qt = (sl.L + BQ - 1) / BQ;
  int bid = blockIdx.x;
  const int mt = bid % n_qt;
  bid /= n_qt;
  const int h = bid % H, z = bid / H;
  const int nq = sl.nq(z), nk = sl.nk(z);
  const size_t rs = (size_t)H * D, base = (sl.row0_q(z) * H + h) * D, base_k = (sl.row0_k(z) * H + h) * D;
  const int rows = sl.rows(nq);
  const int tid = threadIdx.x, q0 = mt * BQ, row = q0 + tid;
  const bool live = row < nq;
  float q[D], g[D], acc[D];
  for (int d = 0; d < D; ++d) {
    q[d] = live ? Q[base + (size_t)row * rs + d] : 0.0f;
    g[d] = live ? dO[base + (size_t)row * rs + d] : 0.0f;
    acc[d] = 0.0f;
  }
  float2 st = live ? stats[(sl.row0_q(z) + row) * H + h] : make_float2(0.0f, 0.0f);
  st.x *= c1;  // LSE / alpha -> LSE log2 e
  const int nkt = q0 < nq ? (nk + BK - 1) / BK : 0;
  for (int t = 0; t < nkt; ++t) {
    for (int c = tid; c < BK * D; c += 64) {
      const int r = c / D, d = c % D, kr = t * BK + r;
      sK[r][d] = kr < nk ? K[base_k + (size_t)kr * rs + d] : 0.0f;
      sV[r][d] = kr < nk ? V[base_k + (size_t)kr * rs + d] : 0.0f;
    }
    __syncthreads();
    for (int j = 0; j < BK && t * BK + j < nk; ++j) {
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < D; ++d) {
        s = __builtin_fmaf(q[d], sK[j][d], s);
        dp = __builtin_fmaf(g[d], sV[j][d], dp);
      }
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s, c1, -st.x));
      const float ds = p * (dp - st.y);
      for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(ds, sK[j][d], acc[d]);
    }
    __syncthreads();
  }
  if (row < rows)
    for (int d = 0; d < D; ++d) dQ[base + (size_t)row * rs + d] = live ? alpha * acc[d] : 0.0f;
}

template <int D>
__global__ __launch_bounds__(64) void sm_dkdv_fp32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                          const float* __restrict__ V, const float* __restrict__ dO,
                                                          const float2* __restrict__ stats, float* __restrict__ dK,
                                                          float* __restrict__ dV, SeqLayout sl, int H, float alpha,
                                                          float c1) {
  constexpr int BK = 64, BQ = 32;
  __shared__ float sQ[BQ][D];
  __shared__ float sG[BQ][D];
  __shared__ float2 sSt[BQ];
  const int n_kt = (sl.L + BK - 1) / BK;
  int bid = blockIdx.x;
  const int t = bid % n_kt;
  bid /= n_kt;
  const int h = bid % H, z = bid / H;
  const int nq = sl.nq(z), nk = sl.nk(z);
  const size_t rs = (size_t)H * D, base = (sl.row0_k(z) * H + h) * D, base_q = (sl.row0_q(z) * H + h) * D;
  const size_t srow0 = sl.row0_q(z);
  const int rows = sl.rows(nk);
  const int tid = threadIdx.x, k0 = t * BK, row = k0 + tid;
  const bool live = row < nk;
  float kk[D], vv[D], dk[D], dv[D];
  for (int d = 0; d < D; ++d) {
    kk[d] = live ? K[base + (size_t)row * rs + d] : 0.0f;
    vv[d] = live ? V[base + (size_t)row * rs + d] : 0.0f;
    dk[d] = dv[d] = 0.0f;
  }
  const int nqt = k0 < nk ? (nq + BQ - 1) / BQ : 0;
  for (int u = 0; u < nqt; ++u) {
    for (int c = tid; c < BQ * D; c += 64) {
      const int r = c / D, d = c % D, qr = u * BQ + r;
      sQ[r][d] = qr < nq ? Q[base_q + (size_t)qr * rs + d] : 0.0f;
      sG[r][d] = qr < nq ? dO[base_q + (size_t)qr * rs + d] : 0.0f;
    }
    if (tid < BQ) {
      const int qr = u * BQ + tid;
      sSt[tid] = qr < nq ? stats[(srow0 + qr) * H + h] : make_float2(0.0f, 0.0f);
      sSt[tid].x *= c1;  // LSE / alpha -> LSE log2 e
    }
    __syncthreads();
    for (int i = 0; i < BQ && u * BQ + i < nq; ++i) {
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < D; ++d) {
        s = __builtin_fmaf(sQ[i][d], kk[d], s);
        dp = __builtin_fmaf(sG[i][d], vv[d], dp);
      }
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s, c1, -sSt[i].x));
      const float ds = p * (dp - sSt[i].y);
      for (int d = 0; d < D; ++d) {
        dv[d] = __builtin_fmaf(p, sG[i][d], dv[d]);
        dk[d] = __builtin_fmaf(ds, sQ[i][d], dk[d]);
      }
    }
    __syncthreads();
  }
  if (row < rows)
    for (int d = 0; d < D; ++d) {
      dK[base + (size_t)row * rs + d] = live ? alpha * dk[d] : 0.0f;
      dV[base + (size_t)row * rs + d] = live ? dv[d] : 0.0f;
    }
}

// -------------------------------------------------------------------------------------- fp32 forward
// Validation build: one thread per query row, online softmax in fp32.
template <int D>
__global__ __launch_bounds__(64) void sm_fwd_fp32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                         const float* __restrict__ V, float* __restrict__ O,
                                                         float* __restrict__ LSE, SeqLayout sl, int H, float c1) {
  constexpr int BQ = 64, BK = 32;
  __shared__ float sK[BK][D];
  __shared__ float sV[BK][D];
  const int n_qt = (sl.L + BQ - 1) / BQ;
  int bid = blockIdx.x;
  const int mt = bid % n_qt;
  bid /= n_qt;
  const int h = bid % H, z = bid / H;
  const int nq = sl.nq(z), nk = sl.nk(z);
  const size_t rs = (size_t)H * D, base = (sl.row0_q(z) * H + h) * D, base_k = (sl.row0_k(z) * H + h) * D;
  const size_t lbase = sl.row0_q(z) * H + h;
  const int rows = sl.rows(nq);
  const int tid = threadIdx.x, q0 = mt * BQ, row = q0 + tid;
  const bool live = row < nq;
  float q[D], o[D];
  for (int d = 0; d < D; ++d) {
    q[d] = live ? Q[base + (size_t)row * rs + d] : 0.0f;
    o[d] = 0.0f;
  }
  float m = -__builtin_inff(), l = 0.0f;
  const int nkt = q0 < nq ? (nk + BK - 1) / BK : 0;
  for (int t = 0; t < nkt; ++t) {
    for (int c = tid; c < BK * D; c += 64) {
      const int r = c / D, d = c % D, kr = t * BK + r;
      sK[r][d] = kr < nk ? K[base_k + (size_t)kr * rs + d] : 0.0f;
      sV[r][d] = kr < nk ? V[base_k + (size_t)kr * rs + d] : 0.0f;
    }
    __syncthreads();
    for (int j = 0; j < BK && t * BK + j < nk; ++j) {
      float s = 0.0f;
      for (int d = 0; d < D; ++d) s = __builtin_fmaf(q[d], sK[j][d], s);
      s *= c1;  // log2 units
      const float mn = fmaxf(m, s);
      const float f = __builtin_amdgcn_exp2f(m - mn), p = __builtin_amdgcn_exp2f(s - mn);
      l = l * f + p;
      for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(p, sV[j][d], o[d] * f);
      m = mn;
    }
    __syncthreads();
  }
  if (row < rows) {
    const bool ok = live && l > 0.0f;
    const float inv = ok ? 1.0f / l : 0.0f;
    for (int d = 0; d < D; ++d) O[base + (size_t)row * rs + d] = o[d] * inv;
    LSE[lbase + (size_t)row * H] = ok ? (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f : 0.0f;
  }
}

// ------------------------------------------------------------------------------------------ launchers
template <int D>
hipError_t launch_sm_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse, SeqLayout sl, int Z,
                              int H, float c1, hipStream_t st) {
  using C = SmCfg<D>;
  const long long blocks = (long long)Z * H * ((sl.L + C::BQ - 1) / C::BQ);
  hipLaunchKernelGGL(sm_fwd_bf16_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)q,
                     (const __bf16*)k, (const __bf16*)v, (__bf16*)o, lse, sl, Z, H, c1);
  return hipGetLastError();
}

template <int D>
hipError_t launch_sm_fwd_fp32(const void* q, const void* k, const void* v, void* o, float* lse, SeqLayout sl, int Z,
                              int H, float c1, hipStream_t st) {
  const long long blocks = (long long)Z * H * ((sl.L + 63) / 64);
  hipLaunchKernelGGL(sm_fwd_fp32_kernel<D>, dim3((unsigned)blocks), dim3(64), 0, st, (const float*)q,
                     (const float*)k, (const float*)v, (float*)o, lse, sl, H, c1);
  return hipGetLastError();
}

template <int D>
hipError_t launch_sm_rowstats(int bf16, const void* o, const void* dout, const float* lse, void* stats,
                              SeqLayout sl, int Z, int H, float alpha, hipStream_t st) {
  const long long items = (long long)Z * sl.L * H;
  const int per_block = bf16 ? 256 / (D / 8) : 256 / (D / 4);
  const unsigned blocks = (unsigned)std::min<long long>((items + per_block - 1) / per_block, 1 << 16);
  if (bf16)
    hipLaunchKernelGGL((sm_rowstats_kernel<__bf16, D>), dim3(blocks), dim3(256), 0, st, (const __bf16*)o,
                       (const __bf16*)dout, lse, (float2*)stats, sl, Z, H, alpha);
  else
    hipLaunchKernelGGL((sm_rowstats_kernel<float, D>), dim3(blocks), dim3(256), 0, st, (const float*)o,
                       (const float*)dout, lse, (float2*)stats, sl, Z, H, alpha);
  return hipGetLastError();
}

template <int D>
hipError_t launch_sm_bwd_fp32(const void* q, const void* k, const void* v, const void* dout, const void* stats,
                              void* dq, void* dk, void* dv, SeqLayout sl, int Z, int H, float alpha, float c1,
                              hipStream_t st) {
  const long long blocks = (long long)Z * H * ((sl.L + 63) / 64);
  hipLaunchKernelGGL(sm_dkdv_fp32_kernel<D>, dim3((unsigned)blocks), dim3(64), 0, st, (const float*)q,
                     (const float*)k, (const float*)v, (const float*)dout, (const float2*)stats, (float*)dk,
                     (float*)dv, sl, H, alpha, c1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sm_dq_fp32_kernel<D>, dim3((unsigned)blocks), dim3(64), 0, st, (const float*)q,
                     (const float*)k, (const float*)v, (const float*)dout, (const float2*)stats, (float*)dq, sl, H,
                     alpha, c1);
  return hipGetLastError();
}

#define SIGATTN_INST_SM(D)                                                                                      \
  template hipError_t launch_sm_fwd_bf16<D>(const void*, const void*, const void*, void*, float*, SeqLayout, int, \
                                            int, float, hipStream_t);                                          \
  template hipError_t launch_sm_fwd_fp32<D>(const void*, const void*, const void*, void*, float*, SeqLayout, int, \
                                            int, float, hipStream_t);                                          \
  template hipError_t launch_sm_rowstats<D>(int, const void*, const void*, const float*, void*, SeqLayout, int,  \
                                            int, float, hipStream_t);                                          \
  template hipError_t launch_sm_bwd_fp32<D>(const void*, const void*, const void*, const void*, const void*,    \
                                            void*, void*, void*, SeqLayout, int, int, float, float, hipStream_t);
SIGATTN_INST_SM(64)
SIGATTN_INST_SM(128)

}  // namespace sigattn
