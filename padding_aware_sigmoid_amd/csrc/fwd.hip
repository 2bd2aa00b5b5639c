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
//  - sigma takes one v_exp_f32 and one v_rcp_f32 per score.
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

// P = sigma(S) in registers, packed as the A operands (two k-steps of 16 keys) of P V.
__device__ __forceinline__ void sigma_pack(bf16x8 (&p)[2][2], const f32x16 (&sacc)[2], float c1, float c0) {
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int r = 0; r < 16; ++r) p[qb][r >> 3][r & 7] = (__bf16)sigmoid_dot(sacc[qb][r], c1, c0);
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

// One pipeline phase of the forward for one wave, written as a fixed step
// schedule. With one wave per SIMD, latency can only be hidden inside the
// wave's own instruction stream.
// The phase does three independent jobs:
//   S_out = K(kb_s) Q^T   (KS steps of 2 MFMAs; A operand = a K row chunk)
//   O += P_in V(kb_v)     (2*NB steps of 2 MFMAs; B operand = a V tr-read pair)
//   P_out = sigma(S_in)   (32 values per lane, spread evenly over the steps)
// The LDS operand of step j+2 is requested at step j (a 3-deep ring of
// operand registers). An MFMA therefore never waits on a read issued just
// before it, and the sigma work fills the MFMA pipe's busy cycles.
template <int D>
__device__ __forceinline__ void fwd_phase(f32x16 (&s_out)[2], const __bf16* sK, int kb_s,
                                          f32x16 (&oacc)[2][FwdCfg<D>::NB], const bf16x8 (&p_in)[2][2],
                                          const __bf16* sV, int kb_v, bf16x8 (&p_out)[2][2], const f32x16 (&s_in)[2],
                                          const bf16x8 (&qf)[2][FwdCfg<D>::KS], float c1, float c0, int l32,
                                          int half, int lane) {
  using C = FwdCfg<D>;
  constexpr int NSTEP = C::KS + 2 * C::NB;  // 16 at D = 128, 8 at D = 64
  constexpr int EPS = 32 / NSTEP;           // sigma values per step
  auto read = [&](auto jc) -> bf16x8 {
    constexpr int j = decltype(jc)::value;
    if constexpr (j < C::KS) {
      return lds_nat<D>(sK, kb_s * 32 + l32, 2 * j + half);
    } else {
      constexpr int i = j - C::KS;
      return lds_tr<D>(sV, kb_v * 32 + (i & 1) * 16, (i >> 1) * 32, lane);
    }
  };
#pragma unroll
  for (int r = 0; r < 16; ++r) s_out[0][r] = s_out[1][r] = 0.0f;
  bf16x8 ops[3];
  ops[0] = read(std::integral_constant<int, 0>{});
  ops[1] = read(std::integral_constant<int, 1>{});
  static_for<0, NSTEP>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if constexpr (j + 2 < NSTEP) ops[(j + 2) % 3] = read(std::integral_constant<int, j + 2>{});
    const bf16x8 op = ops[j % 3];
    if constexpr (j < C::KS) {
      s_out[0] = mfma32(op, qf[0][j], s_out[0]);
      s_out[1] = mfma32(op, qf[1][j], s_out[1]);
    } else {
      constexpr int i = j - C::KS, db = i >> 1, ks = i & 1;
      oacc[0][db] = mfma32(p_in[0][ks], op, oacc[0][db]);
      oacc[1][db] = mfma32(p_in[1][ks], op, oacc[1][db]);
    }
    static_for<j * EPS, (j + 1) * EPS>([&](auto ec) {
      constexpr int e = decltype(ec)::value, qb = e >> 4, r = e & 15;
      p_out[qb][r >> 3][r & 7] = (__bf16)sigmoid_dot(s_in[qb][r], c1, c0);
    });
    sched_step<j, (j + 2 < NSTEP) ? ((j + 2 < C::KS) ? 1 : 2) : 0, 2, 5 * EPS, 2>();
  });
}

// Forward. Each wave owns 64 query rows. The key loop is software-pipelined in
// half-tiles (32 keys) so that the MFMAs of one half-tile run beside the sigma
// of another. In key tile t:
//   phase A: S(t, 2nd half) and O += P(t-1, 2nd half) V   ||   P(t, 1st half) = sigma(S)
//   barrier; the DMA of tile t+2 into the slot tile t-1 held starts
//   phase B: S(t+1, 1st half) and O += P(t, 1st half) V   ||   P(t, 2nd half) = sigma(S)
// The LDS ring holds tiles t-1, t and t+1. There is one barrier per key tile.
// K and V come straight from global memory into LDS by DMA, with padded key
// rows replaced by zeros on the way. Each ring slot is its own LDS variable
// and the key loop is unrolled by three, so every access names its slot at
// compile time; the compiler then sees that phase B's reads cannot touch the
// slot the DMA is filling and does not wait for the DMA before them.
template <int D>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                       const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                                       const int32_t* __restrict__ seqlens_q,
                                                       const int32_t* __restrict__ seqlens_k, int Z, int L, int H,
                                                       float c1, float c0, int32_t* __restrict__ tile_counts) {
  using C = FwdCfg<D>;
  static_assert(C::NBUF == 3, "the key loop is unrolled over a ring of three slots");
  __shared__ __attribute__((aligned(1024))) __bf16 sK0[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sK1[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sK2[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV0[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV1[C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV2[C::TILE];

  __shared__ int rank_lds[kMaxRankedSamples];
  const int n_qt = (L + C::BQ - 1) / C::BQ;
  const TileCoord tc = schedule_tile(blockIdx.x, Z, H, n_qt, L, seqlens_q, seqlens_k, rank_lds);
  const int z = tc.z, h = tc.h, m = tc.m;
  const int nq = clamp_len(seqlens_q[z], L);
  const int nk = clamp_len(seqlens_k[z], L);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)H * D;
  const size_t base = ((size_t)z * L * H + h) * D;
  __bf16* Ob = O + base;
  const int q0 = m * C::BQ;

  if (q0 >= nq) {  // wholly padded query tile: write zeros, skip all work
    const int rows_here = min(C::BQ, L - q0);
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

  const int nkt = (nk + C::BK - 1) / C::BK;
  // The loop runs a multiple of three tiles. Tiles past n_k arrive as zeros
  // (every DMA lane is out of range): their V rows are 0, so they add exactly
  // nothing to O.
  const int nkt3 = (nkt + 2) / 3 * 3;
  if (nkt > 0) {
    const uint32_t row_bytes = (uint32_t)(rs * 2);
    const __bf16* Kb = K + base;
    const __bf16* Vb = V + base;
    auto fetch = [&](__bf16* sk, __bf16* sv, int tile) {  // DMA key tile `tile` into one slot
      const int k0 = tile * C::BK;
      const size_t off = (size_t)(k0 < nk ? k0 : 0) * rs;  // no row is read past n_k
      dma_tile<D, C::BK, 256>(sk, Kb + off, row_bytes, nk - k0, tid);
      dma_tile<D, C::BK, 256>(sv, Vb + off, row_bytes, nk - k0, tid);
    };
    fetch(sK0, sV0, 0);
    fetch(sK1, sV1, 1);
    // Slot 2's V is read by the first phase A with P = 0 (there is no tile -1).
    // It must hold finite values then, so it starts as zeros.
    for (int c = tid; c < C::TILE / 8; c += 256) *(bf16x8*)(sV2 + c * 8) = zero_bf16x8();
    dma_wait();
    __syncthreads();

    f32x16 s_cur[2], s_nxt[2];
    bf16x8 p0[2][2], p1[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) p1[qb][0] = p1[qb][1] = zero_bf16x8();
    scores_t<D>(s_cur, sK0, 0, qf, l32, half);
    // Key tile t in slot T; slot P holds tile t-1 and slot N tile t+1.
    auto iteration = [&](auto t_c, auto p_c, auto n_c, int t) {
      constexpr int T = decltype(t_c)::value, P = decltype(p_c)::value, N = decltype(n_c)::value;
      // phase A: 32 MFMAs beside 32 sigmoids per lane
      fwd_phase<D>(s_nxt, ring<T>(sK0, sK1, sK2), 1, oacc, p1, ring<P>(sV0, sV1, sV2), 1, p0, s_cur, qf, c1, c0,
                   l32, half, lane);
      pin_before_barrier(p0);
      dma_wait();       // this wave's DMA of tile t+1 has landed
      __syncthreads();  // ... everyone's has, and every wave is done with slot P
      if (t + 2 < nkt3) fetch(ring<P>(sK0, sK1, sK2), ring<P>(sV0, sV1, sV2), t + 2);
      // phase B. At the last tile the new S comes from a stale slot and is never used.
      fwd_phase<D>(s_cur, ring<N>(sK0, sK1, sK2), 0, oacc, p0, ring<T>(sV0, sV1, sV2), 0, p1, s_nxt, qf, c1, c0,
                   l32, half, lane);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    for (int t = 0; t < nkt3; t += 3) {
      iteration(I0{}, I2{}, I1{}, t);
      iteration(I1{}, I0{}, I2{}, t + 1);
      iteration(I2{}, I1{}, I0{}, t + 2);
    }
    // the second half of tile nkt3 - 1 (slot 2)
    accumulate_pv<D>(oacc, p1, sV2, 1, lane);
  }

  // Epilogue. Register r of oacc[qb][db] holds query row 64w + 32qb + acc_row(r, half), column 32db + l%32.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < C::NB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = q0 + 64 * w + 32 * qb + acc_row(r, half);
        if (row < L) Ob[(size_t)row * rs + db * 32 + l32] = (__bf16)(row < nq ? oacc[qb][db][r] : 0.0f);
      }
  if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = nkt;
}

// ---------------------------------------------------------------------------------------------
// fp32 validation forward: scalar fp32 arithmetic, one thread per query row.
// The tile logic is the same (BQ = 64 rows per workgroup, BK = 32 keys per LDS tile).
template <int D>
__global__ __launch_bounds__(64) void fwd_fp32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                      const float* __restrict__ V, float* __restrict__ O,
                                                      const int32_t* __restrict__ seqlens_q,
                                                      const int32_t* __restrict__ seqlens_k, int L, int H, float c1,
                                                      float c0, int32_t* __restrict__ tile_counts) {
  constexpr int BQ = 64, BK = 32;
  __shared__ float sK[BK][D];
  __shared__ float sV[BK][D];
  const int n_qt = (L + BQ - 1) / BQ;
  int bid = blockIdx.x;
  const int m = bid % n_qt;
  bid /= n_qt;
  const int h = bid % H;
  const int z = bid / H;
  const int nq = clamp_len(seqlens_q[z], L);
  const int nk = clamp_len(seqlens_k[z], L);
  const size_t rs = (size_t)H * D;
  const size_t base = ((size_t)z * L * H + h) * D;
  const int tid = threadIdx.x;
  const int q0 = m * BQ;
  const int row = q0 + tid;
  if (q0 >= nq) {
    if (row < L)
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
      sK[r][d] = kr < nk ? K[base + (size_t)kr * rs + d] : 0.0f;
      sV[r][d] = kr < nk ? V[base + (size_t)kr * rs + d] : 0.0f;
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
  if (row < L)
    for (int d = 0; d < D; ++d) O[base + (size_t)row * rs + d] = live ? o[d] : 0.0f;
  if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = nkt;
}

// Launchers (called from api.cpp). They return the hipError_t of the launch.
template <int D>
hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, const int32_t* nq, const int32_t* nk,
                           int Z, int L, int H, float c1, float c0, int32_t* tc, hipStream_t st) {
  using C = FwdCfg<D>;
  const long long blocks = (long long)Z * H * ((L + C::BQ - 1) / C::BQ);
  hipLaunchKernelGGL(fwd_bf16_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)q,
                     (const __bf16*)k, (const __bf16*)v, (__bf16*)o, nq, nk, Z, L, H, c1, c0, tc);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_fp32(const void* q, const void* k, const void* v, void* o, const int32_t* nq, const int32_t* nk,
                           int Z, int L, int H, float c1, float c0, int32_t* tc, hipStream_t st) {
  const long long blocks = (long long)Z * H * ((L + 63) / 64);
  hipLaunchKernelGGL(fwd_fp32_kernel<D>, dim3((unsigned)blocks), dim3(64), 0, st, (const float*)q, (const float*)k,
                     (const float*)v, (float*)o, nq, nk, L, H, c1, c0, tc);
  return hipGetLastError();
}

template hipError_t launch_fwd_bf16<64>(const void*, const void*, const void*, void*, const int32_t*, const int32_t*,
                                        int, int, int, float, float, int32_t*, hipStream_t);
template hipError_t launch_fwd_bf16<128>(const void*, const void*, const void*, void*, const int32_t*, const int32_t*,
                                         int, int, int, float, float, int32_t*, hipStream_t);
template hipError_t launch_fwd_fp32<64>(const void*, const void*, const void*, void*, const int32_t*, const int32_t*,
                                        int, int, int, float, float, int32_t*, hipStream_t);
template hipError_t launch_fwd_fp32<128>(const void*, const void*, const void*, void*, const int32_t*, const int32_t*,
                                         int, int, int, float, float, int32_t*, hipStream_t);

}  // namespace sigattn
