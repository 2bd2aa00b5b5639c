// Backward kernels of padding-aware sigmoid attention.
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
#include "common.hpp"

namespace sigattn {

template <int D>
struct BwdCfg {
  static constexpr int W = 64;          // rows a wave owns: queries (dQ kernel) or keys (dK/dV kernel)
  static constexpr int NWAVE = 4;       // one wave per SIMD
  static constexpr int BQ_DQ = 256;     // dQ kernel: query rows per workgroup
  static constexpr int BK_DQ = 64;      // dQ kernel: keys per LDS tile
  static constexpr int BK_KV = 256;     // dK/dV kernel: key rows per workgroup
  static constexpr int BQ_KV = 64;      // dK/dV kernel: queries per LDS tile
  static constexpr int KS = D / 16;     // MFMA k-steps over the head dim
  static constexpr int NB = D / 32;     // 32-wide column blocks of the gradients
  static constexpr int TILE = 64 * D;   // elements of one 64-row LDS tile (swizzled, unpadded)
};

// ------------------------------------------------------------------------------------------ dQ
// Wave w owns 64 query rows (two 32-row blocks). It holds Q and dO as B
// operands, for:
//   S^T  = K Q^T   (A = K from LDS)
//   dP^T = V dO^T  (A = V from LDS)
// dS^T = P (1 - P) dP^T is built in registers and fed as the A operand of
// dQ += dS K. That product takes K from LDS through transposed reads.
// Key tiles of 64 rows stream through a 2-slot LDS ring by DMA.
// Per 32-key block, the next block's S^T / dP^T MFMAs run beside this block's
// sigma and dS, and the previous block's dQ MFMAs run beside them too.
template <int D>
__global__ __launch_bounds__(256) void dq_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                      const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                                                      __bf16* __restrict__ dQ, const int32_t* __restrict__ seqlens_q,
                                                      const int32_t* __restrict__ seqlens_k, int L, int H, float alpha,
                                                      float c1, float c0, int32_t* __restrict__ tile_counts) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 sK[2][C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sV[2][C::TILE];
  const int n_qt = (L + C::BQ_DQ - 1) / C::BQ_DQ;
  int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int m = bid % n_qt;
  bid /= n_qt;
  const int h = bid % H;
  const int z = bid / H;
  const int nq = clamp_len(seqlens_q[z], L);
  const int nk = clamp_len(seqlens_k[z], L);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)H * D;
  const size_t base = ((size_t)z * L * H + h) * D;
  const int q0 = m * C::BQ_DQ;
  __bf16* dQb = dQ + base;

  if (q0 >= nq) {
    const int rows_here = min(C::BQ_DQ, L - q0);
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

  const int nkt = (nk + C::BK_DQ - 1) / C::BK_DQ;
  if (nkt > 0) {
    const uint32_t row_bytes = (uint32_t)(rs * 2);
    const __bf16* Kb = K + base;
    const __bf16* Vb = V + base;
    auto fetch = [&](int slot, int tile) {
      const int k0 = tile * C::BK_DQ;
      dma_tile<D, 64, 256>(sK[slot], Kb + (size_t)k0 * rs, row_bytes, nk - k0, tid);
      dma_tile<D, 64, 256>(sV[slot], Vb + (size_t)k0 * rs, row_bytes, nk - k0, tid);
    };
    fetch(0, 0);
    // dS of the previous 32-key block, waiting for its dQ MFMAs (zero before the first block).
    bf16x8 ds_prev[2][2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) ds_prev[qb][0] = ds_prev[qb][1] = zero_bf16x8();
    int slot_prev = 0;
    for (int t = 0; t < nkt; ++t) {
      const int slot = t & 1;
      dma_wait();
      __syncthreads();  // tile t is in LDS; every wave is done with tile t-1's dQ reads below
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // S^T, dP^T for this block (32 MFMAs)
        f32x16 sacc[2], pacc[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[qb][r] = pacc[qb][r] = 0.0f;
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
          const bf16x8 ak = lds_nat<D>(sK[slot], kb * 32 + l32, 2 * s + half);
          const bf16x8 av = lds_nat<D>(sV[slot], kb * 32 + l32, 2 * s + half);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            sacc[qb] = mfma32(ak, qf[qb][s], sacc[qb]);
            pacc[qb] = mfma32(av, dof[qb][s], pacc[qb]);
          }
        }
        // the previous block's dQ (16 MFMAs), beside this block's sigma and dS
        {
          const __bf16* kt = (kb == 0) ? sK[slot_prev] : sK[slot];
          const int kbp = (kb == 0) ? 1 : 0;
#pragma unroll
          for (int db = 0; db < C::NB; ++db)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
              const bf16x8 b = lds_tr<D>(kt, kbp * 32 + ks * 16, db * 32, lane);
              acc[0][db] = mfma32(ds_prev[0][ks], b, acc[0][db]);
              acc[1][db] = mfma32(ds_prev[1][ks], b, acc[1][db]);
            }
        }
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = sigmoid_dot(sacc[qb][r], c1, c0);
            ds_prev[qb][r >> 3][r & 7] = (__bf16)(__builtin_fmaf(-p, p, p) * pacc[qb][r]);
          }
        interleave_mfma_valu<4 * C::KS + 2 * C::NB * 2, 6>();
        if (kb == 0 && t + 1 < nkt) fetch(slot ^ 1, t + 1);  // slot ^ 1 held tile t-1, finished above
      }
      slot_prev = slot;
    }
    // dQ of the last block
#pragma unroll
    for (int db = 0; db < C::NB; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16x8 b = lds_tr<D>(sK[slot_prev], 32 + ks * 16, db * 32, lane);
        acc[0][db] = mfma32(ds_prev[0][ks], b, acc[0][db]);
        acc[1][db] = mfma32(ds_prev[1][ks], b, acc[1][db]);
      }
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < C::NB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = q0 + 64 * w + 32 * qb + acc_row(r, half);
        if (row < L) dQb[(size_t)row * rs + db * 32 + l32] = (__bf16)(row < nq ? alpha * acc[qb][db][r] : 0.0f);
      }
  if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = nkt;
}

// ---------------------------------------------------------------------------------------- dK/dV
// Wave w owns 64 key rows (two 32-row blocks). It holds K and V as B operands, for:
//   S  = Q K^T   (A = Q from LDS)
//   dP = dO V^T  (A = dO from LDS)
// P^T and dS^T come straight from those accumulators as A operands, for:
//   dV += P^T dO   (B = dO through transposed LDS reads)
//   dK += dS^T Q   (B = Q through transposed LDS reads)
// Query tiles of 64 rows stream through a 2-slot LDS ring by DMA.
//
// MODE selects what one launch computes:
//   KV_BOTH (dK and dV together) shares S between them: 8*D MFMA FLOP per pair.
//   KV_DK (S, dP, dK: 6*D) and KV_DV (S, dV: 4*D) split the work over two
//   launches.
// At D = 128 the K and V operands plus both accumulators do not fit one
// wave's registers (the fused form spills), so D = 128 runs the split form.
enum KvMode { KV_BOTH = 0, KV_DK = 1, KV_DV = 2 };

template <int D, int MODE>
__global__ __launch_bounds__(256) void dkdv_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                        const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                                                        __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                                                        const int32_t* __restrict__ seqlens_q,
                                                        const int32_t* __restrict__ seqlens_k, int L, int H,
                                                        float alpha, float c1, float c0,
                                                        int32_t* __restrict__ tile_counts) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(1024))) __bf16 sQ[2][C::TILE];
  __shared__ __attribute__((aligned(1024))) __bf16 sdO[2][C::TILE];
  const int n_kt = (L + C::BK_KV - 1) / C::BK_KV;
  int bid = xcd_remap(blockIdx.x, gridDim.x);
  const int t = bid % n_kt;
  bid /= n_kt;
  const int h = bid % H;
  const int z = bid / H;
  const int nq = clamp_len(seqlens_q[z], L);
  const int nk = clamp_len(seqlens_k[z], L);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, half = lane >> 5, l32 = lane & 31;
  const size_t rs = (size_t)H * D;
  const size_t base = ((size_t)z * L * H + h) * D;
  const int k0 = t * C::BK_KV;
  __bf16* dKb = dK + base;
  __bf16* dVb = dV + base;

  constexpr bool DO_DK = MODE != KV_DV, DO_DV = MODE != KV_DK;
  if (k0 >= nk) {
    const int rows_here = min(C::BK_KV, L - k0);
    const bf16x8 zz = zero_bf16x8();
    for (int c = tid; c < rows_here * (D / 8); c += 256) {
      const size_t off = (size_t)(k0 + c / (D / 8)) * rs + (c % (D / 8)) * 8;
      if (DO_DK) *(bf16x8*)(dKb + off) = zz;
      if (DO_DV) *(bf16x8*)(dVb + off) = zz;
    }
    if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_kt + t] = 0;
    return;
  }

  bf16x8 kf[2][C::KS], vf[2][C::KS];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int kr = k0 + 64 * w + 32 * kb + l32;
    const bool ok = kr < nk;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      kf[kb][s] = ok ? *(const bf16x8*)(K + base + (size_t)kr * rs + 16 * s + 8 * half) : zero_bf16x8();
      if (DO_DK) vf[kb][s] = ok ? *(const bf16x8*)(V + base + (size_t)kr * rs + 16 * s + 8 * half) : zero_bf16x8();
    }
  }
  f32x16 dkacc[2][C::NB], dvacc[2][C::NB];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < C::NB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) dkacc[kb][db][r] = dvacc[kb][db][r] = 0.0f;

  const int nqt = (nq + C::BQ_KV - 1) / C::BQ_KV;
  if (nqt > 0) {
    const uint32_t row_bytes = (uint32_t)(rs * 2);
    const __bf16* Qb = Q + base;
    const __bf16* dOb = dO + base;
    auto fetch = [&](int slot, int tile) {
      const int r0 = tile * C::BQ_KV;
      dma_tile<D, 64, 256>(sQ[slot], Qb + (size_t)r0 * rs, row_bytes, nq - r0, tid);
      dma_tile<D, 64, 256>(sdO[slot], dOb + (size_t)r0 * rs, row_bytes, nq - r0, tid);  // dV: B operand; dK: A of dP
    };
    fetch(0, 0);
    for (int u = 0; u < nqt; ++u) {
      const int slot = u & 1;
      dma_wait();
      __syncthreads();  // tile u is in LDS; every wave is done with tile u-1
      if (u + 1 < nqt) fetch(slot ^ 1, u + 1);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        f32x16 sacc[2], pacc[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) sacc[kb][r] = pacc[kb][r] = 0.0f;
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
          const bf16x8 aq = lds_nat<D>(sQ[slot], qb * 32 + l32, 2 * s + half);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) sacc[kb] = mfma32(aq, kf[kb][s], sacc[kb]);
          if (DO_DK) {
            const bf16x8 ag = lds_nat<D>(sdO[slot], qb * 32 + l32, 2 * s + half);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) pacc[kb] = mfma32(ag, vf[kb][s], pacc[kb]);
          }
        }
        bf16x8 pt[2][2], dst[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = sigmoid_dot(sacc[kb][r], c1, c0);
            if (DO_DV) pt[kb][r >> 3][r & 7] = (__bf16)p;
            if (DO_DK) dst[kb][r >> 3][r & 7] = (__bf16)(__builtin_fmaf(-p, p, p) * pacc[kb][r]);
          }
#pragma unroll
        for (int db = 0; db < C::NB; ++db)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            if (DO_DV) {
              const bf16x8 bg = lds_tr<D>(sdO[slot], qb * 32 + ks * 16, db * 32, lane);
#pragma unroll
              for (int kb = 0; kb < 2; ++kb) dvacc[kb][db] = mfma32(pt[kb][ks], bg, dvacc[kb][db]);
            }
            if (DO_DK) {
              const bf16x8 bq = lds_tr<D>(sQ[slot], qb * 32 + ks * 16, db * 32, lane);
#pragma unroll
              for (int kb = 0; kb < 2; ++kb) dkacc[kb][db] = mfma32(dst[kb][ks], bq, dkacc[kb][db]);
            }
          }
        interleave_mfma_valu<(DO_DK ? 6 : 3) * C::KS, (DO_DK ? 8 : 6)>();
      }
    }
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int db = 0; db < C::NB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = k0 + 64 * w + 32 * kb + acc_row(r, half);
        if (row < L) {
          const bool ok = row < nk;
          if (DO_DK) dKb[(size_t)row * rs + db * 32 + l32] = (__bf16)(ok ? alpha * dkacc[kb][db][r] : 0.0f);
          if (DO_DV) dVb[(size_t)row * rs + db * 32 + l32] = (__bf16)(ok ? dvacc[kb][db][r] : 0.0f);
        }
      }
  if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_kt + t] = nqt;
}

// ------------------------------------------------------------------------------ fp32 validation
// Scalar fp32. The dQ kernel has one thread per query row (BQ = 64, BK = 32).
// The dK/dV kernel has one thread per key row (BK = 64, BQ = 32). Each row's
// K and V sit in LDS so the register count stays small.
template <int D>
__global__ __launch_bounds__(64) void dq_fp32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                     const float* __restrict__ V, const float* __restrict__ dO,
                                                     float* __restrict__ dQ, const int32_t* __restrict__ seqlens_q,
                                                     const int32_t* __restrict__ seqlens_k, int L, int H, float alpha,
                                                     float c1, float c0, int32_t* __restrict__ tile_counts) {
  constexpr int BQ = 64, BK = 32;
  __shared__ float sK[BK][D];
  __shared__ float sV[BK][D];
  __shared__ float sQr[BQ][D + 1];  // this workgroup's own query rows and dO rows
  __shared__ float sGr[BQ][D + 1];
  const int n_qt = (L + BQ - 1) / BQ;
  int bid = blockIdx.x;
  const int m = bid % n_qt;
  bid /= n_qt;
  const int h = bid % H, z = bid / H;
  const int nq = clamp_len(seqlens_q[z], L), nk = clamp_len(seqlens_k[z], L);
  const size_t rs = (size_t)H * D, base = ((size_t)z * L * H + h) * D;
  const int tid = threadIdx.x, q0 = m * BQ, row = q0 + tid;
  if (q0 >= nq) {
    if (row < L)
      for (int d = 0; d < D; ++d) dQ[base + (size_t)row * rs + d] = 0.0f;
    if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = 0;
    return;
  }
  const bool live = row < nq;
  for (int c = tid; c < BQ * D; c += 64) {
    const int r = c / D, d = c % D, qr = q0 + r;
    sQr[r][d] = qr < nq ? Q[base + (size_t)qr * rs + d] : 0.0f;
    sGr[r][d] = qr < nq ? dO[base + (size_t)qr * rs + d] : 0.0f;
  }
  float acc[D];
  for (int d = 0; d < D; ++d) acc[d] = 0.0f;
  const int nkt = (nk + BK - 1) / BK;
  for (int t = 0; t < nkt; ++t) {
    __syncthreads();
    for (int c = tid; c < BK * D; c += 64) {
      const int r = c / D, d = c % D, kr = t * BK + r;
      sK[r][d] = kr < nk ? K[base + (size_t)kr * rs + d] : 0.0f;
      sV[r][d] = kr < nk ? V[base + (size_t)kr * rs + d] : 0.0f;
    }
    __syncthreads();
    for (int j = 0; j < BK; ++j) {
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < D; ++d) {
        s = __builtin_fmaf(sQr[tid][d], sK[j][d], s);
        dp = __builtin_fmaf(sGr[tid][d], sV[j][d], dp);
      }
      const float p = sigmoid_dot(s, c1, c0);
      const float ds = (p - p * p) * dp;
      for (int d = 0; d < D; ++d) acc[d] = __builtin_fmaf(ds, sK[j][d], acc[d]);
    }
  }
  if (row < L)
    for (int d = 0; d < D; ++d) dQ[base + (size_t)row * rs + d] = live ? alpha * acc[d] : 0.0f;
  if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = nkt;
}

template <int D>
__global__ __launch_bounds__(64) void dkdv_fp32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                       const float* __restrict__ V, const float* __restrict__ dO,
                                                       float* __restrict__ dK, float* __restrict__ dV,
                                                       const int32_t* __restrict__ seqlens_q,
                                                       const int32_t* __restrict__ seqlens_k, int L, int H,
                                                       float alpha, float c1, float c0,
                                                       int32_t* __restrict__ tile_counts) {
  constexpr int BK = 64, BQ = 32;
  __shared__ float sQ[BQ][D];
  __shared__ float sdO[BQ][D];
  __shared__ float sKr[BK][D + 1];  // this workgroup's own key rows (+1 pad: conflict-free column walk)
  __shared__ float sVr[BK][D + 1];
  const int n_kt = (L + BK - 1) / BK;
  int bid = blockIdx.x;
  const int t = bid % n_kt;
  bid /= n_kt;
  const int h = bid % H, z = bid / H;
  const int nq = clamp_len(seqlens_q[z], L), nk = clamp_len(seqlens_k[z], L);
  const size_t rs = (size_t)H * D, base = ((size_t)z * L * H + h) * D;
  const int tid = threadIdx.x, k0 = t * BK, row = k0 + tid;
  if (k0 >= nk) {
    if (row < L)
      for (int d = 0; d < D; ++d) dK[base + (size_t)row * rs + d] = dV[base + (size_t)row * rs + d] = 0.0f;
    if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_kt + t] = 0;
    return;
  }
  const bool live = row < nk;
  for (int c = tid; c < BK * D; c += 64) {
    const int r = c / D, d = c % D, kr = k0 + r;
    sKr[r][d] = kr < nk ? K[base + (size_t)kr * rs + d] : 0.0f;
    sVr[r][d] = kr < nk ? V[base + (size_t)kr * rs + d] : 0.0f;
  }
  float dk[D], dv[D];
  for (int d = 0; d < D; ++d) dk[d] = dv[d] = 0.0f;
  const int nqt = (nq + BQ - 1) / BQ;
  for (int u = 0; u < nqt; ++u) {
    __syncthreads();
    for (int c = tid; c < BQ * D; c += 64) {
      const int r = c / D, d = c % D, qr = u * BQ + r;
      sQ[r][d] = qr < nq ? Q[base + (size_t)qr * rs + d] : 0.0f;
      sdO[r][d] = qr < nq ? dO[base + (size_t)qr * rs + d] : 0.0f;
    }
    __syncthreads();
    for (int i = 0; i < BQ; ++i) {
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < D; ++d) {
        s = __builtin_fmaf(sQ[i][d], sKr[tid][d], s);
        dp = __builtin_fmaf(sdO[i][d], sVr[tid][d], dp);
      }
      const float p = sigmoid_dot(s, c1, c0);
      const float ds = (p - p * p) * dp;
      for (int d = 0; d < D; ++d) {
        dv[d] = __builtin_fmaf(p, sdO[i][d], dv[d]);
        dk[d] = __builtin_fmaf(ds, sQ[i][d], dk[d]);
      }
    }
  }
  if (row < L)
    for (int d = 0; d < D; ++d) {
      dK[base + (size_t)row * rs + d] = live ? alpha * dk[d] : 0.0f;
      dV[base + (size_t)row * rs + d] = live ? dv[d] : 0.0f;
    }
  if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_kt + t] = nqt;
}

// --------------------------------------------------------------------------------- launchers
template <int D>
hipError_t launch_dkdv_bf16(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                            const int32_t* nq, const int32_t* nk, int Z, int L, int H, float alpha, float c1,
                            float c0, int32_t* tc, hipStream_t st) {
  using C = BwdCfg<D>;
  const long long blocks = (long long)Z * H * ((L + C::BK_KV - 1) / C::BK_KV);
  if constexpr (D == 64) {
    hipLaunchKernelGGL((dkdv_bf16_kernel<D, KV_BOTH>), dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, (__bf16*)dk, (__bf16*)dv, nq, nk, L,
                       H, alpha, c1, c0, tc);
  } else {
    // Both launches see the same lengths, so both write the same counters.
    hipLaunchKernelGGL((dkdv_bf16_kernel<D, KV_DK>), dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, (__bf16*)dk, (__bf16*)dv, nq, nk, L,
                       H, alpha, c1, c0, tc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dkdv_bf16_kernel<D, KV_DV>), dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, (__bf16*)dk, (__bf16*)dv, nq, nk, L,
                       H, alpha, c1, c0, tc);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_dq_bf16(const void* q, const void* k, const void* v, const void* dout, void* dq, const int32_t* nq,
                          const int32_t* nk, int Z, int L, int H, float alpha, float c1, float c0, int32_t* tc,
                          hipStream_t st) {
  using C = BwdCfg<D>;
  const long long blocks = (long long)Z * H * ((L + C::BQ_DQ - 1) / C::BQ_DQ);
  hipLaunchKernelGGL(dq_bf16_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)q, (const __bf16*)k,
                     (const __bf16*)v, (const __bf16*)dout, (__bf16*)dq, nq, nk, L, H, alpha, c1, c0, tc);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dkdv_fp32(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                            const int32_t* nq, const int32_t* nk, int Z, int L, int H, float alpha, float c1,
                            float c0, int32_t* tc, hipStream_t st) {
  const long long blocks = (long long)Z * H * ((L + 63) / 64);
  hipLaunchKernelGGL(dkdv_fp32_kernel<D>, dim3((unsigned)blocks), dim3(64), 0, st, (const float*)q, (const float*)k,
                     (const float*)v, (const float*)dout, (float*)dk, (float*)dv, nq, nk, L, H, alpha, c1, c0, tc);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dq_fp32(const void* q, const void* k, const void* v, const void* dout, void* dq, const int32_t* nq,
                          const int32_t* nk, int Z, int L, int H, float alpha, float c1, float c0, int32_t* tc,
                          hipStream_t st) {
  const long long blocks = (long long)Z * H * ((L + 63) / 64);
  hipLaunchKernelGGL(dq_fp32_kernel<D>, dim3((unsigned)blocks), dim3(64), 0, st, (const float*)q, (const float*)k,
                     (const float*)v, (const float*)dout, (float*)dq, nq, nk, L, H, alpha, c1, c0, tc);
  return hipGetLastError();
}

#define SIGATTN_INST_BWD(D)                                                                                   \
  template hipError_t launch_dkdv_bf16<D>(const void*, const void*, const void*, const void*, void*, void*,      \
                                          const int32_t*, const int32_t*, int, int, int, float, float, float,  \
                                          int32_t*, hipStream_t);                                              \
  template hipError_t launch_dq_bf16<D>(const void*, const void*, const void*, const void*, void*,              \
                                        const int32_t*, const int32_t*, int, int, int, float, float, float,    \
                                        int32_t*, hipStream_t);                                                \
  template hipError_t launch_dkdv_fp32<D>(const void*, const void*, const void*, const void*, void*, void*,      \
                                          const int32_t*, const int32_t*, int, int, int, float, float, float,  \
                                          int32_t*, hipStream_t);                                              \
  template hipError_t launch_dq_fp32<D>(const void*, const void*, const void*, const void*, void*,              \
                                        const int32_t*, const int32_t*, int, int, int, float, float, float,    \
                                        int32_t*, hipStream_t);
SIGATTN_INST_BWD(64)
SIGATTN_INST_BWD(128)

}  // namespace sigattn
