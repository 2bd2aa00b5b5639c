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
  static constexpr int BQ_DQ = 128;   // dQ kernel: query rows per workgroup (4 waves x 32)
  static constexpr int BK_DQ = 64;    // dQ kernel: keys per LDS tile
  static constexpr int BK_KV = 128;   // dK/dV kernel: key rows per workgroup (4 waves x 32)
  static constexpr int BQ_KV = 64;    // dK/dV kernel: queries per LDS tile
  static constexpr int KS = D / 16;
  static constexpr int NB = D / 32;
  static constexpr int LD = D + 8;
};

// ------------------------------------------------------------------------------------------ dQ
// Wave w owns 32 query rows. It holds Q and dO as B operands, for:
//   S^T  = K Q^T   (A = K from LDS)
//   dP^T = V dO^T  (A = V from LDS)
// dS^T is built elementwise in registers and fed as the A operand of
// dQ += dS K. That product takes K from LDS through transposed reads.
template <int D>
__global__ __launch_bounds__(256) void dq_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                      const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                                                      __bf16* __restrict__ dQ, const int32_t* __restrict__ seqlens_q,
                                                      const int32_t* __restrict__ seqlens_k, int L, int H, float alpha,
                                                      float c1, float c0, int32_t* __restrict__ tile_counts) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sK[C::BK_DQ * C::LD];
  __shared__ __attribute__((aligned(16))) __bf16 sV[C::BK_DQ * C::LD];
  const int n_qt = (L + C::BQ_DQ - 1) / C::BQ_DQ;
  int bid = blockIdx.x;
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
  const int rows_here = min(C::BQ_DQ, L - q0);
  __bf16* dQb = dQ + base;

  if (q0 >= nq) {
    const bf16x8 zz = zero_bf16x8();
    for (int c = tid; c < rows_here * (D / 8); c += 256) {
      const int r = c / (D / 8), cc = c % (D / 8);
      *(bf16x8*)(dQb + (size_t)(q0 + r) * rs + cc * 8) = zz;
    }
    if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = 0;
    return;
  }

  const int qr = q0 + 32 * w + l32;
  bf16x8 qf[C::KS], dof[C::KS];
#pragma unroll
  for (int s = 0; s < C::KS; ++s) {
    const bool ok = qr < nq;
    qf[s] = ok ? *(const bf16x8*)(Q + base + (size_t)qr * rs + 16 * s + 8 * half) : zero_bf16x8();
    dof[s] = ok ? *(const bf16x8*)(dO + base + (size_t)qr * rs + 16 * s + 8 * half) : zero_bf16x8();
  }
  f32x16 acc[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[nb][r] = 0.0f;

  const int nkt = (nk + C::BK_DQ - 1) / C::BK_DQ;
  for (int t = 0; t < nkt; ++t) {
    const int k0 = t * C::BK_DQ;
    for (int c = tid; c < C::BK_DQ * (D / 8); c += 256) {
      const int r = c / (D / 8), cc = c % (D / 8);
      const int kr = k0 + r;
      bf16x8 kv = zero_bf16x8(), vv = zero_bf16x8();
      if (kr < nk) {
        kv = *(const bf16x8*)(K + base + (size_t)kr * rs + cc * 8);
        vv = *(const bf16x8*)(V + base + (size_t)kr * rs + cc * 8);
      }
      *(bf16x8*)(sK + r * C::LD + cc * 8) = kv;
      *(bf16x8*)(sV + r * C::LD + cc * 8) = vv;
    }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < C::BK_DQ / 32; ++kb) {
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.0f;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const int off = (kb * 32 + l32) * C::LD + 16 * s + 8 * half;
        sacc = mfma32(*(const bf16x8*)(sK + off), qf[s], sacc);
        pacc = mfma32(*(const bf16x8*)(sV + off), dof[s], pacc);
      }
      bf16x8 ds[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = sigmoid_dot(sacc[r], c1, c0);
        ds[r >> 3][r & 7] = (__bf16)(__builtin_fmaf(-p, p, p) * pacc[r]);
      }
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          acc[nb] = mfma32(ds[ks], lds_read_b_tr(sK, C::LD, kb * 32 + ks * 16, nb * 32, lane), acc[nb]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = q0 + 32 * w + acc_row(r, half);
      if (row < L) dQb[(size_t)row * rs + nb * 32 + l32] = (__bf16)(row < nq ? alpha * acc[nb][r] : 0.0f);
    }
  if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = nkt;
}

// ---------------------------------------------------------------------------------------- dK/dV
// Wave w owns 32 key rows. It holds K and V as B operands, for:
//   S  = Q K^T   (A = Q from LDS)
//   dP = dO V^T  (A = dO from LDS)
// P^T and dS^T come straight from those accumulators as A operands, for:
//   dV += P^T dO   (B = dO through transposed LDS reads)
//   dK += dS^T Q   (B = Q through transposed LDS reads)
template <int D>
__global__ __launch_bounds__(256) void dkdv_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                        const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                                                        __bf16* __restrict__ dK, __bf16* __restrict__ dV,
                                                        const int32_t* __restrict__ seqlens_q,
                                                        const int32_t* __restrict__ seqlens_k, int L, int H,
                                                        float alpha, float c1, float c0,
                                                        int32_t* __restrict__ tile_counts) {
  using C = BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sQ[C::BQ_KV * C::LD];
  __shared__ __attribute__((aligned(16))) __bf16 sdO[C::BQ_KV * C::LD];
  const int n_kt = (L + C::BK_KV - 1) / C::BK_KV;
  int bid = blockIdx.x;
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
  const int rows_here = min(C::BK_KV, L - k0);
  __bf16* dKb = dK + base;
  __bf16* dVb = dV + base;

  if (k0 >= nk) {
    const bf16x8 zz = zero_bf16x8();
    for (int c = tid; c < rows_here * (D / 8); c += 256) {
      const int r = c / (D / 8), cc = c % (D / 8);
      *(bf16x8*)(dKb + (size_t)(k0 + r) * rs + cc * 8) = zz;
      *(bf16x8*)(dVb + (size_t)(k0 + r) * rs + cc * 8) = zz;
    }
    if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_kt + t] = 0;
    return;
  }

  const int kr = k0 + 32 * w + l32;
  bf16x8 kf[C::KS], vf[C::KS];
#pragma unroll
  for (int s = 0; s < C::KS; ++s) {
    const bool ok = kr < nk;
    kf[s] = ok ? *(const bf16x8*)(K + base + (size_t)kr * rs + 16 * s + 8 * half) : zero_bf16x8();
    vf[s] = ok ? *(const bf16x8*)(V + base + (size_t)kr * rs + 16 * s + 8 * half) : zero_bf16x8();
  }
  f32x16 dkacc[C::NB], dvacc[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkacc[nb][r] = dvacc[nb][r] = 0.0f;

  const int nqt = (nq + C::BQ_KV - 1) / C::BQ_KV;
  for (int u = 0; u < nqt; ++u) {
    const int qbase = u * C::BQ_KV;
    for (int c = tid; c < C::BQ_KV * (D / 8); c += 256) {
      const int r = c / (D / 8), cc = c % (D / 8);
      const int qrow = qbase + r;
      bf16x8 qv = zero_bf16x8(), dv = zero_bf16x8();
      if (qrow < nq) {
        qv = *(const bf16x8*)(Q + base + (size_t)qrow * rs + cc * 8);
        dv = *(const bf16x8*)(dO + base + (size_t)qrow * rs + cc * 8);
      }
      *(bf16x8*)(sQ + r * C::LD + cc * 8) = qv;
      *(bf16x8*)(sdO + r * C::LD + cc * 8) = dv;
    }
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < C::BQ_KV / 32; ++qb) {
      f32x16 sacc, pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = pacc[r] = 0.0f;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const int off = (qb * 32 + l32) * C::LD + 16 * s + 8 * half;
        sacc = mfma32(*(const bf16x8*)(sQ + off), kf[s], sacc);
        pacc = mfma32(*(const bf16x8*)(sdO + off), vf[s], pacc);
      }
      bf16x8 pt[2], dst[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = sigmoid_dot(sacc[r], c1, c0);
        pt[r >> 3][r & 7] = (__bf16)p;
        dst[r >> 3][r & 7] = (__bf16)(__builtin_fmaf(-p, p, p) * pacc[r]);
      }
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          dvacc[nb] = mfma32(pt[ks], lds_read_b_tr(sdO, C::LD, qb * 32 + ks * 16, nb * 32, lane), dvacc[nb]);
          dkacc[nb] = mfma32(dst[ks], lds_read_b_tr(sQ, C::LD, qb * 32 + ks * 16, nb * 32, lane), dkacc[nb]);
        }
    }
    __syncthreads();
  }
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = k0 + 32 * w + acc_row(r, half);
      if (row < L) {
        const bool ok = row < nk;
        dKb[(size_t)row * rs + nb * 32 + l32] = (__bf16)(ok ? alpha * dkacc[nb][r] : 0.0f);
        dVb[(size_t)row * rs + nb * 32 + l32] = (__bf16)(ok ? dvacc[nb][r] : 0.0f);
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
  hipLaunchKernelGGL(dkdv_bf16_kernel<D>, dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)q,
                     (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, (__bf16*)dk, (__bf16*)dv, nq, nk, L, H,
                     alpha, c1, c0, tc);
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
