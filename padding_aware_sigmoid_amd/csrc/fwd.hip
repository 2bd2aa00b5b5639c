// Forward kernels: O = sigma(alpha Q K^T + b) V with padding-aware tile skipping.
//
// Method: rainbus.top summary of arXiv:2604.27124, section "方法步骤详情",
// steps 1-3 (blocking of [Z,L,H,D] tensors, skipping of query blocks wholly in
// padding, -inf at padded keys, sigma accumulated into O); gist.science summary
// section 2.A (forward formula).
//
// CDNA4 design (bf16):
//  - One workgroup computes one query tile of BQ = 128 rows for one (z, h).
//    It has 4 waves of 32 query rows each.
//  - A query tile at or past n_q writes zeros and exits.
//  - Only key tiles below n_k are visited, so wholly padded key tiles are
//    skipped.
//  - K and V tiles are staged through LDS with coalesced 16-byte loads.
//  - A padded key row is never read: its LDS row is filled with zeros. Its
//    score is then b, and its weight is multiplied by V = 0. Its contribution
//    is therefore exactly 0, whatever the padding holds.
//  - Scores are computed transposed, S^T = K Q^T, so the accumulator already
//    has the layout of the A operand of P V. P never leaves registers.
//  - V reaches the MFMA through ds_read_b64_tr_b16.
//  - sigma takes one v_exp_f32 and one v_rcp_f32 per score.
#include "common.hpp"

namespace sigattn {

template <int D>
struct FwdCfg {
  static constexpr int BQ = 128;  // query rows per workgroup
  static constexpr int BK = 64;   // keys per LDS tile
  static constexpr int NWAVE = 4;
  static constexpr int KS = D / 16;  // MFMA k-steps over the head dim
  static constexpr int NB = D / 32;  // 32-wide column blocks of O
  static constexpr int LD = D + 8;   // LDS row pitch (bf16), +16 B against bank conflicts
};

template <int D>
__global__ __launch_bounds__(256) void fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                                                       const __bf16* __restrict__ V, __bf16* __restrict__ O,
                                                       const int32_t* __restrict__ seqlens_q,
                                                       const int32_t* __restrict__ seqlens_k, int L, int H, float c1,
                                                       float c0, int32_t* __restrict__ tile_counts) {
  using C = FwdCfg<D>;
  __shared__ __attribute__((aligned(16))) __bf16 sK[C::BK * C::LD];
  __shared__ __attribute__((aligned(16))) __bf16 sV[C::BK * C::LD];

  const int n_qt = (L + C::BQ - 1) / C::BQ;
  int bid = blockIdx.x;
  const int m = bid % n_qt;
  bid /= n_qt;
  const int h = bid % H;
  const int z = bid / H;
  const int nq = clamp_len(seqlens_q[z], L);
  const int nk = clamp_len(seqlens_k[z], L);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int half = lane >> 5;
  const int l32 = lane & 31;
  const size_t rs = (size_t)H * D;  // elements between consecutive rows of one head
  const size_t base = ((size_t)z * L * H + h) * D;
  const __bf16* Qb = Q + base;
  const __bf16* Kb = K + base;
  const __bf16* Vb = V + base;
  __bf16* Ob = O + base;
  const int q0 = m * C::BQ;
  const int rows_here = min(C::BQ, L - q0);

  if (q0 >= nq) {  // wholly padded query tile: write zeros, skip all work
    const bf16x8 zz = zero_bf16x8();
    for (int c = tid; c < rows_here * (D / 8); c += 256) {
      const int r = c / (D / 8), cc = c % (D / 8);
      *(bf16x8*)(Ob + (size_t)(q0 + r) * rs + cc * 8) = zz;
    }
    if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = 0;
    return;
  }

  // Q fragment as the B operand of S^T = K Q^T: query row q0 + 32w + l%32, d = 16s + 8*half + 0..7.
  const int qr = q0 + 32 * w + l32;
  bf16x8 qf[C::KS];
#pragma unroll
  for (int s = 0; s < C::KS; ++s)
    qf[s] = (qr < nq) ? *(const bf16x8*)(Qb + (size_t)qr * rs + 16 * s + 8 * half) : zero_bf16x8();

  f32x16 oacc[C::NB];
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[nb][r] = 0.0f;

  const int nkt = (nk + C::BK - 1) / C::BK;
  for (int t = 0; t < nkt; ++t) {
    const int k0 = t * C::BK;
    for (int c = tid; c < C::BK * (D / 8); c += 256) {
      const int r = c / (D / 8), cc = c % (D / 8);
      const int kr = k0 + r;
      bf16x8 kv = zero_bf16x8(), vv = zero_bf16x8();
      if (kr < nk) {
        kv = *(const bf16x8*)(Kb + (size_t)kr * rs + cc * 8);
        vv = *(const bf16x8*)(Vb + (size_t)kr * rs + cc * 8);
      }
      *(bf16x8*)(sK + r * C::LD + cc * 8) = kv;
      *(bf16x8*)(sV + r * C::LD + cc * 8) = vv;
    }
    __syncthreads();
#pragma unroll
    for (int kb = 0; kb < C::BK / 32; ++kb) {
      f32x16 sacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        const bf16x8 a = *(const bf16x8*)(sK + (kb * 32 + l32) * C::LD + 16 * s + 8 * half);
        sacc = mfma32(a, qf[s], sacc);
      }
      bf16x8 p[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r >> 3][r & 7] = (__bf16)sigmoid_dot(sacc[r], c1, c0);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x8 b = lds_read_b_tr(sV, C::LD, kb * 32 + ks * 16, nb * 32, lane);
          oacc[nb] = mfma32(p[ks], b, oacc[nb]);
        }
    }
    __syncthreads();
  }

  // Epilogue. Register r of oacc[nb] holds query row 32w + acc_row(r, half) and column nb*32 + l%32.
#pragma unroll
  for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = q0 + 32 * w + acc_row(r, half);
      if (row < L) Ob[(size_t)row * rs + nb * 32 + l32] = (__bf16)(row < nq ? oacc[nb][r] : 0.0f);
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
                     (const __bf16*)k, (const __bf16*)v, (__bf16*)o, nq, nk, L, H, c1, c0, tc);
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
