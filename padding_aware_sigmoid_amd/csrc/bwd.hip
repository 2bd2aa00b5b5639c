// Backward: the fp32 validation kernels and the launchers of every backward
// kernel. The bf16 kernels are templates in bwd_kernels.hpp.
#include "bwd_kernels.hpp"

namespace sigattn {

// ------------------------------------------------------------------------------ fp32 validation
// Scalar fp32. The dQ kernel has one thread per query row (BQ = 64, BK = 32).
// The dK/dV kernel has one thread per key row (BK = 64, BQ = 32). Each row's
// K and V sit in LDS so the register count stays small.
template <int D>
__global__ __launch_bounds__(64) void dq_fp32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                     const float* __restrict__ V, const float* __restrict__ dO,
                                                     float* __restrict__ dQ, SeqLayout sl, int H, float alpha,
                                                     float c1, float c0_base, int32_t* __restrict__ tile_counts) {
  constexpr int BQ = 64, BK = 32;
  __shared__ float sK[BK][D];
  __shared__ float sV[BK][D];
  __shared__ float sQr[BQ][D + 1];  // this workgroup's own query rows and dO rows
  __shared__ float sGr[BQ][D + 1];
  const int n_qt = (sl.L + BQ - 1) / BQ;
  int bid = blockIdx.x;
  const int m = bid % n_qt;
  bid /= n_qt;
  const int h = bid % H, z = bid / H;
  const int nq = sl.nq(z), nk = sl.nk(z);
  const float c0 = sl.c0_for(c0_base, nk);
  const size_t rs = (size_t)H * D, base = (sl.row0_q(z) * H + h) * D, base_k = (sl.row0_k(z) * H + h) * D;
  const int rows = sl.rows(nq);
  const int tid = threadIdx.x, q0 = m * BQ, row = q0 + tid;
  if (q0 >= nq) {
    if (row < rows)
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
      sK[r][d] = kr < nk ? K[base_k + (size_t)kr * rs + d] : 0.0f;
      sV[r][d] = kr < nk ? V[base_k + (size_t)kr * rs + d] : 0.0f;
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
  if (row < rows)
    for (int d = 0; d < D; ++d) dQ[base + (size_t)row * rs + d] = live ? alpha * acc[d] : 0.0f;
  if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_qt + m] = nkt;
}

template <int D>
__global__ __launch_bounds__(64) void dkdv_fp32_kernel(const float* __restrict__ Q, const float* __restrict__ K,
                                                       const float* __restrict__ V, const float* __restrict__ dO,
                                                       float* __restrict__ dK, float* __restrict__ dV,
                                                       SeqLayout sl, int H, float alpha, float c1, float c0_base,
                                                       int32_t* __restrict__ tile_counts) {
  constexpr int BK = 64, BQ = 32;
  __shared__ float sQ[BQ][D];
  __shared__ float sdO[BQ][D];
  __shared__ float sKr[BK][D + 1];  // this workgroup's own key rows (+1 pad: conflict-free column walk)
  __shared__ float sVr[BK][D + 1];
  const int n_kt = (sl.L + BK - 1) / BK;
  int bid = blockIdx.x;
  const int t = bid % n_kt;
  bid /= n_kt;
  const int h = bid % H, z = bid / H;
  const int nq = sl.nq(z), nk = sl.nk(z);
  const float c0 = sl.c0_for(c0_base, nk);
  const size_t rs = (size_t)H * D, base = (sl.row0_k(z) * H + h) * D, base_q = (sl.row0_q(z) * H + h) * D;
  const int rows = sl.rows(nk);
  const int tid = threadIdx.x, k0 = t * BK, row = k0 + tid;
  if (k0 >= nk) {
    if (row < rows)
      for (int d = 0; d < D; ++d) {
        if (dK != nullptr) dK[base + (size_t)row * rs + d] = 0.0f;
        if (dV != nullptr) dV[base + (size_t)row * rs + d] = 0.0f;
      }
    if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_kt + t] = 0;
    return;
  }
  const bool live = row < nk;
  for (int c = tid; c < BK * D; c += 64) {
    const int r = c / D, d = c % D, kr = k0 + r;
    sKr[r][d] = kr < nk ? K[base + (size_t)kr * rs + d] : 0.0f;
    // V only feeds dK. A dV-only launch passes V = NULL.
    sVr[r][d] = (kr < nk && dK != nullptr) ? V[base + (size_t)kr * rs + d] : 0.0f;
  }
  float dk[D], dv[D];
  for (int d = 0; d < D; ++d) dk[d] = dv[d] = 0.0f;
  const int nqt = (nq + BQ - 1) / BQ;
  for (int u = 0; u < nqt; ++u) {
    __syncthreads();
    for (int c = tid; c < BQ * D; c += 64) {
      const int r = c / D, d = c % D, qr = u * BQ + r;
      sQ[r][d] = qr < nq ? Q[base_q + (size_t)qr * rs + d] : 0.0f;
      sdO[r][d] = qr < nq ? dO[base_q + (size_t)qr * rs + d] : 0.0f;
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
  if (row < rows)
    for (int d = 0; d < D; ++d) {
      if (dK != nullptr) dK[base + (size_t)row * rs + d] = live ? alpha * dk[d] : 0.0f;
      if (dV != nullptr) dV[base + (size_t)row * rs + d] = live ? dv[d] : 0.0f;
    }
  if (tile_counts != nullptr && tid == 0) tile_counts[((size_t)z * H + h) * n_kt + t] = nqt;
}

// --------------------------------------------------------------------------------- launchers
// MODE: KV_BOTH (dk and dv), KV_DK (dk only) or KV_DV (dv only; v is not read).
// act: ACT_SIGMOID (stats unused) or ACT_SOFTMAX (stats: {LSE / alpha, D} per query row and head).
template <int D>
hipError_t launch_dkdv_bf16(int act, int mode, const void* q, const void* k, const void* v, const void* dout,
                            void* dk, void* dv, const void* stats, SeqLayout sl, int Z, int H, float alpha, float c1,
                            float c0, int32_t* tc, hipStream_t st) {
  using C = BwdCfg<D>;
  // One workgroup per kKeysPerWg keys of each (sample, head) pair.
  auto go = [&](auto kern, int keys_per_wg) {
    const long long blocks = (long long)Z * H * ((sl.L + keys_per_wg - 1) / keys_per_wg);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)q,
                       (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, (__bf16*)dk, (__bf16*)dv,
                       (const float2*)stats, sl, Z, H, alpha, c1, c0, tc);
    return hipGetLastError();
  };
  auto only_dk = [&](auto act_c) -> hipError_t {
    constexpr int A = decltype(act_c)::value;
    if constexpr (D == 128 && A == ACT_SOFTMAX)
      return launch_dk_bf16_softmax_d128(q, k, v, dout, dk, stats, sl, Z, H, alpha, c1, tc, st);
    else
      return go(dkdv_bf16_kernel<D, KV_DK, A>, kKeysPerWg<D, KV_DK, false>);
  };
  auto run = [&](auto act_c) -> hipError_t {
    constexpr int A = decltype(act_c)::value;
    if (mode == KV_DK) return only_dk(act_c);
    if (mode == KV_DV) return go(dkdv_bf16_kernel<D, KV_DV, A>, kKeysPerWg<D, KV_DV, false>);
    return go(dkdv_bf16_kernel<D, KV_BOTH, A>, kKeysPerWg<D, KV_BOTH, false>);
  };
  return act == ACT_SOFTMAX ? run(std::integral_constant<int, ACT_SOFTMAX>{})
                            : run(std::integral_constant<int, ACT_SIGMOID>{});
}

template <int D>
hipError_t launch_dq_bf16(int act, const void* q, const void* k, const void* v, const void* dout, void* dq,
                          const void* stats, SeqLayout sl, int Z, int H, float alpha, float c1, float c0,
                          int32_t* tc, hipStream_t st) {
  using C = BwdCfg<D>;
  const long long blocks = (long long)Z * H * ((sl.L + C::BQ_DQ - 1) / C::BQ_DQ);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)q, (const __bf16*)k,
                       (const __bf16*)v, (const __bf16*)dout, (__bf16*)dq, (const float2*)stats, sl, Z, H, alpha, c1,
                       c0, tc);
    return hipGetLastError();
  };
  if constexpr (D == 64) {
    if (act == ACT_SIGMOID) {
      // Sigmoid dQ at D = 64 runs the dK/dV kernel with queries and keys
      // exchanged: a workgroup owns 128 query rows (one 32-row block per
      // wave), streams K and V, and its "dK" is dQ. dS is
      // symmetric in the exchange (sigma of the same score, dP^T = V dO^T).
      // At 240 registers two waves share a SIMD; 14% faster than
      // dq_bf16_kernel on stress8k. At D = 128 it measured 3% slower, and
      // softmax needs row statistics per owned row, which that kernel does
      // not take.
      static_assert(C::BQ_DQ == C::BK_KV, "the exchanged kernel tiles the queries as the dK/dV kernel tiles keys");
      constexpr int R = kKeysPerWg<D, KV_DK, true>;  // query rows per workgroup
      const long long wgs = (long long)Z * H * ((sl.L + R - 1) / R);
      hipLaunchKernelGGL((dkdv_bf16_kernel<D, KV_DK, ACT_SIGMOID, true>), dim3((unsigned)wgs), dim3(256), 0, st,
                         (const __bf16*)k, (const __bf16*)q, (const __bf16*)dout, (const __bf16*)v, (__bf16*)dq,
                         (__bf16*)nullptr, (const float2*)nullptr, sl, Z, H, alpha, c1, c0, tc);
      return hipGetLastError();
    }
  }
  return act == ACT_SOFTMAX ? go(dq_bf16_kernel<D, ACT_SOFTMAX>) : go(dq_bf16_kernel<D, ACT_SIGMOID>);
}

template <int D>
hipError_t launch_dkdv_fp32(int mode, const void* q, const void* k, const void* v, const void* dout, void* dk,
                            void* dv, SeqLayout sl, int Z, int H, float alpha, float c1, float c0, int32_t* tc,
                            hipStream_t st) {
  if (mode == KV_DK) dv = nullptr;
  if (mode == KV_DV) dk = nullptr;
  const long long blocks = (long long)Z * H * ((sl.L + 63) / 64);
  hipLaunchKernelGGL(dkdv_fp32_kernel<D>, dim3((unsigned)blocks), dim3(64), 0, st, (const float*)q, (const float*)k,
                     (const float*)v, (const float*)dout, (float*)dk, (float*)dv, sl, H, alpha, c1, c0, tc);
  return hipGetLastError();
}

template <int D>
hipError_t launch_dq_fp32(const void* q, const void* k, const void* v, const void* dout, void* dq, SeqLayout sl,
                          int Z, int H, float alpha, float c1, float c0, int32_t* tc, hipStream_t st) {
  const long long blocks = (long long)Z * H * ((sl.L + 63) / 64);
  hipLaunchKernelGGL(dq_fp32_kernel<D>, dim3((unsigned)blocks), dim3(64), 0, st, (const float*)q, (const float*)k,
                     (const float*)v, (const float*)dout, (float*)dq, sl, H, alpha, c1, c0, tc);
  return hipGetLastError();
}

#define SIGATTN_INST_BWD(D)                                                                                        \
  template hipError_t launch_dkdv_bf16<D>(int, int, const void*, const void*, const void*, const void*, void*,   \
                                          void*, const void*, SeqLayout, int, int, float, float, float, int32_t*, \
                                          hipStream_t);                                                         \
  template hipError_t launch_dkdv_fp32<D>(int, const void*, const void*, const void*, const void*, void*, void*, \
                                          SeqLayout, int, int, float, float, float, int32_t*, hipStream_t);     \
  template hipError_t launch_dq_bf16<D>(int, const void*, const void*, const void*, const void*, void*,          \
                                        const void*, SeqLayout, int, int, float, float, float, int32_t*,        \
                                        hipStream_t);                                                           \
  template hipError_t launch_dq_fp32<D>(const void*, const void*, const void*, const void*, void*, SeqLayout,    \
                                        int, int, float, float, float, int32_t*, hipStream_t);
SIGATTN_INST_BWD(64)
SIGATTN_INST_BWD(128)

}  // namespace sigattn
