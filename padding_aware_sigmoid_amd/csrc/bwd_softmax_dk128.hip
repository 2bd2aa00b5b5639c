// The softmax dK kernel at D = 128 (dK only; dV runs as its own launch).
// It holds K and V for 64 keys, the dK accumulators and two blocks of S and
// dP, at the 512-register limit. With MFMA results in VGPRs the compiler
// fails on it among the other backward kernels and spills 350 registers on
// its own, so this file is built with accumulators in AGPRs and the max-ILP
// scheduler, which leaves no spill.
#include "bwd_kernels.hpp"

namespace sigattn {

hipError_t launch_dk_bf16_softmax_d128(const void* q, const void* k, const void* v, const void* dout, void* dk,
                                       const void* stats, SeqLayout sl, int Z, int H, float alpha, float c1,
                                       int32_t* tc, hipStream_t st) {
  using C = BwdCfg<128>;
  const long long blocks = (long long)Z * H * ((sl.L + C::BK_KV - 1) / C::BK_KV);
  static_assert(kKeysPerWg<128, KV_DK, false> == C::BK_KV, "one workgroup per key tile");
  hipLaunchKernelGGL((dkdv_bf16_kernel<128, KV_DK, ACT_SOFTMAX>), dim3((unsigned)blocks), dim3(256), 0, st,
                     (const __bf16*)q, (const __bf16*)k, (const __bf16*)v, (const __bf16*)dout, (__bf16*)dk,
                     (__bf16*)nullptr, (const float2*)stats, sl, Z, H, alpha, c1, 0.0f, tc);
  return hipGetLastError();
}

}  // namespace sigattn
