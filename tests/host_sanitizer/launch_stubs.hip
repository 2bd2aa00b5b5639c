// Stand-ins for the kernel launchers, so that the host code of api.hip can be
// built with host sanitizers without compiling the kernels. Each one reports
// that the launch is not supported; the C entry points turn that into
// SIGATTN_EHIP. Signatures as declared at the top of csrc/api.hip.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace sigattn {
template <int D>
hipError_t launch_fwd_bf16(const void*, const void*, const void*, void*, SeqLayout, int, int, float, float, int32_t*,
                           hipStream_t) { return hipErrorNotSupported; }
template <int D>
hipError_t launch_fwd_fp32(const void*, const void*, const void*, void*, SeqLayout, int, int, float, float, int32_t*,
                           hipStream_t) { return hipErrorNotSupported; }
template <int D>
hipError_t launch_dkdv_bf16(int, int, const void*, const void*, const void*, const void*, void*, void*, const void*,
                            SeqLayout, int, int, float, float, float, int32_t*, hipStream_t) {
  return hipErrorNotSupported;
}
template <int D>
hipError_t launch_dkdv_fp32(int, const void*, const void*, const void*, const void*, void*, void*, SeqLayout, int, int,
                            float, float, float, int32_t*, hipStream_t) { return hipErrorNotSupported; }
template <int D>
hipError_t launch_dq_bf16(int, const void*, const void*, const void*, const void*, void*, const void*, SeqLayout, int,
                          int, float, float, float, int32_t*, hipStream_t) { return hipErrorNotSupported; }
template <int D>
hipError_t launch_dq_fp32(const void*, const void*, const void*, const void*, void*, SeqLayout, int, int, float,
                          float, float, int32_t*, hipStream_t) { return hipErrorNotSupported; }
template <int D>
hipError_t launch_sm_fwd_bf16(const void*, const void*, const void*, void*, float*, SeqLayout, int, int, float,
                              hipStream_t) { return hipErrorNotSupported; }
template <int D>
hipError_t launch_sm_fwd_fp32(const void*, const void*, const void*, void*, float*, SeqLayout, int, int, float,
                              hipStream_t) { return hipErrorNotSupported; }
template <int D>
hipError_t launch_sm_rowstats(int, const void*, const void*, const float*, void*, SeqLayout, int, int, float,
                              hipStream_t) { return hipErrorNotSupported; }
template <int D>
hipError_t launch_sm_bwd_fp32(const void*, const void*, const void*, const void*, const void*, void*, void*, void*,
                              SeqLayout, int, int, float, float, hipStream_t) { return hipErrorNotSupported; }
template <int D>
hipError_t launch_quantize_fp8(const void*, void*, uint8_t*, SeqLayout, int, int, int, hipStream_t) {
  return hipErrorNotSupported;
}
template <int D>
hipError_t launch_fwd_fp8(const void*, const void*, const void*, const uint8_t*, const uint8_t*, const uint8_t*,
                          void*, SeqLayout, int, int, float, float, hipStream_t) { return hipErrorNotSupported; }

#define SIGATTN_STUBS(D)                                                                                          \
  template hipError_t launch_fwd_bf16<D>(const void*, const void*, const void*, void*, SeqLayout, int, int, float, \
                                         float, int32_t*, hipStream_t);                                           \
  template hipError_t launch_fwd_fp32<D>(const void*, const void*, const void*, void*, SeqLayout, int, int, float, \
                                         float, int32_t*, hipStream_t);                                           \
  template hipError_t launch_dkdv_bf16<D>(int, int, const void*, const void*, const void*, const void*, void*,      \
                                          void*, const void*, SeqLayout, int, int, float, float, float, int32_t*,   \
                                          hipStream_t);                                                            \
  template hipError_t launch_dkdv_fp32<D>(int, const void*, const void*, const void*, const void*, void*, void*,    \
                                          SeqLayout, int, int, float, float, float, int32_t*, hipStream_t);        \
  template hipError_t launch_dq_bf16<D>(int, const void*, const void*, const void*, const void*, void*,             \
                                        const void*, SeqLayout, int, int, float, float, float, int32_t*,           \
                                        hipStream_t);                                                              \
  template hipError_t launch_dq_fp32<D>(const void*, const void*, const void*, const void*, void*, SeqLayout, int,  \
                                        int, float, float, float, int32_t*, hipStream_t);                          \
  template hipError_t launch_sm_fwd_bf16<D>(const void*, const void*, const void*, void*, float*, SeqLayout, int,   \
                                            int, float, hipStream_t);                                              \
  template hipError_t launch_sm_fwd_fp32<D>(const void*, const void*, const void*, void*, float*, SeqLayout, int,   \
                                            int, float, hipStream_t);                                              \
  template hipError_t launch_sm_rowstats<D>(int, const void*, const void*, const float*, void*, SeqLayout, int,     \
                                            int, float, hipStream_t);                                              \
  template hipError_t launch_sm_bwd_fp32<D>(const void*, const void*, const void*, const void*, const void*, void*, \
                                            void*, void*, SeqLayout, int, int, float, float, hipStream_t);         \
  template hipError_t launch_quantize_fp8<D>(const void*, void*, uint8_t*, SeqLayout, int, int, int, hipStream_t); \
  template hipError_t launch_fwd_fp8<D>(const void*, const void*, const void*, const uint8_t*, const uint8_t*,      \
                                        const uint8_t*, void*, SeqLayout, int, int, float, float, hipStream_t);
SIGATTN_STUBS(64)
SIGATTN_STUBS(128)
}  // namespace sigattn
