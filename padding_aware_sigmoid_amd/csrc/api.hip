// C ABI of the sigmoid-attention library: argument checks and dispatch.
// Declarations and the contract live in include/sigattn.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "sigattn.h"
#include "common.hpp"

namespace sigattn {
template <int D>
hipError_t launch_fwd_bf16(const void*, const void*, const void*, void*, SeqLayout, int, int, float, float, int32_t*,
                           hipStream_t);
template <int D>
hipError_t launch_fwd_fp32(const void*, const void*, const void*, void*, SeqLayout, int, int, float, float, int32_t*,
                           hipStream_t);
template <int D>
hipError_t launch_dkdv_bf16(int, int, const void*, const void*, const void*, const void*, void*, void*, const void*,
                            SeqLayout, int, int, float, float, float, int32_t*, hipStream_t);
template <int D>
hipError_t launch_dkdv_fp32(int, const void*, const void*, const void*, const void*, void*, void*, SeqLayout, int, int,
                            float, float, float, int32_t*, hipStream_t);
template <int D>
hipError_t launch_dq_bf16(int, const void*, const void*, const void*, const void*, void*, const void*, SeqLayout, int,
                          int, float, float, float, int32_t*, hipStream_t);
template <int D>
hipError_t launch_dq_fp32(const void*, const void*, const void*, const void*, void*, SeqLayout, int, int, float,
                          float, float, int32_t*, hipStream_t);
template <int D>
hipError_t launch_sm_fwd_bf16(const void*, const void*, const void*, void*, float*, SeqLayout, int, int, float,
                              hipStream_t);
template <int D>
hipError_t launch_sm_fwd_fp32(const void*, const void*, const void*, void*, float*, SeqLayout, int, int, float,
                              hipStream_t);
template <int D>
hipError_t launch_sm_rowstats(int, const void*, const void*, const float*, void*, SeqLayout, int, int, float,
                              hipStream_t);
template <int D>
hipError_t launch_sm_bwd_fp32(const void*, const void*, const void*, const void*, const void*, void*, void*, void*,
                              SeqLayout, int, int, float, float, hipStream_t);
template <int D>
hipError_t launch_quantize_fp8(const void*, void*, uint8_t*, SeqLayout, int, int, int, hipStream_t);
template <int D>
hipError_t launch_fwd_fp8(const void*, const void*, const void*, const uint8_t*, const uint8_t*, const uint8_t*,
                          void*, SeqLayout, int, int, float, float, hipStream_t);
}  // namespace sigattn

namespace {

constexpr int kFp8MaxL = 262144;  // the FP8 forward stages one scale byte per 64-key tile in LDS

thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, const char* detail = "") {
  std::snprintf(g_last_error, sizeof(g_last_error), fmt, detail);
  return status;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Tile sizes per kernel, D and dtype. They must match the kernels' constants.
bool tile_config(int kernel, int dtype, int* bq, int* bk) {
  if (dtype == SIGATTN_BF16) {
    switch (kernel) {
      case SIGATTN_KERNEL_FWD: *bq = 256; *bk = 64; return true;
      case SIGATTN_KERNEL_DQ: *bq = 256; *bk = 64; return true;
      case SIGATTN_KERNEL_DKDV: *bq = 64; *bk = 256; return true;
    }
  } else if (dtype == SIGATTN_FP32) {
    switch (kernel) {
      case SIGATTN_KERNEL_FWD: *bq = 64; *bk = 32; return true;
      case SIGATTN_KERNEL_DQ: *bq = 64; *bk = 32; return true;
      case SIGATTN_KERNEL_DKDV: *bq = 32; *bk = 64; return true;
    }
  }
  return false;
}

// Shared checks. Returns 0 when the call may proceed, 1 when there is nothing
// to do (an empty batch), or a negative status.
int check_common(int Z, int L, int H, int D, float alpha, float bias, int dtype, const int32_t* nq, const int32_t* nk) {
  if (dtype != SIGATTN_BF16 && dtype != SIGATTN_FP32) return fail(SIGATTN_EUNSUPPORTED, "unsupported dtype%s");
  if (Z < 0 || L < 0 || H < 0) return fail(SIGATTN_EINVAL, "Z, L and H must be >= 0%s");
  if (D != 64 && D != 128) return fail(SIGATTN_EINVAL, "D must be 64 or 128%s");
  if (!std::isfinite(alpha) || !std::isfinite(bias)) return fail(SIGATTN_EINVAL, "alpha and bias must be finite%s");
  if (Z == 0 || L == 0 || H == 0) return 1;
  if (nq == nullptr || nk == nullptr) return fail(SIGATTN_EINVAL, "seqlens_q and seqlens_k must not be NULL%s");
  // The largest grid has one workgroup of 256 work-items per 128 rows of each
  // (sample, head) pair: the fused dK/dV kernel and the exchanged sigmoid dQ
  // at D = 64 own 128 rows per workgroup, every other bf16 kernel 256, and
  // the fp32 kernels 64 rows per workgroup of 64 work-items. A dispatch holds
  // at most 2^32 - 1 work-items. Element offsets are 64-bit.
  const long long items = (long long)Z * H * ((L + 127) / 128) * 256;
  if (items > 0xffffffffLL) return fail(SIGATTN_EINVAL, "problem too large for one grid%s");
  // Tiles reach LDS through buffer loads with 32-bit offsets below 256 rows.
  if ((long long)H * D * 2 * 256 >= 0x80000000LL) return fail(SIGATTN_EINVAL, "H * D too large%s");
  return 0;
}

int check_tensor(const void* p, const char* name) {
  if (p == nullptr) return fail(SIGATTN_EINVAL, "tensor %s is NULL", name);
  if (!aligned16(p)) return fail(SIGATTN_EINVAL, "tensor %s is not 16-byte aligned", name);
  return 0;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return SIGATTN_OK;
  return fail(SIGATTN_EHIP, "HIP launch failed: %s", hipGetErrorString(e));
}

// log2(e), for sigma(x) = 1 / (1 + 2^(-x log2 e))
constexpr float kLog2e = 1.4426950408889634f;

// What a dK/dV launch writes. The values match the kernels' KvMode.
constexpr int kKvBoth = 0, kKvDk = 1, kKvDv = 2;

}  // namespace

namespace {

int launch_dkdv(int mode, const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                sigattn::SeqLayout sl, int Z, int H, int D, float alpha, float bias, int dtype, int32_t* tc,
                hipStream_t st) {
  const float c1 = -alpha * kLog2e, c0 = -bias * kLog2e;
  hipError_t e;
  if (dtype == SIGATTN_BF16)
    e = (D == 64) ? sigattn::launch_dkdv_bf16<64>(0, mode, q, k, v, dout, dk, dv, nullptr, sl, Z, H, alpha, c1, c0,
                                                  tc, st)
                  : sigattn::launch_dkdv_bf16<128>(0, mode, q, k, v, dout, dk, dv, nullptr, sl, Z, H, alpha, c1, c0,
                                                   tc, st);
  else
    e = (D == 64) ? sigattn::launch_dkdv_fp32<64>(mode, q, k, v, dout, dk, dv, sl, Z, H, alpha, c1, c0, tc, st)
                  : sigattn::launch_dkdv_fp32<128>(mode, q, k, v, dout, dk, dv, sl, Z, H, alpha, c1, c0, tc, st);
  return hip_status(e);
}

int launch_dq(const void* q, const void* k, const void* v, const void* dout, void* dq, sigattn::SeqLayout sl, int Z,
              int H, int D, float alpha, float bias, int dtype, int32_t* tc, hipStream_t st) {
  const float c1 = -alpha * kLog2e, c0 = -bias * kLog2e;
  hipError_t e;
  if (dtype == SIGATTN_BF16)
    e = (D == 64) ? sigattn::launch_dq_bf16<64>(0, q, k, v, dout, dq, nullptr, sl, Z, H, alpha, c1, c0, tc, st)
                  : sigattn::launch_dq_bf16<128>(0, q, k, v, dout, dq, nullptr, sl, Z, H, alpha, c1, c0, tc, st);
  else
    e = (D == 64) ? sigattn::launch_dq_fp32<64>(q, k, v, dout, dq, sl, Z, H, alpha, c1, c0, tc, st)
                  : sigattn::launch_dq_fp32<128>(q, k, v, dout, dq, sl, Z, H, alpha, c1, c0, tc, st);
  return hip_status(e);
}

int launch_fwd(const void* q, const void* k, const void* v, void* o, sigattn::SeqLayout sl, int Z, int H, int D,
               float alpha, float bias, int dtype, int32_t* tc, hipStream_t st) {
  const float c1 = -alpha * kLog2e, c0 = -bias * kLog2e;
  hipError_t e;
  if (dtype == SIGATTN_BF16)
    e = (D == 64) ? sigattn::launch_fwd_bf16<64>(q, k, v, o, sl, Z, H, c1, c0, tc, st)
                  : sigattn::launch_fwd_bf16<128>(q, k, v, o, sl, Z, H, c1, c0, tc, st);
  else
    e = (D == 64) ? sigattn::launch_fwd_fp32<64>(q, k, v, o, sl, Z, H, c1, c0, tc, st)
                  : sigattn::launch_fwd_fp32<128>(q, k, v, o, sl, Z, H, c1, c0, tc, st);
  return hip_status(e);
}

// The layout of the original entry points: padded [Z, L, H, D], one bias.
sigattn::SeqLayout padded(const int32_t* nq, const int32_t* nk, int L) { return {nq, nk, L, 0, 0}; }

int check_modes(int layout, int bias_mode) {
  if (layout != SIGATTN_LAYOUT_PADDED && layout != SIGATTN_LAYOUT_PACKED)
    return fail(SIGATTN_EINVAL, "unknown layout%s");
  if (bias_mode != SIGATTN_BIAS_CONSTANT && bias_mode != SIGATTN_BIAS_NEG_LOG_NK)
    return fail(SIGATTN_EINVAL, "unknown bias mode%s");
  return 0;
}

}  // namespace

extern "C" {

int sigattn_fwd(const void* q, const void* k, const void* v, void* o, const int32_t* seqlens_q,
                const int32_t* seqlens_k, int Z, int L, int H, int D, float alpha, float bias, sigattn_dtype dtype,
                int32_t* tile_counts, void* stream) {
  return sigattn_fwd_ex(q, k, v, o, seqlens_q, seqlens_k, SIGATTN_LAYOUT_PADDED, SIGATTN_BIAS_CONSTANT, Z, L, H, D,
                        alpha, bias, dtype, tile_counts, stream);
}

int sigattn_fwd_ex(const void* q, const void* k, const void* v, void* o, const int32_t* seq_q, const int32_t* seq_k,
                   sigattn_layout layout, sigattn_bias_mode bias_mode, int Z, int L, int H, int D, float alpha,
                   float bias, sigattn_dtype dtype, int32_t* tile_counts, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_modes(layout, bias_mode);
  if (rc != 0) return rc;
  rc = check_common(Z, L, H, D, alpha, bias, dtype, seq_q, seq_k);
  if (rc != 0) return rc > 0 ? SIGATTN_OK : rc;
  if ((rc = check_tensor(q, "q")) || (rc = check_tensor(k, "k")) || (rc = check_tensor(v, "v")) ||
      (rc = check_tensor(o, "o")))
    return rc;
  return launch_fwd(q, k, v, o, {seq_q, seq_k, L, layout, bias_mode}, Z, H, D, alpha, bias, dtype, tile_counts,
                    reinterpret_cast<hipStream_t>(stream));
}

int sigattn_bwd(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk, void* dv,
                const int32_t* seqlens_q, const int32_t* seqlens_k, int Z, int L, int H, int D, float alpha,
                float bias, sigattn_dtype dtype, int32_t* tile_counts_dq, int32_t* tile_counts_dkdv, void* stream) {
  return sigattn_bwd_ex(q, k, v, dout, dq, dk, dv, seqlens_q, seqlens_k, SIGATTN_LAYOUT_PADDED,
                        SIGATTN_BIAS_CONSTANT, Z, L, H, D, alpha, bias, dtype, tile_counts_dq, tile_counts_dkdv,
                        stream);
}

int sigattn_bwd_ex(const void* q, const void* k, const void* v, const void* dout, void* dq, void* dk, void* dv,
                   const int32_t* seq_q, const int32_t* seq_k, sigattn_layout layout, sigattn_bias_mode bias_mode,
                   int Z, int L, int H, int D, float alpha, float bias, sigattn_dtype dtype,
                   int32_t* tile_counts_dq, int32_t* tile_counts_dkdv, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_modes(layout, bias_mode);
  if (rc != 0) return rc;
  rc = check_common(Z, L, H, D, alpha, bias, dtype, seq_q, seq_k);
  if (rc != 0) return rc > 0 ? SIGATTN_OK : rc;
  if ((rc = check_tensor(q, "q")) || (rc = check_tensor(k, "k")) || (rc = check_tensor(v, "v")) ||
      (rc = check_tensor(dout, "dout")) || (rc = check_tensor(dq, "dq")) || (rc = check_tensor(dk, "dk")) ||
      (rc = check_tensor(dv, "dv")))
    return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const sigattn::SeqLayout sl{seq_q, seq_k, L, layout, bias_mode};
  rc = launch_dkdv(kKvBoth, q, k, v, dout, dk, dv, sl, Z, H, D, alpha, bias, dtype, tile_counts_dkdv, st);
  if (rc != SIGATTN_OK) return rc;
  return launch_dq(q, k, v, dout, dq, sl, Z, H, D, alpha, bias, dtype, tile_counts_dq, st);
}

int sigattn_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                     const int32_t* seqlens_q, const int32_t* seqlens_k, int Z, int L, int H, int D, float alpha,
                     float bias, sigattn_dtype dtype, int32_t* tile_counts_dkdv, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_common(Z, L, H, D, alpha, bias, dtype, seqlens_q, seqlens_k);
  if (rc != 0) return rc > 0 ? SIGATTN_OK : rc;
  if ((rc = check_tensor(q, "q")) || (rc = check_tensor(k, "k")) || (rc = check_tensor(v, "v")) ||
      (rc = check_tensor(dout, "dout")) || (rc = check_tensor(dk, "dk")) || (rc = check_tensor(dv, "dv")))
    return rc;
  return launch_dkdv(kKvBoth, q, k, v, dout, dk, dv, padded(seqlens_q, seqlens_k, L), Z, H, D, alpha, bias, dtype,
                     tile_counts_dkdv, reinterpret_cast<hipStream_t>(stream));
}

int sigattn_bwd_dk(const void* q, const void* k, const void* v, const void* dout, void* dk,
                   const int32_t* seqlens_q, const int32_t* seqlens_k, int Z, int L, int H, int D, float alpha,
                   float bias, sigattn_dtype dtype, int32_t* tile_counts_dkdv, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_common(Z, L, H, D, alpha, bias, dtype, seqlens_q, seqlens_k);
  if (rc != 0) return rc > 0 ? SIGATTN_OK : rc;
  if ((rc = check_tensor(q, "q")) || (rc = check_tensor(k, "k")) || (rc = check_tensor(v, "v")) ||
      (rc = check_tensor(dout, "dout")) || (rc = check_tensor(dk, "dk")))
    return rc;
  return launch_dkdv(kKvDk, q, k, v, dout, dk, nullptr, padded(seqlens_q, seqlens_k, L), Z, H, D, alpha, bias, dtype,
                     tile_counts_dkdv, reinterpret_cast<hipStream_t>(stream));
}

int sigattn_bwd_dv(const void* q, const void* k, const void* dout, void* dv, const int32_t* seqlens_q,
                   const int32_t* seqlens_k, int Z, int L, int H, int D, float alpha, float bias,
                   sigattn_dtype dtype, int32_t* tile_counts_dkdv, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_common(Z, L, H, D, alpha, bias, dtype, seqlens_q, seqlens_k);
  if (rc != 0) return rc > 0 ? SIGATTN_OK : rc;
  if ((rc = check_tensor(q, "q")) || (rc = check_tensor(k, "k")) || (rc = check_tensor(dout, "dout")) ||
      (rc = check_tensor(dv, "dv")))
    return rc;
  return launch_dkdv(kKvDv, q, k, nullptr, dout, nullptr, dv, padded(seqlens_q, seqlens_k, L), Z, H, D, alpha, bias,
                     dtype, tile_counts_dkdv, reinterpret_cast<hipStream_t>(stream));
}

int sigattn_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq,
                   const int32_t* seqlens_q, const int32_t* seqlens_k, int Z, int L, int H, int D, float alpha,
                   float bias, sigattn_dtype dtype, int32_t* tile_counts_dq, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_common(Z, L, H, D, alpha, bias, dtype, seqlens_q, seqlens_k);
  if (rc != 0) return rc > 0 ? SIGATTN_OK : rc;
  if ((rc = check_tensor(q, "q")) || (rc = check_tensor(k, "k")) || (rc = check_tensor(v, "v")) ||
      (rc = check_tensor(dout, "dout")) || (rc = check_tensor(dq, "dq")))
    return rc;
  return launch_dq(q, k, v, dout, dq, padded(seqlens_q, seqlens_k, L), Z, H, D, alpha, bias, dtype, tile_counts_dq,
                   reinterpret_cast<hipStream_t>(stream));
}

int sigattn_softmax_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* seq_q,
                        const int32_t* seq_k, sigattn_layout layout, int Z, int L, int H, int D, float alpha,
                        sigattn_dtype dtype, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_modes(layout, SIGATTN_BIAS_CONSTANT);
  if (rc != 0) return rc;
  if (!(alpha > 0.0f)) return fail(SIGATTN_EINVAL, "softmax needs alpha > 0%s");
  rc = check_common(Z, L, H, D, alpha, 0.0f, dtype, seq_q, seq_k);
  if (rc != 0) return rc > 0 ? SIGATTN_OK : rc;
  if ((rc = check_tensor(q, "q")) || (rc = check_tensor(k, "k")) || (rc = check_tensor(v, "v")) ||
      (rc = check_tensor(o, "o")) || (rc = check_tensor(lse, "lse")))
    return rc;
  const sigattn::SeqLayout sl{seq_q, seq_k, L, layout, 0};
  const float c1 = alpha * kLog2e;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (dtype == SIGATTN_BF16)
    e = (D == 64) ? sigattn::launch_sm_fwd_bf16<64>(q, k, v, o, lse, sl, Z, H, c1, st)
                  : sigattn::launch_sm_fwd_bf16<128>(q, k, v, o, lse, sl, Z, H, c1, st);
  else
    e = (D == 64) ? sigattn::launch_sm_fwd_fp32<64>(q, k, v, o, lse, sl, Z, H, c1, st)
                  : sigattn::launch_sm_fwd_fp32<128>(q, k, v, o, lse, sl, Z, H, c1, st);
  return hip_status(e);
}

size_t sigattn_softmax_bwd_workspace_size(long long rows_q, int H) {
  return rows_q > 0 && H > 0 ? (size_t)rows_q * (size_t)H * 8 : 0;
}

}  // extern "C"

namespace {

// The row statistics pass, then the fused dK/dV and the dQ kernels (bf16), or
// the fp32 validation kernels, with the row statistics in `workspace`.
int run_softmax_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                    void* dq, void* dk, void* dv, const sigattn::SeqLayout& sl, int Z, int H, int D, float alpha,
                    int dtype, void* workspace, hipStream_t st) {
  const float c1 = alpha * kLog2e;
  const int bf = dtype == SIGATTN_BF16;
  hipError_t e = (D == 64) ? sigattn::launch_sm_rowstats<64>(bf, o, dout, lse, workspace, sl, Z, H, alpha, st)
                           : sigattn::launch_sm_rowstats<128>(bf, o, dout, lse, workspace, sl, Z, H, alpha, st);
  if (e != hipSuccess) return hip_status(e);
  if (bf) {
    e = (D == 64) ? sigattn::launch_dkdv_bf16<64>(1, kKvBoth, q, k, v, dout, dk, dv, workspace, sl, Z, H, alpha, c1,
                                                  0.0f, nullptr, st)
                  : sigattn::launch_dkdv_bf16<128>(1, kKvBoth, q, k, v, dout, dk, dv, workspace, sl, Z, H, alpha, c1,
                                                   0.0f, nullptr, st);
    if (e != hipSuccess) return hip_status(e);
    e = (D == 64) ? sigattn::launch_dq_bf16<64>(1, q, k, v, dout, dq, workspace, sl, Z, H, alpha, c1, 0.0f, nullptr, st)
                  : sigattn::launch_dq_bf16<128>(1, q, k, v, dout, dq, workspace, sl, Z, H, alpha, c1, 0.0f, nullptr,
                                                 st);
  } else {
    e = (D == 64) ? sigattn::launch_sm_bwd_fp32<64>(q, k, v, dout, workspace, dq, dk, dv, sl, Z, H, alpha, c1, st)
                  : sigattn::launch_sm_bwd_fp32<128>(q, k, v, dout, workspace, dq, dk, dv, sl, Z, H, alpha, c1, st);
  }
  return hip_status(e);
}

// Checks shared by both softmax backward entry points. Returns 0 to proceed,
// 1 for an empty batch, or a negative status.
int check_softmax_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                      void* dq, void* dk, void* dv, const int32_t* seq_q, const int32_t* seq_k, int layout, int Z,
                      int L, int H, int D, float alpha, int dtype) {
  int rc = check_modes(layout, SIGATTN_BIAS_CONSTANT);
  if (rc != 0) return rc;
  if (!(alpha > 0.0f)) return fail(SIGATTN_EINVAL, "softmax needs alpha > 0%s");
  rc = check_common(Z, L, H, D, alpha, 0.0f, dtype, seq_q, seq_k);
  if (rc != 0) return rc;
  if ((rc = check_tensor(q, "q")) || (rc = check_tensor(k, "k")) || (rc = check_tensor(v, "v")) ||
      (rc = check_tensor(o, "o")) || (rc = check_tensor(dout, "dout")) || (rc = check_tensor(lse, "lse")) ||
      (rc = check_tensor(dq, "dq")) || (rc = check_tensor(dk, "dk")) || (rc = check_tensor(dv, "dv")))
    return rc;
  return 0;
}

// The device-resident row statistics of sigattn_softmax_bwd_noalloc: one
// array per GPU, of fixed size, for the life of the process. Host code never
// uses the array's name as an address: each device's address comes from
// hipGetSymbolAddress, looked up once per device with that device current,
// and kept in scratch_ptr.
constexpr size_t kScratchPairs = (size_t)SIGATTN_NOALLOC_ROWS;
static_assert(kScratchPairs * sizeof(float2) == ((size_t)16 << 20), "16 MiB of row statistics per GPU");
static __device__ __align__(256) float2 scratch[kScratchPairs];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The address of `scratch` on the device that runs `st` (the current device
// for the null stream).
int scratch_address(hipStream_t st, void** out) {
  int dev = 0;
  hipError_t e = st != nullptr ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return fail(SIGATTN_EINVAL, "device index out of the supported range%s");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_status(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t back = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_status(e);
    if (back != hipSuccess) return hip_status(back);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SIGATTN_OK;
}

}  // namespace

extern "C" {

int sigattn_softmax_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                        const float* lse, void* dq, void* dk, void* dv, const int32_t* seq_q, const int32_t* seq_k,
                        sigattn_layout layout, int Z, int L, int H, int D, float alpha, sigattn_dtype dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_softmax_bwd(q, k, v, o, dout, lse, dq, dk, dv, seq_q, seq_k, layout, Z, L, H, D, alpha, dtype);
  if (rc != 0) return rc > 0 ? SIGATTN_OK : rc;
  if ((rc = check_tensor(workspace, "workspace"))) return rc;
  // The padded layout has Z * L query rows. The packed layout's row count sits
  // in device memory (the last offset): there only the one-row-per-sample floor
  // is checked here, and the caller sizes the buffer for all of its rows.
  const size_t rows = layout == SIGATTN_LAYOUT_PADDED ? (size_t)Z * L : (size_t)Z;
  if (workspace_bytes < rows * (size_t)H * 8)
    return fail(SIGATTN_EWORKSPACE, "workspace smaller than query rows * H * 8 bytes%s");
  return run_softmax_bwd(q, k, v, o, dout, lse, dq, dk, dv, {seq_q, seq_k, L, layout, 0}, Z, H, D, alpha, dtype,
                         workspace, reinterpret_cast<hipStream_t>(stream));
}

int sigattn_softmax_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, const int32_t* seq_q,
                                const int32_t* seq_k, sigattn_layout layout, int Z, int L, int H, int D, float alpha,
                                sigattn_dtype dtype, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_softmax_bwd(q, k, v, o, dout, lse, dq, dk, dv, seq_q, seq_k, layout, Z, L, H, D, alpha, dtype);
  if (rc != 0) return rc > 0 ? SIGATTN_OK : rc;
  // Both layouts hold at most Z * L query rows (a packed batch within its
  // contract: no sample longer than L).
  if ((unsigned long long)Z * (unsigned long long)L * (unsigned long long)H > kScratchPairs)
    return fail(SIGATTN_EINVAL, "Z * L * H exceeds the fixed row-statistics buffer (SIGATTN_NOALLOC_ROWS)%s");
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if ((rc = scratch_address(st, &ws)) != SIGATTN_OK) return rc;
  return run_softmax_bwd(q, k, v, o, dout, lse, dq, dk, dv, {seq_q, seq_k, L, layout, 0}, Z, H, D, alpha, dtype, ws,
                         st);
}

int sigattn_quantize_fp8(const void* x, void* x8, uint8_t* scales, const int32_t* seq, sigattn_layout layout,
                         int Z, int L, int H, int D, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_modes(layout, SIGATTN_BIAS_CONSTANT);
  if (rc != 0) return rc;
  rc = check_common(Z, L, H, D, 1.0f, 0.0f, SIGATTN_BF16, seq, seq);
  if (rc != 0) return rc > 0 ? SIGATTN_OK : rc;
  if ((rc = check_tensor(x, "x")) || (rc = check_tensor(x8, "x8"))) return rc;
  if (scales == nullptr) return fail(SIGATTN_EINVAL, "scales is NULL%s");
  const sigattn::SeqLayout sl{seq, seq, L, layout, 0};
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_status(D == 64 ? sigattn::launch_quantize_fp8<64>(x, x8, scales, sl, Z, H, 0, st)
                            : sigattn::launch_quantize_fp8<128>(x, x8, scales, sl, Z, H, 0, st));
}

int sigattn_fwd_fp8(const void* q8, const void* k8, const void* v8, const uint8_t* sq, const uint8_t* sk,
                    const uint8_t* sv, void* o, const int32_t* seq_q, const int32_t* seq_k, sigattn_layout layout,
                    sigattn_bias_mode bias_mode, int Z, int L, int H, int D, float alpha, float bias, void* stream) {
  g_last_error[0] = '\0';
  int rc = check_modes(layout, bias_mode);
  if (rc != 0) return rc;
  if (!(alpha > 0.0f)) return fail(SIGATTN_EINVAL, "the FP8 forward needs alpha > 0%s");
  rc = check_common(Z, L, H, D, alpha, bias, SIGATTN_BF16, seq_q, seq_k);
  if (rc != 0) return rc > 0 ? SIGATTN_OK : rc;
  if (L > kFp8MaxL) return fail(SIGATTN_EINVAL, "the FP8 forward takes L <= 262144%s");
  if ((rc = check_tensor(q8, "q8")) || (rc = check_tensor(k8, "k8")) || (rc = check_tensor(v8, "v8")) ||
      (rc = check_tensor(o, "o")))
    return rc;
  if (sq == nullptr || sk == nullptr || sv == nullptr) return fail(SIGATTN_EINVAL, "a scale array is NULL%s");
  const sigattn::SeqLayout sl{seq_q, seq_k, L, layout, bias_mode};
  const float c1 = -alpha * kLog2e, c0 = -bias * kLog2e;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  return hip_status(D == 64 ? sigattn::launch_fwd_fp8<64>(q8, k8, v8, sq, sk, sv, o, sl, Z, H, c1, c0, st)
                            : sigattn::launch_fwd_fp8<128>(q8, k8, v8, sq, sk, sv, o, sl, Z, H, c1, c0, st));
}

int sigattn_tile_config(sigattn_kernel kernel, int D, sigattn_dtype dtype, int* block_q, int* block_k) {
  if (block_q == nullptr || block_k == nullptr || (D != 64 && D != 128)) return SIGATTN_EINVAL;
  return tile_config(kernel, dtype, block_q, block_k) ? SIGATTN_OK : SIGATTN_EINVAL;
}

const char* sigattn_strerror(int status) {
  switch (status) {
    case SIGATTN_OK: return "ok";
    case SIGATTN_EINVAL: return "invalid argument";
    case SIGATTN_EUNSUPPORTED: return "unsupported dtype";
    case SIGATTN_EHIP: return "HIP error";
    case SIGATTN_EWORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* sigattn_last_error(void) { return g_last_error; }

const char* sigattn_version(void) { return "sigattn-mi355x 0.2 (gfx950)"; }

}  // extern "C"
