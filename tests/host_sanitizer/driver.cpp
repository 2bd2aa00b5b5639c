// Host-side checks of the C ABI under AddressSanitizer and UBSan. Every call
// here is rejected by the argument checks, or passes them and reaches a
// stand-in launcher that reports failure, so no kernel runs and no pointer is
// dereferenced: the tensor pointers are host buffers standing in for device
// memory. The process exits non-zero on any wrong status; the sanitizers
// abort it on any memory or undefined-behaviour error in the host code.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <vector>

#include "sigattn.h"

static int g_failures = 0;

static void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "FAIL line %d: %s (last error: %s)\n", line, what, sigattn_last_error());
    ++g_failures;
  }
}
#define EXPECT(cond) expect((cond), #cond, __LINE__)

static bool last_error_has(const char* s) { return std::strstr(sigattn_last_error(), s) != nullptr; }

alignas(16) static unsigned char g_buf[12][64];
alignas(16) static int32_t g_lens[8] = {1, 2, 3, 4, 5, 6, 7, 8};
alignas(16) static float g_lse[64];

int main() {
  const void* q = g_buf[0];
  const void* k = g_buf[1];
  const void* v = g_buf[2];
  const void* dout = g_buf[3];
  void* o = g_buf[4];
  void* dq = g_buf[5];
  void* dk = g_buf[6];
  void* dv = g_buf[7];
  const void* misaligned = g_buf[8] + 1;
  const int32_t* n = g_lens;
  const sigattn_dtype bf16 = SIGATTN_BF16, fp32 = SIGATTN_FP32;
  const float a = 0.125f, b = -3.0f;

  // status strings and version
  for (int s = -6; s <= 2; ++s) EXPECT(sigattn_strerror(s) != nullptr && sigattn_strerror(s)[0] != 0);
  EXPECT(sigattn_version() != nullptr && sigattn_version()[0] != 0);

  // forward: every rejection, then a call that reaches the launcher
  EXPECT(sigattn_fwd(q, k, v, o, n, n, 2, 64, 2, 64, a, b, (sigattn_dtype)7, nullptr, nullptr) == SIGATTN_EUNSUPPORTED);
  EXPECT(sigattn_fwd(q, k, v, o, n, n, -1, 64, 2, 64, a, b, bf16, nullptr, nullptr) == SIGATTN_EINVAL);
  EXPECT(sigattn_fwd(q, k, v, o, n, n, 2, -64, 2, 64, a, b, bf16, nullptr, nullptr) == SIGATTN_EINVAL);
  EXPECT(sigattn_fwd(q, k, v, o, n, n, 2, 64, 2, 96, a, b, bf16, nullptr, nullptr) == SIGATTN_EINVAL);
  EXPECT(last_error_has("D must be"));
  EXPECT(sigattn_fwd(q, k, v, o, n, n, 2, 64, 2, 64, NAN, b, bf16, nullptr, nullptr) == SIGATTN_EINVAL);
  EXPECT(sigattn_fwd(q, k, v, o, n, n, 2, 64, 2, 64, a, INFINITY, bf16, nullptr, nullptr) == SIGATTN_EINVAL);
  EXPECT(sigattn_fwd(q, k, v, o, nullptr, n, 2, 64, 2, 64, a, b, bf16, nullptr, nullptr) == SIGATTN_EINVAL);
  EXPECT(sigattn_fwd(nullptr, k, v, o, n, n, 2, 64, 2, 64, a, b, bf16, nullptr, nullptr) == SIGATTN_EINVAL);
  EXPECT(last_error_has("NULL"));
  EXPECT(sigattn_fwd(misaligned, k, v, o, n, n, 2, 64, 2, 64, a, b, bf16, nullptr, nullptr) == SIGATTN_EINVAL);
  EXPECT(last_error_has("aligned"));
  EXPECT(sigattn_fwd(q, k, v, o, n, n, 0, 64, 2, 64, a, b, bf16, nullptr, nullptr) == SIGATTN_OK);  // empty batch
  EXPECT(sigattn_fwd(q, k, v, o, n, n, 65536, 1 << 20, 64, 128, a, b, bf16, nullptr, nullptr) == SIGATTN_EINVAL);
  EXPECT(last_error_has("too large"));
  EXPECT(sigattn_fwd(q, k, v, o, n, n, 1, 64, 1 << 23, 128, a, b, bf16, nullptr, nullptr) == SIGATTN_EINVAL);
  for (int D : {64, 128})
    for (sigattn_dtype t : {bf16, fp32}) {
      EXPECT(sigattn_fwd(q, k, v, o, n, n, 2, 300, 3, D, a, b, t, nullptr, nullptr) == SIGATTN_EHIP);
      EXPECT(last_error_has("HIP launch failed"));
    }

  // layouts and bias modes
  EXPECT(sigattn_fwd_ex(q, k, v, o, n, n, (sigattn_layout)5, SIGATTN_BIAS_CONSTANT, 2, 64, 2, 64, a, b, bf16, nullptr,
                        nullptr) == SIGATTN_EINVAL);
  EXPECT(sigattn_fwd_ex(q, k, v, o, n, n, SIGATTN_LAYOUT_PACKED, (sigattn_bias_mode)9, 2, 64, 2, 64, a, b, bf16,
                        nullptr, nullptr) == SIGATTN_EINVAL);
  EXPECT(sigattn_fwd_ex(q, k, v, o, n, n, SIGATTN_LAYOUT_PACKED, SIGATTN_BIAS_NEG_LOG_NK, 2, 64, 2, 64, a, 0.0f, bf16,
                        nullptr, nullptr) == SIGATTN_EHIP);

  // backward entry points
  EXPECT(sigattn_bwd(q, k, v, dout, nullptr, dk, dv, n, n, 2, 64, 2, 64, a, b, bf16, nullptr, nullptr, nullptr) ==
         SIGATTN_EINVAL);
  EXPECT(sigattn_bwd(q, k, v, dout, dq, dk, dv, n, n, 2, 64, 2, 64, a, b, bf16, nullptr, nullptr, nullptr) ==
         SIGATTN_EHIP);
  EXPECT(sigattn_bwd_ex(q, k, v, dout, dq, dk, dv, n, n, SIGATTN_LAYOUT_PACKED, SIGATTN_BIAS_CONSTANT, 2, 64, 2, 128,
                        a, b, fp32, nullptr, nullptr, nullptr) == SIGATTN_EHIP);
  EXPECT(sigattn_bwd_dkdv(q, k, v, dout, dk, nullptr, n, n, 2, 64, 2, 64, a, b, bf16, nullptr, nullptr) ==
         SIGATTN_EINVAL);
  EXPECT(sigattn_bwd_dkdv(q, k, v, dout, dk, dv, n, n, 2, 64, 2, 64, a, b, bf16, nullptr, nullptr) == SIGATTN_EHIP);
  EXPECT(sigattn_bwd_dq(q, k, v, misaligned, dq, n, n, 2, 64, 2, 64, a, b, bf16, nullptr, nullptr) == SIGATTN_EINVAL);
  EXPECT(sigattn_bwd_dq(q, k, v, dout, dq, n, n, 2, 64, 2, 128, a, b, bf16, nullptr, nullptr) == SIGATTN_EHIP);
  EXPECT(sigattn_bwd_dk(q, k, v, dout, dk, n, n, 2, 64, 2, 64, a, b, bf16, nullptr, nullptr) == SIGATTN_EHIP);
  EXPECT(sigattn_bwd_dv(q, k, dout, dv, n, n, 2, 64, 2, 64, a, b, (sigattn_dtype)3, nullptr, nullptr) ==
         SIGATTN_EUNSUPPORTED);
  EXPECT(sigattn_bwd_dv(q, k, dout, dv, n, n, 2, 64, 2, 64, a, b, bf16, nullptr, nullptr) == SIGATTN_EHIP);

  // softmax: forward, workspace size and check, and the allocation-free backward
  float* lse = g_lse;
  EXPECT(sigattn_softmax_fwd(q, k, v, o, nullptr, n, n, SIGATTN_LAYOUT_PADDED, 2, 64, 2, 64, a, bf16, nullptr) ==
         SIGATTN_EINVAL);
  EXPECT(sigattn_softmax_fwd(q, k, v, o, lse, n, n, SIGATTN_LAYOUT_PADDED, 2, 64, 2, 64, a, bf16, nullptr) ==
         SIGATTN_EHIP);
  const size_t ws = sigattn_softmax_bwd_workspace_size(2 * 64, 2);
  EXPECT(ws >= (size_t)2 * 64 * 2 * 8);
  std::vector<unsigned char> wsbuf(ws + 16);
  void* wsp = wsbuf.data() + ((16 - (reinterpret_cast<uintptr_t>(wsbuf.data()) & 15)) & 15);
  EXPECT(sigattn_softmax_bwd(q, k, v, o, dout, lse, dq, dk, dv, n, n, SIGATTN_LAYOUT_PADDED, 2, 64, 2, 64, a, bf16, wsp,
                             ws - 1, nullptr) == SIGATTN_EWORKSPACE);
  EXPECT(sigattn_softmax_bwd(q, k, v, o, dout, lse, dq, dk, dv, n, n, SIGATTN_LAYOUT_PADDED, 2, 64, 2, 64, a, bf16, wsp,
                             ws, nullptr) == SIGATTN_EHIP);
  EXPECT(sigattn_softmax_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, n, n, SIGATTN_LAYOUT_PADDED, 64, 8192, 8, 64,
                                     a, bf16, nullptr) == SIGATTN_EINVAL);
  EXPECT(last_error_has("SIGATTN_NOALLOC_ROWS"));
  // Within the limit the call asks HIP for the device of the stream and the
  // buffer's address; with no device present that fails cleanly.
  const int na = sigattn_softmax_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, n, n, SIGATTN_LAYOUT_PADDED, 2, 64, 2,
                                             64, a, bf16, nullptr);
  EXPECT(na == SIGATTN_EHIP || na == SIGATTN_OK);

  // FP8
  uint8_t* sc = reinterpret_cast<uint8_t*>(g_buf[9]);
  EXPECT(sigattn_quantize_fp8(q, g_buf[10], nullptr, n, SIGATTN_LAYOUT_PADDED, 2, 64, 2, 64, nullptr) ==
         SIGATTN_EINVAL);
  EXPECT(sigattn_quantize_fp8(q, g_buf[10], sc, n, SIGATTN_LAYOUT_PADDED, 2, 64, 2, 64, nullptr) == SIGATTN_EHIP);
  EXPECT(sigattn_fwd_fp8(q, k, v, sc, sc, sc, o, n, n, SIGATTN_LAYOUT_PADDED, SIGATTN_BIAS_CONSTANT, 2, 64, 2, 96, a, b,
                         nullptr) == SIGATTN_EINVAL);
  EXPECT(sigattn_fwd_fp8(q, k, v, sc, sc, sc, o, n, n, SIGATTN_LAYOUT_PADDED, SIGATTN_BIAS_CONSTANT, 2, 64, 2, 128, a,
                         b, nullptr) == SIGATTN_EHIP);

  // tile configuration
  int bq = 0, bk = 0;
  for (sigattn_kernel kern : {SIGATTN_KERNEL_FWD, SIGATTN_KERNEL_DQ, SIGATTN_KERNEL_DKDV})
    for (int D : {64, 128})
      for (sigattn_dtype t : {bf16, fp32}) {
        bq = bk = 0;
        EXPECT(sigattn_tile_config(kern, D, t, &bq, &bk) == SIGATTN_OK && bq > 0 && bk > 0);
      }
  EXPECT(sigattn_tile_config((sigattn_kernel)7, 64, bf16, &bq, &bk) != SIGATTN_OK);
  EXPECT(sigattn_tile_config(SIGATTN_KERNEL_FWD, 64, bf16, nullptr, &bk) == SIGATTN_EINVAL);

  // The last-error text belongs to the calling thread.
  std::vector<std::thread> pool;
  std::vector<int> bad(8, 0);
  for (int t = 0; t < 8; ++t)
    pool.emplace_back([&, t] {
      for (int i = 0; i < 2000; ++i) {
        if (t % 2 == 0) {
          if (sigattn_fwd(q, k, v, o, n, n, 2, 64, 2, 96, a, b, bf16, nullptr, nullptr) != SIGATTN_EINVAL ||
              std::strstr(sigattn_last_error(), "D must be") == nullptr)
            ++bad[t];
        } else {
          if (sigattn_fwd(misaligned, k, v, o, n, n, 2, 64, 2, 64, a, b, bf16, nullptr, nullptr) != SIGATTN_EINVAL ||
              std::strstr(sigattn_last_error(), "aligned") == nullptr)
            ++bad[t];
        }
      }
    });
  for (auto& th : pool) th.join();
  for (int t = 0; t < 8; ++t) EXPECT(bad[t] == 0);

  if (g_failures == 0) std::printf("host sanitizer driver: all checks passed\n");
  return g_failures == 0 ? 0 : 1;
}
