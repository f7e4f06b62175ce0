// Host-side driver for the sanitizer build of the C ABI (AddressSanitizer +
// UndefinedBehaviorSanitizer on the API layer's host code).  It runs every
// validation path of include/ffn.h that returns before a launch, the
// per-thread timing state from two threads, the error text, workspace
// sizes and the no-allocation entry point's size check.  No GPU is needed:
// every call below fails validation or is a no-op.  Exit status 0 and the
// line "abi driver ok" on success.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <thread>

#include "ffn.h"

static int failures = 0;
#define EXPECT(cond)                                                         \
  do {                                                                       \
    if (!(cond)) {                                                           \
      std::fprintf(stderr, "FAILED line %d: %s (last error: %s)\n", __LINE__, \
                   #cond, ffn_last_error());                                 \
      ++failures;                                                            \
    }                                                                        \
  } while (0)

// fake device addresses, never dereferenced
static void* P(unsigned long v) { return reinterpret_cast<void*>(v); }
static const unsigned long A = 0x10000000, B = 0x20000000, C = 0x30000000, D = 0x40000000,
                           E = 0x50000000, Y = 0x60000000, WS = 0x70000000;

static ffn_status block(ffn_dtype dt, unsigned long x, unsigned long y, int64_t M, int64_t d, int64_t f,
                        float eps, int v, unsigned long ws, size_t wsb) {
  return ffn_swiglu_block(dt, P(x), P(B), P(C), P(D), P(E), P(y), M, d, f, eps, (ffn_variant)v, P(ws),
                          wsb, nullptr);
}

int main() {
  const size_t big = (size_t)1 << 30;
  // ---- block validation
  EXPECT(block(FFN_BF16, 0, Y, 16, 4096, 11008, 1e-6f, 0, WS, big) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(block((ffn_dtype)7, A, Y, 16, 4096, 11008, 1e-6f, 0, WS, big) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(block(FFN_BF16, A, Y, 16, 4096, 11008, 1e-6f, 9, WS, big) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(block(FFN_BF16, A, Y, -1, 4096, 11008, 1e-6f, 0, WS, big) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(block(FFN_BF16, A, Y, 16, 0, 11008, 1e-6f, 0, WS, big) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(block(FFN_BF16, A, Y, 16, 4096, 11008, -1.f, 0, WS, big) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(block(FFN_BF16, A, Y, 16, 4096, 11008, NAN, 0, WS, big) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(block(FFN_BF16, A, Y, 16, 4096, 11008, INFINITY, 0, WS, big) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(block(FFN_BF16, A, Y, 16, 4100, 11008, 1e-6f, 0, WS, big) == FFN_ERR_UNSUPPORTED);
  EXPECT(block(FFN_BF16, A + 2, Y, 16, 4096, 11008, 1e-6f, 0, WS, big) == FFN_ERR_UNSUPPORTED);
  EXPECT(block(FFN_BF16, A, Y, 16, 4096, 11008, 1e-6f, 0, WS + 16, big) == FFN_ERR_UNSUPPORTED);
  EXPECT(block(FFN_BF16, A, Y, 16, 4096, 11008, 1e-6f, 0, WS, 100) == FFN_ERR_WORKSPACE);
  EXPECT(std::strstr(ffn_last_error(), "workspace") != nullptr);
  EXPECT(block(FFN_BF16, A, A, 16, 4096, 11008, 1e-6f, 0, WS, big) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(block(FFN_BF16, A, WS, 16, 4096, 11008, 1e-6f, 0, WS, big) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(block(FFN_BF16, A, Y, 17, 4096, 11008, 1e-6f, 3, WS, big) == FFN_ERR_UNSUPPORTED);
  EXPECT(block(FFN_BF16, A, Y, (int64_t)1 << 40, 4096, 11008, 1e-6f, 0, WS, big) == FFN_ERR_UNSUPPORTED);
  EXPECT(block(FFN_BF16, A, Y, 16, (int64_t)1 << 33, 8, 1e-6f, 0, WS, big) == FFN_ERR_UNSUPPORTED);
  EXPECT(block(FFN_BF16, A, Y, 0, 4096, 11008, 1e-6f, 0, 0, 0) == FFN_OK);
  EXPECT(std::strcmp(ffn_last_error(), "") == 0);
  // ---- workspace sizes, including extreme and invalid shapes
  EXPECT(ffn_swiglu_block_workspace_size(FFN_BF16, 16, 4096, 11008, FFN_VARIANT_FUSED) > 0);
  EXPECT(ffn_swiglu_block_workspace_size((ffn_dtype)5, 16, 4096, 11008, FFN_VARIANT_FUSED) == 0);
  EXPECT(ffn_swiglu_block_workspace_size(FFN_BF16, -1, 4096, 11008, FFN_VARIANT_FUSED) == 0);
  EXPECT(ffn_swiglu_block_workspace_size(FFN_BF16, 16, 4096, 11008, (ffn_variant)17) == 0);
  EXPECT(ffn_swiglu_block_workspace_size(FFN_BF16, 17, 4096, 11008, FFN_VARIANT_PERSISTENT) == 0);
  EXPECT(ffn_swiglu_block_persistent_status_offset(16, 4096, 11008) > 0);
  EXPECT(ffn_swiglu_block_persistent_status_offset(0, 4096, 11008) == 0);
  EXPECT(ffn_swiglu_block_q8_workspace_size(8, 5120, 17408) > 0);
  EXPECT(ffn_swiglu_block_q8_workspace_size(65, 5120, 17408) == 0);
  EXPECT(ffn_swiglu_block_q4_workspace_size(8, 5120, (int64_t)1 << 40) == 0);
  // ---- rmsnorm
  EXPECT(ffn_rmsnorm(FFN_BF16, nullptr, P(B), P(Y), 4, 64, 1e-6f, nullptr) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(ffn_rmsnorm(FFN_BF16, P(A), P(B), P(Y), 4, 60, 1e-6f, nullptr) == FFN_ERR_UNSUPPORTED);
  EXPECT(ffn_rmsnorm(FFN_F32, P(A), P(B), P(A + 16), 4, 64, 1e-6f, nullptr) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(ffn_rmsnorm(FFN_BF16, P(A), P(B), P(Y), 0, 64, 1e-6f, nullptr) == FFN_OK);
  // ---- quantised blocks
  ffn_q8_matrix q8a = {(const int8_t*)P(C), (const uint16_t*)P(D)};
  ffn_q8_matrix q8b = {(const int8_t*)P(E), (const uint16_t*)P(E + 0x1000000)};
  ffn_q8_matrix q8c = {(const int8_t*)P(E + 0x2000000), (const uint16_t*)P(E + 0x3000000)};
  ffn_q8_matrix q8bad = {(const int8_t*)P(C + 8), (const uint16_t*)P(D)};
  EXPECT(ffn_swiglu_block_q8(P(A), P(B), &q8a, &q8b, &q8c, P(Y), 8, 5128, 17408, 1e-6f, P(WS), big, nullptr) ==
         FFN_ERR_UNSUPPORTED);
  EXPECT(ffn_swiglu_block_q8(P(A), P(B), &q8bad, &q8b, &q8c, P(Y), 8, 5120, 17408, 1e-6f, P(WS), big, nullptr) ==
         FFN_ERR_UNSUPPORTED);
  EXPECT(ffn_swiglu_block_q8(P(A), P(B), nullptr, &q8b, &q8c, P(Y), 8, 5120, 17408, 1e-6f, P(WS), big, nullptr) ==
         FFN_ERR_INVALID_ARGUMENT);
  EXPECT(ffn_swiglu_block_q8(P(A), P(B), &q8a, &q8b, &q8c, P(Y), 65, 5120, 17408, 1e-6f, P(WS), big, nullptr) ==
         FFN_ERR_UNSUPPORTED);
  ffn_q4_matrix q4a = {(const uint8_t*)P(C), (const uint16_t*)P(D)};
  ffn_q4_matrix q4b = {(const uint8_t*)P(E), (const uint16_t*)P(E + 0x1000001)};
  EXPECT(ffn_swiglu_block_q4(P(A), P(B), &q4a, &q4b, &q4a, P(Y), 8, 5120, 17408, 1e-6f, P(WS), big, nullptr) ==
         FFN_ERR_UNSUPPORTED);
  EXPECT(ffn_swiglu_block_q4(P(A), P(B), &q4a, &q4a, &q4a, P(Y), 0, 5120, 17408, 1e-6f, nullptr, 0, nullptr) ==
         FFN_OK);
  // ---- no-allocation entry point: sizes beyond its array, invalid calls, no-ops
  EXPECT(ffn_swiglu_block_noalloc(FFN_BF16, P(A), P(B), P(C), P(D), P(E), P(Y), 8192, 4096, 14336, 1e-6f,
                                  FFN_VARIANT_FUSED, nullptr) == FFN_ERR_UNSUPPORTED);
  EXPECT(std::strstr(ffn_last_error(), "scratch") != nullptr);
  EXPECT(ffn_swiglu_block_noalloc(FFN_BF16, nullptr, P(B), P(C), P(D), P(E), P(Y), 16, 4096, 11008, 1e-6f,
                                  FFN_VARIANT_FUSED, nullptr) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(ffn_swiglu_block_noalloc(FFN_BF16, P(A), P(B), P(C), P(D), P(E), P(Y), 0, 4096, 11008, 1e-6f,
                                  FFN_VARIANT_FUSED, nullptr) == FFN_OK);
  // ---- probes
  EXPECT(ffn_probe_read(P(A), 15, P(B), 4, nullptr) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(ffn_probe_copy(P(A), P(A + 16), 64, 0, 0, nullptr) == FFN_ERR_INVALID_ARGUMENT);
  EXPECT(ffn_probe_mfma(0, 8, P(A), nullptr) == FFN_ERR_INVALID_ARGUMENT);
  // ---- status strings
  for (int s = 0; s < 6; ++s) EXPECT(ffn_status_string((ffn_status)s) != nullptr);
  EXPECT(std::strcmp(ffn_status_string((ffn_status)99), "FFN_ERR_UNKNOWN") == 0);
  // ---- timing state per thread (enable, query, collect with nothing
  // recorded, get out of range, reset, disable)
  EXPECT(ffn_timing_enable(1, 0) == FFN_ERR_INVALID_ARGUMENT);
  int a_on = -1, b_on = -1, a_after = -1;
  std::thread ta([&] {
    if (ffn_timing_enable(1, 1024) != FFN_OK) ++failures;
    a_on = ffn_timing_enabled();
    std::thread tb([&] {
      b_on = ffn_timing_enabled();
      if (ffn_timing_enable(0, 0) != FFN_OK) ++failures;
    });
    tb.join();
    a_after = ffn_timing_enabled();
    if (ffn_timing_collect() != FFN_OK) ++failures;
    if (ffn_timing_count() != 0) ++failures;
    const char* nm = nullptr;
    int64_t n = 0;
    double ms = 0;
    if (ffn_timing_get(0, &nm, &n, &ms) != FFN_ERR_INVALID_ARGUMENT) ++failures;
    ffn_timing_reset();
    if (ffn_timing_enable(0, 0) != FFN_OK) ++failures;
  });
  ta.join();
  EXPECT(a_on == 1 && b_on == 0 && a_after == 1);
  EXPECT(ffn_timing_enabled() == 0);
  if (failures) {
    std::fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  std::printf("abi driver ok\n");
  return 0;
}
