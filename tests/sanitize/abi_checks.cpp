// Host-side checks of the C ABI's argument validation, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of abi.cpp (test infrastructure).  Every
// call below must be refused (or accepted as an empty no-op) by the argument checks,
// so no device is touched: fake pointers stand in for device buffers and are never
// dereferenced.  Exit status 0 when every status matches, 1 otherwise.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "pql.h"

static int failures = 0;

static void expect(const char* what, pql_status got, pql_status want) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, (int)got, (int)want, pql_last_error());
    ++failures;
  }
}

static void* P(uintptr_t off = 0) { return reinterpret_cast<void*>((uintptr_t)1 << 20 | off); }

int main() {
  const int A = PQL_ACTIVATION, W = PQL_WEIGHT;
  size_t c = 0, s = 0, z = 0;
  // sizes
  expect("sizes fp8_row", pql_quantized_sizes(PQL_FP8_ROW, W, 12288, 3072, &c, &s, &z), PQL_OK);
  if (c != 12288u * 3072u || s != 4u * 12288u || z != 0) { std::printf("FAIL sizes values\n"); ++failures; }
  expect("sizes mxfp4_dual", pql_quantized_sizes(PQL_MXFP4_DUAL, A, 20280, 5120, &c, &s, &z), PQL_OK);
  expect("sizes K % 32", pql_quantized_sizes(PQL_FP8_ROW, A, 4, 48, &c, &s, &z), PQL_ERR_INVALID_ARGUMENT);
  expect("sizes block weight rows", pql_quantized_sizes(PQL_FP8_BLOCK128, W, 64, 128, &c, &s, &z),
         PQL_ERR_INVALID_ARGUMENT);
  expect("sizes negative", pql_quantized_sizes(PQL_FP8_ROW, A, -1, 64, &c, &s, &z), PQL_ERR_INVALID_ARGUMENT);
  expect("sizes 2^51", pql_quantized_sizes(PQL_FP8_BLOCK128, W, (int64_t(1) << 31) - 128, 1 << 20, &c, &s, &z),
         PQL_ERR_INVALID_ARGUMENT);
  expect("sizes int64 extremes", pql_quantized_sizes(PQL_FP8_ROW, A, INT64_MAX, INT64_MAX, &c, &s, &z),
         PQL_ERR_INVALID_ARGUMENT);
  expect("sizes w4a16 activation", pql_quantized_sizes(PQL_W4A16_ASYM, A, 4, 128, &c, &s, &z), PQL_ERR_UNSUPPORTED);
  expect("sizes unknown scheme", pql_quantized_sizes(99, A, 4, 128, &c, &s, &z), PQL_ERR_UNSUPPORTED);
  expect("sizes unknown role", pql_quantized_sizes(PQL_FP8_ROW, 7, 4, 128, &c, &s, &z), PQL_ERR_UNSUPPORTED);
  expect("layout sizes bad layout", pql_layout_sizes(PQL_MXFP8, W, 2, 4, 64, &c, &s, &z), PQL_ERR_INVALID_ARGUMENT);
  expect("workspace unknown op", pql_workspace_size(17, PQL_FP8_ROW, A, 16, 128, 128, &c), PQL_ERR_INVALID_ARGUMENT);
  expect("workspace NULL", pql_workspace_size(PQL_OP_QLINEAR, PQL_FP8_ROW, A, 16, 128, 128, nullptr),
         PQL_ERR_INVALID_ARGUMENT);
  expect("workspace qlinear K", pql_workspace_size(PQL_OP_QLINEAR, PQL_FP8_ROW, A, 16, 128, 100, &c),
         PQL_ERR_INVALID_ARGUMENT);
  expect("workspace fused", pql_workspace_size(PQL_OP_QLINEAR, PQL_FP8_ROW, A, 16, 12288, 3072, &c), PQL_OK);
  if (c != 0) { std::printf("FAIL fused workspace %zu\n", c); ++failures; }

  // quantize
  auto q = [&](int scheme, int role, void* x, int64_t rows, int64_t cols, int64_t ldx, void* zeros, void* ws,
               size_t wsb) { return pql_quantize(scheme, role, x, rows, cols, ldx, P(4096), P(8192), zeros, ws, wsb,
                                                 nullptr); };
  expect("quantize NULL x", q(PQL_FP8_ROW, A, nullptr, 16, 128, 128, nullptr, nullptr, 0), PQL_ERR_INVALID_ARGUMENT);
  expect("quantize ldx < cols", q(PQL_FP8_ROW, A, P(), 16, 128, 120, nullptr, nullptr, 0), PQL_ERR_INVALID_ARGUMENT);
  expect("quantize ldx % 8", q(PQL_FP8_ROW, A, P(), 16, 128, 132, nullptr, nullptr, 0), PQL_ERR_INVALID_ARGUMENT);
  expect("quantize misaligned", q(PQL_FP8_ROW, A, P(4), 16, 128, 128, nullptr, nullptr, 0), PQL_ERR_INVALID_ARGUMENT);
  expect("quantize w4a16 zeros", q(PQL_W4A16_ASYM, W, P(), 16, 128, 128, nullptr, nullptr, 0),
         PQL_ERR_INVALID_ARGUMENT);
  expect("quantize tensor workspace", q(PQL_FP8_TENSOR, A, P(), 16, 128, 128, nullptr, nullptr, 0), PQL_ERR_WORKSPACE);
  expect("quantize tensor small ws", q(PQL_FP8_TENSOR, A, P(), 16, 128, 128, nullptr, P(16384), 64),
         PQL_ERR_WORKSPACE);
  expect("quantize empty", q(PQL_FP8_ROW, A, P(), 0, 128, 128, nullptr, nullptr, 0), PQL_OK);
  expect("quantize huge ldx", q(PQL_FP8_ROW, A, P(), 16, 128, INT64_MAX - 7, nullptr, nullptr, 0),
         PQL_ERR_INVALID_ARGUMENT);
  expect("static per-row", pql_quantize_static(PQL_FP8_ROW, A, P(), 16, 128, 128, P(4096), P(8192), nullptr),
         PQL_ERR_UNSUPPORTED);
  expect("static misaligned", pql_quantize_static(PQL_FP8_TENSOR, A, P(), 16, 128, 128, P(4100), P(8192), nullptr),
         PQL_ERR_INVALID_ARGUMENT);

  // dequantize
  expect("dequantize NULL", pql_dequantize(PQL_MXFP4, A, nullptr, P(4096), nullptr, 16, 128, P(8192), 128, nullptr),
         PQL_ERR_INVALID_ARGUMENT);
  expect("dequantize ldy", pql_dequantize(PQL_MXFP4, A, P(), P(4096), nullptr, 16, 128, P(8192), 64, nullptr),
         PQL_ERR_INVALID_ARGUMENT);

  // GEMMs
  auto g = [&](int scheme, int64_t M, int64_t N, int64_t K, int64_t ldc, void* wz, float alpha, void* bias) {
    return pql_qgemm_ex(scheme, P(), P(1024), P(2048), P(3072), wz, M, N, K, alpha, bias, P(8192), ldc, nullptr);
  };
  expect("qgemm K", g(PQL_FP8_ROW, 16, 256, 200, 256, nullptr, 1.f, nullptr), PQL_ERR_INVALID_ARGUMENT);
  expect("qgemm N 0", g(PQL_FP8_ROW, 16, 0, 256, 256, nullptr, 1.f, nullptr), PQL_ERR_INVALID_ARGUMENT);
  expect("qgemm ldc", g(PQL_FP8_ROW, 16, 256, 256, 100, nullptr, 1.f, nullptr), PQL_ERR_INVALID_ARGUMENT);
  expect("qgemm w4a16 zeros", g(PQL_W4A16_ASYM, 16, 256, 256, 256, nullptr, 1.f, nullptr), PQL_ERR_INVALID_ARGUMENT);
  expect("qgemm block N", g(PQL_FP8_BLOCK128, 16, 200, 256, 200, nullptr, 1.f, nullptr), PQL_ERR_INVALID_ARGUMENT);
  expect("qgemm tiles", g(PQL_FP8_ROW, int64_t(1) << 30, int64_t(1) << 30, 256, int64_t(1) << 30, nullptr, 1.f,
                          nullptr), PQL_ERR_INVALID_ARGUMENT);
  expect("qgemm int64 M", g(PQL_FP8_ROW, INT64_MAX, 256, 256, 256, nullptr, 1.f, nullptr), PQL_ERR_INVALID_ARGUMENT);
  expect("qgemm MX alpha", g(PQL_MXFP8, 16, 256, 256, 256, nullptr, 2.f, nullptr), PQL_ERR_UNSUPPORTED);
  expect("qgemm NaN alpha", g(PQL_FP8_ROW, 16, 256, 256, 256, nullptr, std::nanf(""), nullptr),
         PQL_ERR_INVALID_ARGUMENT);
  expect("qgemm odd N bias", g(PQL_FP8_ROW, 16, 255, 256, 256, nullptr, 1.f, P(4096)), PQL_ERR_INVALID_ARGUMENT);
  expect("qgemm empty", g(PQL_MXFP8, 0, 256, 256, 256, nullptr, 1.f, nullptr), PQL_OK);
  expect("qgemm dual K", g(PQL_MXFP4_DUAL, 16, 256, 256, 256, nullptr, 1.f, nullptr), PQL_ERR_INVALID_ARGUMENT);

  auto l = [&](int scheme, int64_t M, int64_t K, int64_t lda, void* st, void* ws, size_t wsb) {
    return pql_qlinear_ex(scheme, P(), M, K, lda, st, P(2048), P(3072), nullptr, 256, 1.f, nullptr, P(8192), 256, ws,
                          wsb, nullptr);
  };
  expect("qlinear workspace", l(PQL_MXFP8, 16, 256, 256, nullptr, P(16384), 64), PQL_ERR_WORKSPACE);
  expect("qlinear no workspace", l(PQL_MXFP8, 16, 256, 256, nullptr, nullptr, 0), PQL_ERR_WORKSPACE);
  expect("qlinear lda", l(PQL_MXFP8, 16, 256, 250, nullptr, P(16384), 1 << 20), PQL_ERR_INVALID_ARGUMENT);
  expect("qlinear static row", l(PQL_FP8_ROW, 16, 256, 256, P(512), P(16384), 1 << 20), PQL_ERR_UNSUPPORTED);
  expect("qlinear static misaligned", l(PQL_FP8_TENSOR, 16, 256, 256, P(516), P(16384), 1 << 20),
         PQL_ERR_INVALID_ARGUMENT);
  expect("qlinear empty", l(PQL_FP8_ROW, 0, 256, 256, nullptr, nullptr, 0), PQL_OK);
  const int64_t Mbig = int64_t(pql_noalloc_scratch_bytes() / 4096 + 1);
  expect("noalloc limit", pql_qlinear_noalloc(PQL_FP8_ROW, P(), Mbig, 4096, 4096, nullptr, P(), P(), nullptr, 128, 1.f,
                                              nullptr, P(), 128, nullptr), PQL_ERR_WORKSPACE);

  // repack
  expect("repack layout", pql_repack(PQL_MXFP8, W, 0, 3, P(), nullptr, P(4096), nullptr, 4, 64, nullptr),
         PQL_ERR_INVALID_ARGUMENT);
  expect("repack in place", pql_repack(PQL_MXFP4, W, 0, 1, P(), nullptr, P(), nullptr, 4, 64, nullptr),
         PQL_ERR_INVALID_ARGUMENT);
  expect("repack w4a16 zeros", pql_repack(PQL_W4A16_ASYM, W, 1, 0, P(), nullptr, P(4096), P(8192), 4, 128, nullptr),
         PQL_ERR_INVALID_ARGUMENT);

  // introspection over every op, scheme and a spread of shapes (string lifetimes and formatting)
  for (int op = 0; op <= 4; ++op)
    for (int scheme = 0; scheme <= 9; ++scheme)
      for (int64_t M : {int64_t(0), int64_t(1), int64_t(16), int64_t(17), int64_t(4096), int64_t(1) << 30}) {
        const char* n = pql_kernel_name(op, scheme, A, M, 12288, 3072);
        if (!n) { std::printf("FAIL kernel_name NULL\n"); ++failures; }
        else (void)std::strlen(n);
      }
  (void)std::strlen(pql_last_error());
  if (pql_version() < 1) { std::printf("FAIL version\n"); ++failures; }
  std::printf("%s: %d failures\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
