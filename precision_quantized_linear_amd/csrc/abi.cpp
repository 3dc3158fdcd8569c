// C ABI of libpql (declared in include/pql.h): argument validation, size
// queries, device checks and dispatch to the kernel launchers.
//
// Every check runs before anything is enqueued; errors raise instead of
// silently reinterpreting data, in the spirit of the pages' own loaders (an
// unknown method or an unsupported platform is an error, never a fallback:
// "vLLM-Omni Online Quantization complete guide", sections "Hardware support
// matrix" and "Configuration").
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "../../include/pql.h"
#include "pql_internal.hpp"

namespace {

thread_local std::string g_error;

pql_status fail(pql_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

pql_status ok() {
  g_error.clear();
  return PQL_OK;
}

const char* scheme_name(int s) {
  switch (s) {
    case PQL_FP8_TENSOR: return "FP8_TENSOR";
    case PQL_FP8_ROW: return "FP8_ROW";
    case PQL_FP8_BLOCK128: return "FP8_BLOCK128";
    case PQL_MXFP8: return "MXFP8";
    case PQL_MXFP4: return "MXFP4";
    case PQL_W4A16_ASYM: return "W4A16_ASYM";
    case PQL_W4A16_SYM: return "W4A16_SYM";
    case PQL_INT8_ROW: return "INT8_ROW";
    case PQL_MXFP4_DUAL: return "MXFP4_DUAL";
  }
  return "?";
}

bool is_w4a16(int s) { return s == PQL_W4A16_ASYM || s == PQL_W4A16_SYM; }
bool is_mx(int s) { return s == PQL_MXFP8 || s == PQL_MXFP4; }
bool valid_scheme(int s) { return s >= PQL_FP8_TENSOR && s <= PQL_MXFP4_DUAL; }
// Schemes whose GEMM takes the fused epilogue alpha * (A W^T) + bias.
bool has_epilogue(int s) { return s == PQL_FP8_TENSOR || s == PQL_FP8_ROW || s == PQL_FP8_BLOCK128 || s == PQL_INT8_ROW; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

// A leading dimension: at least `cols`, a multiple of 8 where asked, and the addressed
// span (rows - 1) * ld + cols at most 2^40 elements, so that every in-kernel offset
// (row * ld in 64-bit arithmetic) stays in range.
constexpr int64_t kMaxSpan = int64_t(1) << 40;
pql_status check_ld(const char* name, int64_t ld, int64_t rows, int64_t cols, bool mult8) {
  if (ld < cols || (mult8 && ld % 8))
    return fail(PQL_ERR_INVALID_ARGUMENT, "%s must be >= %lld%s (got %lld)", name, (long long)cols,
                mult8 ? " and a multiple of 8" : "", (long long)ld);
  if (rows > 1 && ld > (kMaxSpan - cols) / (rows - 1))
    return fail(PQL_ERR_INVALID_ARGUMENT, "%s = %lld spans more than 2^40 elements over %lld rows", name,
                (long long)ld, (long long)rows);
  return PQL_OK;
}

int64_t k_granule(int scheme) {
  return scheme == PQL_MXFP4_DUAL ? 512 : (scheme == PQL_FP8_BLOCK128 || is_w4a16(scheme)) ? 128 : 32;
}

// Dual-scale MXFP4 keeps both scale levels in its scales buffer: the fine e8m0
// exponents (rows * cols / 32 bytes), then, from the next 256-byte boundary,
// the coarse fp32 scales (rows * cols / 512 of them).
size_t dual_coarse_offset(int64_t rows, int64_t cols) { return ((size_t)rows * (size_t)(cols / 32) + 255) & ~size_t(255); }

pql_status check_scheme_role(int scheme, int role) {
  if (!valid_scheme(scheme)) return fail(PQL_ERR_UNSUPPORTED, "unknown scheme %d", scheme);
  if (role != PQL_ACTIVATION && role != PQL_WEIGHT) return fail(PQL_ERR_UNSUPPORTED, "unknown role %d", role);
  if (is_w4a16(scheme) && role == PQL_ACTIVATION)
    return fail(PQL_ERR_UNSUPPORTED, "%s quantizes weights only; activations stay bf16", scheme_name(scheme));
  return PQL_OK;
}

// Shape rules shared by quantize / dequantize / sizes.
pql_status check_shape(int scheme, int role, int64_t rows, int64_t cols) {
  if (rows < 0 || cols <= 0) return fail(PQL_ERR_INVALID_ARGUMENT, "rows must be >= 0 and cols > 0 (got %lld, %lld)",
                                         (long long)rows, (long long)cols);
  const int64_t gk = k_granule(scheme);
  if (cols % gk) return fail(PQL_ERR_INVALID_ARGUMENT, "%s needs cols %% %lld == 0 (got %lld)", scheme_name(scheme),
                             (long long)gk, (long long)cols);
  if (scheme == PQL_FP8_BLOCK128 && role == PQL_WEIGHT && rows % 128)
    return fail(PQL_ERR_INVALID_ARGUMENT, "FP8_BLOCK128 weights need rows %% 128 == 0 (got %lld)", (long long)rows);
  if (cols > (int64_t(1) << 20)) return fail(PQL_ERR_INVALID_ARGUMENT, "cols above 2^20 is not supported");
  if (rows > (int64_t(1) << 31) - 1) return fail(PQL_ERR_INVALID_ARGUMENT, "rows above 2^31-1 is not supported");
  // Launch grids are counted in 32-bit integers; 2^40 elements (2 TiB of bf16)
  // is far beyond any device's memory.
  if (rows > ((int64_t(1) << 40) / cols))
    return fail(PQL_ERR_INVALID_ARGUMENT, "a %lld x %lld tensor is too large", (long long)rows, (long long)cols);
  return PQL_OK;
}

struct Sizes { size_t codes, scales, zeros; };

Sizes sizes_of(int scheme, int role, int64_t rows, int64_t cols) {
  Sizes s{0, 0, 0};
  const size_t R = (size_t)rows, C = (size_t)cols;
  switch (scheme) {
    case PQL_FP8_TENSOR: s.codes = R * C; s.scales = 4; break;
    case PQL_FP8_ROW:
    case PQL_INT8_ROW: s.codes = R * C; s.scales = 4 * R; break;
    case PQL_FP8_BLOCK128:
      s.codes = R * C;
      s.scales = role == PQL_ACTIVATION ? 4 * R * (C / 128) : 4 * (R / 128) * (C / 128);
      break;
    case PQL_MXFP8: s.codes = R * C; s.scales = R * pql::mx_packed_row_bytes(C, false); break;
    case PQL_MXFP4: s.codes = R * C / 2; s.scales = R * pql::mx_packed_row_bytes(C, true); break;
    case PQL_MXFP4_DUAL: s.codes = R * C / 2; s.scales = dual_coarse_offset(rows, cols) + 4 * R * (C / 512); break;
    default: s.codes = R * C / 2; s.scales = 2 * R * (C / 128); s.zeros = R * (C / 128); break;
  }
  return s;
}

constexpr size_t kTensorWs = 4 * (size_t)pql::kTensorAmaxBlocks;

// gfx950 check, cached per device.
std::atomic<int> g_dev_state[64];

pql_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PQL_ERR_HIP, "no usable HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(PQL_ERR_HIP, "device index %d out of range", dev);
  int st = g_dev_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail(PQL_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
    st = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_relaxed);
    if (st == 2) return fail(PQL_ERR_UNSUPPORTED, "device %d is %s; libpql targets gfx950 only", dev, prop.gcnArchName);
  }
  if (st == 2) return fail(PQL_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return PQL_OK;
}

pql_status launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PQL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// Launch log: with the environment variable PQL_LOG set (to anything but "" or
// "0"; read once per process), every call of the entry points that enqueue work
// writes one line to stderr: the call, scheme, role and shape, the kernel it
// runs (the name pql_kernel_name reports) and the outcome, with the error
// message when a check rejected it.
bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("PQL_LOG");
    return v != nullptr && *v != '\0' && std::strcmp(v, "0") != 0;
  }();
  return on;
}

void log_call(pql_status st, const char* call, int scheme, int role, int64_t M, int64_t N, int64_t K,
              const char* kernel, const void* stream) {
  const char* role_name = role == PQL_ACTIVATION ? " activation" : role == PQL_WEIGHT ? " weight" : "";
  if (st != PQL_OK)
    std::fprintf(stderr, "[pql] %s %s%s M=%lld N=%lld K=%lld: rejected (status %d): %s\n", call, scheme_name(scheme),
                 role_name, (long long)M, (long long)N, (long long)K, (int)st, g_error.c_str());
  else if (M == 0)
    std::fprintf(stderr, "[pql] %s %s%s M=0 N=%lld K=%lld: nothing to do\n", call, scheme_name(scheme), role_name,
                 (long long)N, (long long)K);
  else
    std::fprintf(stderr, "[pql] %s %s%s M=%lld N=%lld K=%lld -> %s on stream %p\n", call, scheme_name(scheme),
                 role_name, (long long)M, (long long)N, (long long)K, kernel, stream);
}

// Quantize without re-validating (shared by pql_quantize and pql_qlinear).
hipError_t do_quantize(int scheme, int role, const void* x, int64_t rows, int64_t cols, int64_t ldx, void* codes,
                       void* scales, void* zeros, void* ws, hipStream_t st) {
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  uint8_t* cb = static_cast<uint8_t*>(codes);
  switch (scheme) {
    case PQL_FP8_TENSOR:
      return pql::launch_quant_fp8_tensor(xb, rows, cols, ldx, cb, static_cast<float*>(scales),
                                          static_cast<float*>(ws), st);
    case PQL_FP8_ROW: return pql::launch_quant_fp8_row(xb, rows, cols, ldx, cb, static_cast<float*>(scales), st);
    case PQL_INT8_ROW: return pql::launch_quant_int8_row(xb, rows, cols, ldx, cb, static_cast<float*>(scales), st);
    case PQL_FP8_BLOCK128:
      return role == PQL_ACTIVATION
                 ? pql::launch_quant_fp8_block_act(xb, rows, cols, ldx, cb, static_cast<float*>(scales), st)
                 : pql::launch_quant_fp8_block_wt(xb, rows, cols, ldx, cb, static_cast<float*>(scales), st);
    case PQL_MXFP8:
    case PQL_MXFP4:
      return pql::launch_quant_mx(scheme == PQL_MXFP4, xb, rows, cols, ldx, cb, static_cast<uint8_t*>(scales), st);
    case PQL_MXFP4_DUAL:
      return pql::launch_quant_mx4_dual(xb, rows, cols, ldx, cb, static_cast<uint8_t*>(scales),
                                        reinterpret_cast<float*>(static_cast<uint8_t*>(scales) +
                                                                 dual_coarse_offset(rows, cols)),
                                        st);
    default:
      return pql::launch_quant_int4(scheme == PQL_W4A16_SYM, xb, rows, cols, ldx, static_cast<uint32_t*>(codes),
                                    static_cast<uint16_t*>(scales), static_cast<uint8_t*>(zeros), st);
  }
}

pql::GemmKind gemm_kind(int scheme) {
  return scheme == PQL_FP8_BLOCK128 ? pql::GEMM_FP8_BLOCK
         : scheme == PQL_MXFP8      ? pql::GEMM_MXFP8
         : scheme == PQL_MXFP4      ? pql::GEMM_MXFP4
         : scheme == PQL_INT8_ROW   ? pql::GEMM_INT8_ROW
                                    : pql::GEMM_FP8_ROWSCALE;
}

hipError_t do_qgemm(int scheme, const void* a, const void* a_scales, const void* w_codes, const void* w_scales,
                    const void* w_zeros, int64_t M, int64_t N, int64_t K, float alpha, const void* bias, void* c,
                    int64_t ldc, hipStream_t st) {
  if (scheme == PQL_MXFP4_DUAL) {   // alpha = 1 and no bias here (checked by the callers)
    pql::GemmArgs g{};
    g.a = static_cast<const uint8_t*>(a);
    g.w = static_cast<const uint8_t*>(w_codes);
    g.a_scales = a_scales;
    g.w_scales = w_scales;
    g.M = M;
    g.N = N;
    g.K = K;
    g.c = static_cast<uint16_t*>(c);
    g.ldc = ldc;
    g.vec_store = aligned16(c) && ldc % 8 == 0;
    g.alpha = 1.0f;
    const float* ac = reinterpret_cast<const float*>(static_cast<const uint8_t*>(a_scales) + dual_coarse_offset(M, K));
    const float* wc = reinterpret_cast<const float*>(static_cast<const uint8_t*>(w_scales) + dual_coarse_offset(N, K));
    return pql::launch_gemm_mx4_dual(g, ac, wc, st);
  }
  if (is_w4a16(scheme))   // alpha = 1 and no bias here (checked by the callers)
    return pql::launch_gemm_w4a16(static_cast<const uint16_t*>(a), static_cast<const uint32_t*>(w_codes),
                                  static_cast<const uint16_t*>(w_scales), static_cast<const uint8_t*>(w_zeros), M, N,
                                  K, static_cast<uint16_t*>(c), ldc, st);
  pql::GemmArgs g;
  g.a = static_cast<const uint8_t*>(a);
  g.w = static_cast<const uint8_t*>(w_codes);
  g.a_scales = a_scales;
  g.w_scales = w_scales;
  g.a_scale_stride = scheme == PQL_FP8_TENSOR ? 0 : 1;
  g.w_scale_stride = scheme == PQL_FP8_TENSOR ? 0 : 1;
  g.M = M;
  g.N = N;
  g.K = K;
  g.c = static_cast<uint16_t*>(c);
  g.ldc = ldc;
  g.vec_store = aligned16(c) && ldc % 8 == 0;
  g.alpha = alpha;
  g.bias = static_cast<const uint16_t*>(bias);
  return pql::launch_gemm(gemm_kind(scheme), g, st);
}

pql_status check_gemm_shape(int scheme, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N <= 0 || K <= 0)
    return fail(PQL_ERR_INVALID_ARGUMENT, "need M >= 0, N > 0, K > 0 (got %lld, %lld, %lld)", (long long)M,
                (long long)N, (long long)K);
  if (K % 128) return fail(PQL_ERR_INVALID_ARGUMENT, "qgemm needs K %% 128 == 0 (got %lld)", (long long)K);
  if (K > (int64_t(1) << 20)) return fail(PQL_ERR_INVALID_ARGUMENT, "K above 2^20 is not supported");
  if (M > (int64_t(1) << 30) || N > (int64_t(1) << 30))
    return fail(PQL_ERR_INVALID_ARGUMENT, "M and N above 2^30 are not supported");
  // The launchers count output tiles (at least 64 x 64 elements each) in 32-bit
  // integers; an output with more tiles could not be allocated anyway.
  if (((M + 63) / 64) * ((N + 63) / 64) > (int64_t(1) << 31) - 1)
    return fail(PQL_ERR_INVALID_ARGUMENT, "an M x N output of %lld x %lld is too large", (long long)M, (long long)N);
  if (scheme == PQL_FP8_BLOCK128 && N % 128)
    return fail(PQL_ERR_INVALID_ARGUMENT, "FP8_BLOCK128 needs N %% 128 == 0 (got %lld)", (long long)N);
  if (scheme == PQL_MXFP4_DUAL && K % 512)
    return fail(PQL_ERR_INVALID_ARGUMENT, "MXFP4_DUAL needs K %% 512 == 0 (got %lld)", (long long)K);
  return PQL_OK;
}

// The fused small-M kernel's kind for a scheme, or -1 when it does not apply.
int small_kind(int scheme, int64_t M, int64_t K) {
  if (!pql::qlinear_small_applies(M, K)) return -1;
  switch (scheme) {
    case PQL_FP8_TENSOR: return pql::SMALL_TENSOR;
    case PQL_FP8_ROW: return pql::SMALL_ROW;
    case PQL_INT8_ROW: return pql::SMALL_INT8;
    case PQL_FP8_BLOCK128: return pql::SMALL_BLOCK;
  }
  return -1;
}

size_t qlinear_ws_bytes(int scheme, int64_t M, int64_t K) {
  if (small_kind(scheme, M, K) >= 0) return 0;   // the fused kernel keeps the quantized activation on chip
  const Sizes s = sizes_of(scheme, PQL_ACTIVATION, M, K);
  return round256(s.codes) + round256(s.scales) + (scheme == PQL_FP8_TENSOR ? kTensorWs : 0);
}

}  // namespace

extern "C" {

int pql_version(void) { return PQL_VERSION; }

const char* pql_last_error(void) { return g_error.c_str(); }

pql_status pql_quantized_sizes(int scheme, int role, int64_t rows, int64_t cols, size_t* codes_bytes,
                               size_t* scales_bytes, size_t* zeros_bytes) {
  pql_status st = check_scheme_role(scheme, role);
  if (st != PQL_OK) return st;
  if ((st = check_shape(scheme, role, rows, cols)) != PQL_OK) return st;
  const Sizes s = sizes_of(scheme, role, rows, cols);
  if (codes_bytes) *codes_bytes = s.codes;
  if (scales_bytes) *scales_bytes = s.scales;
  if (zeros_bytes) *zeros_bytes = s.zeros;
  return ok();
}

pql_status pql_workspace_size(int op, int scheme, int role, int64_t M, int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(PQL_ERR_INVALID_ARGUMENT, "bytes is NULL");
  if (op < PQL_OP_QUANTIZE || op > PQL_OP_QLINEAR) return fail(PQL_ERR_INVALID_ARGUMENT, "unknown op %d", op);
  *bytes = 0;
  if (op == PQL_OP_QUANTIZE) {
    pql_status st = check_scheme_role(scheme, role);
    if (st != PQL_OK) return st;
    if (scheme == PQL_FP8_TENSOR) *bytes = kTensorWs;
    return ok();
  }
  if (op == PQL_OP_QLINEAR) {
    if (!valid_scheme(scheme)) return fail(PQL_ERR_UNSUPPORTED, "unknown scheme %d", scheme);
    pql_status st = check_gemm_shape(scheme, M, N, K);
    if (st != PQL_OK) return st;
    if (!is_w4a16(scheme)) *bytes = qlinear_ws_bytes(scheme, M, K);
    return ok();
  }
  return ok();
}

static pql_status quantize_impl(int scheme, int role, const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                void* codes, void* scales, void* zeros, void* workspace, size_t workspace_bytes,
                                void* stream) {
  pql_status st = check_scheme_role(scheme, role);
  if (st != PQL_OK) return st;
  if ((st = check_shape(scheme, role, rows, cols)) != PQL_OK) return st;
  if ((st = check_ld("ldx", ldx, rows, cols, true)) != PQL_OK) return st;
  if (rows == 0) return ok();
  if (!x || !codes || !scales) return fail(PQL_ERR_INVALID_ARGUMENT, "x, codes and scales must be non-NULL");
  if (is_w4a16(scheme) && !zeros) return fail(PQL_ERR_INVALID_ARGUMENT, "zeros must be non-NULL for W4A16");
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || (zeros && !aligned16(zeros)))
    return fail(PQL_ERR_INVALID_ARGUMENT, "x, codes, scales and zeros must be 16-byte aligned");
  if (scheme == PQL_FP8_TENSOR) {
    if (!workspace || workspace_bytes < kTensorWs)
      return fail(PQL_ERR_WORKSPACE, "FP8_TENSOR needs a %zu-byte workspace (got %zu)", kTensorWs,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(PQL_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  }
  if ((st = check_device()) != PQL_OK) return st;
  return launched(do_quantize(scheme, role, x, rows, cols, ldx, codes, scales, zeros, workspace,
                              static_cast<hipStream_t>(stream)),
                  "quantize launch");
}

pql_status pql_quantize(int scheme, int role, const void* x, int64_t rows, int64_t cols, int64_t ldx, void* codes,
                        void* scales, void* zeros, void* workspace, size_t workspace_bytes, void* stream) {
  const pql_status st =
      quantize_impl(scheme, role, x, rows, cols, ldx, codes, scales, zeros, workspace, workspace_bytes, stream);
  if (log_enabled())
    log_call(st, "quantize", scheme, role, rows, 0, cols, pql_kernel_name(PQL_OP_QUANTIZE, scheme, role, rows, 0, cols),
             stream);
  return st;
}

static pql_status dequantize_impl(int scheme, int role, const void* codes, const void* scales, const void* zeros,
                                  int64_t rows, int64_t cols, void* y, int64_t ldy, void* stream) {
  pql_status st = check_scheme_role(scheme, role);
  if (st != PQL_OK) return st;
  if ((st = check_shape(scheme, role, rows, cols)) != PQL_OK) return st;
  if ((st = check_ld("ldy", ldy, rows, cols, true)) != PQL_OK) return st;
  if (rows == 0) return ok();
  if (!codes || !scales || !y) return fail(PQL_ERR_INVALID_ARGUMENT, "codes, scales and y must be non-NULL");
  if (is_w4a16(scheme) && !zeros) return fail(PQL_ERR_INVALID_ARGUMENT, "zeros must be non-NULL for W4A16");
  if (!aligned16(codes) || !aligned16(scales) || !aligned16(y) || (zeros && !aligned16(zeros)))
    return fail(PQL_ERR_INVALID_ARGUMENT, "codes, scales, zeros and y must be 16-byte aligned");
  if ((st = check_device()) != PQL_OK) return st;
  int kind;
  switch (scheme) {
    case PQL_FP8_TENSOR: kind = 0; break;
    case PQL_FP8_ROW: kind = 1; break;
    case PQL_FP8_BLOCK128: kind = role == PQL_ACTIVATION ? 2 : 3; break;
    case PQL_MXFP8: kind = 4; break;
    case PQL_MXFP4: kind = 5; break;
    case PQL_INT8_ROW: kind = 7; break;
    case PQL_MXFP4_DUAL: kind = 8; break;
    default: kind = 6; break;
  }
  if (scheme == PQL_MXFP4_DUAL)   // the coarse scales follow the fine exponents in the scales buffer
    zeros = static_cast<const uint8_t*>(scales) + dual_coarse_offset(rows, cols);
  return launched(pql::launch_dequant(kind, codes, scales, static_cast<const uint8_t*>(zeros), rows, cols,
                                      static_cast<uint16_t*>(y), ldy, static_cast<hipStream_t>(stream)),
                  "dequantize launch");
}

pql_status pql_dequantize(int scheme, int role, const void* codes, const void* scales, const void* zeros,
                          int64_t rows, int64_t cols, void* y, int64_t ldy, void* stream) {
  const pql_status st = dequantize_impl(scheme, role, codes, scales, zeros, rows, cols, y, ldy, stream);
  if (log_enabled()) log_call(st, "dequantize", scheme, role, rows, 0, cols, "k_dequant", stream);
  return st;
}

}  // extern "C"

namespace {

// Checks of the fused epilogue (alpha, bias) shared by qgemm_ex and qlinear_ex.
pql_status check_epilogue(int scheme, int64_t N, float alpha, const void* bias) {
  if (!(alpha == alpha) || alpha - alpha != 0.0f) return fail(PQL_ERR_INVALID_ARGUMENT, "alpha must be finite");
  if ((alpha != 1.0f || bias) && !has_epilogue(scheme))
    return fail(PQL_ERR_UNSUPPORTED, "%s has no fused alpha / bias epilogue (FP8 and INT8_ROW only)",
                scheme_name(scheme));
  if (bias && !aligned16(bias)) return fail(PQL_ERR_INVALID_ARGUMENT, "bias must be 16-byte aligned");
  if (bias && N % 2) return fail(PQL_ERR_INVALID_ARGUMENT, "a bias needs an even N (got %lld)", (long long)N);
  return PQL_OK;
}

}  // namespace

extern "C" {

static pql_status quantize_static_impl(int scheme, int role, const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                       const void* scales, void* codes, void* stream) {
  pql_status st = check_scheme_role(scheme, role);
  if (st != PQL_OK) return st;
  if (scheme != PQL_FP8_TENSOR && scheme != PQL_FP8_BLOCK128)
    return fail(PQL_ERR_UNSUPPORTED, "static scales are defined for FP8_TENSOR and FP8_BLOCK128 only (got %s)",
                scheme_name(scheme));
  if ((st = check_shape(scheme, role, rows, cols)) != PQL_OK) return st;
  if ((st = check_ld("ldx", ldx, rows, cols, true)) != PQL_OK) return st;
  if (rows == 0) return ok();
  if (!x || !codes || !scales) return fail(PQL_ERR_INVALID_ARGUMENT, "x, scales and codes must be non-NULL");
  if (!aligned16(x) || !aligned16(codes) || !aligned16(scales))
    return fail(PQL_ERR_INVALID_ARGUMENT, "x, scales and codes must be 16-byte aligned");
  if ((st = check_device()) != PQL_OK) return st;
  const int mode = scheme == PQL_FP8_TENSOR ? 0 : role == PQL_ACTIVATION ? 1 : 2;
  return launched(pql::launch_quant_fp8_static(mode, static_cast<const uint16_t*>(x), rows, cols, ldx,
                                               static_cast<const float*>(scales), static_cast<uint8_t*>(codes),
                                               static_cast<hipStream_t>(stream)),
                  "static quantize launch");
}

pql_status pql_quantize_static(int scheme, int role, const void* x, int64_t rows, int64_t cols, int64_t ldx,
                               const void* scales, void* codes, void* stream) {
  const pql_status st = quantize_static_impl(scheme, role, x, rows, cols, ldx, scales, codes, stream);
  if (log_enabled())
    log_call(st, "quantize_static", scheme, role, rows, 0, cols,
             scheme == PQL_FP8_TENSOR ? "k_fp8_static<tensor>" : "k_fp8_static<block128>", stream);
  return st;
}

static pql_status qgemm_ex_impl(int scheme, const void* a, const void* a_scales, const void* w_codes,
                                const void* w_scales, const void* w_zeros, int64_t M, int64_t N, int64_t K,
                                float alpha, const void* bias, void* c, int64_t ldc, void* stream) {
  if (!valid_scheme(scheme)) return fail(PQL_ERR_UNSUPPORTED, "unknown scheme %d", scheme);
  pql_status st = check_gemm_shape(scheme, M, N, K);
  if (st != PQL_OK) return st;
  if ((st = check_epilogue(scheme, N, alpha, bias)) != PQL_OK) return st;
  if ((st = check_ld("ldc", ldc, M, N, false)) != PQL_OK) return st;
  if (M == 0) return ok();
  if (!a || !w_codes || !w_scales || !c) return fail(PQL_ERR_INVALID_ARGUMENT, "a, w_codes, w_scales and c must be non-NULL");
  if (!is_w4a16(scheme) && !a_scales) return fail(PQL_ERR_INVALID_ARGUMENT, "a_scales must be non-NULL");
  if (is_w4a16(scheme) && !w_zeros) return fail(PQL_ERR_INVALID_ARGUMENT, "w_zeros must be non-NULL for W4A16");
  if (!aligned16(a) || !aligned16(w_codes) || !aligned16(w_scales) || (a_scales && !aligned16(a_scales)) ||
      (w_zeros && !aligned16(w_zeros)))
    return fail(PQL_ERR_INVALID_ARGUMENT, "operands, scales and zero-points must be 16-byte aligned");
  if ((st = check_device()) != PQL_OK) return st;
  return launched(do_qgemm(scheme, a, a_scales, w_codes, w_scales, w_zeros, M, N, K, alpha, bias, c, ldc,
                           static_cast<hipStream_t>(stream)),
                  "qgemm launch");
}

pql_status pql_qgemm_ex(int scheme, const void* a, const void* a_scales, const void* w_codes, const void* w_scales,
                        const void* w_zeros, int64_t M, int64_t N, int64_t K, float alpha, const void* bias,
                        void* c, int64_t ldc, void* stream) {
  const pql_status st =
      qgemm_ex_impl(scheme, a, a_scales, w_codes, w_scales, w_zeros, M, N, K, alpha, bias, c, ldc, stream);
  if (log_enabled())
    log_call(st, "qgemm", scheme, -1, M, N, K, pql_kernel_name(PQL_OP_QGEMM, scheme, PQL_ACTIVATION, M, N, K), stream);
  return st;
}

pql_status pql_qgemm(int scheme, const void* a, const void* a_scales, const void* w_codes, const void* w_scales,
                     const void* w_zeros, int64_t M, int64_t N, int64_t K, void* c, int64_t ldc, void* stream) {
  return pql_qgemm_ex(scheme, a, a_scales, w_codes, w_scales, w_zeros, M, N, K, 1.0f, nullptr, c, ldc, stream);
}

}  // extern "C"

namespace {

// Argument checks of qlinear (both entry points) that precede the workspace check.
pql_status check_qlinear(int scheme, const void* a, int64_t M, int64_t K, int64_t lda, const void* a_static_scales,
                         const void* w_codes, const void* w_scales, const void* w_zeros, int64_t N, float alpha,
                         const void* bias, const void* c, int64_t ldc) {
  if (!valid_scheme(scheme)) return fail(PQL_ERR_UNSUPPORTED, "unknown scheme %d", scheme);
  pql_status st = check_gemm_shape(scheme, M, N, K);
  if (st != PQL_OK) return st;
  if ((st = check_epilogue(scheme, N, alpha, bias)) != PQL_OK) return st;
  if (a_static_scales && scheme != PQL_FP8_TENSOR && scheme != PQL_FP8_BLOCK128)
    return fail(PQL_ERR_UNSUPPORTED, "static activation scales are defined for FP8_TENSOR and FP8_BLOCK128 only (got %s)",
                scheme_name(scheme));
  if ((st = check_ld("ldc", ldc, M, N, false)) != PQL_OK) return st;
  if (is_w4a16(scheme) && lda != K) return fail(PQL_ERR_INVALID_ARGUMENT, "W4A16 needs lda == K");
  if ((st = check_ld("lda", lda, M, K, true)) != PQL_OK) return st;
  if (M == 0) return ok();
  if (!a || !w_codes || !w_scales || !c) return fail(PQL_ERR_INVALID_ARGUMENT, "a, w_codes, w_scales and c must be non-NULL");
  if (is_w4a16(scheme) && !w_zeros) return fail(PQL_ERR_INVALID_ARGUMENT, "w_zeros must be non-NULL for W4A16");
  if (!aligned16(a) || !aligned16(w_codes) || !aligned16(w_scales) || (a_static_scales && !aligned16(a_static_scales)) ||
      (w_zeros && !aligned16(w_zeros)))
    return fail(PQL_ERR_INVALID_ARGUMENT, "operands, scales and zero-points must be 16-byte aligned");
  return PQL_OK;
}

// qlinear's launches, after every check (the workspace holds at least qlinear_ws_bytes).
pql_status run_qlinear(int scheme, const void* a, int64_t M, int64_t K, int64_t lda, const void* a_static_scales,
                       const void* w_codes, const void* w_scales, const void* w_zeros, int64_t N, float alpha,
                       const void* bias, void* c, int64_t ldc, void* workspace, void* stream) {
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int sk = small_kind(scheme, M, K);
  if (sk >= 0) {   // a few tokens: quantize inside the GEMM, one launch, no workspace traffic
    pql::SmallArgs s;
    s.a = static_cast<const uint16_t*>(a);
    s.M = M;
    s.K = K;
    s.lda = lda;
    s.a_static = static_cast<const float*>(a_static_scales);
    s.w = static_cast<const uint8_t*>(w_codes);
    s.w_scales = static_cast<const float*>(w_scales);
    s.N = N;
    s.alpha = alpha;
    s.bias = static_cast<const uint16_t*>(bias);
    s.c = static_cast<uint16_t*>(c);
    s.ldc = ldc;
    return launched(pql::launch_qlinear_small(sk, s, hs), "qlinear launch");
  }
  if (is_w4a16(scheme))
    return launched(do_qgemm(scheme, a, nullptr, w_codes, w_scales, w_zeros, M, N, K, 1.0f, nullptr, c, ldc, hs),
                    "qlinear launch");
  const Sizes s = sizes_of(scheme, PQL_ACTIVATION, M, K);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  void* a_codes = ws;
  void* a_scales = ws + round256(s.codes);
  void* partials = ws + round256(s.codes) + round256(s.scales);
  hipError_t e;
  if (a_static_scales) {
    a_scales = const_cast<void*>(a_static_scales);
    e = pql::launch_quant_fp8_static(scheme == PQL_FP8_TENSOR ? 0 : 1, static_cast<const uint16_t*>(a), M, K, lda,
                                     static_cast<const float*>(a_static_scales), static_cast<uint8_t*>(a_codes), hs);
  } else {
    e = do_quantize(scheme, PQL_ACTIVATION, a, M, K, lda, a_codes, a_scales, nullptr, partials, hs);
  }
  if (e != hipSuccess) return launched(e, "qlinear activation quantize");
  return launched(do_qgemm(scheme, a_codes, a_scales, w_codes, w_scales, w_zeros, M, N, K, alpha, bias, c, ldc, hs),
                  "qlinear gemm");
}

// ---- the entry point that allocates nothing: its activation codes and scales
// live in this file-scope device array.  The host-side name `scratch` is only a
// stand-in: kernels get the per-device address from hipGetSymbolAddress.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];   // per device, filled on the device's first call

pql_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PQL_ERR_HIP, "no usable HIP device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return fail(PQL_ERR_HIP, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(PQL_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PQL_OK;
}

}  // namespace

extern "C" {

static pql_status qlinear_ex_impl(int scheme, const void* a, int64_t M, int64_t K, int64_t lda,
                                  const void* a_static_scales, const void* w_codes, const void* w_scales,
                                  const void* w_zeros, int64_t N, float alpha, const void* bias, void* c, int64_t ldc,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  pql_status st = check_qlinear(scheme, a, M, K, lda, a_static_scales, w_codes, w_scales, w_zeros, N, alpha, bias,
                                c, ldc);
  if (st != PQL_OK || M == 0) return st == PQL_OK ? ok() : st;
  const size_t need = is_w4a16(scheme) ? 0 : qlinear_ws_bytes(scheme, M, K);
  if (need) {   // W4A16 and the fused few-token kernel need none (the pointer may then be NULL)
    if (!workspace || workspace_bytes < need)
      return fail(PQL_ERR_WORKSPACE, "qlinear needs a %zu-byte workspace (got %zu)", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(PQL_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  }
  if ((st = check_device()) != PQL_OK) return st;
  return run_qlinear(scheme, a, M, K, lda, a_static_scales, w_codes, w_scales, w_zeros, N, alpha, bias, c, ldc,
                     workspace, stream);
}

pql_status pql_qlinear_ex(int scheme, const void* a, int64_t M, int64_t K, int64_t lda, const void* a_static_scales,
                          const void* w_codes, const void* w_scales, const void* w_zeros, int64_t N, float alpha,
                          const void* bias, void* c, int64_t ldc, void* workspace, size_t workspace_bytes,
                          void* stream) {
  const pql_status st = qlinear_ex_impl(scheme, a, M, K, lda, a_static_scales, w_codes, w_scales, w_zeros, N, alpha,
                                        bias, c, ldc, workspace, workspace_bytes, stream);
  if (log_enabled())
    log_call(st, "qlinear", scheme, -1, M, N, K, pql_kernel_name(PQL_OP_QLINEAR, scheme, PQL_ACTIVATION, M, N, K),
             stream);
  return st;
}

size_t pql_noalloc_scratch_bytes(void) { return kScratchBytes; }

static pql_status qlinear_noalloc_impl(int scheme, const void* a, int64_t M, int64_t K, int64_t lda,
                                       const void* a_static_scales, const void* w_codes, const void* w_scales,
                                       const void* w_zeros, int64_t N, float alpha, const void* bias, void* c,
                                       int64_t ldc, void* stream) {
  pql_status st = check_qlinear(scheme, a, M, K, lda, a_static_scales, w_codes, w_scales, w_zeros, N, alpha, bias,
                                c, ldc);
  if (st != PQL_OK || M == 0) return st == PQL_OK ? ok() : st;
  const size_t need = is_w4a16(scheme) ? 0 : qlinear_ws_bytes(scheme, M, K);
  if (need > kScratchBytes)
    return fail(PQL_ERR_WORKSPACE, "the activation's codes and scales need %zu bytes, more than the %zu-byte "
                "static scratch of pql_qlinear_noalloc; use pql_qlinear_ex with a workspace", need, kScratchBytes);
  if ((st = check_device()) != PQL_OK) return st;
  void* ws = nullptr;
  if (need && (st = scratch_address(&ws)) != PQL_OK) return st;
  return run_qlinear(scheme, a, M, K, lda, a_static_scales, w_codes, w_scales, w_zeros, N, alpha, bias, c, ldc, ws,
                     stream);
}

pql_status pql_qlinear_noalloc(int scheme, const void* a, int64_t M, int64_t K, int64_t lda,
                               const void* a_static_scales, const void* w_codes, const void* w_scales,
                               const void* w_zeros, int64_t N, float alpha, const void* bias, void* c, int64_t ldc,
                               void* stream) {
  const pql_status st = qlinear_noalloc_impl(scheme, a, M, K, lda, a_static_scales, w_codes, w_scales, w_zeros, N,
                                             alpha, bias, c, ldc, stream);
  if (log_enabled())
    log_call(st, "qlinear_noalloc", scheme, -1, M, N, K,
             pql_kernel_name(PQL_OP_QLINEAR, scheme, PQL_ACTIVATION, M, N, K), stream);
  return st;
}

pql_status pql_qlinear(int scheme, const void* a, int64_t M, int64_t K, int64_t lda, const void* w_codes,
                       const void* w_scales, const void* w_zeros, int64_t N, void* c, int64_t ldc, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return pql_qlinear_ex(scheme, a, M, K, lda, nullptr, w_codes, w_scales, w_zeros, N, 1.0f, nullptr, c, ldc,
                        workspace, workspace_bytes, stream);
}

pql_status pql_layout_sizes(int scheme, int role, int layout, int64_t rows, int64_t cols, size_t* codes_bytes,
                            size_t* scales_bytes, size_t* zeros_bytes) {
  if (layout != PQL_LAYOUT_CANONICAL && layout != PQL_LAYOUT_PACKED)
    return fail(PQL_ERR_INVALID_ARGUMENT, "unknown layout %d", layout);
  pql_status st = pql_quantized_sizes(scheme, role, rows, cols, codes_bytes, scales_bytes, zeros_bytes);
  if (st != PQL_OK || layout == PQL_LAYOUT_PACKED) return st;
  if (is_mx(scheme) && scales_bytes) *scales_bytes = (size_t)rows * (size_t)(cols / 32);   // u8 [rows, cols / 32]
  return ok();
}

static pql_status repack_impl(int scheme, int role, int from_layout, int to_layout, const void* scales_in,
                              const void* zeros_in, void* scales_out, void* zeros_out, int64_t rows, int64_t cols,
                              void* stream) {
  pql_status st = check_scheme_role(scheme, role);
  if (st != PQL_OK) return st;
  if ((st = check_shape(scheme, role, rows, cols)) != PQL_OK) return st;
  for (int l : {from_layout, to_layout})
    if (l != PQL_LAYOUT_CANONICAL && l != PQL_LAYOUT_PACKED)
      return fail(PQL_ERR_INVALID_ARGUMENT, "unknown layout %d", l);
  if (rows == 0) return ok();
  if (!scales_in || !scales_out) return fail(PQL_ERR_INVALID_ARGUMENT, "scales_in and scales_out must be non-NULL");
  if (is_w4a16(scheme) && (!zeros_in || !zeros_out))
    return fail(PQL_ERR_INVALID_ARGUMENT, "W4A16 needs zeros_in and zeros_out");
  const bool differs = from_layout != to_layout && (is_mx(scheme) || is_w4a16(scheme) || scheme == PQL_MXFP4_DUAL);
  if (differs && (scales_in == scales_out || (zeros_in && zeros_in == zeros_out)))
    return fail(PQL_ERR_INVALID_ARGUMENT, "%s scales change layout; input and output must be distinct buffers",
                scheme_name(scheme));
  if ((st = check_device()) != PQL_OK) return st;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool to_packed = to_layout == PQL_LAYOUT_PACKED;
  if (differs && scheme == PQL_MXFP4_DUAL) {   // fine exponents as MXFP4, coarse scales transposed
    const size_t off = dual_coarse_offset(rows, cols);
    const uint8_t* in = static_cast<const uint8_t*>(scales_in);
    uint8_t* out = static_cast<uint8_t*>(scales_out);
    hipError_t e = pql::launch_mx_repack(to_packed, true, in, rows, cols, out, hs);
    // canonical coarse [rows, cols / 512], packed group-major [cols / 512, rows]
    if (e == hipSuccess)
      e = pql::launch_transpose_f32(reinterpret_cast<const float*>(in + off), to_packed ? rows : cols / 512,
                                    to_packed ? cols / 512 : rows, reinterpret_cast<float*>(out + off), hs);
    return launched(e, "repack launch");
  }
  if (differs && is_mx(scheme))
    return launched(pql::launch_mx_repack(to_packed, scheme == PQL_MXFP4, static_cast<const uint8_t*>(scales_in),
                                          rows, cols, static_cast<uint8_t*>(scales_out), hs),
                    "repack launch");
  if (differs)
    return launched(pql::launch_group_repack(to_packed, static_cast<const uint16_t*>(scales_in),
                                             static_cast<const uint8_t*>(zeros_in), rows, cols / 128,
                                             static_cast<uint16_t*>(scales_out), static_cast<uint8_t*>(zeros_out), hs),
                    "repack launch");
  // the same layout: a copy (nothing to do in place)
  const Sizes sz = sizes_of(scheme, role, rows, cols);
  hipError_t e = hipSuccess;
  if (scales_in != scales_out) e = hipMemcpyAsync(scales_out, scales_in, sz.scales, hipMemcpyDeviceToDevice, hs);
  if (e == hipSuccess && zeros_in && zeros_out && zeros_in != zeros_out)
    e = hipMemcpyAsync(zeros_out, zeros_in, sz.zeros, hipMemcpyDeviceToDevice, hs);
  return launched(e, "repack copy");
}

pql_status pql_repack(int scheme, int role, int from_layout, int to_layout, const void* scales_in,
                      const void* zeros_in, void* scales_out, void* zeros_out, int64_t rows, int64_t cols,
                      void* stream) {
  const pql_status st =
      repack_impl(scheme, role, from_layout, to_layout, scales_in, zeros_in, scales_out, zeros_out, rows, cols, stream);
  if (log_enabled()) log_call(st, "repack", scheme, role, rows, 0, cols, "k_repack", stream);
  return st;
}

const char* pql_kernel_name(int op, int scheme, int role, int64_t M, int64_t N, int64_t K) {
  if (!valid_scheme(scheme)) return "";
  switch (op) {
    case PQL_OP_QUANTIZE:
      if (is_w4a16(scheme) && role == PQL_ACTIVATION) return "";
      switch (scheme) {
        case PQL_FP8_TENSOR: return "k_amax_partial+k_fp8_tensor";
        case PQL_FP8_ROW: return "k_fp8_row";
        case PQL_INT8_ROW: return "k_fp8_row<int8>";
        case PQL_FP8_BLOCK128: return role == PQL_ACTIVATION ? "k_fp8_block_act" : "k_fp8_block_wt";
        case PQL_MXFP8: return "k_mx<e4m3>";
        case PQL_MXFP4: return "k_mx<e2m1>";
        case PQL_MXFP4_DUAL: return "k_mx4_dual";
        default: return scheme == PQL_W4A16_SYM ? "k_int4<sym>" : "k_int4<asym>";
      }
    case PQL_OP_DEQUANTIZE: return "k_dequant";
    case PQL_OP_QLINEAR: {
      const bool few = pql::qlinear_few_applies(M, K);
      switch (small_kind(scheme, M, K)) {
        case pql::SMALL_TENSOR: return few ? "k_qlinear_few<fp8_tensor>" : "k_qlinear_small<fp8_tensor>";
        case pql::SMALL_ROW: return few ? "k_qlinear_few<fp8_row>" : "k_qlinear_small<fp8_row>";
        case pql::SMALL_INT8: return few ? "k_qlinear_few<int8_row>" : "k_qlinear_small<int8_row>";
        case pql::SMALL_BLOCK: return few ? "k_qlinear_few<fp8_block128>" : "k_qlinear_small<fp8_block128>";
      }
    }
      [[fallthrough]];
    case PQL_OP_QGEMM:
      if (is_w4a16(scheme)) return pql::gemm_w4a16_kernel_name(M, N, K);
      if (scheme == PQL_MXFP4_DUAL) return "k_gemm_mx4_dual";
      return pql::gemm_kernel_name(gemm_kind(scheme), M, N, K);
  }
  return "";
}

}  // extern "C"
