/*
 * pql.h -- C ABI of libpql, the quantized-linear hot path for AMD MI355X (gfx950).
 *
 * Two steps, as the pages describe the online-quantized linear layer:
 *   1. quantize bf16 activations (every call) and weights (once, at load) into
 *      block-scaled low-precision codes plus scales;
 *   2. a scaled GEMM on those codes, C = A * W^T, returning bf16.
 * ("vLLM-Omni Online Quantization complete guide", section "How online
 *  quantization works underneath", steps 1-3; "[vLLM] Other quantization: FP8,
 *  ModelOpt, INC, TorchAO, Quark", section "FP8"; "vLLM-Omni accelerates
 *  inference with AutoRound quantization", section "Usage".)
 *
 * Conventions for every call:
 *   - Operands: A is [M, K] (tokens x input channels), W is [N, K] (output x
 *     input channels, a linear layer's own layout), C is [M, N].  K is the
 *     contraction axis and is contiguous in every operand.
 *   - All pointers except the size outputs are DEVICE pointers on the current
 *     HIP device.  The caller allocates and owns every buffer, including
 *     workspace; the library allocates no device memory and keeps no state
 *     besides a per-device property cache, a thread-local error message and
 *     the static device buffer of pql_qlinear_noalloc (see there).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the null stream)
 *     and the call returns without synchronizing.  Calls are re-entrant.
 *   - Every argument check runs before anything is enqueued; on any error
 *     nothing is enqueued and pql_last_error() describes the problem.
 *   - Launch log: with the environment variable PQL_LOG set to anything but
 *     "" or "0" (read once, at the first call), pql_quantize,
 *     pql_quantize_static, pql_dequantize, pql_qgemm(_ex), pql_qlinear(_ex),
 *     pql_qlinear_noalloc and pql_repack each write one line to stderr: the
 *     call, scheme, role and shape, then the kernel enqueued (the name
 *     pql_kernel_name gives) and the stream, "nothing to do" for an empty
 *     operand, or "rejected (status S)" with the pql_last_error() text.
 *   - Element sizes: bf16 = 2 bytes, fp32 = 4 bytes.  Leading dimensions
 *     (ldx, ldy, lda, ldc) are in elements.  Device pointers must be 16-byte
 *     aligned and leading dimensions multiples of 8 elements (ldc: any value
 *     >= N).  The span a leading dimension addresses, (rows - 1) * ld + cols,
 *     must stay within 2^40 elements (INVALID_ARGUMENT otherwise).
 *
 * Packed layouts: what every call below except pql_repack produces and
 * consumes, laid out for the GEMM kernels (per scheme; rows = M for
 * activations, N for weights, cols = K):
 *   FP8_TENSOR    codes u8 e4m3fn [rows, cols]          scales f32 [1]
 *   FP8_ROW       codes u8 e4m3fn [rows, cols]          scales f32 [rows]
 *   FP8_BLOCK128  codes u8 e4m3fn [rows, cols]          scales f32 [rows, cols/128] (activation)
 *                                                       scales f32 [rows/128, cols/128] (weight)
 *   MXFP8         codes u8 e4m3fn [rows, cols]          scales u8 e8m0, packed [G, rows, 4]
 *   MXFP4         codes u8 [rows, cols/2], two e2m1,    scales u8 e8m0, packed [G, rows, 8]
 *                 element 2j in the low nibble
 *   W4A16_ASYM    codes u32 [rows, cols/8], element k   scales bf16 [cols/128, rows]
 *                 at bits 4*(k mod 8)                   zeros u8 [cols/128, rows] (0..15)
 *   W4A16_SYM     as W4A16_ASYM with every zero-point 8
 *   INT8_ROW      codes i8 [rows, cols] (two's         scales f32 [rows]
 *                 complement)
 *   MXFP4_DUAL    codes as MXFP4                       scales: fine e8m0 packed [G, rows, 8], then
 *                                                       from the next 256-byte boundary coarse
 *                                                       f32 [cols/512, rows] (group-major)
 * All codes are K-contiguous, which is the operand order the matrix cores
 * consume, so weights need no re-layout after quantization.
 * W4A16 scales and zero-points are group-major ([group, row]): one K-group's
 * values for consecutive weight rows are consecutive, which is how the GEMM
 * stages them.
 * MX scales are packed for the GEMM's staging: with c = 4 (MXFP8) or 8
 * (MXFP4) and G = ceil(cols / (32 c)), byte [g, r, b] is the exponent of row
 * r's 32-element block c g + b (K-elements 32 (c g + b) .. + 31); bytes past
 * the row's last block are 127.  A chunk covers 128 bytes of codes, so the
 * exponents one GEMM step needs for consecutive rows are consecutive bytes.
 *
 * Canonical layouts (PQL_LAYOUT_CANONICAL): the same codes, with the scales
 * and zero-points of every row together: MX exponents u8 [rows, cols/32],
 * W4A16 scales bf16 [rows, cols/128] and zero-points u8 [rows, cols/128],
 * MXFP4_DUAL fine exponents u8 [rows, cols/32] then (from the next 256-byte
 * boundary, as packed) coarse f32 [rows, cols/512]; for every other scheme the
 * canonical and packed layouts are the same bytes.
 * pql_repack converts between the two on the device.
 */
#ifndef PQL_H
#define PQL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PQL_VERSION 2

typedef enum pql_status {
  PQL_OK = 0,
  PQL_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, stride or alignment */
  PQL_ERR_UNSUPPORTED = 2,      /* scheme x role not defined, or device is not gfx950 */
  PQL_ERR_WORKSPACE = 3,        /* workspace missing or smaller than pql_workspace_size() */
  PQL_ERR_HIP = 4               /* HIP runtime error (no device, launch failure) */
} pql_status;

/* Quantization schemes.
 *   FP8_TENSOR / FP8_ROW / FP8_BLOCK128: dynamic symmetric FP8 e4m3fn with an
 *     fp32 scale per tensor, per row (per token for activations, per output
 *     channel for weights) or per block (1x128 for activations, 128x128 for
 *     weights) ("[vLLM] Other quantization...", section "FP8").
 *     s = fp32(amax / 448) (1 if that is 0); code = e4m3fn(fp32(x / s)),
 *     round to nearest even, saturating at +-448, sign of zero kept.
 *   MXFP8 / MXFP4: OCP MX, one e8m0 exponent per 32 consecutive K-elements
 *     ("vLLM-Omni Online Quantization complete guide", section "How online
 *     quantization works underneath", steps 2-3).
 *     X = clamp(floor(log2 amax) - emax, -127, 127) (emax 8 for e4m3, 2 for
 *     e2m1; amax = 0 gives -127), scale code X + 127, code = RNE_sat(x * 2^-X).
 *   W4A16_ASYM / W4A16_SYM: int4 weights, group 128 along K, bf16 scale and
 *     4-bit zero-point per group; activations stay bf16 ("vLLM-Omni
 *     accelerates inference with AutoRound quantization", section "Usage").
 *     Weight quantization is round-to-nearest:
 *       asym: s = bf16(fp32(fp32(max(0,max x) - min(0,min x)) / 15)),
 *             z = clamp(rne(fp32(-min(0,min x) / s)), 0, 15)
 *       sym:  s = bf16(fp32(max|x| / 7)), z = 8
 *       q = clamp(rne(fp32(x / s)) + z, 0, 15); s = 0 is replaced by 1 (z = 0 asym).
 *   INT8_ROW: int8 W8A8, symmetric, one fp32 scale per row (per token for
 *     activations, per output channel for weights), dynamic only ("vLLM-Omni
 *     Online Quantization complete guide", sections "Key parameters in
 *     detail" and "How online quantization works underneath": the int8
 *     online path quantizes weights with weight scales; its activation
 *     scales are dynamic, a static activation scheme is an error).
 *     s = fp32(amax / 127) (1 if that is 0); code = clamp(rne(fp32(x / s)), -128, 127).
 *   MXFP4_DUAL: MXFP4 with two online scale levels, a coarse fp32 scale per
 *     512 K-elements and a fine e8m0 exponent per 32 ("vLLM-Omni Online
 *     Quantization complete guide", section "How online quantization works
 *     underneath", MXFP4 paragraph; the calibrated multiplier of offline
 *     checkpoints is all ones online and leaves x unchanged).  K % 512 == 0.
 *     s_c = fp32(amax_512 / 6) (1 if 0); v = fp32(x / s_c) (correctly
 *     rounded); X = clamp(floor(log2 max|v|) - 2, -127, 127) per 32-block;
 *     code = RNE_sat_e2m1(v * 2^-X).  Dequantized: fp32(decode * 2^X) * s_c.
 *     No fused alpha / bias epilogue.
 */
typedef enum pql_scheme {
  PQL_FP8_TENSOR = 0,
  PQL_FP8_ROW = 1,
  PQL_FP8_BLOCK128 = 2,
  PQL_MXFP8 = 3,
  PQL_MXFP4 = 4,
  PQL_W4A16_ASYM = 5,
  PQL_W4A16_SYM = 6,
  PQL_INT8_ROW = 7,
  PQL_MXFP4_DUAL = 8
} pql_scheme;

typedef enum pql_role { PQL_ACTIVATION = 0, PQL_WEIGHT = 1 } pql_role;

typedef enum pql_layout { PQL_LAYOUT_CANONICAL = 0, PQL_LAYOUT_PACKED = 1 } pql_layout;

typedef enum pql_op {
  PQL_OP_QUANTIZE = 0,
  PQL_OP_DEQUANTIZE = 1,
  PQL_OP_QGEMM = 2,
  PQL_OP_QLINEAR = 3
} pql_op;

/* Library version (PQL_VERSION). */
int pql_version(void);

/* Text of the last error on the calling thread ("" if none).  The pointer
 * stays valid until the thread's next pql call. */
const char* pql_last_error(void);

/* Byte sizes of the codes, scales and zero-point buffers of a quantized
 * [rows, cols] tensor in the packed layout (zeros_bytes is 0 except for
 * W4A16).  Size outputs are host pointers; any may be NULL.
 * Errors: INVALID_ARGUMENT for negative sizes or cols / rows that the scheme
 * cannot block (cols % 32 for FP8 tensor/row, INT8_ROW and MX, cols % 128 for
 * FP8_BLOCK128 and W4A16, rows % 128 for FP8_BLOCK128 weights), and for
 * cols > 2^20, rows > 2^31 - 1 or rows * cols > 2^40 (the same limits hold for
 * every quantize and dequantize call; GEMMs take K <= 2^20, M, N <= 2^30 and
 * at most 2^31 - 1 output tiles of 64 x 64);
 * UNSUPPORTED for W4A16 activations or an unknown scheme / role. */
pql_status pql_quantized_sizes(int scheme, int role, int64_t rows, int64_t cols,
                               size_t* codes_bytes, size_t* scales_bytes,
                               size_t* zeros_bytes);

/* pql_quantized_sizes for either layout (PQL_LAYOUT_PACKED gives the same
 * sizes as pql_quantized_sizes; canonical MX scales take rows * cols / 32
 * bytes, without the packed layout's padding).  Same errors, plus
 * INVALID_ARGUMENT for an unknown layout. */
pql_status pql_layout_sizes(int scheme, int role, int layout, int64_t rows, int64_t cols, size_t* codes_bytes,
                            size_t* scales_bytes, size_t* zeros_bytes);

/* Convert a quantized tensor's scales (and W4A16 zero-points) from one layout
 * to the other on the device ("vLLM-Omni Online Quantization complete
 * guide", section "How online quantization works underneath", step 2: online
 * weights are brought into the layout the GEMM consumes, with the scales
 * rearranged to match).  Codes are the same bytes in both layouts and are not
 * touched.  scales_in / zeros_in are in `from_layout`, scales_out /
 * zeros_out (caller-allocated, pql_layout_sizes(to_layout) bytes) receive
 * `to_layout`; zeros are required for W4A16 and ignored otherwise.  When the
 * two layouts are the same bytes (the layouts are equal, or the scheme has
 * one layout) this is a device copy, nothing if input and output coincide;
 * otherwise input and output must be distinct buffers.  Errors: as
 * pql_quantize's shape checks, INVALID_ARGUMENT for an unknown layout, NULL
 * buffers or overlapping buffers of a transposing repack. */
pql_status pql_repack(int scheme, int role, int from_layout, int to_layout, const void* scales_in,
                      const void* zeros_in, void* scales_out, void* zeros_out, int64_t rows, int64_t cols,
                      void* stream);

/* Workspace bytes a call needs (host output).  op = PQL_OP_QUANTIZE: the
 * per-tensor scheme needs a small partial-maximum buffer, the others 0.
 * op = PQL_OP_QLINEAR: room for the activation's codes and scales (0 for
 * W4A16).  Other ops need none.  `role` matters for QUANTIZE only. */
pql_status pql_workspace_size(int op, int scheme, int role, int64_t M, int64_t N,
                              int64_t K, size_t* bytes);

/* Quantize a bf16 tensor x[rows, cols] (row stride ldx elements) into the
 * packed layout.  Activation role: rows = M; weight role: rows = N.
 * `zeros` is written for W4A16 only (may be NULL otherwise).  The scales are
 * dynamic (computed from x).  FP8_TENSOR needs `workspace` of at least
 * pql_workspace_size(PQL_OP_QUANTIZE, ...) bytes; other schemes ignore it.
 * rows = 0 is a no-op. */
pql_status pql_quantize(int scheme, int role, const void* x, int64_t rows, int64_t cols,
                        int64_t ldx, void* codes, void* scales, void* zeros,
                        void* workspace, size_t workspace_bytes, void* stream);

/* y[rows, cols] (bf16, row stride ldy) = bf16_RNE(fp32(decode(code) * scale))
 * (W4A16: bf16_RNE((q - z) * s)).  Inputs in the packed layout. */
pql_status pql_dequantize(int scheme, int role, const void* codes, const void* scales,
                          const void* zeros, int64_t rows, int64_t cols, void* y,
                          int64_t ldy, void* stream);

/* C[M, N] (bf16, row stride ldc) = A_hat * W_hat^T on already-quantized
 * operands, fp32 accumulation, bf16 round-to-nearest-even output.
 *   FP8 / MX schemes: a = activation codes [M, K], a_scales its scales
 *   (packed activation layout); w_codes / w_scales the weight's.
 *   W4A16: a = bf16 activation [M, K] (contiguous), a_scales unused (NULL),
 *   w_zeros required.
 * K must be a multiple of 128; M, N >= 1 may be ragged (tails are masked);
 * FP8_BLOCK128 needs N % 128 == 0 (the weight's 128-row blocks). */
pql_status pql_qgemm(int scheme, const void* a, const void* a_scales, const void* w_codes,
                     const void* w_scales, const void* w_zeros, int64_t M, int64_t N,
                     int64_t K, void* c, int64_t ldc, void* stream);

/* The linear layer's forward: quantize the bf16 activation a[M, K] (row
 * stride lda) with the scheme's activation rule into `workspace`, then
 * qgemm against the quantized weight.  W4A16 uses a as-is (lda must equal K)
 * and needs no workspace.  C as for pql_qgemm.
 * A few tokens (1 <= M <= 16) under FP8_TENSOR, FP8_ROW, FP8_BLOCK128 or
 * INT8_ROW take one fused launch instead ("vLLM-Omni Online Quantization
 * complete guide", section "How online quantization works underneath": the
 * activation quantize fused into the GEMM): each workgroup recomputes the
 * activation's scales and codes on chip, with the same rule and the same
 * codes as pql_quantize, and the workspace is neither needed nor touched
 * (pql_workspace_size gives 0 for these shapes).  The result differs from
 * quantize + qgemm only in the order of the fp32 partial sums. */
pql_status pql_qlinear(int scheme, const void* a, int64_t M, int64_t K, int64_t lda,
                       const void* w_codes, const void* w_scales, const void* w_zeros,
                       int64_t N, void* c, int64_t ldc, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Static-scale FP8 quantization (FP8_TENSOR and FP8_BLOCK128 only): the
 * scale is supplied instead of computed from x ("[vLLM] Other quantization:
 * FP8, ModelOpt, INC, TorchAO, Quark", section "FP8": the static tensor-wise
 * and static 128-block symmetric scheme keys).  `scales` (device, read only)
 * is in the scheme's scale layout for `role` (f32 [1]; f32
 * [rows, cols/128] for activations, f32 [rows/128, cols/128] for weights) and
 * must hold finite positive values (not checked on the device: a zero, NaN or
 * infinite scale gives meaningless codes).  codes = e4m3fn(fp32(x / s)),
 * round to nearest even, saturating at +-448: values beyond 448 s clamp,
 * which a calibrated scale makes possible.  Same shape rules as
 * pql_quantize; rows = 0 is a no-op.  UNSUPPORTED for other schemes
 * (INT8_ROW has no static scheme). */
pql_status pql_quantize_static(int scheme, int role, const void* x, int64_t rows, int64_t cols, int64_t ldx,
                               const void* scales, void* codes, void* stream);

/* pql_qgemm with the fused epilogue ("vLLM-Omni Online Quantization complete
 * guide", section "How online quantization works underneath": the FP8 path's
 * alpha * (A @ B) + bias):
 *   C[m, n] = bf16_RNE(alpha * (A_hat W_hat^T)[m, n] + bias[n])
 * computed in fp32 with one rounding to bf16.  alpha is a finite host fp32;
 * bias is a device bf16 [N] vector (16-byte aligned, N even) or NULL.
 * Defined for FP8_TENSOR, FP8_ROW, FP8_BLOCK128 and INT8_ROW; other schemes
 * are UNSUPPORTED unless alpha == 1 and bias == NULL (then identical to
 * pql_qgemm).  INT8_ROW sums in int32, then scales in fp32.  Other arguments
 * and errors as pql_qgemm. */
pql_status pql_qgemm_ex(int scheme, const void* a, const void* a_scales, const void* w_codes, const void* w_scales,
                        const void* w_zeros, int64_t M, int64_t N, int64_t K, float alpha, const void* bias,
                        void* c, int64_t ldc, void* stream);

/* pql_qlinear with the fused epilogue (alpha, bias as pql_qgemm_ex) and,
 * optionally, static activation scales: with `a_static_scales` non-NULL
 * (FP8_TENSOR: f32 [1]; FP8_BLOCK128: f32 [M, K/128]; device, read only,
 * finite and positive) the activation is quantized with those scales as
 * pql_quantize_static does, and the GEMM reads them in place; NULL means
 * dynamic scales, as pql_qlinear.  Static scales for any other scheme are
 * UNSUPPORTED.  The workspace is the one pql_workspace_size(PQL_OP_QLINEAR)
 * gives, in both cases. */
pql_status pql_qlinear_ex(int scheme, const void* a, int64_t M, int64_t K, int64_t lda, const void* a_static_scales,
                          const void* w_codes, const void* w_scales, const void* w_zeros, int64_t N, float alpha,
                          const void* bias, void* c, int64_t ldc, void* workspace, size_t workspace_bytes,
                          void* stream);

/* pql_qlinear_ex for callers that cannot allocate device memory at call
 * time -- code being captured into a HIP graph, tight serving loops, harnesses
 * that forbid allocation -- and so cannot hand over a workspace.  Arguments,
 * results and errors are those of pql_qlinear_ex without the workspace: the
 * activation's codes and scales go to a static device buffer of the library
 * (pql_noalloc_scratch_bytes(), 64 MiB, held on every device the library runs
 * on until the process ends).  Nothing is allocated or freed, by the library
 * or anything it calls.  An activation whose codes and scales need more than
 * that (pql_workspace_size(PQL_OP_QLINEAR, ...) > pql_noalloc_scratch_bytes())
 * is rejected with PQL_ERR_WORKSPACE before anything is enqueued.  Every call
 * on one device shares that device's buffer and leaves its contents behind
 * (nothing in it needs to start at zero): calls that overlap in time on one
 * device -- on different streams, or from different threads without ordering
 * -- race and give undefined results.  W4A16 uses no buffer. */
pql_status pql_qlinear_noalloc(int scheme, const void* a, int64_t M, int64_t K, int64_t lda, const void* a_static_scales,
                               const void* w_codes, const void* w_scales, const void* w_zeros, int64_t N, float alpha,
                               const void* bias, void* c, int64_t ldc, void* stream);

/* Size in bytes of pql_qlinear_noalloc's static device buffer. */
size_t pql_noalloc_scratch_bytes(void);

/* Name of the kernel that `op` would launch for these sizes (for "no silent
 * fallback" checks); "" if the combination is invalid.  Static string. */
const char* pql_kernel_name(int op, int scheme, int role, int64_t M, int64_t N, int64_t K);

#ifdef __cplusplus
}
#endif

#endif /* PQL_H */
