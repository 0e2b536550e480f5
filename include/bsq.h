/*
 * bsq.h - block-scaled quantized matmul for AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Conventions shared by every call:
 *
 *   - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees or keeps a pointer after the call
 *     returns.  Tensors are dense row-major; base addresses must be 16-byte
 *     aligned.  Sizes are int64_t element counts.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Each call validates its arguments on the host, enqueues its kernels
 *     on `stream` and returns without synchronising.  Kernel errors that
 *     the launch itself reports are returned as BSQ_ERR_HIP.
 *   - Every call returns a bsq_status.  On failure nothing has been
 *     enqueued and bsq_last_error() (thread-local) describes the cause.
 *   - A call with an empty extent (a zero size) is a valid no-op unless the
 *     call's own rules say otherwise.
 *   - Matmul extents are at most 2^30, a contraction length (K of a
 *     matmul; M and N of the mxfp8 backward, whose two products contract
 *     over them) at most 2^24, a batch of products at most 65535, and one
 *     product's output at most 2^31 - 1 tiles of 128 x 256 (far beyond any
 *     output that fits in memory); larger -> BSQ_ERR_UNSUPPORTED.
 *   - No array a call reads or writes may hold more than 2^60 elements
 *     (so that no size or offset overflows 64 bits); larger ->
 *     BSQ_ERR_UNSUPPORTED.
 *   - A *_workspace_bytes query returns 0 for negative sizes and SIZE_MAX
 *     for sizes whose byte count would not fit (its call rejects them).
 *   - Non-finite inputs give unspecified results (the pages state all
 *     values are finite).
 *   - Format names: E4M3 = OCP float8_e4m3fn, E5M2 = OCP float8_e5m2,
 *     E8M0 = OCP float8_e8m0fnu (scale 2^(b-127)), BF16 = bfloat16.
 *
 * Citations name the web page and the part of it that defines the
 * operation: "scaled_matmul" = jax.nn.scaled_matmul documentation;
 * "block_scaled_mm" = atrex-bench operator #002; "int8 per-channel" =
 * TensorTonic "Int8 Matmul with Per-Channel Scales"; "mxfp8 backward" =
 * AWS Neuron NKI matmul_mxfp8_backward API reference.
 */
#ifndef BSQ_H
#define BSQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bsq_status {
  BSQ_OK = 0,
  BSQ_ERR_NULL = 1,        /* a required pointer is NULL */
  BSQ_ERR_SHAPE = 2,       /* sizes negative, not divisible, or inconsistent */
  BSQ_ERR_DTYPE = 3,       /* a format code outside the enum */
  BSQ_ERR_UNSUPPORTED = 4, /* a valid combination this library does not run */
  BSQ_ERR_ALIGN = 5,       /* a pointer is not 16-byte aligned */
  BSQ_ERR_DEVICE = 6,      /* no HIP device, or the current device is not gfx950 */
  BSQ_ERR_HIP = 7          /* the HIP runtime reported an error */
} bsq_status;

typedef enum bsq_dtype {
  BSQ_F32 = 0,
  BSQ_BF16 = 1,
  BSQ_E4M3 = 2,
  BSQ_E5M2 = 3,
  BSQ_E8M0 = 4,
  BSQ_I8 = 5,
  BSQ_I32 = 6
} bsq_dtype;

/* ---------------------------------------------------------------- misc -- */

/* Library version string, e.g. "0.1.0". Static storage. */
const char* bsq_version(void);
/* Static description of a status code. */
const char* bsq_status_string(int status);
/* Thread-local message for the last failing call on this thread ("" if
 * none).  Valid until the next call on the same thread. */
const char* bsq_last_error(void);
/* Checks that a HIP device is present and the current one is gfx950.
 * Returns BSQ_OK or BSQ_ERR_DEVICE. */
bsq_status bsq_device_check(void);
/* Timing hook for benchmarks.  The next GEMM kernel that this thread
 * launches, through any matmul entry point, is launched with
 * hipExtLaunchKernel and records `start_event` as it begins and
 * `stop_event` as it ends, so that hipEventElapsedTime(start, stop) is that
 * kernel's own duration, with no marker packets around it.  Both are
 * hipEvent_t handles owned by the caller (hipEventCreate); either may be
 * NULL.  The request covers one kernel launch and is then cleared; both NULL
 * clears a pending request.  Returns BSQ_OK. */
bsq_status bsq_time_next_gemm(void* start_event, void* stop_event);

/* ---------------------------------------------------------- quantizers -- */

/* FP8 activation quantizer with 1 x `group` blocks along each row.
 * block_scaled_mm, "Input Generation" (activation path): per block
 * amax = max|x|, s = max(amax / 448, 1e-10) (float32), codes =
 * e4m3fn(clamp(x / s, -448, 448)) with a true float32 division and
 * round-to-nearest-even.
 *   src    float32 [rows, cols]
 *   codes  uint8   [rows, cols]          (E4M3 bytes, out)
 *   scales float32 [rows, cols / group]  (out)
 * Rules: cols % group == 0 (else BSQ_ERR_SHAPE); group is 32, 64, 128 or
 * 256 (else BSQ_ERR_UNSUPPORTED); rows may be 0. */
bsq_status bsq_quant_fp8_rowblock(int64_t rows, int64_t cols, int64_t group,
                                  const float* src, uint8_t* codes, float* scales,
                                  void* stream);

/* FP8 weight quantizer with one scale per group_r x group_c tile.
 * block_scaled_mm, "Input Generation" (weight path), with the tile
 * maximum taken over absolute values (the page's weight path omits abs();
 * the activation path and the workload description use it).
 *   src    float32 [rows, cols]
 *   codes  uint8   [rows, cols]                        (E4M3, out)
 *   scales float32 [rows / group_r, cols / group_c]    (out)
 * Rules: rows % group_r == 0, cols % group_c == 0; the library runs
 * group_r == group_c == 128, at most 2^31 - 1 tiles. */
bsq_status bsq_quant_fp8_tile(int64_t rows, int64_t cols, int64_t group_r, int64_t group_c,
                              const float* src, uint8_t* codes, float* scales, void* stream);

/* MX quantizer: 32-element blocks with an E8M0 scale.
 * scaled_matmul, Notes (mxfp8: e4m3fn or e5m2 codes, e8m0 scales, block
 * 32); mxfp8 backward, Parameters (float8_dtype).  The pages do not state
 * the scale rule; this library's: E = the smallest integer with
 * max(amax, 1e-10) <= fmax * 2^E (fmax 448 for E4M3, 57344 for E5M2),
 * scale byte E + 127, codes = fp8(x * 2^-E) rounded to nearest even.
 *   axis = 1: blocks run along each row.  codes [rows, cols],
 *             scales [rows, cols / 32].
 *   axis = 0: blocks run down each column and the output is written
 *             transposed: codes [cols, rows], scales [cols, rows / 32]
 *             (the layout the backward products consume).
 *   src_dtype  BSQ_F32 or BSQ_BF16;  code_dtype BSQ_E4M3 or BSQ_E5M2.
 * Rules: the blocked extent is a multiple of 32; for axis = 0 both rows
 * and cols are multiples of 32. */
bsq_status bsq_quant_mx(int64_t rows, int64_t cols, int axis, const void* src, int src_dtype,
                        uint8_t* codes, int code_dtype, uint8_t* scales, void* stream);

/* INT8 per-channel quantizer for activations, one scale per row.
 * int8 per-channel, scale and code formulas: s_b = max_i |x_bi| / 127
 * (float32), s_b = 1 when the row is all zero, q = clip(round(x / s),
 * -127, 127), round = nearest with ties to even.
 *   x [B, D] float32 -> x_q [B, D] int8, x_s [B] float32.
 * Rules: B <= 2^31 - 1 (one workgroup per row), else UNSUPPORTED. */
bsq_status bsq_int8_quant_rows(int64_t B, int64_t D, const float* x, int8_t* x_q, float* x_s,
                               void* stream);

/* INT8 per-channel quantizer for weights, one scale per column.
 * int8 per-channel, as above with the max over each column of w.
 *   w    [D_in, D_out] float32
 *   w_q  [D_in, D_out] int8 (w's layout, out)
 *   w_s  [D_out] float32 (out)
 *   w_qT [D_out, D_in] int8, the same codes transposed (K-contiguous, for
 *        bsq_int8_matmul), or NULL to skip.
 * Rules: D_in <= 4194304 (2^22), else UNSUPPORTED. */
bsq_status bsq_int8_quant_cols(int64_t D_in, int64_t D_out, const float* w, int8_t* w_q,
                               float* w_s, int8_t* w_qT, void* stream);

/* -------------------------------------------------------------- matmuls -- */

/* block_scaled_mm: y[m, n] = sum over K-blocks kb of
 *   a_scales[m, kb] * b_scales[n / group_n, kb] * sum_{k in kb} a[m,k] b[n,k]
 * (block_scaled_mm, "Reference Implementation").
 *   a        E4M3 [M, K]            b        E4M3 [N, K]  (both K-contiguous)
 *   a_scales float32 [M, K / group_k]
 *   b_scales float32 [N / group_n, K / group_k]
 *   out      [M, N], out_dtype BSQ_F32 or BSQ_BF16 (nearest even)
 * Rules: N % group_n == 0, K % group_k == 0; M >= 0 arbitrary.  The library
 * runs any group_n (N % 16 == 0) and group_k a multiple of 64 with K % 128
 * == 0; other group_k -> UNSUPPORTED.  group_k == 128 with group_n 1 or
 * 128 is the tuned kernel; other groups run the same kernel with general
 * scale indexing (slower scale handling), and a group_k that is not a
 * multiple of 128 takes two matrix-core products per 128-wide K-step
 * (about half the rate). */
bsq_status bsq_blockwise_fp8_matmul(int64_t M, int64_t N, int64_t K, int64_t group_n,
                                    int64_t group_k, const uint8_t* a, const uint8_t* b,
                                    const float* a_scales, const float* b_scales, void* out,
                                    int out_dtype, void* stream);

/* scaled_matmul: out[b, m, n] = sum_k lhs[b,m,k] lhs_scales[b,m,k/(K/K_a)]
 *                                     rhs[b,n,k] rhs_scales[b,n,k/(K/K_b)]
 * (scaled_matmul, "Mathematically" and Parameters; block size K / K_a).
 *   lhs [B, M, K], rhs [B, N, K] codes (lhs_dtype / rhs_dtype E4M3 or E5M2)
 *   lhs_scales [B, M, K_a], rhs_scales [B, N, K_b] of scale_dtype
 *   out [B, M, N] of out_dtype (BSQ_F32, the page's default, or BSQ_BF16)
 * Rules: K % K_a == 0 and K % K_b == 0 (else SHAPE).  The library runs
 * (K % 128 == 0, N % 16 == 0): scale_dtype E8M0 with blocks K / K_a and
 * K / K_b multiples of 16 (they may differ; unless both are 32, K_a and
 * K_b must be multiples of 4); scale_dtype F32 with E4M3 operands and
 * blocks multiples of 64 (may differ).  Blocks that are not multiples of
 * 32 (E8M0) or 128 (F32) take two matrix-core products per 128-wide
 * K-step (about half the rate).  Other valid combinations (e.g. E8M0
 * block 8) -> UNSUPPORTED. */
bsq_status bsq_scaled_matmul(int64_t B, int64_t M, int64_t N, int64_t K, int64_t K_a,
                             int64_t K_b, const void* lhs, int lhs_dtype, const void* rhs,
                             int rhs_dtype, const void* lhs_scales, const void* rhs_scales,
                             int scale_dtype, void* out, int out_dtype, void* stream);

/* INT8 matmul with per-channel scales (int8 per-channel, output formula and
 * Requirements): a[b, j] = sum_i x_q[b,i] w_q[i,j] accumulated in int32,
 * y[b, j] = float32(a[b, j]) * (x_s[b] * w_s[j]) in float32.
 *   x_q  [B, D_in] int8;  w_qT [D_out, D_in] int8 (w_q transposed, as
 *   written by bsq_int8_quant_cols);  x_s [B], w_s [D_out] float32
 *   y [B, D_out] float32 (out); acc [B, D_out] int32 (out) or NULL.
 * Rules: D_in <= 133144, so that no int32 sum can wrap (127^2 D_in <=
 * 2^31 - 1); larger -> UNSUPPORTED.  Shapes with D_in % 128 == 0,
 * D_out % 16 == 0 and 16-byte aligned x_q, w_qT, w_s run on the int8 matrix
 * core; any other shape runs a plain per-output kernel with the same
 * arithmetic (slower, same results). */
bsq_status bsq_int8_matmul(int64_t B, int64_t D_in, int64_t D_out, const int8_t* x_q,
                           const int8_t* w_qT, const float* x_s, const float* w_s, float* y,
                           int32_t* acc, void* stream);

/* The whole int8 per-channel problem: quantize x by rows and w by
 * columns, multiply in int8 with int32 sums, apply the float32 epilogue.
 * Writes the five results the problem returns (w_q, w_scales, x_q,
 * x_scales, y).  `workspace` holds the transposed weight codes: at least
 * bsq_int8_workspace_bytes(D_in, D_out) bytes, 16-byte aligned.  Rules:
 * those of bsq_int8_quant_rows, bsq_int8_quant_cols and bsq_int8_matmul
 * (D_in <= 133144), all checked before any of the three steps is
 * enqueued. */
size_t bsq_int8_workspace_bytes(int64_t D_in, int64_t D_out);
bsq_status bsq_int8_per_channel_matmul(int64_t B, int64_t D_in, int64_t D_out, const float* x,
                                       const float* w, int8_t* w_q, float* w_s, int8_t* x_q,
                                       float* x_s, float* y, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* The same int8 composite for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument; the transposed weight codes go to a
 * scratch array of bsq_int8_noalloc_max_bytes() bytes (16 MiB) that the
 * library holds on each GPU it runs on until the process ends.  The call
 * allocates and frees nothing.  Outputs are identical to
 * bsq_int8_per_channel_matmul's.
 * Rules: as bsq_int8_per_channel_matmul, and D_in * D_out <= 2^24 (the
 * scratch) else BSQ_ERR_UNSUPPORTED.  Every call on one GPU shares that
 * GPU's scratch: calls that overlap in time on one GPU (e.g. on two
 * streams) race and give undefined results; calls ordered on one stream do
 * not. */
size_t bsq_int8_noalloc_max_bytes(void);
bsq_status bsq_int8_per_channel_matmul_noalloc(int64_t B, int64_t D_in, int64_t D_out, const float* x,
                                               const float* w, int8_t* w_q, float* w_s, int8_t* x_q,
                                               float* x_s, float* y, void* stream);

/* MXFP8 linear-layer backward (mxfp8 backward: forward Y = X W^T with X
 * [M, K], W [N, K]; dX = dY W [M, K] contracting over N; dW = dY^T X [N, K]
 * contracting over M; bf16 inputs quantized on the fly).
 *   dY [M, N], W [N, K], X [M, K]: BSQ_BF16
 *   code_dtype: BSQ_E5M2 (the page's default) or BSQ_E4M3
 *   out_dtype:  BSQ_BF16 (the page's default) or BSQ_F32
 *   dX [M, K], dW [N, K] (out)
 * The MX blocks run along each product's contraction axis.  `workspace`
 * receives the quantized operands: at least
 * bsq_mxfp8_backward_workspace_bytes(M, N, K) bytes.
 * Rules: M, N, K multiples of 128 (else UNSUPPORTED; negative -> SHAPE);
 * a smaller workspace -> SHAPE. */
size_t bsq_mxfp8_backward_workspace_bytes(int64_t M, int64_t N, int64_t K);
bsq_status bsq_mxfp8_backward(int64_t M, int64_t N, int64_t K, const void* dY, const void* W,
                              const void* X, int code_dtype, int out_dtype, void* dX, void* dW,
                              void* workspace, size_t workspace_bytes, void* stream);

/* The same backward in two calls, for pre-quantized operands and for
 * quantizing an operand once and reusing it (mxfp8 backward, parameters:
 * the optional pre-computed scales of output_grad, weights and
 * input_activation; packed scales for pre-quantized inputs; spilling the
 * quantized blocks to HBM and reloading them).  The four operands of the
 * two products, each a codes array plus an E8M0 scale array (one byte per
 * 32-element block, rows of blocks contiguous: four scales to a 32-bit
 * word), all row-major and K-contiguous along the product's contraction:
 *   dyn: dY blocked along N,  codes [M, N], scales [M, N/32]   (A of dX)
 *   wt:  W blocked along N, transposed,  codes [K, N], scales [K, N/32]
 *        (B of dX)
 *   dyt: dY blocked along M, transposed, codes [N, M], scales [N, M/32]
 *        (A of dW)
 *   xt:  X blocked along M, transposed,  codes [K, M], scales [K, M/32]
 *        (B of dW)
 * bsq_mxfp8_backward computes exactly these four (into its workspace) and
 * then exactly these two products, so the two-call path gives the same
 * bits.
 *
 * bsq_mxfp8_backward_quantize: bf16 dY [M, N], W [N, K], X [M, K] ->
 * each operand whose codes pointer is non-NULL (its scales then must be
 * non-NULL too, and its source).  E.g. W's operand once per weight update,
 * dY's two per micro-batch.  A NULL codes pointer with non-NULL scales ->
 * BSQ_ERR_NULL.
 *
 * bsq_mxfp8_backward_gemms: dX [M, K] = dyn . wt (contract N) when dX is
 * non-NULL, dW [N, K] = dyt . xt (contract M) when dW is non-NULL; the
 * operands of a requested product must be non-NULL.  out_dtype BSQ_BF16 or
 * BSQ_F32 for both.  An empty contraction (N = 0 for dX, M = 0 for dW)
 * writes zeros.
 * Rules for both: M, N, K multiples of 128 (else UNSUPPORTED; negative ->
 * SHAPE); code_dtype BSQ_E5M2 or BSQ_E4M3 for every operand. */
bsq_status bsq_mxfp8_backward_quantize(int64_t M, int64_t N, int64_t K, const void* dY, const void* W,
                                       const void* X, int code_dtype, uint8_t* dyn_codes,
                                       uint8_t* dyn_scales, uint8_t* wt_codes, uint8_t* wt_scales,
                                       uint8_t* dyt_codes, uint8_t* dyt_scales, uint8_t* xt_codes,
                                       uint8_t* xt_scales, void* stream);
bsq_status bsq_mxfp8_backward_gemms(int64_t M, int64_t N, int64_t K, int code_dtype, int out_dtype,
                                    const uint8_t* dyn_codes, const uint8_t* dyn_scales,
                                    const uint8_t* wt_codes, const uint8_t* wt_scales,
                                    const uint8_t* dyt_codes, const uint8_t* dyt_scales,
                                    const uint8_t* xt_codes, const uint8_t* xt_scales, void* dX, void* dW,
                                    void* stream);

/* scaled_matmul with nvfp4 operands (scaled_matmul, Notes: float4_e2m1fn
 * operands, float8_e4m3fn scales, block 16; the sum as in
 * bsq_scaled_matmul with K_a = K_b = K / 16).
 *   lhs [B, M, K/2], rhs [B, N, K/2]: e2m1 codes, two per byte, the element
 *       with the lower K index in the low nibble
 *   lhs_scales [B, M, K/16], rhs_scales [B, N, K/16]: e4m3 (OCP e4m3fn)
 *   out [B, M, N], out_dtype BSQ_F32 or BSQ_BF16
 *   workspace: at least bsq_nvfp4_workspace_bytes(B, M, N, K) bytes; it
 *       receives both operands dequantized to bfloat16 (exact: an e2m1
 *       value times an e4m3 scale has at most 6 significant bits), which
 *       a bf16 matrix-core product then multiplies in float32.
 * Rules: K % 16 == 0 (else SHAPE); the library needs K % 128 == 0,
 * N % 16 == 0 and B * M * K, B * N * K <= 2^40 (else UNSUPPORTED); a
 * smaller workspace -> SHAPE. */
size_t bsq_nvfp4_workspace_bytes(int64_t B, int64_t M, int64_t N, int64_t K);
bsq_status bsq_scaled_matmul_nvfp4(int64_t B, int64_t M, int64_t N, int64_t K, const uint8_t* lhs,
                                   const uint8_t* rhs, const uint8_t* lhs_scales,
                                   const uint8_t* rhs_scales, void* out, int out_dtype, void* workspace,
                                   size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BSQ_H */
