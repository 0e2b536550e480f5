// Launcher of the block-scaled GEMM kernels (arguments already validated).
#pragma once

#include "common.h"

namespace bsq {

// MODE_BF16: bfloat16 operands without scales (the operand dequantized
// from nvfp4), K counted in elements; float32 accumulation.
enum GemmMode { MODE_FP8G = 0, MODE_MX = 1, MODE_I8 = 2, MODE_BF16 = 3 };

struct GemmLaunch {
  int mode;          // GemmMode
  int64_t batch, M, N, K;
  const void* A;     // [batch, M, K] codes, K-contiguous
  const void* B;     // [batch, N, K] codes, K-contiguous
  const void* SA;    // FP8G: float [batch, M, K/128]; MX: e8m0 [batch, M, K/32]; I8: float [M]
  const void* SB;    // FP8G: float [batch, N/128 or N, K/128]; MX: e8m0 [batch, N, K/32]; I8: float [N]
  void* out;         // [batch, M, N] float32 or bf16
  int32_t* acc_out;  // I8 only, optional [M, N] int32
  bool out_bf16;
  bool gn1;          // FP8G: one B scale per row instead of per 128 rows
  bool fa_e5m2, fb_e5m2;
  // General scale blocks (gen = true): SA [batch, M, sc_a], SB [batch, N /
  // gn (FP8G; gn a multiple of 128 takes one scale per 128 columns, others
  // one per column) or N (MX), sc_b]; a scale covers sg_a / sg_b granules:
  // K-steps of 128 (FP8G, float32 scales, e4m3 operands) or 32-element
  // blocks (MX, e8m0); with sub = true, half steps of 64 (FP8G) or
  // 16-element blocks (MX).  sc_a * sg_a * granule == K, likewise for B; MX
  // needs sc_a and sc_b multiples of 4 (word-aligned scale rows).
  bool gen;
  bool sub;
  int sc_a, sc_b, sg_a, sg_b, gn;
};

// Requires K % 128 == 0 (MODE_BF16: K % 64 == 0) and N % 16 == 0; M, N,
// batch >= 0.
bsq_status launch_gemm(const GemmLaunch& L, hipStream_t st);

// Exact int8 matmul for any D_in, D_out (one thread per output): the same
// int32 sums and the same float32 epilogue as the MFMA path.
bsq_status launch_int8_matmul_small(int64_t B, int64_t D_in, int64_t D_out, const int8_t* xq,
                                    const int8_t* wqT, const float* xs, const float* ws, float* y,
                                    int32_t* acc, hipStream_t st);

}  // namespace bsq
