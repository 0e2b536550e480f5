// Launchers of the quantizer kernels (arguments already validated).
#pragma once

#include "common.h"

namespace bsq {

bsq_status launch_fp8_rowblock(int64_t rows, int64_t cols, int64_t group, const float* src,
                               uint8_t* codes, float* scales, hipStream_t st);
bsq_status launch_fp8_tile128(int64_t rows, int64_t cols, const float* src, uint8_t* codes,
                              float* scales, hipStream_t st);
bsq_status launch_mx(int64_t rows, int64_t cols, int axis, const void* src, bool src_bf16,
                     uint8_t* codes, bool e5m2, uint8_t* scales, hipStream_t st);
// Blocks of 32 down the columns of up to three matrices in one launch, each
// rows x cols (both multiples of 32) from src: codes_t [cols, rows] and
// scales_t [cols, rows / 32], the bytes of launch_mx with axis 0.  A job
// with row_codes set also writes blocks of 32 along its rows into
// row_codes [rows, cols] / row_scales [rows, cols / 32] (the bytes of
// launch_mx with axis 1) from the same read of src.
struct MxT {
  const void* src;
  int64_t rows, cols;
  uint8_t* codes_t;
  uint8_t* scales_t;
  uint8_t* row_codes;
  uint8_t* row_scales;
};
bsq_status launch_mx_cols(const MxT* jobs, int n, bool src_bf16, bool e5m2, hipStream_t st);
bsq_status launch_int8_rows(int64_t B, int64_t D, const float* x, int8_t* xq, float* xs,
                            hipStream_t st);
bsq_status launch_int8_cols(int64_t D_in, int64_t D_out, const float* w, int8_t* wq, float* ws,
                            int8_t* wqT, hipStream_t st);
// nvfp4 rows (K/2 bytes of e2m1 codes, low nibble first, and K/16 e4m3
// scales per row) -> bf16 [rows, K]; exact.  K % 16 == 0.
bsq_status launch_nvfp4_to_bf16(int64_t rows, int64_t K, const uint8_t* codes, const uint8_t* scales,
                                uint16_t* out, hipStream_t st);

}  // namespace bsq
