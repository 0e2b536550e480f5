// The C ABI of libbsq (declared in include/bsq.h): argument validation on
// the host, then kernel launches on the caller's stream.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "gemm.h"
#include "quant.h"

namespace bsq {

namespace {
thread_local std::string g_last_error;
thread_local GemmEvents g_gemm_events;
std::mutex g_dev_mu;
std::vector<int> g_dev_state;  // per device: 0 unknown, 1 gfx950, 2 other
}  // namespace

bsq_status fail(bsq_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

bsq_status ok() {
  g_last_error.clear();
  return BSQ_OK;
}

GemmEvents take_gemm_events() {
  const GemmEvents e = g_gemm_events;
  g_gemm_events = GemmEvents{};
  return e;
}

bsq_status require_gfx950() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(BSQ_ERR_DEVICE, "no HIP device available");
  }
  std::lock_guard<std::mutex> lk(g_dev_mu);
  if (size_t(dev) >= g_dev_state.size()) g_dev_state.resize(size_t(dev) + 1, 0);
  if (g_dev_state[size_t(dev)] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(BSQ_ERR_DEVICE, "hipGetDeviceProperties failed");
    }
    g_dev_state[size_t(dev)] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  if (g_dev_state[size_t(dev)] != 1) return fail(BSQ_ERR_DEVICE, "the current device is not gfx950");
  return BSQ_OK;
}

bsq_status launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BSQ_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return ok();
}

}  // namespace bsq

using namespace bsq;

namespace {

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

bool is_fp8(int d) { return d == BSQ_E4M3 || d == BSQ_E5M2; }
bool known_dtype(int d) { return d >= BSQ_F32 && d <= BSQ_I32; }

// Shared tail of every call: the device check comes after the host-side
// argument checks, so argument errors are reported without a GPU.
#define BSQ_DEVICE()                                 \
  do {                                               \
    bsq_status _s = ::bsq::require_gfx950();         \
    if (_s != BSQ_OK) return _s;                     \
  } while (0)

}  // namespace

extern "C" {

const char* bsq_version(void) { return "0.1.0"; }

const char* bsq_status_string(int status) {
  switch (status) {
    case BSQ_OK: return "ok";
    case BSQ_ERR_NULL: return "null pointer";
    case BSQ_ERR_SHAPE: return "invalid shape";
    case BSQ_ERR_DTYPE: return "invalid dtype";
    case BSQ_ERR_UNSUPPORTED: return "unsupported combination";
    case BSQ_ERR_ALIGN: return "misaligned pointer";
    case BSQ_ERR_DEVICE: return "no gfx950 device";
    case BSQ_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* bsq_last_error(void) { return g_last_error.c_str(); }

bsq_status bsq_device_check(void) {
  const bsq_status s = require_gfx950();
  return s == BSQ_OK ? ok() : s;
}

bsq_status bsq_time_next_gemm(void* start_event, void* stop_event) {
  g_gemm_events.start = static_cast<hipEvent_t>(start_event);
  g_gemm_events.stop = static_cast<hipEvent_t>(stop_event);
  return ok();
}

// Largest array the calls take, in elements: far beyond device memory, and
// small enough that every byte offset derived from it fits 64 bits.
constexpr int64_t kMaxElems = int64_t(1) << 60;
// a * b * c <= kMaxElems for non-negative factors, without overflow
static inline bool elems_fit(int64_t a, int64_t b, int64_t c = 1) {
  int64_t n = 0;
  return !__builtin_mul_overflow(a, b, &n) && !__builtin_mul_overflow(n, c, &n) && n <= kMaxElems;
}

// ------------------------------------------------------------ quantizers --

bsq_status bsq_quant_fp8_rowblock(int64_t rows, int64_t cols, int64_t group, const float* src,
                                  uint8_t* codes, float* scales, void* stream) {
  BSQ_CHECK(rows >= 0 && cols >= 0 && group > 0, BSQ_ERR_SHAPE, "negative size or group <= 0");
  BSQ_CHECK(elems_fit(rows, cols), BSQ_ERR_UNSUPPORTED, "more than 2^60 elements");
  BSQ_CHECK(cols % group == 0, BSQ_ERR_SHAPE, "cols must be a multiple of group");
  BSQ_CHECK(group == 32 || group == 64 || group == 128 || group == 256, BSQ_ERR_UNSUPPORTED,
            "group must be 32, 64, 128 or 256");
  if (rows == 0 || cols == 0) return ok();
  BSQ_CHECK_PTR(src);
  BSQ_CHECK_PTR(codes);
  BSQ_CHECK_PTR(scales);
  BSQ_DEVICE();
  return launch_fp8_rowblock(rows, cols, group, src, codes, scales, as_stream(stream));
}

bsq_status bsq_quant_fp8_tile(int64_t rows, int64_t cols, int64_t group_r, int64_t group_c,
                              const float* src, uint8_t* codes, float* scales, void* stream) {
  BSQ_CHECK(rows >= 0 && cols >= 0 && group_r > 0 && group_c > 0, BSQ_ERR_SHAPE,
            "negative size or group <= 0");
  BSQ_CHECK(elems_fit(rows, cols), BSQ_ERR_UNSUPPORTED, "more than 2^60 elements");
  BSQ_CHECK(rows % group_r == 0 && cols % group_c == 0, BSQ_ERR_SHAPE,
            "rows and cols must be multiples of the tile");
  BSQ_CHECK(group_r == 128 && group_c == 128, BSQ_ERR_UNSUPPORTED, "tile must be 128 x 128");
  // one workgroup per tile along a one-dimensional grid
  BSQ_CHECK((rows / 128) * (cols / 128) <= int64_t(0x7FFFFFFF), BSQ_ERR_UNSUPPORTED,
            "more than 2^31 - 1 tiles");
  if (rows == 0 || cols == 0) return ok();
  BSQ_CHECK_PTR(src);
  BSQ_CHECK_PTR(codes);
  BSQ_CHECK_PTR(scales);
  BSQ_DEVICE();
  return launch_fp8_tile128(rows, cols, src, codes, scales, as_stream(stream));
}

bsq_status bsq_quant_mx(int64_t rows, int64_t cols, int axis, const void* src, int src_dtype,
                        uint8_t* codes, int code_dtype, uint8_t* scales, void* stream) {
  BSQ_CHECK(rows >= 0 && cols >= 0, BSQ_ERR_SHAPE, "negative size");
  BSQ_CHECK(elems_fit(rows, cols), BSQ_ERR_UNSUPPORTED, "more than 2^60 elements");
  BSQ_CHECK(axis == 0 || axis == 1, BSQ_ERR_SHAPE, "axis must be 0 or 1");
  BSQ_CHECK(known_dtype(src_dtype) && known_dtype(code_dtype), BSQ_ERR_DTYPE, "unknown dtype");
  BSQ_CHECK(src_dtype == BSQ_F32 || src_dtype == BSQ_BF16, BSQ_ERR_UNSUPPORTED,
            "src_dtype must be F32 or BF16");
  BSQ_CHECK(is_fp8(code_dtype), BSQ_ERR_UNSUPPORTED, "code_dtype must be E4M3 or E5M2");
  if (axis == 1) {
    BSQ_CHECK(cols % 32 == 0, BSQ_ERR_SHAPE, "cols must be a multiple of 32 (axis 1)");
  } else {
    BSQ_CHECK(rows % 32 == 0 && cols % 32 == 0, BSQ_ERR_SHAPE,
              "rows and cols must be multiples of 32 (axis 0)");
  }
  if (rows == 0 || cols == 0) return ok();
  BSQ_CHECK_PTR(src);
  BSQ_CHECK_PTR(codes);
  BSQ_CHECK(scales != nullptr, BSQ_ERR_NULL, "scales is NULL");
  BSQ_DEVICE();
  return launch_mx(rows, cols, axis, src, src_dtype == BSQ_BF16, codes, code_dtype == BSQ_E5M2,
                   scales, as_stream(stream));
}

bsq_status bsq_int8_quant_rows(int64_t B, int64_t D, const float* x, int8_t* x_q, float* x_s,
                               void* stream) {
  BSQ_CHECK(B >= 0 && D >= 0, BSQ_ERR_SHAPE, "negative size");
  // one workgroup per row along the grid's x
  BSQ_CHECK(B <= int64_t(0x7FFFFFFF), BSQ_ERR_UNSUPPORTED, "B > 2^31 - 1 rows");
  BSQ_CHECK(elems_fit(B, D), BSQ_ERR_UNSUPPORTED, "more than 2^60 elements");
  if (B == 0) return ok();
  BSQ_CHECK_PTR(x_s);
  if (D > 0) {
    BSQ_CHECK_PTR(x);
    BSQ_CHECK_PTR(x_q);
  }
  BSQ_DEVICE();
  return launch_int8_rows(B, D, x, x_q, x_s, as_stream(stream));
}

// Longest column the int8 column quantizer takes: its two-pass grids hold
// D_in / 64 row blocks along y.
constexpr int64_t kMaxInt8ColsRows = int64_t(64) * 65536;

bsq_status bsq_int8_quant_cols(int64_t D_in, int64_t D_out, const float* w, int8_t* w_q,
                               float* w_s, int8_t* w_qT, void* stream) {
  BSQ_CHECK(D_in >= 0 && D_out >= 0, BSQ_ERR_SHAPE, "negative size");
  BSQ_CHECK(D_in <= kMaxInt8ColsRows, BSQ_ERR_UNSUPPORTED,
            "D_in > 4194304: beyond the column quantizer's grid");
  BSQ_CHECK(elems_fit(D_in, D_out), BSQ_ERR_UNSUPPORTED, "more than 2^60 elements");
  if (D_out == 0) return ok();
  BSQ_CHECK_PTR(w_s);
  if (D_in > 0) {
    BSQ_CHECK_PTR(w);
    BSQ_CHECK_PTR(w_q);
    if (w_qT != nullptr) BSQ_CHECK(aligned16(w_qT), BSQ_ERR_ALIGN, "w_qT is not 16-byte aligned");
  }
  BSQ_DEVICE();
  return launch_int8_cols(D_in, D_out, w, w_q, w_s, D_in > 0 ? w_qT : nullptr, as_stream(stream));
}

// --------------------------------------------------------------- matmuls --

// Longest contraction the GEMM kernels address: their per-lane buffer
// offsets reach 64 rows of K bytes in 32 bits.
constexpr int64_t kMaxContraction = int64_t(1) << 24;
// Longest batch of products: the GEMM grids put the batch along z.
constexpr int64_t kMaxBatch = 65535;
// The GEMM grids number one product's output tiles (down to 128 x 256) along
// x, which holds at most 2^31 - 1.  Composites check this before their first
// step; a lone product's launcher checks it too.
static inline bool gemm_tiles_fit(int64_t M, int64_t N) {
  return ((M + 127) / 128) * ((N + 255) / 256) <= int64_t(0x7FFFFFFF);
}

bsq_status bsq_blockwise_fp8_matmul(int64_t M, int64_t N, int64_t K, int64_t group_n,
                                    int64_t group_k, const uint8_t* a, const uint8_t* b,
                                    const float* a_scales, const float* b_scales, void* out,
                                    int out_dtype, void* stream) {
  BSQ_CHECK(M >= 0 && N >= 0 && K >= 0 && group_n > 0 && group_k > 0, BSQ_ERR_SHAPE,
            "negative size or group <= 0");
  BSQ_CHECK(N % group_n == 0 && K % group_k == 0, BSQ_ERR_SHAPE,
            "N and K must be multiples of group_n and group_k");
  BSQ_CHECK(known_dtype(out_dtype), BSQ_ERR_DTYPE, "unknown out_dtype");
  BSQ_CHECK(out_dtype == BSQ_F32 || out_dtype == BSQ_BF16, BSQ_ERR_UNSUPPORTED,
            "out_dtype must be F32 or BF16");
  BSQ_CHECK(group_k % 64 == 0, BSQ_ERR_UNSUPPORTED, "the library runs group_k multiples of 64");
  BSQ_CHECK(N % 16 == 0, BSQ_ERR_UNSUPPORTED, "N must be a multiple of 16");
  BSQ_CHECK(M <= (int64_t(1) << 30) && N <= (int64_t(1) << 30) && K <= kMaxContraction,
            BSQ_ERR_UNSUPPORTED, "extent too large");
  if (M == 0 || N == 0) return ok();
  BSQ_CHECK_PTR(out);
  if (K > 0) {
    BSQ_CHECK_PTR(a);
    BSQ_CHECK_PTR(b);
    BSQ_CHECK(a_scales != nullptr && b_scales != nullptr, BSQ_ERR_NULL, "scales are NULL");
  }
  BSQ_DEVICE();
  GemmLaunch L{};
  L.mode = MODE_FP8G;
  L.batch = 1;
  L.M = M; L.N = N; L.K = K;
  L.A = a; L.B = b; L.SA = a_scales; L.SB = b_scales;
  L.out = out;
  L.out_bf16 = out_dtype == BSQ_BF16;
  L.gn1 = group_n == 1;
  if (group_k != 128 || (group_n != 1 && group_n != 128)) {
    // general groups: per-column B scale rows n / group_n, group_k / 128
    // K-steps per scale (group_k / 64 half steps when group_k is not a
    // multiple of 128)
    L.gen = true;
    L.gn1 = true;
    L.gn = int(group_n);
    L.sc_a = L.sc_b = int(K / group_k);
    L.sub = group_k % 128 != 0;
    L.sg_a = L.sg_b = int(group_k / (L.sub ? 64 : 128));
  }
  return launch_gemm(L, as_stream(stream));
}

bsq_status bsq_scaled_matmul(int64_t B, int64_t M, int64_t N, int64_t K, int64_t K_a,
                             int64_t K_b, const void* lhs, int lhs_dtype, const void* rhs,
                             int rhs_dtype, const void* lhs_scales, const void* rhs_scales,
                             int scale_dtype, void* out, int out_dtype, void* stream) {
  BSQ_CHECK(B >= 0 && M >= 0 && N >= 0 && K >= 0 && K_a >= 0 && K_b >= 0, BSQ_ERR_SHAPE,
            "negative size");
  BSQ_CHECK(K_a > 0 && K_b > 0 && K % K_a == 0 && K % K_b == 0, BSQ_ERR_SHAPE,
            "K must be a multiple of K_a and of K_b");
  BSQ_CHECK(known_dtype(lhs_dtype) && known_dtype(rhs_dtype) && known_dtype(scale_dtype) &&
                known_dtype(out_dtype),
            BSQ_ERR_DTYPE, "unknown dtype");
  BSQ_CHECK(is_fp8(lhs_dtype) && is_fp8(rhs_dtype), BSQ_ERR_UNSUPPORTED,
            "operands must be E4M3 or E5M2");
  BSQ_CHECK(out_dtype == BSQ_F32 || out_dtype == BSQ_BF16, BSQ_ERR_UNSUPPORTED,
            "out_dtype must be F32 or BF16");
  BSQ_CHECK(K % 128 == 0 && N % 16 == 0, BSQ_ERR_UNSUPPORTED,
            "the library needs K % 128 == 0 and N % 16 == 0");
  BSQ_CHECK(M <= (int64_t(1) << 30) && N <= (int64_t(1) << 30) && K <= kMaxContraction,
            BSQ_ERR_UNSUPPORTED, "extent too large");
  BSQ_CHECK(B <= kMaxBatch, BSQ_ERR_UNSUPPORTED, "batch over 65535");
  BSQ_CHECK(elems_fit(B, M, K) && elems_fit(B, N, K) && elems_fit(B, M, N), BSQ_ERR_UNSUPPORTED,
            "an operand or the output of more than 2^60 elements");
  GemmLaunch L{};
  const int64_t blk_a = K / K_a, blk_b = K / K_b;  // elements per scale along K
  if (scale_dtype == BSQ_E8M0) {
    BSQ_CHECK(blk_a % 16 == 0 && blk_b % 16 == 0, BSQ_ERR_UNSUPPORTED,
              "E8M0 scale blocks must be multiples of 16");
    L.mode = MODE_MX;
    if (blk_a != 32 || blk_b != 32) {
      BSQ_CHECK(K_a % 4 == 0 && K_b % 4 == 0, BSQ_ERR_UNSUPPORTED,
                "with E8M0 blocks other than 32, K_a and K_b must be multiples of 4");
      L.gen = true;
      L.sc_a = int(K_a); L.sc_b = int(K_b);
      // blocks that are not multiples of 32 count in 16-element granules
      L.sub = blk_a % 32 != 0 || blk_b % 32 != 0;
      L.sg_a = int(blk_a / (L.sub ? 16 : 32)); L.sg_b = int(blk_b / (L.sub ? 16 : 32));
    }
  } else if (scale_dtype == BSQ_F32) {
    BSQ_CHECK(blk_a % 64 == 0 && blk_b % 64 == 0, BSQ_ERR_UNSUPPORTED,
              "F32 scale blocks must be multiples of 64");
    BSQ_CHECK(lhs_dtype == BSQ_E4M3 && rhs_dtype == BSQ_E4M3, BSQ_ERR_UNSUPPORTED,
              "F32-scaled operands must be E4M3");
    L.mode = MODE_FP8G;
    L.gn1 = true;
    if (blk_a != 128 || blk_b != 128) {
      L.gen = true;
      L.gn = 1;
      L.sc_a = int(K_a); L.sc_b = int(K_b);
      // blocks that are not multiples of 128 count in 64-wide half steps
      L.sub = blk_a % 128 != 0 || blk_b % 128 != 0;
      L.sg_a = int(blk_a / (L.sub ? 64 : 128)); L.sg_b = int(blk_b / (L.sub ? 64 : 128));
    }
  } else {
    return fail(BSQ_ERR_UNSUPPORTED, "scale_dtype must be E8M0 or F32");
  }
  if (B == 0 || M == 0 || N == 0) return ok();
  BSQ_CHECK_PTR(out);
  if (K > 0) {
    BSQ_CHECK_PTR(lhs);
    BSQ_CHECK_PTR(rhs);
    BSQ_CHECK(lhs_scales != nullptr && rhs_scales != nullptr, BSQ_ERR_NULL, "scales are NULL");
    if (scale_dtype == BSQ_E8M0)
      BSQ_CHECK((reinterpret_cast<uintptr_t>(lhs_scales) & 3) == 0 &&
                    (reinterpret_cast<uintptr_t>(rhs_scales) & 3) == 0,
                BSQ_ERR_ALIGN, "scales must be 4-byte aligned");
  }
  BSQ_DEVICE();
  L.batch = B;
  L.M = M; L.N = N; L.K = K;
  L.A = lhs; L.B = rhs; L.SA = lhs_scales; L.SB = rhs_scales;
  L.out = out;
  L.out_bf16 = out_dtype == BSQ_BF16;
  L.fa_e5m2 = lhs_dtype == BSQ_E5M2;
  L.fb_e5m2 = rhs_dtype == BSQ_E5M2;
  return launch_gemm(L, as_stream(stream));
}

// Longest int8 contraction whose int32 sums cannot wrap: |a| <= 127^2 D_in
// stays at or below 2^31 - 1 (the problem's sums are int32).
constexpr int64_t kMaxInt8Contraction = (int64_t(0x7FFFFFFF)) / (127 * 127);  // 133144

bsq_status bsq_int8_matmul(int64_t B, int64_t D_in, int64_t D_out, const int8_t* x_q,
                           const int8_t* w_qT, const float* x_s, const float* w_s, float* y,
                           int32_t* acc, void* stream) {
  BSQ_CHECK(B >= 0 && D_in >= 0 && D_out >= 0, BSQ_ERR_SHAPE, "negative size");
  BSQ_CHECK(B <= (int64_t(1) << 30) && D_out <= (int64_t(1) << 30), BSQ_ERR_UNSUPPORTED,
            "extent too large");
  BSQ_CHECK(D_in <= kMaxInt8Contraction, BSQ_ERR_UNSUPPORTED,
            "D_in > 133144: int32 sums of int8 products could wrap");
  if (B == 0 || D_out == 0) return ok();
  BSQ_CHECK_PTR(y);
  BSQ_CHECK(x_s != nullptr && w_s != nullptr, BSQ_ERR_NULL, "scales are NULL");
  if (D_in > 0) {
    BSQ_CHECK(x_q != nullptr && w_qT != nullptr, BSQ_ERR_NULL, "codes are NULL");
  }
  if (acc != nullptr) BSQ_CHECK(aligned16(acc), BSQ_ERR_ALIGN, "acc is not 16-byte aligned");
  BSQ_DEVICE();
  const bool mfma = D_in % 128 == 0 && D_out % 16 == 0 && aligned16(x_q) && aligned16(w_qT) &&
                    aligned16(w_s) && D_in > 0;
  if (!mfma)
    return launch_int8_matmul_small(B, D_in, D_out, x_q, w_qT, x_s, w_s, y, acc, as_stream(stream));
  GemmLaunch L{};
  L.mode = MODE_I8;
  L.batch = 1;
  L.M = B; L.N = D_out; L.K = D_in;
  L.A = x_q; L.B = w_qT; L.SA = x_s; L.SB = w_s;
  L.out = y;
  L.acc_out = acc;
  return launch_gemm(L, as_stream(stream));
}

size_t bsq_int8_workspace_bytes(int64_t D_in, int64_t D_out) {
  if (D_in <= 0 || D_out <= 0) return 0;
  int64_t n = 0;
  if (__builtin_mul_overflow(D_in, D_out, &n) || n > (int64_t(1) << 62)) return SIZE_MAX;
  return size_t((n + 255) / 256 * 256);
}

bsq_status bsq_int8_per_channel_matmul(int64_t B, int64_t D_in, int64_t D_out, const float* x,
                                       const float* w, int8_t* w_q, float* w_s, int8_t* x_q,
                                       float* x_s, float* y, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  BSQ_CHECK(B >= 0 && D_in >= 0 && D_out >= 0, BSQ_ERR_SHAPE, "negative size");
  BSQ_CHECK(D_in <= kMaxInt8Contraction, BSQ_ERR_UNSUPPORTED,
            "D_in > 133144: int32 sums of int8 products could wrap");
  BSQ_CHECK(B <= (int64_t(1) << 30) && D_out <= (int64_t(1) << 30), BSQ_ERR_UNSUPPORTED,
            "extent too large");
  BSQ_CHECK(workspace_bytes >= bsq_int8_workspace_bytes(D_in, D_out), BSQ_ERR_SHAPE,
            "workspace too small");
  // every step's pointer rules, checked before anything is enqueued
  if (B > 0) BSQ_CHECK_PTR(x_s);
  if (B > 0 && D_in > 0) {
    BSQ_CHECK_PTR(x);
    BSQ_CHECK_PTR(x_q);
  }
  if (D_out > 0) BSQ_CHECK_PTR(w_s);
  if (D_in > 0 && D_out > 0) {
    BSQ_CHECK_PTR(w);
    BSQ_CHECK_PTR(w_q);
    BSQ_CHECK_PTR(workspace);
  }
  if (B > 0 && D_out > 0) BSQ_CHECK_PTR(y);
  int8_t* wqT = static_cast<int8_t*>(workspace);
  bsq_status s = bsq_int8_quant_rows(B, D_in, x, x_q, x_s, stream);
  if (s != BSQ_OK) return s;
  s = bsq_int8_quant_cols(D_in, D_out, w, w_q, w_s, D_in > 0 ? wqT : nullptr, stream);
  if (s != BSQ_OK) return s;
  return bsq_int8_matmul(B, D_in, D_out, x_q, wqT, x_s, w_s, y, nullptr, stream);
}

}  // extern "C"

// ---------------------------------------------- the composite, no allocation --
// For callers that cannot allocate (HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc): the int8 composite with its workspace
// (the transposed weight codes) in a file-scope device array instead of a
// caller buffer.  The array exists once per GPU for the life of the process;
// host code never uses its name as an address, only the address that
// hipGetSymbolAddress returns for the current device (each GPU holds its own
// copy at its own address).
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;  // 16 MiB: D_in * D_out <= 2^24
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device: the address of `scratch`, or null before its first use

// The current device's copy of `scratch`, looked up once per device with
// that device current.
bsq_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(BSQ_ERR_DEVICE, "no HIP device available");
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (size_t(dev) >= g_scratch_ptr.size()) g_scratch_ptr.resize(size_t(dev) + 1, nullptr);
  if (g_scratch_ptr[size_t(dev)] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return fail(BSQ_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    }
    g_scratch_ptr[size_t(dev)] = ptr;
  }
  *out = g_scratch_ptr[size_t(dev)];
  return BSQ_OK;
}

}  // namespace

extern "C" {

size_t bsq_int8_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

bsq_status bsq_int8_per_channel_matmul_noalloc(int64_t B, int64_t D_in, int64_t D_out, const float* x,
                                               const float* w, int8_t* w_q, float* w_s, int8_t* x_q,
                                               float* x_s, float* y, void* stream) {
  BSQ_CHECK(B >= 0 && D_in >= 0 && D_out >= 0, BSQ_ERR_SHAPE, "negative size");
  BSQ_CHECK(D_in <= kMaxInt8Contraction, BSQ_ERR_UNSUPPORTED,
            "D_in > 133144: int32 sums of int8 products could wrap");
  BSQ_CHECK(B <= (int64_t(1) << 30) && D_out <= (int64_t(1) << 30), BSQ_ERR_UNSUPPORTED,
            "extent too large");
  const size_t need = bsq_int8_workspace_bytes(D_in, D_out);
  BSQ_CHECK(need <= kNoAllocScratchBytes, BSQ_ERR_UNSUPPORTED,
            "D_in * D_out exceeds the 16 MiB scratch of the no-allocation entry point");
  // the composite's pointer rules, checked before the device is touched
  if (B > 0) BSQ_CHECK_PTR(x_s);
  if (B > 0 && D_in > 0) {
    BSQ_CHECK_PTR(x);
    BSQ_CHECK_PTR(x_q);
  }
  if (D_out > 0) BSQ_CHECK_PTR(w_s);
  if (D_in > 0 && D_out > 0) {
    BSQ_CHECK_PTR(w);
    BSQ_CHECK_PTR(w_q);
  }
  if (B > 0 && D_out > 0) BSQ_CHECK_PTR(y);
  void* ws = nullptr;
  if (need > 0) {
    BSQ_DEVICE();
    const bsq_status s = scratch_for_current_device(&ws);
    if (s != BSQ_OK) return s;
  }
  // the transposed codes are written in full by the column quantizer before
  // the GEMM reads them: nothing in the scratch needs clearing
  return bsq_int8_per_channel_matmul(B, D_in, D_out, x, w, w_q, w_s, x_q, x_s, y, ws, need, stream);
}

}  // extern "C"

extern "C" {

// MXFP8 backward: four MX quantizations into the workspace, then two
// scaled GEMMs on K-contiguous operands.
namespace {
struct BwdLayout {
  size_t dyn_codes, dyn_scales, wt_codes, wt_scales, dyt_codes, dyt_scales, xt_codes, xt_scales,
      total;
};
size_t up256(size_t v) { return (v + 255) / 256 * 256; }
// The four MX operands of the two backward products, each K-contiguous
// (blocks of 32 along the product's contraction axis):
//   dyn: dY blocked along N [M, N] (+ [M, N/32] scales)      A of dX
//   wt:  W blocked along N, transposed [K, N] (+ [K, N/32])   B of dX
//   dyt: dY blocked along M, transposed [N, M] (+ [N, M/32])  A of dW
//   xt:  X blocked along M, transposed [K, M] (+ [K, M/32])   B of dW
struct BwdOps {
  const uint8_t *dyn_c, *dyn_s, *wt_c, *wt_s, *dyt_c, *dyt_s, *xt_c, *xt_s;
};

bsq_status bwd_check_dims(int64_t M, int64_t N, int64_t K, int code_dtype) {
  BSQ_CHECK(M >= 0 && N >= 0 && K >= 0, BSQ_ERR_SHAPE, "negative size");
  BSQ_CHECK(known_dtype(code_dtype), BSQ_ERR_DTYPE, "unknown dtype");
  BSQ_CHECK(is_fp8(code_dtype), BSQ_ERR_UNSUPPORTED, "code_dtype must be E4M3 or E5M2");
  BSQ_CHECK(M % 128 == 0 && N % 128 == 0 && K % 128 == 0, BSQ_ERR_UNSUPPORTED,
            "M, N and K must be multiples of 128");
  BSQ_CHECK(M <= kMaxContraction && N <= kMaxContraction && K <= (int64_t(1) << 30),
            BSQ_ERR_UNSUPPORTED, "extent too large");
  BSQ_CHECK(gemm_tiles_fit(M, K) && gemm_tiles_fit(N, K), BSQ_ERR_UNSUPPORTED,
            "more than 2^31 - 1 output tiles");
  return BSQ_OK;
}

// Quantizes the bf16 sources into whichever operands have codes != NULL.
bsq_status bwd_quantize(int64_t M, int64_t N, int64_t K, const void* dY, const void* W, const void* X,
                        bool e5, uint8_t* dyn_c, uint8_t* dyn_s, uint8_t* wt_c, uint8_t* wt_s,
                        uint8_t* dyt_c, uint8_t* dyt_s, uint8_t* xt_c, uint8_t* xt_s, hipStream_t st) {
  // the transposed operands in one launch; dY in both orientations from
  // one read of dY when both are wanted
  MxT jobs[3];
  int n = 0;
  const bool dy_both = dyn_c != nullptr && dyt_c != nullptr;
  if (dyt_c != nullptr) jobs[n++] = MxT{dY, M, N, dyt_c, dyt_s, dy_both ? dyn_c : nullptr, dyn_s};
  if (wt_c != nullptr) jobs[n++] = MxT{W, N, K, wt_c, wt_s, nullptr, nullptr};
  if (xt_c != nullptr) jobs[n++] = MxT{X, M, K, xt_c, xt_s, nullptr, nullptr};
  bsq_status s = launch_mx_cols(jobs, n, true, e5, st);
  if (s != BSQ_OK) return s;
  if (dyn_c != nullptr && !dy_both && (s = launch_mx(M, N, 1, dY, true, dyn_c, e5, dyn_s, st)) != BSQ_OK)
    return s;
  return ok();
}

// dX = dyn . wt (contract N) if dX != NULL; dW = dyt . xt (contract M) if
// dW != NULL.  An empty contraction writes zeros.
bsq_status bwd_gemms(int64_t M, int64_t N, int64_t K, bool e5, bool out_bf16, const BwdOps& o, void* dX,
                     void* dW, hipStream_t st) {
  GemmLaunch L{};
  L.mode = MODE_MX;
  L.batch = 1;
  L.out_bf16 = out_bf16;
  L.fa_e5m2 = L.fb_e5m2 = e5;
  if (dX != nullptr && M > 0 && K > 0) {
    L.M = M; L.N = K; L.K = N;
    L.A = o.dyn_c; L.SA = o.dyn_s;
    L.B = o.wt_c; L.SB = o.wt_s;
    L.out = dX;
    const bsq_status s = launch_gemm(L, st);
    if (s != BSQ_OK) return s;
  }
  if (dW != nullptr && N > 0 && K > 0) {
    L.M = N; L.N = K; L.K = M;
    L.A = o.dyt_c; L.SA = o.dyt_s;
    L.B = o.xt_c; L.SB = o.xt_s;
    L.out = dW;
    const bsq_status s = launch_gemm(L, st);
    if (s != BSQ_OK) return s;
  }
  return ok();
}

BwdLayout bwd_layout(int64_t M, int64_t N, int64_t K) {
  BwdLayout L{};
  size_t o = 0;
  auto take = [&o](size_t bytes) {
    const size_t at = o;
    o += up256(bytes);
    return at;
  };
  L.dyn_codes = take(size_t(M * N));        // dY blocked along N: [M, N]
  L.dyn_scales = take(size_t(M * (N / 32)));
  L.wt_codes = take(size_t(K * N));         // W blocked along N, transposed: [K, N]
  L.wt_scales = take(size_t(K * (N / 32)));
  L.dyt_codes = take(size_t(N * M));        // dY blocked along M, transposed: [N, M]
  L.dyt_scales = take(size_t(N * (M / 32)));
  L.xt_codes = take(size_t(K * M));         // X blocked along M, transposed: [K, M]
  L.xt_scales = take(size_t(K * (M / 32)));
  L.total = o;
  return L;
}
}  // namespace

size_t bsq_mxfp8_backward_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return 0;
  // beyond the call's extents the byte count could overflow; no buffer is
  // large enough for such sizes
  if (M > kMaxContraction || N > kMaxContraction || K > (int64_t(1) << 30)) return SIZE_MAX;
  return bwd_layout(M, N, K).total;
}

bsq_status bsq_mxfp8_backward(int64_t M, int64_t N, int64_t K, const void* dY, const void* W,
                              const void* X, int code_dtype, int out_dtype, void* dX, void* dW,
                              void* workspace, size_t workspace_bytes, void* stream) {
  bsq_status s = bwd_check_dims(M, N, K, code_dtype);
  if (s != BSQ_OK) return s;
  BSQ_CHECK(known_dtype(out_dtype), BSQ_ERR_DTYPE, "unknown dtype");
  BSQ_CHECK(out_dtype == BSQ_BF16 || out_dtype == BSQ_F32, BSQ_ERR_UNSUPPORTED,
            "out_dtype must be BF16 or F32");
  const BwdLayout lay = bwd_layout(M, N, K);
  BSQ_CHECK(workspace_bytes >= lay.total, BSQ_ERR_SHAPE, "workspace too small");
  if (K == 0 || (M == 0 && N == 0)) return ok();  // both outputs are empty
  if (M > 0) BSQ_CHECK_PTR(dX);
  if (N > 0) BSQ_CHECK_PTR(dW);
  if (M > 0 && N > 0) {
    BSQ_CHECK_PTR(dY);
    BSQ_CHECK_PTR(W);
    BSQ_CHECK_PTR(X);
    BSQ_CHECK_PTR(workspace);
  }
  BSQ_DEVICE();
  hipStream_t st = as_stream(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const bool e5 = code_dtype == BSQ_E5M2;
  if (M > 0 && N > 0) {
    s = bwd_quantize(M, N, K, dY, W, X, e5, ws + lay.dyn_codes, ws + lay.dyn_scales, ws + lay.wt_codes,
                     ws + lay.wt_scales, ws + lay.dyt_codes, ws + lay.dyt_scales, ws + lay.xt_codes,
                     ws + lay.xt_scales, st);
    if (s != BSQ_OK) return s;
  }
  const BwdOps o{ws + lay.dyn_codes, ws + lay.dyn_scales, ws + lay.wt_codes, ws + lay.wt_scales,
                 ws + lay.dyt_codes, ws + lay.dyt_scales, ws + lay.xt_codes, ws + lay.xt_scales};
  return bwd_gemms(M, N, K, e5, out_dtype == BSQ_BF16, o, M > 0 ? dX : nullptr, N > 0 ? dW : nullptr, st);
}

bsq_status bsq_mxfp8_backward_quantize(int64_t M, int64_t N, int64_t K, const void* dY, const void* W,
                                       const void* X, int code_dtype, uint8_t* dyn_codes,
                                       uint8_t* dyn_scales, uint8_t* wt_codes, uint8_t* wt_scales,
                                       uint8_t* dyt_codes, uint8_t* dyt_scales, uint8_t* xt_codes,
                                       uint8_t* xt_scales, void* stream) {
  bsq_status s = bwd_check_dims(M, N, K, code_dtype);
  if (s != BSQ_OK) return s;
  // an operand is produced iff its codes pointer is given; it then needs its
  // scales and its source (unless it is empty)
  struct Req {
    uint8_t* c;
    uint8_t* sc;
    const void* src;
    int64_t r, cl;
    const char* what;
  };
  const Req req[4] = {{dyn_codes, dyn_scales, dY, M, N, "dY blocked along N"},
                      {wt_codes, wt_scales, W, N, K, "W blocked along N"},
                      {dyt_codes, dyt_scales, dY, M, N, "dY blocked along M"},
                      {xt_codes, xt_scales, X, M, K, "X blocked along M"}};
  bool live[4] = {false, false, false, false};
  for (int i = 0; i < 4; ++i) {
    const Req& q = req[i];
    if (q.c == nullptr) {
      BSQ_CHECK(q.sc == nullptr, BSQ_ERR_NULL, std::string(q.what) + ": scales given without codes");
      continue;
    }
    if (q.r == 0 || q.cl == 0) continue;
    BSQ_CHECK(q.sc != nullptr, BSQ_ERR_NULL, std::string(q.what) + ": scales are NULL");
    BSQ_CHECK(aligned16(q.c) && aligned16(q.sc), BSQ_ERR_ALIGN,
              std::string(q.what) + ": codes or scales not 16-byte aligned");
    BSQ_CHECK(q.src != nullptr, BSQ_ERR_NULL, std::string(q.what) + ": source is NULL");
    BSQ_CHECK(aligned16(q.src), BSQ_ERR_ALIGN, std::string(q.what) + ": source not 16-byte aligned");
    live[i] = true;
  }
  if (!(live[0] || live[1] || live[2] || live[3])) return ok();
  BSQ_DEVICE();
  return bwd_quantize(M, N, K, dY, W, X, code_dtype == BSQ_E5M2, live[0] ? dyn_codes : nullptr, dyn_scales,
                      live[1] ? wt_codes : nullptr, wt_scales, live[2] ? dyt_codes : nullptr, dyt_scales,
                      live[3] ? xt_codes : nullptr, xt_scales, as_stream(stream));
}

bsq_status bsq_mxfp8_backward_gemms(int64_t M, int64_t N, int64_t K, int code_dtype, int out_dtype,
                                    const uint8_t* dyn_codes, const uint8_t* dyn_scales,
                                    const uint8_t* wt_codes, const uint8_t* wt_scales,
                                    const uint8_t* dyt_codes, const uint8_t* dyt_scales,
                                    const uint8_t* xt_codes, const uint8_t* xt_scales, void* dX, void* dW,
                                    void* stream) {
  bsq_status s = bwd_check_dims(M, N, K, code_dtype);
  if (s != BSQ_OK) return s;
  BSQ_CHECK(known_dtype(out_dtype), BSQ_ERR_DTYPE, "unknown dtype");
  BSQ_CHECK(out_dtype == BSQ_BF16 || out_dtype == BSQ_F32, BSQ_ERR_UNSUPPORTED,
            "out_dtype must be BF16 or F32");
  const bool want_dx = dX != nullptr && M > 0 && K > 0;
  const bool want_dw = dW != nullptr && N > 0 && K > 0;
  if (want_dx) {
    BSQ_CHECK(aligned16(dX), BSQ_ERR_ALIGN, "dX is not 16-byte aligned");
    if (N > 0) {
      BSQ_CHECK_PTR(dyn_codes);
      BSQ_CHECK_PTR(dyn_scales);
      BSQ_CHECK_PTR(wt_codes);
      BSQ_CHECK_PTR(wt_scales);
    }
  }
  if (want_dw) {
    BSQ_CHECK(aligned16(dW), BSQ_ERR_ALIGN, "dW is not 16-byte aligned");
    if (M > 0) {
      BSQ_CHECK_PTR(dyt_codes);
      BSQ_CHECK_PTR(dyt_scales);
      BSQ_CHECK_PTR(xt_codes);
      BSQ_CHECK_PTR(xt_scales);
    }
  }
  if (!want_dx && !want_dw) return ok();
  BSQ_DEVICE();
  const BwdOps o{dyn_codes, dyn_scales, wt_codes, wt_scales, dyt_codes, dyt_scales, xt_codes, xt_scales};
  return bwd_gemms(M, N, K, code_dtype == BSQ_E5M2, out_dtype == BSQ_BF16, o, want_dx ? dX : nullptr,
                   want_dw ? dW : nullptr, as_stream(stream));
}

// ------------------------------------------------------------- nvfp4 --

// Largest operand of the nvfp4 product, in values (B * M * K and B * N * K):
// its bfloat16 copy then takes at most 2 TiB, far beyond device memory,
// and every size derived from it fits 64 bits.
constexpr int64_t kMaxNvfp4Values = int64_t(1) << 40;
static inline bool nvfp4_operand_fits(int64_t B, int64_t R, int64_t K) {
  int64_t n = 0;
  return !__builtin_mul_overflow(B, R, &n) && !__builtin_mul_overflow(n, K, &n) && n <= kMaxNvfp4Values;
}

size_t bsq_nvfp4_workspace_bytes(int64_t B, int64_t M, int64_t N, int64_t K) {
  if (B < 0 || M < 0 || N < 0 || K < 0) return 0;
  if (!nvfp4_operand_fits(B, M, K) || !nvfp4_operand_fits(B, N, K)) return SIZE_MAX;
  return up256(size_t(B * M * K * 2)) + up256(size_t(B * N * K * 2));
}

bsq_status bsq_scaled_matmul_nvfp4(int64_t B, int64_t M, int64_t N, int64_t K, const uint8_t* lhs,
                                   const uint8_t* rhs, const uint8_t* lhs_scales,
                                   const uint8_t* rhs_scales, void* out, int out_dtype, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  BSQ_CHECK(B >= 0 && M >= 0 && N >= 0 && K >= 0, BSQ_ERR_SHAPE, "negative size");
  BSQ_CHECK(K % 16 == 0, BSQ_ERR_SHAPE, "K must be a multiple of the block (16)");
  BSQ_CHECK(known_dtype(out_dtype), BSQ_ERR_DTYPE, "unknown out_dtype");
  BSQ_CHECK(out_dtype == BSQ_F32 || out_dtype == BSQ_BF16, BSQ_ERR_UNSUPPORTED,
            "out_dtype must be F32 or BF16");
  BSQ_CHECK(K % 128 == 0 && N % 16 == 0, BSQ_ERR_UNSUPPORTED,
            "the library needs K % 128 == 0 and N % 16 == 0");
  BSQ_CHECK(M <= (int64_t(1) << 30) && N <= (int64_t(1) << 30) && K <= kMaxContraction / 2,
            BSQ_ERR_UNSUPPORTED, "extent too large");
  BSQ_CHECK(B <= kMaxBatch, BSQ_ERR_UNSUPPORTED, "batch over 65535");
  BSQ_CHECK(gemm_tiles_fit(M, N), BSQ_ERR_UNSUPPORTED, "more than 2^31 - 1 output tiles");
  BSQ_CHECK(nvfp4_operand_fits(B, M, K) && nvfp4_operand_fits(B, N, K), BSQ_ERR_UNSUPPORTED,
            "an operand of more than 2^40 values");
  BSQ_CHECK(elems_fit(B, M, N), BSQ_ERR_UNSUPPORTED, "an output of more than 2^60 elements");
  const size_t need = bsq_nvfp4_workspace_bytes(B, M, N, K);
  BSQ_CHECK(workspace_bytes >= need, BSQ_ERR_SHAPE, "workspace too small");
  if (B == 0 || M == 0 || N == 0) return ok();
  BSQ_CHECK_PTR(out);
  if (K > 0) {
    BSQ_CHECK_PTR(lhs);
    BSQ_CHECK_PTR(rhs);
    BSQ_CHECK(lhs_scales != nullptr && rhs_scales != nullptr, BSQ_ERR_NULL, "scales are NULL");
    BSQ_CHECK_PTR(workspace);
  }
  BSQ_DEVICE();
  hipStream_t st = as_stream(stream);
  uint16_t* wa = static_cast<uint16_t*>(workspace);
  uint16_t* wb = reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(workspace) + up256(size_t(B * M * K * 2)));
  bsq_status s = BSQ_OK;
  if (K > 0) {
    if ((s = launch_nvfp4_to_bf16(B * M, K, lhs, lhs_scales, wa, st)) != BSQ_OK) return s;
    if ((s = launch_nvfp4_to_bf16(B * N, K, rhs, rhs_scales, wb, st)) != BSQ_OK) return s;
  }
  GemmLaunch L{};
  L.mode = MODE_BF16;
  L.batch = B;
  L.M = M; L.N = N; L.K = K;
  L.A = wa; L.B = wb;
  L.out = out;
  L.out_bf16 = out_dtype == BSQ_BF16;
  return launch_gemm(L, st);
}

}  // extern "C"
