// Quantizer kernels: float values -> fp8 / int8 codes plus scales.
//
// All of them are bound by HBM: one streaming read of the input, one write
// of the codes.  The pages divide each value by the block scale; the code is
// that of the correctly rounded float32 quotient x / s, obtained without a
// division per element: with r = 1 / s correctly rounded, q0 = x * r is
// within an ulp of x / s, the residual x - q0 * s is exact in one FMA, and
// q0 + (x - q0 * s) * r rounds to the correctly rounded quotient whenever
// nothing underflows (Markstein's theorem on division by a correctly
// rounded reciprocal).  Where the residual underflows (|x| below about
// 2^-102) the quotient is below 2^-60 and still encodes to a zero of x's
// sign (see quot).  The per-block scale amax / 448 and its reciprocal are
// formed the same way without a division instruction sequence (see
// fp8_block_scale and recip).  float32 -> fp8 uses the gfx950 conversion
// instructions (nearest, ties to even; inputs already clamped to the
// format's range).  Block maxima are taken on the bits of |x| (for finite
// values their unsigned order is the order of |x|) and exchanged between
// lanes with DPP and permlane operations, which stay in the VALU.
#include "common.h"
#include "quant.h"

namespace bsq {

namespace {

constexpr float kE4M3Max = 448.0f;
constexpr float kE5M2Max = 57344.0f;

// |x| as bits: for finite x the unsigned order of these is the order of |x|.
__device__ __forceinline__ uint32_t abs_bits(float x) { return __float_as_uint(x) & 0x7FFFFFFFu; }
__device__ __forceinline__ uint32_t amax4_bits(float4 v) {
  return max(max(abs_bits(v.x), abs_bits(v.y)), max(abs_bits(v.z), abs_bits(v.w)));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}

// Maximum over aligned groups of WIDTH lanes (2 .. 64), left in every lane of
// the group.  Quad permutations give the maximum of each 4 lanes; mirroring
// each half row (lane i <-> 7 - i) then each row (i <-> 15 - i) pairs every
// 4- then 8-lane group with its neighbour; v_permlane16_swap exchanges rows
// 0 <-> 1 and 2 <-> 3, v_permlane32_swap the two halves of the wave.
template <int WIDTH>
__device__ __forceinline__ uint32_t group_max_bits(uint32_t v) {
  static_assert(WIDTH >= 2 && WIDTH <= 64 && (WIDTH & (WIDTH - 1)) == 0, "group width");
  v = max(v, dpp_mov<0xB1>(v));  // quad_perm [1, 0, 3, 2]
  if constexpr (WIDTH >= 4) v = max(v, dpp_mov<0x4E>(v));   // quad_perm [2, 3, 0, 1]
  if constexpr (WIDTH >= 8) v = max(v, dpp_mov<0x141>(v));  // row_half_mirror
  if constexpr (WIDTH >= 16) v = max(v, dpp_mov<0x140>(v));  // row_mirror
  if constexpr (WIDTH >= 32) {
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = max(uint32_t(p[0]), uint32_t(p[1]));
  }
  if constexpr (WIDTH >= 64) {
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = max(uint32_t(p[0]), uint32_t(p[1]));
  }
  return v;
}

// fp32 block scale of the block_scaled_mm recipe: max(amax / 448, 1e-10),
// the quotient correctly rounded.  Markstein's form with the correctly
// rounded constant 1/448: q0 = amax * (1/448) is within an ulp, the residual
// amax - 448 q0 is exact in one FMA, and the corrected quotient is the
// correctly rounded amax / 448 (no underflow matters: below 448e-10 the
// floor is taken).  Checked bit for bit against IEEE division on every
// float32 amax from 2^-40 to the largest float.
__device__ __forceinline__ float fp8_block_scale(float amax) {
  constexpr float kInv = 1.0f / kE4M3Max;
  const float q0 = amax * kInv;
  const float q = __builtin_fmaf(__builtin_fmaf(-q0, kE4M3Max, amax), kInv, q0);
  return fmaxf(q, scale_floor());
}

// 1 / s correctly rounded for the scales above (normal, 1e-10 <= s < 2^120):
// the hardware reciprocal (within an ulp) and one Newton step whose
// residual 1 - s y0 is exact in the FMA.  Checked bit for bit against IEEE
// division on every float32 s in that range.
__device__ __forceinline__ float recip(float s) {
  const float y0 = __builtin_amdgcn_rcpf(s);
  return __builtin_fmaf(__builtin_fmaf(-s, y0, 1.0f), y0, y0);
}

// Four float32 in [-fmax, fmax] to four fp8 codes (first value in the low
// byte), nearest with ties to even.
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true));
}
__device__ __forceinline__ uint32_t cvt4_e5m2(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
  return uint32_t(__builtin_amdgcn_cvt_pk_bf8_f32(c, d, lo, true));
}

// x / s correctly rounded (r = 1 / s correctly rounded, s > 0 normal).  The
// residual is formed as t = q0 s - x and subtracted, q0 - t r: the same
// value as q0 + (x - q0 s) r, but a zero quotient keeps x's sign without a
// separate copysign (x = -0: q0 = -0, t = +0, -0 - 0 = -0; the other order
// gives +0).  Checked bit for bit against that order with copysign on every
// finite x with |x| <= 1000 s, for nine scales from 1e-10 to 1e30.
__device__ __forceinline__ float quot(float x, float s, float r) {
  const float q0 = x * r;
  return __builtin_fmaf(-__builtin_fmaf(q0, s, -x), r, q0);
}

__device__ __forceinline__ uint32_t quant4_e4m3(float4 v, float s, float r) {
  auto q = [s, r](float x) { return __builtin_amdgcn_fmed3f(quot(x, s, r), -kE4M3Max, kE4M3Max); };
  return cvt4_e4m3(q(v.x), q(v.y), q(v.z), q(v.w));
}

// ------------------------------------------------ fp8 1 x G row blocks ----
// One float4 per lane, G/4 lanes per block; a workgroup handles U chunks of
// 256 float4 per grid-stride step, all loads issued before any use.
template <int G, int U>
__global__ void __launch_bounds__(256) k_fp8_rowblock(const float4* __restrict__ src,
                                                      uint32_t* __restrict__ codes,
                                                      float* __restrict__ scales, int64_t n4) {
  constexpr int LPB = G / 4;
  const int64_t chunk = int64_t(256) * U;
  for (int64_t base = int64_t(blockIdx.x) * chunk; base < n4; base += int64_t(gridDim.x) * chunk) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t f = base + u * 256 + threadIdx.x;
      v[u] = f < n4 ? ldnt(src + f) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t f = base + u * 256 + threadIdx.x;
      const float amax = __uint_as_float(group_max_bits<LPB>(amax4_bits(v[u])));
      const float s = fp8_block_scale(amax);
      const float r = recip(s);
      if (f < n4) {
        codes[f] = quant4_e4m3(v[u], s, r);
        if ((threadIdx.x % LPB) == 0) scales[f / LPB] = s;
      }
    }
  }
}

// ------------------------------------------------ fp8 128 x 128 tiles ----
// One workgroup per tile along a one-dimensional grid; each thread holds 64
// values (16 float4) of the tile in registers between the reduction and the
// encode.  Workgroups are dealt to the 8 XCDs round-robin by linear id, and
// linear id L takes tile (L % 8) * (T / 8) + L / 8 of the row-major order,
// so each XCD works through a contiguous run of tiles (tiles past 8 (T / 8)
// keep their own index).  Measured at 4096^2 with cold inputs: 15.5 us
// against 15.6 us for the plain row-major order, same bytes.
__global__ void __launch_bounds__(256) k_fp8_tile128(const float* __restrict__ src,
                                                     uint8_t* __restrict__ codes,
                                                     float* __restrict__ scales, int64_t cols) {
  __shared__ uint32_t wmax[4];
  const int tx = threadIdx.x;
  const int c4 = tx & 31;
  const int r0 = tx >> 5;
  const int64_t tiles_c = cols / 128;
  const int64_t T = gridDim.x, per = T / 8, L = blockIdx.x;
  const int64_t t = L < 8 * per ? (L % 8) * per + L / 8 : L;
  const int64_t row0 = (t / tiles_c) * 128;
  const int64_t col0 = (t % tiles_c) * 128 + 4 * c4;
  float4 v[16];
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4* p = reinterpret_cast<const float4*>(src + (row0 + r0 + 8 * i) * cols + col0);
    v[i] = ldnt(p);
    m = max(m, amax4_bits(v[i]));
  }
  m = group_max_bits<64>(m);
  if ((tx & 63) == 0) wmax[tx >> 6] = m;
  __syncthreads();
  const float amax = __uint_as_float(max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3])));
  const float s = fp8_block_scale(amax);
  const float r = recip(s);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    uint32_t* q = reinterpret_cast<uint32_t*>(codes + (row0 + r0 + 8 * i) * cols + col0);
    *q = quant4_e4m3(v[i], s, r);
  }
  if (tx == 0) scales[t] = s;
}

// ------------------------------------------------------------ MX (e8m0) --
// Exponent of the block scale: the smallest E with max(amax, 1e-10) <=
// fmax * 2^E, read off the float32 fields.  fmax = 1.75 * 2^EMAX for both
// formats (448 = 1.75 * 2^8, 57344 = 1.75 * 2^15).
template <int EMAX>
__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t u = __float_as_uint(fmaxf(amax, scale_floor()));
  const int e = int((u >> 23) & 0xFFu) - 127;
  const int E = e - EMAX + ((u & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return min(max(E, -127), 127);
}

// x * 2^-E (exact) clamped to the format's range, four at a time.
template <int CODE>  // 0 = e4m3, 1 = e5m2
__device__ __forceinline__ uint32_t mx_encode4(const float* x, int E) {
  constexpr float fmax = CODE == 0 ? kE4M3Max : kE5M2Max;
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = __builtin_amdgcn_fmed3f(ldexpf(x[i], -E), -fmax, fmax);
  return CODE == 0 ? cvt4_e4m3(y[0], y[1], y[2], y[3]) : cvt4_e5m2(y[0], y[1], y[2], y[3]);
}

// Loads 8 consecutive source values as float (from f32 or bf16).
template <int SRC_BF16>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&x)[8]) {
  if (SRC_BF16) {
    const uint4 w = ldnt(
        reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem));
    const uint32_t p[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = decode_bf16(p[i] & 0xFFFFu);
      x[2 * i + 1] = decode_bf16(p[i] >> 16);
    }
  } else {
    const float4* f = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
    const float4 a = ldnt(f);
    const float4 b = ldnt(f + 1);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Blocks of 32 along rows (axis = 1): 4 lanes per block, 8 values each.
template <int SRC_BF16, int CODE, int U>
__global__ void __launch_bounds__(256) k_mx_rows(const void* __restrict__ src,
                                                 uint2* __restrict__ codes,
                                                 uint8_t* __restrict__ scales, int64_t n8) {
  constexpr int EMAX = CODE == 0 ? 8 : 15;
  const int64_t chunk = int64_t(256) * U;
  for (int64_t base = int64_t(blockIdx.x) * chunk; base < n8; base += int64_t(gridDim.x) * chunk) {
    float x[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t f = base + u * 256 + threadIdx.x;
      if (f < n8) {
        load8<SRC_BF16>(src, f * 8, x[u]);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[u][i] = 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t f = base + u * 256 + threadIdx.x;
      uint32_t m = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = max(m, abs_bits(x[u][i]));
      const int E = mx_exponent<EMAX>(__uint_as_float(group_max_bits<4>(m)));
      if (f < n8) {
        codes[f] = make_uint2(mx_encode4<CODE>(&x[u][0], E), mx_encode4<CODE>(&x[u][4], E));
        if ((threadIdx.x & 3) == 0) scales[f >> 2] = uint8_t(E + 127);
      }
    }
  }
}

// Blocks of 32 down columns (axis = 0), output transposed.  A workgroup
// takes a 64 x 64 tile through LDS; thread t writes 16 codes of output row
// (input column) t / 4, two threads per 32-block.  A launch covers up to
// kMxJobs matrices (the backward's three transposed operands in one grid):
// workgroup b belongs to the job whose range of tiles holds it.  A job with
// row_codes set also quantizes along rows (axis = 1, blocks of 32 along a
// row: four consecutive lanes of 8 values each) in the same pass, exactly
// as k_mx_rows does, so that a matrix needed in both orientations is read
// once.
constexpr int kMxJobs = 3;
struct MxJob {
  const void* src;
  uint8_t* codes;      // [cols, rows]
  uint8_t* scales;     // [cols, rows / 32]
  uint2* row_codes;    // [rows, cols] or null
  uint8_t* row_scales; // [rows, cols / 32]
  int64_t rows, cols;
  int tiles_x;         // 64-column tiles
  int first;           // first workgroup of the job
};
struct MxJobs {
  MxJob j[kMxJobs];
  int n;
  // 1: a lone job that writes only the transposed output takes its tiles
  // column by column, each XCD a contiguous run of them (workgroups are
  // dealt to the 8 XCDs round-robin by linear id), so that the two tiles
  // writing the halves of one output line run side by side on one XCD;
  // 0: tiles row by row in launch order
  int order;
};

template <int SRC_BF16, int CODE>
__global__ void __launch_bounds__(256) k_mx_cols_t(MxJobs jobs) {
  constexpr int EMAX = CODE == 0 ? 8 : 15;
  __shared__ float tile[64][65];
  int b = blockIdx.x;
  if (jobs.order == 1) {
    const int T = gridDim.x, per = T / 8;
    b = b < 8 * per ? (b % 8) * per + b / 8 : b;
  }
  int ji = 0;
#pragma unroll
  for (int q = 1; q < kMxJobs; ++q)
    if (q < jobs.n && b >= jobs.j[q].first) ji = q;
  const MxJob& J = jobs.j[ji];
  const int t = b - J.first;
  const int64_t rows = J.rows, cols = J.cols;
  const int tx = threadIdx.x;
  int64_t r0, c0;
  if (jobs.order == 1) {
    const int tiles_y = int((rows + 63) / 64);
    r0 = int64_t(t % tiles_y) * 64;
    c0 = int64_t(t / tiles_y) * 64;
  } else {
    r0 = int64_t(t / J.tiles_x) * 64;
    c0 = int64_t(t % J.tiles_x) * 64;
  }
  const bool both = J.row_codes != nullptr;
  // load: 64 rows x 64 cols, 8 values per thread-step, 2 steps
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int idx = tx + 256 * s;  // 0..511: row idx / 8, col group idx % 8
    const int r = idx >> 3, cg = (idx & 7) * 8;
    const bool in = r0 + r < rows && c0 + cg < cols;
    float x[8];
    if (in) {
      load8<SRC_BF16>(J.src, (r0 + r) * cols + c0 + cg, x);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.f;
    }
    if (both) {
      // lanes 4 q .. 4 q + 3 hold one row's 32-block (idx % 8 = lane % 8)
      uint32_t m = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) m = max(m, abs_bits(x[i]));
      const int E = mx_exponent<EMAX>(__uint_as_float(group_max_bits<4>(m)));
      if (in) {
        const int64_t f = ((r0 + r) * cols + c0 + cg) / 8;
        J.row_codes[f] = make_uint2(mx_encode4<CODE>(&x[0], E), mx_encode4<CODE>(&x[4], E));
        if ((tx & 3) == 0) J.row_scales[f >> 2] = uint8_t(E + 127);
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) tile[r][cg + i] = x[i];
  }
  __syncthreads();
  const int oc = tx >> 2, seg = tx & 3;
  float x[16];
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    x[i] = tile[16 * seg + i][oc];
    m = max(m, abs_bits(x[i]));
  }
  const int E = mx_exponent<EMAX>(__uint_as_float(group_max_bits<2>(m)));
  const int64_t orow = c0 + oc;
  const int64_t ocol = r0 + 16 * seg;
  if (orow < cols && ocol < rows) {
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = mx_encode4<CODE>(&x[4 * q], E);
    *reinterpret_cast<uint4*>(J.codes + orow * rows + ocol) = make_uint4(w[0], w[1], w[2], w[3]);
    if ((seg & 1) == 0) J.scales[orow * (rows / 32) + (ocol >> 5)] = uint8_t(E + 127);
  }
}

// ------------------------------------------------------ int8 per-channel --

__device__ __forceinline__ float int8_scale(float amax) {
  return amax == 0.f ? 1.0f : amax / 127.0f;
}

// round(x / s) with ties to even, clamped to +-127 (r = 1 / s).  The
// Markstein quotient q1 is correctly rounded except where |x * r| < 2^-11
// (possible underflow); there |q1| < 2^-10 all the same and rounds to the
// integer 0, so no special case is needed for integer codes.
__device__ __forceinline__ int32_t int8_code(float x, float s, float r) {
  const float q0 = x * r;
  const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, s, x), r, q0);
  return int32_t(fminf(fmaxf(__builtin_rintf(q1), -127.f), 127.f));
}

__device__ __forceinline__ uint32_t int8_pack4(float4 v, float s, float r) {
  return (uint32_t(int8_code(v.x, s, r)) & 0xFFu) | ((uint32_t(int8_code(v.y, s, r)) & 0xFFu) << 8) |
         ((uint32_t(int8_code(v.z, s, r)) & 0xFFu) << 16) | ((uint32_t(int8_code(v.w, s, r)) & 0xFFu) << 24);
}

// Maximum of |x| bits over the workgroup's N waves, as a float.
template <int N>
__device__ __forceinline__ float block_max(uint32_t m, uint32_t* red) {
  m = group_max_bits<64>(m);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = m;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < N; ++i) r = max(r, red[i]);
  return __uint_as_float(r);
}

// One workgroup per row, D % 4 == 0, the row held in registers (V float4
// per thread).
template <int V>
__global__ void __launch_bounds__(256) k_int8_rows_vec(const float* __restrict__ x,
                                                       uint32_t* __restrict__ xq,
                                                       float* __restrict__ xs, int64_t D) {
  __shared__ uint32_t red[4];
  const int64_t d4 = D / 4;
  const float4* row = reinterpret_cast<const float4*>(x + int64_t(blockIdx.x) * D);
  float4 v[V];
  uint32_t m = 0u;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int64_t c = threadIdx.x + 256 * i;
    v[i] = c < d4 ? ldnt(row + c) : make_float4(0.f, 0.f, 0.f, 0.f);
    m = max(m, amax4_bits(v[i]));
  }
  const float s = int8_scale(block_max<4>(m, red));
  const float r = 1.0f / s;
  uint32_t* out = xq + int64_t(blockIdx.x) * d4;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int64_t c = threadIdx.x + 256 * i;
    if (c < d4) out[c] = int8_pack4(v[i], s, r);
  }
  if (threadIdx.x == 0) xs[blockIdx.x] = s;
}

// Any D: two passes over the row (the second from cache).
__global__ void __launch_bounds__(256) k_int8_rows_any(const float* __restrict__ x,
                                                       int8_t* __restrict__ xq,
                                                       float* __restrict__ xs, int64_t D) {
  __shared__ uint32_t red[4];
  const float* row = x + int64_t(blockIdx.x) * D;
  uint32_t m = 0u;
  for (int64_t c = threadIdx.x; c < D; c += 256) m = max(m, abs_bits(row[c]));
  const float s = int8_scale(block_max<4>(m, red));
  const float r = 1.0f / s;
  int8_t* out = xq + int64_t(blockIdx.x) * D;
  for (int64_t c = threadIdx.x; c < D; c += 256) out[c] = int8_t(int8_code(row[c], s, r));
  if (threadIdx.x == 0) xs[blockIdx.x] = s;
}

// Column maxima of w[D_in, D_out] by atomic max on the float bits (all
// values are >= 0, so the unsigned order is the float order).  A workgroup
// covers up to 256 columns and `rows_per_wg` rows.
__global__ void __launch_bounds__(256) k_int8_colmax(const float* __restrict__ w,
                                                     uint32_t* __restrict__ cmax, int64_t D_in,
                                                     int64_t D_out, int rows_per_wg) {
  const int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t r_begin = int64_t(blockIdx.y) * rows_per_wg;
  const int64_t r_end = min(r_begin + rows_per_wg, D_in);
  // 256 threads walk 256 consecutive columns one row at a time
  float m = 0.f;
  if (c < D_out) {
    for (int64_t r = r_begin; r < r_end; ++r) m = fmaxf(m, fabsf(w[r * D_out + c]));
    atomicMax(cmax + c, __float_as_uint(m));
  }
}

// Vector variant: D_out % 4 == 0; 64 float4 columns x 4 row phases.
__global__ void __launch_bounds__(256) k_int8_colmax_vec(const float4* __restrict__ w,
                                                         uint32_t* __restrict__ cmax,
                                                         int64_t D_in, int64_t d4,
                                                         int rows_per_wg) {
  __shared__ float4 part[4][64];
  const int tx = threadIdx.x;
  const int cx = tx & 63, ph = tx >> 6;
  const int64_t c = int64_t(blockIdx.x) * 64 + cx;
  const int64_t r_begin = int64_t(blockIdx.y) * rows_per_wg;
  const int64_t r_end = min(r_begin + rows_per_wg, D_in);
  float4 m = make_float4(0.f, 0.f, 0.f, 0.f);
  if (c < d4) {
    // rows r_begin + ph + 4 n; 16 loads in flight per thread when the
    // workgroup's 64 rows are all there
    int64_t r = r_begin + ph;
    if (rows_per_wg == 64 && r_begin + 64 <= r_end) {
      float4 a[16];
#pragma unroll
      for (int n = 0; n < 16; ++n) a[n] = ldnt(w + (r + 4 * n) * d4 + c);
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        m.x = fmaxf(m.x, fabsf(a[n].x));
        m.y = fmaxf(m.y, fabsf(a[n].y));
        m.z = fmaxf(m.z, fabsf(a[n].z));
        m.w = fmaxf(m.w, fabsf(a[n].w));
      }
    } else {
      for (; r < r_end; r += 4) {
        const float4 a = ldnt(w + r * d4 + c);
        m.x = fmaxf(m.x, fabsf(a.x));
        m.y = fmaxf(m.y, fabsf(a.y));
        m.z = fmaxf(m.z, fabsf(a.z));
        m.w = fmaxf(m.w, fabsf(a.w));
      }
    }
  }
  part[ph][cx] = m;
  __syncthreads();
  if (ph == 0 && c < d4) {
#pragma unroll
    for (int p = 1; p < 4; ++p) {
      const float4 o = part[p][cx];
      m.x = fmaxf(m.x, o.x);
      m.y = fmaxf(m.y, o.y);
      m.z = fmaxf(m.z, o.z);
      m.w = fmaxf(m.w, o.w);
    }
    uint32_t* dst = cmax + 4 * c;
    atomicMax(dst + 0, __float_as_uint(m.x));
    atomicMax(dst + 1, __float_as_uint(m.y));
    atomicMax(dst + 2, __float_as_uint(m.z));
    atomicMax(dst + 3, __float_as_uint(m.w));
  }
}

__global__ void __launch_bounds__(256) k_fill_u32(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    p[i] = v;
}

// Codes of w with the column scales derived from the column maxima; also
// the transposed codes w_qT[D_out, D_in] when requested.  Tiles of 128 x
// 128 (D_in x D_out); any sizes (edges guarded).  Thread (cx, rg) owns
// columns 4 cx .. 4 cx + 3 and the four runs of 4 consecutive rows
// 4 (rg + 8 kk) .. + 3, kk = 0..3; all 16 row loads are issued first.  For
// the transpose, a column's 4 codes of one run form one word in LDS
// (tq[column][row / 4]), read back 16 bytes at a time.
__global__ void __launch_bounds__(256) k_int8_cols_quant(const float* __restrict__ w,
                                                         const uint32_t* __restrict__ cmax,
                                                         int8_t* __restrict__ wq,
                                                         int8_t* __restrict__ wqT, int64_t D_in,
                                                         int64_t D_out) {
  __shared__ __attribute__((aligned(16))) uint32_t tq[128][36];  // 144-byte rows
  const int tx = threadIdx.x;
  const int64_t i0 = int64_t(blockIdx.y) * 128;  // rows of w (D_in)
  const int64_t j0 = int64_t(blockIdx.x) * 128;  // cols of w (D_out)
  const int cx = tx & 31;
  const int rg = tx >> 5;
  const int64_t j = j0 + 4 * cx;
  const bool vec = (D_out % 4) == 0 && j < D_out;
  float s[4], rs[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s[q] = j + q < D_out ? int8_scale(__uint_as_float(cmax[j + q])) : 1.0f;
    rs[q] = 1.0f / s[q];
  }
  float4 v[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    const int64_t i = i0 + 4 * (rg + 8 * (n >> 2)) + (n & 3);
    v[n] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < D_in) {
      if (vec) {
        v[n] = ldnt(reinterpret_cast<const float4*>(w + i * D_out + j));
      } else {
        float e[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (j + q < D_out) e[q] = w[i * D_out + j + q];
        v[n] = make_float4(e[0], e[1], e[2], e[3]);
      }
    }
  }
  uint32_t packed[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    const int64_t i = i0 + 4 * (rg + 8 * (n >> 2)) + (n & 3);
    const float vv[4] = {v[n].x, v[n].y, v[n].z, v[n].w};
    packed[n] = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) packed[n] |= (uint32_t(int8_code(vv[q], s[q], rs[q])) & 0xFFu) << (8 * q);
    if (i < D_in) {
      if (vec) {
        *reinterpret_cast<uint32_t*>(wq + i * D_out + j) = packed[n];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (j + q < D_out) wq[i * D_out + j + q] = int8_t(packed[n] >> (8 * q));
      }
    }
  }
  if (wqT == nullptr) return;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) word |= ((packed[4 * kk + t] >> (8 * q)) & 0xFFu) << (8 * t);
      tq[4 * cx + q][rg + 8 * kk] = word;
    }
  __syncthreads();
  // 128 output rows (j) x 128 bytes (i): thread writes 64 bytes of one row
  const int oj = tx >> 1, half = tx & 1;
  const int64_t jo = j0 + oj;
  if (jo >= D_out) return;
  const int64_t ib = i0 + 64 * half;
  int8_t* dst = wqT + jo * D_in + ib;
  if ((D_in % 16) == 0 && ib + 64 <= D_in) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<uint4*>(dst + 16 * q) = *reinterpret_cast<const uint4*>(&tq[oj][16 * half + 4 * q]);
  } else {
    const uint8_t* row = reinterpret_cast<const uint8_t*>(&tq[oj][0]);
    for (int q = 0; q < 64 && ib + q < D_in; ++q) dst[q] = int8_t(row[64 * half + q]);
  }
}

__global__ void __launch_bounds__(256) k_int8_col_scales(const uint32_t* __restrict__ cmax,
                                                         float* __restrict__ ws, int64_t n) {
  const int64_t j = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (j < n) ws[j] = int8_scale(__uint_as_float(cmax[j]));
}

// One pass over w when a whole column stripe fits in a workgroup's
// registers (D_out % 16 == 0, D_in <= 4096): workgroup = one 16-column
// stripe, all rows.  Thread t owns float4 column q4 = t & 3 of the stripe
// and rows 512 p + 4 g + k (g = t >> 2, k < 4, p < 8): 32 float4 in
// registers from one read of w.  The column maxima are reduced in the
// workgroup (shuffles over the 16 lanes of a wave that share q4, then LDS
// across the 8 waves), so no second read and no atomics.  A thread's 4
// consecutive rows of one column pack into one word of the transposed copy.
// Workgroups are dealt to the 8 XCDs by linear id, L % 8; XCD x takes a
// contiguous run of S stripes, consecutive stripes on workgroups L, L + 8,
// ...  So the two 64-byte halves of each 128-byte line of w are read
// through one L2 at about the same time, the eight 16-byte pieces of each
// 128-byte line of w_q meet in that L2 before they are written back, and
// each XCD's share of a row is a contiguous 2 KiB (at D_out = 4096), which
// spans all of its L2 channels (a 512-byte share did not).
constexpr int kOnePassMaxRows = 4096;
// the two-pass path's grids hold D_in / 64 row blocks along y (at most 65536)
constexpr int64_t kTwoPassMaxRows = int64_t(64) * 65536;
__global__ void __launch_bounds__(512) k_int8_cols_onepass(const float* __restrict__ w,
                                                           int8_t* __restrict__ wq,
                                                           float* __restrict__ ws,
                                                           int8_t* __restrict__ wqT, int64_t D_in,
                                                           int64_t D_out) {
  __shared__ float4 red[8][4];
  const int tx = threadIdx.x;
  // workgroup L runs on XCD L % 8; XCD x takes stripes [S x, S x + S)
  const int L = blockIdx.x;
  const int64_t S = gridDim.x / 8;
  const int64_t stripe = S * (L % 8) + L / 8;
  if (16 * stripe >= D_out) return;
  const int q4 = tx & 3, g = tx >> 2;
  const int64_t j = 16 * stripe + 4 * q4;
  const int rows = int(D_in);  // <= 4096
  // rows past D_in re-read the last row and are zeroed afterwards, so no
  // branch separates the loads; they go out in batches of 8 with at most
  // 16 in flight per thread, which keeps the paired half-lines of one XCD
  // inside its L2 until both halves are read
  float4 v[32];
#pragma unroll
  for (int bt = 0; bt < 4; ++bt) {
#pragma unroll
    for (int n = 8 * bt; n < 8 * bt + 8; ++n) {
      const int i = 512 * (n >> 2) + 4 * g + (n & 3);
      v[n] = *reinterpret_cast<const float4*>(w + int64_t(min(i, rows - 1)) * D_out + j);
    }
    if (bt > 0) __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8): batch bt - 1 has landed
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int n = 0; n < 32; ++n) {
    const int i = 512 * (n >> 2) + 4 * g + (n & 3);
    if (i >= rows) v[n] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float4 m = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int n = 0; n < 32; ++n) {
    m.x = fmaxf(m.x, fabsf(v[n].x));
    m.y = fmaxf(m.y, fabsf(v[n].y));
    m.z = fmaxf(m.z, fabsf(v[n].z));
    m.w = fmaxf(m.w, fabsf(v[n].w));
  }
#pragma unroll
  for (int off = 4; off < 64; off <<= 1) {
    m.x = fmaxf(m.x, __shfl_xor(m.x, off));
    m.y = fmaxf(m.y, __shfl_xor(m.y, off));
    m.z = fmaxf(m.z, __shfl_xor(m.z, off));
    m.w = fmaxf(m.w, __shfl_xor(m.w, off));
  }
  if ((tx & 63) < 4) red[tx >> 6][q4] = m;
  __syncthreads();
  m = red[0][q4];
#pragma unroll
  for (int wv = 1; wv < 8; ++wv) {
    const float4 o = red[wv][q4];
    m.x = fmaxf(m.x, o.x);
    m.y = fmaxf(m.y, o.y);
    m.z = fmaxf(m.z, o.z);
    m.w = fmaxf(m.w, o.w);
  }
  const float s[4] = {int8_scale(m.x), int8_scale(m.y), int8_scale(m.z), int8_scale(m.w)};
  const float r[4] = {1.0f / s[0], 1.0f / s[1], 1.0f / s[2], 1.0f / s[3]};
  if (g == 0) *reinterpret_cast<float4*>(ws + j) = make_float4(s[0], s[1], s[2], s[3]);
  int8_t* const wq_t = wq + int64_t(4 * g) * D_out + j;  // row 4 g of this thread's columns
  int8_t* const wqT_t = wqT != nullptr ? wqT + j * D_in + 4 * g : nullptr;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    if (512 * p >= rows) break;
    const bool in = 512 * p + 4 * g < rows;  // D_in % 4 == 0: the 4 rows go together
    uint32_t col[4] = {0u, 0u, 0u, 0u};     // column q's codes of this thread's 4 rows
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float4 x = v[4 * p + k];
      const float e[4] = {x.x, x.y, x.z, x.w};
      uint32_t row = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t c = uint32_t(int8_code(e[q], s[q], r[q])) & 0xFFu;
        row |= c << (8 * q);
        col[q] |= c << (8 * k);
      }
      if (in) *reinterpret_cast<uint32_t*>(wq_t + int64_t(512 * p + k) * D_out) = row;
    }
    if (wqT_t != nullptr && in) {
#pragma unroll
      for (int q = 0; q < 4; ++q) *reinterpret_cast<uint32_t*>(wqT_t + int64_t(q) * D_in + 512 * p) = col[q];
    }
  }
}

// ---------------------------------------------------- nvfp4 -> bf16 ----
// One thread per block of 16 values: 8 bytes of e2m1 codes (the lower index
// in the low nibble) and one e4m3 scale.  An e2m1 magnitude (0, 0.5, 1, 1.5,
// 2, 3, 4, 6) times an e4m3 scale has at most 6 significant bits and lies in
// [2^-10, 2688], so the float32 product is exact and so are its upper 16
// bits as a bfloat16.
__device__ __forceinline__ float e2m1_value(uint32_t nib) {
  const uint32_t e = (nib >> 1) & 3u, m = nib & 1u;
  const uint32_t mag = e ? (((e + 126u) << 23) | (m << 22)) : (m ? (126u << 23) : 0u);
  return __uint_as_float(((nib & 8u) << 28) | mag);
}

__global__ void __launch_bounds__(256) k_nvfp4_to_bf16(const uint2* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       uint4* __restrict__ out, int64_t nblocks) {
  for (int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x; b < nblocks; b += int64_t(gridDim.x) * 256) {
    const uint2 c = codes[b];
    const float s = __builtin_amdgcn_cvt_f32_fp8(int(scales[b]), 0);
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 16; e += 2) {
      const uint32_t word = e < 8 ? c.x : c.y;
      const uint32_t lo = __float_as_uint(e2m1_value((word >> (4 * (e % 8))) & 0xFu) * s) >> 16;
      const uint32_t hi = __float_as_uint(e2m1_value((word >> (4 * (e % 8) + 4)) & 0xFu) * s) >> 16;
      h[e / 2] = lo | (hi << 16);
    }
    out[2 * b] = make_uint4(h[0], h[1], h[2], h[3]);
    out[2 * b + 1] = make_uint4(h[4], h[5], h[6], h[7]);
  }
}

int grid_for(int64_t work_items, int per_wg) {
  int64_t g = (work_items + per_wg - 1) / per_wg;
  // One chunk per workgroup: at 16384 x 4096 fp32 the MX row quantizer
  // reaches 71 % of HBM with 16384 one-chunk workgroups against 66 % with
  // 4096 workgroups looping over four chunks each.  The cap only keeps the
  // grid well inside its limit; the kernels stride over what remains.
  const int64_t cap = int64_t(1) << 24;
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return int(g);
}

}  // namespace

// ------------------------------------------------------------ launchers --

bsq_status launch_fp8_rowblock(int64_t rows, int64_t cols, int64_t group, const float* src,
                               uint8_t* codes, float* scales, hipStream_t st) {
  const int64_t n4 = rows * cols / 4;
  if (n4 == 0) return ok();
  constexpr int U = 4;
  const int grid = grid_for(n4, 256 * U);
  const float4* s4 = reinterpret_cast<const float4*>(src);
  uint32_t* c4 = reinterpret_cast<uint32_t*>(codes);
  switch (group) {
    case 32: hipLaunchKernelGGL((k_fp8_rowblock<32, U>), grid, 256, 0, st, s4, c4, scales, n4); break;
    case 64: hipLaunchKernelGGL((k_fp8_rowblock<64, U>), grid, 256, 0, st, s4, c4, scales, n4); break;
    case 128: hipLaunchKernelGGL((k_fp8_rowblock<128, U>), grid, 256, 0, st, s4, c4, scales, n4); break;
    case 256: hipLaunchKernelGGL((k_fp8_rowblock<256, U>), grid, 256, 0, st, s4, c4, scales, n4); break;
    default: return fail(BSQ_ERR_UNSUPPORTED, "fp8 row-block group must be 32, 64, 128 or 256");
  }
  return launch_status("quant_fp8_rowblock");
}

bsq_status launch_fp8_tile128(int64_t rows, int64_t cols, const float* src, uint8_t* codes,
                              float* scales, hipStream_t st) {
  if (rows == 0 || cols == 0) return ok();
  const dim3 grid{unsigned((rows / 128) * (cols / 128))};  // at most 2^31 - 1 tiles (checked by the caller)
  hipLaunchKernelGGL(k_fp8_tile128, grid, 256, 0, st, src, codes, scales, cols);
  return launch_status("quant_fp8_tile");
}

bsq_status launch_mx(int64_t rows, int64_t cols, int axis, const void* src, bool src_bf16,
                     uint8_t* codes, bool e5m2, uint8_t* scales, hipStream_t st) {
  if (rows == 0 || cols == 0) return ok();
  if (axis == 1) {
    const int64_t n8 = rows * cols / 8;
    constexpr int U = 2;
    const int grid = grid_for(n8, 256 * U);
    uint2* c8 = reinterpret_cast<uint2*>(codes);
#define BSQ_MXR(B, C) hipLaunchKernelGGL((k_mx_rows<B, C, U>), grid, 256, 0, st, src, c8, scales, n8)
    if (src_bf16) {
      if (e5m2) BSQ_MXR(1, 1); else BSQ_MXR(1, 0);
    } else {
      if (e5m2) BSQ_MXR(0, 1); else BSQ_MXR(0, 0);
    }
#undef BSQ_MXR
  } else {
    const MxT job{src, rows, cols, codes, scales, nullptr, nullptr};
    return launch_mx_cols(&job, 1, src_bf16, e5m2, st);
  }
  return launch_status("quant_mx");
}

bsq_status launch_mx_cols(const MxT* jobs, int n, bool src_bf16, bool e5m2, hipStream_t st) {
  MxJobs J{};
  int blocks = 0;
  for (int i = 0; i < n; ++i) {
    if (jobs[i].rows == 0 || jobs[i].cols == 0) continue;
    if (J.n == kMxJobs) return fail(BSQ_ERR_UNSUPPORTED, "quant_mx: too many matrices in one launch");
    MxJob& j = J.j[J.n++];
    j.src = jobs[i].src;
    j.codes = jobs[i].codes_t;
    j.scales = jobs[i].scales_t;
    j.row_codes = reinterpret_cast<uint2*>(jobs[i].row_codes);
    j.row_scales = jobs[i].row_scales;
    j.rows = jobs[i].rows;
    j.cols = jobs[i].cols;
    const int64_t tiles_x = (jobs[i].cols + 63) / 64, tiles_y = (jobs[i].rows + 63) / 64;
    if (tiles_x > INT32_MAX || tiles_y > INT32_MAX)
      return fail(BSQ_ERR_UNSUPPORTED, "quant_mx: too many tiles");
    const int64_t tiles = tiles_x * tiles_y;  // both factors below 2^31
    if (blocks + tiles > int64_t(INT32_MAX)) return fail(BSQ_ERR_UNSUPPORTED, "quant_mx: too many tiles");
    j.tiles_x = int(tiles_x);
    j.first = blocks;
    blocks += int(tiles);
  }
  if (J.n == 0) return ok();
  // measured at 8192x4096 bf16: 23.9 us against 24.8 row by row for a lone
  // transposed job; the backward's three-job launch and a job that also
  // writes rows were slower that way (79.7 against 64.8 us, 38.4 against 36.2)
  J.order = (J.n == 1 && J.j[0].row_codes == nullptr) ? 1 : 0;
#define BSQ_MXC(B, C) hipLaunchKernelGGL((k_mx_cols_t<B, C>), dim3(unsigned(blocks)), 256, 0, st, J)
  if (src_bf16) {
    if (e5m2) BSQ_MXC(1, 1); else BSQ_MXC(1, 0);
  } else {
    if (e5m2) BSQ_MXC(0, 1); else BSQ_MXC(0, 0);
  }
#undef BSQ_MXC
  return launch_status("quant_mx (columns, transposed)");
}

bsq_status launch_int8_rows(int64_t B, int64_t D, const float* x, int8_t* xq, float* xs,
                            hipStream_t st) {
  if (B == 0) return ok();
  if (D == 0) {
    // an empty row is all zero: scale 1
    hipLaunchKernelGGL(k_fill_u32, grid_for(B, 256), 256, 0, st, reinterpret_cast<uint32_t*>(xs), B,
                       0x3F800000u);
    return launch_status("int8_quant_rows");
  }
  const int64_t d4 = D / 4;
  uint32_t* q4 = reinterpret_cast<uint32_t*>(xq);
  const unsigned g = unsigned(B);
  if (D % 4 == 0 && d4 <= 256 * 16) {
    if (d4 <= 256) hipLaunchKernelGGL(k_int8_rows_vec<1>, g, 256, 0, st, x, q4, xs, D);
    else if (d4 <= 512) hipLaunchKernelGGL(k_int8_rows_vec<2>, g, 256, 0, st, x, q4, xs, D);
    else if (d4 <= 1024) hipLaunchKernelGGL(k_int8_rows_vec<4>, g, 256, 0, st, x, q4, xs, D);
    else if (d4 <= 2048) hipLaunchKernelGGL(k_int8_rows_vec<8>, g, 256, 0, st, x, q4, xs, D);
    else hipLaunchKernelGGL(k_int8_rows_vec<16>, g, 256, 0, st, x, q4, xs, D);
  } else {
    hipLaunchKernelGGL(k_int8_rows_any, g, 256, 0, st, x, xq, xs, D);
  }
  return launch_status("int8_quant_rows");
}

bsq_status launch_int8_cols(int64_t D_in, int64_t D_out, const float* w, int8_t* wq, float* ws,
                            int8_t* wqT, hipStream_t st) {
  if (D_out == 0) return ok();
  if (D_in > 0 && D_in <= kOnePassMaxRows && D_in % 4 == 0 && D_out % 16 == 0) {
    const int64_t stripes = D_out / 16;
    hipLaunchKernelGGL(k_int8_cols_onepass, unsigned((stripes + 7) / 8 * 8), 512, 0, st, w, wq, ws, wqT,
                       D_in, D_out);
    return launch_status("int8_quant_cols");
  }
  // the two-pass grids put D_in / 64 and D_in / 128 row blocks along y
  if (D_in > kTwoPassMaxRows) return fail(BSQ_ERR_UNSUPPORTED, "int8 column quantizer: D_in > 4194304");
  uint32_t* cmax = reinterpret_cast<uint32_t*>(ws);  // column maxima live in w_s until the end
  hipLaunchKernelGGL(k_fill_u32, grid_for(D_out, 256), 256, 0, st, cmax, D_out, 0u);
  if (D_in > 0) {
    const int rows_per_wg = 64;
    const unsigned gy = unsigned((D_in + rows_per_wg - 1) / rows_per_wg);
    if (D_out % 4 == 0) {
      const int64_t d4 = D_out / 4;
      dim3 grid(unsigned((d4 + 63) / 64), gy);
      hipLaunchKernelGGL(k_int8_colmax_vec, grid, 256, 0, st, reinterpret_cast<const float4*>(w),
                         cmax, D_in, d4, rows_per_wg);
    } else {
      dim3 grid(unsigned((D_out + 255) / 256), gy);
      hipLaunchKernelGGL(k_int8_colmax, grid, 256, 0, st, w, cmax, D_in, D_out, rows_per_wg);
    }
    dim3 grid(unsigned((D_out + 127) / 128), unsigned((D_in + 127) / 128));
    hipLaunchKernelGGL(k_int8_cols_quant, grid, 256, 0, st, w, cmax, wq, wqT, D_in, D_out);
  }
  hipLaunchKernelGGL(k_int8_col_scales, unsigned((D_out + 255) / 256), 256, 0, st, cmax, ws, D_out);
  return launch_status("int8_quant_cols");
}

bsq_status launch_nvfp4_to_bf16(int64_t rows, int64_t K, const uint8_t* codes, const uint8_t* scales,
                                uint16_t* out, hipStream_t st) {
  const int64_t nblocks = rows * (K / 16);
  if (nblocks == 0) return ok();
  hipLaunchKernelGGL(k_nvfp4_to_bf16, grid_for(nblocks, 256), 256, 0, st, reinterpret_cast<const uint2*>(codes),
                     scales, reinterpret_cast<uint4*>(out), nblocks);
  return launch_status("nvfp4_to_bf16");
}

}  // namespace bsq
