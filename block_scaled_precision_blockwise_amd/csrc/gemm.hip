// Block-scaled GEMM for gfx950: out[m, n] = sum_k A[m, k] B[n, k] with the
// scales of the four modes this library runs.
//
//   FP8G  E4M3 operands, float32 scales per 128-wide K-block: one
//         v_mfma_f32_16x16x128_f8f6f4 per K-block (exactly one 128-group),
//         then a VALU rescale-and-add of the block's partial into the
//         float32 accumulator (block_scaled_mm: dot per K-block, times the
//         two scales, summed over K-blocks).
//   MX    E4M3/E5M2 operands, E8M0 scales per 32 elements: the scaled MFMA
//         v_mfma_scale_f32_16x16x128_f8f6f4 applies both scales in the
//         matrix core and accumulates directly (scaled_matmul with mxfp8).
//   I8    int8 operands, v_mfma_i32_16x16x64_i8 into int32 accumulators,
//         float32 epilogue float(a) * (s_x * s_w) (int8 per-channel).
//   BF16  bfloat16 operands (nvfp4 after its exact dequantization),
//         v_mfma_f32_16x16x32_bf16, no scales.
//
// Both operands are K-contiguous ("TN").  A workgroup of 8 waves owns a
// 256 x 256 output tile (192 or 128 rows when that fills the CUs in fewer
// passes) and walks K in steps of 128 bytes; each step's A and B tiles are
// double-buffered in LDS with a 16-byte-chunk XOR swizzle that spreads the
// 16 rows of a fragment read over the LDS banks.  Wave (wm, wn) owns a
// quarter of the rows and columns 128*wn..+128: 4 (3, 2) x 8 blocks of
// 16 x 16.  Products with few tiles run k_gemm_sk instead (64 x 64 tiles, K
// split over the workgroup's waves).
//
// What sets a K-step's length (measured on gfx950, FP8G at 4096^3): each
// SIMD issues 64 MFMAs, 264 VALU instructions (the rescale) and 48
// fragment reads per step.  Two waves per SIMD issue an MFMA every 24
// cycles alone; with the step's reads and rescale FMAs beside them, about
// every 36 (reads or FMAs alone cost little; together they do), so the
// step's register-side work takes about 2310 cycles of the SIMD's issue
// before its loads and barrier (about 2850 measured).  The tile loads
// arrive within the step.  The 32x32x64 MFMA, with each block's two K
// halves chained for the rescale, took more cycles per step than this
// layout.
//
// Unscaled products (FP8G, and the I8/BF16 modes' own instructions): the
// FP8G calls go through the scaled builtin with all four scale operands
// (format selectors and E8M0 bytes) zero; for constant zero scale operands
// the compiler emits the plain v_mfma_f32_16x16x128_f8f6f4, which applies
// no block scale (the FP8G kernels' code holds no v_mfma_scale or
// v_mfma_ld_scale instruction).  Were a scaled form emitted instead, a zero
// E8M0 byte would mean 2^-127 per operand and every FP8G product would
// vanish, which each FP8G parity test would catch.
//
// Fragment layout (measured on gfx950): for the 16x16x128 f8 MFMA a lane
// l supplies 32 bytes of row l % 16: K [16g, 16g+16) in bytes 0..15 and K
// [64+16g, 64+16g+16) in bytes 16..31, g = l / 16; its E8M0 scale covers
// K [32g, 32g+32).  The two 16x16x64 i8 MFMAs take the same two halves.
// The result lane l holds column l % 16 of rows 4*(l/16) .. +3.  The MFMA's
// first operand is the B fragment, so a lane's four results are four
// consecutive n of one m: one 16-byte store, one A scale per lane.
#include <hip/hip_ext.h>

#include "common.h"
#include "gemm.h"

#include <type_traits>

namespace bsq {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 128;

struct GemmArgs {
  const uint8_t* A;
  const uint8_t* B;
  const void* SA;
  const void* SB;
  void* out;
  int32_t* acc_out;
  int M, N, K;
  int64_t sA, sB, sSA, sSB, sC;  // batch strides in elements of each array
  // general scale blocks (GEN kernels only): scale columns per row of A and
  // B, K-steps of 128 (FP8G) or 32-element blocks (MX) per scale, and B
  // rows (output columns) per B scale row (FP8G)
  int sc_a, sc_b, sg_a, sg_b, gn;
};

__device__ __forceinline__ v8i lds_frag(const uint8_t* tile, int off0, int off1) {
  const uint4 lo = *reinterpret_cast<const uint4*>(tile + off0);
  const uint4 hi = *reinterpret_cast<const uint4*>(tile + off1);
  v8i r;
  r[0] = int(lo.x); r[1] = int(lo.y); r[2] = int(lo.z); r[3] = int(lo.w);
  r[4] = int(hi.x); r[5] = int(hi.y); r[6] = int(hi.z); r[7] = int(hi.w);
  return r;
}

// Buffer resource (V#) of a raw byte buffer: base, no stride, `records`
// bytes in range (clamped to [0, 2^31)); offsets at or past the end read as
// zero.  dword3 0x00020000 = 32-bit data format, the gfx9 raw-buffer value.
__device__ __forceinline__ i32x4 raw_rsrc(const uint8_t* base, int64_t records) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const int n = int(records < 0 ? 0 : (records > 0x7FFFFFFF ? 0x7FFFFFFF : records));
  return i32x4{int(uint32_t(b)), int(uint32_t(b >> 32) & 0xFFFFu), n, 0x00020000};
}

// 16 bytes per lane from buffer `rsrc` at byte offset `voff` straight into
// LDS: lane i writes [lds_addr + 16 i, lds_addr + 16 i + 16).  Issued as
// inline asm so that the compiler does not order it against the fragment
// reads of the other LDS stage; the caller waits with vmcnt(0) before the
// barrier that publishes the stage.
__device__ __forceinline__ void lds_dma16(i32x4 rsrc, int voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// 4 bytes per lane: lane i writes [lds_addr + 4 i, lds_addr + 4 i + 4).
__device__ __forceinline__ void lds_dma4(i32x4 rsrc, int voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// Buffer resource of `records` (>= 0, < 2^31) bytes from `base`.
__device__ __forceinline__ i32x4 rsrc32(const uint8_t* base, int records) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return i32x4{__builtin_amdgcn_readfirstlane(int(uint32_t(b))),
               __builtin_amdgcn_readfirstlane(int(uint32_t(b >> 32) & 0xFFFFu)),
               __builtin_amdgcn_readfirstlane(records), 0x00020000};
}

__device__ __forceinline__ uint32_t lds_addr_of(const uint8_t* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)(p)));
}

// Tile order.  The grid is one-dimensional over the tiles (the batch in
// z): its x extent allows 2^31 - 1 workgroups where y allows 65536.
// Workgroups are dealt to the 8 XCDs round-robin by linear id and each XCD
// has its own L2, so the tiles one XCD receives should share operand rows:
// linear id L goes to XCD L % 8 as its (L / 8)-th workgroup; XCD x gets the
// x-th contiguous eighth of a tile order that walks column-major through
// bands of kBand tile rows, i.e. a compact block of tiles (4 x 8 for a
// 16 x 16 grid).
__device__ __forceinline__ void tile_coords(int& tm, int& tn, int tiles_m, int tiles_n) {
  constexpr int kBand = 4;
  const int T = tiles_n * tiles_m;
  const int L = blockIdx.x;
  const int per = T / 8;
  const int t = (L < 8 * per) ? (L % 8) * per + L / 8 : L;
  const int band = t / (kBand * tiles_n);
  const int rows = min(kBand, tiles_m - band * kBand);
  const int in = t - band * kBand * tiles_n;
  tm = band * kBand + in % rows;
  tn = in / rows;
}

// Epilogue of a (64 MB) x 256 tile held by 8 waves as (16 MB) x 128 wave
// tiles (wave w: rows 16 MB (w % 4), columns 128 (w / 4)), through LDS.  A lane's
// results are 4 columns of one row in 16 different rows per block, so
// direct stores would write 16 row pieces of 64 bytes per instruction.
// Instead each wave stages 32 of its rows at a time in LDS (row-major,
// kStageRowB bytes per row) and reads them back so that one store
// instruction writes two whole 128-column rows.  The caller has finished
// every LDS read and DMA of its main loop and passed a barrier, so the
// stage buffers are free.
constexpr int kStageRowB = 128 * 4 + 16;  // 128 floats + 16 B against bank conflicts
constexpr int kLdsAB = 2 * (BM + BN) * BK > 8 * 32 * kStageRowB ? 2 * (BM + BN) * BK : 8 * 32 * kStageRowB;

template <int MODE, int OUT_BF16, int MB, typename acc_t>
__device__ __forceinline__ void store_tile(const GemmArgs& p, const acc_t (&acc)[8][MB], uint8_t* lds_ab, int w,
                                           int lane, int batch, int m0, int n0) {
  constexpr int NB = 8;
  static_assert(MB >= 2 && MB <= 4, "32, 48 or 64 rows per wave");
  const int M = p.M, N = p.N;
  const int wm = w & 3, wn = w >> 2;
  const int g = lane >> 4, r16 = lane & 15;
  uint8_t* const stg = lds_ab + w * 32 * kStageRowB;
  // the wave's rows in pieces of 32 (the last one 16 rows when MB is odd)
#pragma unroll
  for (int h = 0; h < (MB + 1) / 2; ++h) {
    if (h > 0) __syncthreads();  // the previous piece has been read back
    const int T = 2 * h + 1 < MB ? 16 : 8;  // pairs of rows in this piece
#pragma unroll
    for (int ii = 0; ii < 2; ++ii) {
      const int i = 2 * h + ii;
      if (i >= MB) break;
      const int m = m0 + 16 * MB * wm + 16 * i + r16;
      float xs = 0.f;
      if (MODE == MODE_I8) xs = static_cast<const float*>(p.SA)[int64_t(batch) * p.sSA + min(m, M - 1)];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int n = n0 + 128 * wn + 16 * j + 4 * g;
        float y[4] = {0.f, 0.f, 0.f, 0.f};
        if (MODE == MODE_I8) {
          if (n < N) {
            const float4 ws = *reinterpret_cast<const float4*>(static_cast<const float*>(p.SB) +
                                                               int64_t(batch) * p.sSB + n);
            const float wsv[4] = {ws.x, ws.y, ws.z, ws.w};
#pragma unroll
            for (int r = 0; r < 4; ++r) y[r] = float(acc[j][i][r]) * (xs * wsv[r]);
            if (p.acc_out != nullptr && m < M)
              *reinterpret_cast<int4*>(p.acc_out + int64_t(batch) * p.sC + int64_t(m) * N + n) =
                  make_int4(acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = float(acc[j][i][r]);
        }
        *reinterpret_cast<float4*>(stg + (16 * ii + r16) * kStageRowB + (16 * j + 4 * g) * 4) =
            make_float4(y[0], y[1], y[2], y[3]);
      }
    }
    __syncthreads();
    // rows 32 h + rr of the wave's 16 MB: lanes 0-31 one row, 32-63 the next.
    // A tile inside the matrix stores without bounds checks, so that all
    // 16 reads are issued before the first store.
    auto put = [&](int t, const float4& v) {
      const int rr = 2 * t + (lane >> 5), cc = 4 * (lane & 31);
      const int m = m0 + 16 * MB * wm + 32 * h + rr;
      const int n = n0 + 128 * wn + cc;
      const int64_t o = int64_t(batch) * p.sC + int64_t(m) * N + n;
      // streaming stores: the output is not read again by this kernel
      if (OUT_BF16) {
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        const uint32_t lo = encode_bf16(v.x) | (encode_bf16(v.y) << 16);
        const uint32_t hi = encode_bf16(v.z) | (encode_bf16(v.w) << 16);
        __builtin_nontemporal_store(u32x2_t{lo, hi}, reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(p.out) + o));
      } else {
        __builtin_nontemporal_store(f32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4_t*>(static_cast<float*>(p.out) + o));
      }
    };
    auto get = [&](int t) {
      const int rr = 2 * t + (lane >> 5), cc = 4 * (lane & 31);
      return *reinterpret_cast<const float4*>(stg + rr * kStageRowB + cc * 4);
    };
    if (m0 + 64 * MB <= M && n0 + BN <= N) {
      float4 v[16];
#pragma unroll
      for (int t = 0; t < T; ++t) v[t] = get(t);
#pragma unroll
      for (int t = 0; t < T; ++t) put(t, v[t]);
    } else {
#pragma unroll
      for (int t = 0; t < T; ++t) {
        const int rr = 2 * t + (lane >> 5), cc = 4 * (lane & 31);
        const int m = m0 + 16 * MB * wm + 32 * h + rr;
        const int n = n0 + 128 * wn + cc;
        const float4 v = get(t);
        if (m < M && n < N) put(t, v);
      }
    }
  }
}

// NW = 8 waves per workgroup: waves 4 (M) x 2 (N), each 64 x 128 (4 x 8
// blocks; 48 or 32 rows for TBM = 192 or 128), accumulators in VGPRs - the
// FP8G rescale needs them on the VALU.
// (Measured alternatives that were not faster: 4 waves of 128 x 128 with
// AGPR accumulators; two wave groups alternating between MFMA and memory
// phases with a barrier per phase; an L2 prefetch two steps ahead.)
// SUB (general blocks only): scale blocks shorter than the MFMA's K - FP8G
// float32 blocks that are multiples of 64 (not of 128), E8M0 blocks that
// are multiples of 16 (not of 32).  Each block then takes two MFMAs per
// K-step, each with part of the A fragment zeroed so that it sums exactly
// one sub-block of every 128-wide step (see the loop).
template <int MODE, int OUT_BF16, int FA, int FB, int GN1, int NW, int TBM, int GEN = 0, int SUB = 0>
__global__ void __launch_bounds__(64 * NW, 1) k_gemm(GemmArgs p) {
  static_assert(NW == 8, "8 waves: the wave layout, scale staging and epilogue assume it");
  static_assert(TBM == 256 || TBM == 192 || TBM == 128, "tile rows");
  static_assert(!GEN || MODE == MODE_FP8G || MODE == MODE_MX, "general blocks: FP8G or MX");
  static_assert(!SUB || GEN, "sub-step blocks go through the general scale staging");
  constexpr int NT = 64 * NW;          // threads
  constexpr int WGM = 4;                // waves along M
  constexpr int MB = TBM / WGM / 16;    // 16-row blocks per wave along M
  constexpr int NB = 8;                 // 16-column blocks per wave along N
  constexpr int SPW = 32 / NW;          // 8-row DMA slices per wave of B
  constexpr int SPWA = TBM / 8 / NW;    // 8-row DMA slices per wave of A

  // LDS: the two A stages, then the two B stages; after the main loop the
  // same bytes stage the epilogue
  __shared__ __attribute__((aligned(16))) uint8_t lds_ab[kLdsAB];
  uint8_t* const lds_a = lds_ab;                 // stage st at + st * TBM * BK
  uint8_t* const lds_b = lds_ab + 2 * TBM * BK;  // stage st at + st * BN * BK
  // scales of kGS consecutive K-steps, kSG words (16 bytes) per slot: slot
  // r < 256 holds A row r, slot 256 + r B row r (MX, FP8G with GN1) or B
  // row group r (FP8G); without general blocks the word of step ks sits at
  // [(ks / kSG) & 1][slot * kSG + ks % kSG].  General blocks: a slot's 16
  // bytes start at the first scale of the group (the granule index - 128,
  // or 64 for SUB, K-wide steps for FP8G; 32-, or 16-element blocks for MX -
  // of the group's first granule, over granules per scale); a group is 4
  // steps, 2 for SUB, so that it spans at most 16 bytes of scales.
  constexpr int kSG = 4;
  constexpr int kGS = SUB ? 2 : 4;
  __shared__ __attribute__((aligned(16))) uint32_t lds_s[2][512 * kSG];

  const int tid = threadIdx.x;
  const int batch = blockIdx.z;
  int tm, tn;
  tile_coords(tm, tn, (p.M + TBM - 1) / TBM, (p.N + BN - 1) / BN);
  const int m0 = tm * TBM;
  const int n0 = tn * BN;
  const int M = p.M, N = p.N, K = p.K;
  const int nk = K / BK;

  const uint8_t* A = p.A + int64_t(batch) * p.sA;
  const uint8_t* B = p.B + int64_t(batch) * p.sB;

  // ---- global -> LDS: direct 16-byte buffer loads.  Lane i of a wave
  // fills LDS bytes [16 i, 16 i + 16) of one 1 KiB slice (8 rows x 128
  // bytes), i.e. row (slice_row0 + i / 8), physical chunk i % 8; it fetches
  // the logical chunk that the XOR swizzle stores there.  Wave w moves
  // slices w, w + NW, ... of A and of B per K-step.  One descriptor per
  // slice (scalar registers), built once: it starts at the slice's first
  // row and covers its rows inside the operand, so rows at or past M (N)
  // fall outside its range and read as zero and tails need no clamping.
  // A K-step only moves the lane offset, which all slices share.
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lrow = 8 * w + (lane >> 3);
  const int llog = (lane & 7) ^ (lrow & 7);
  const int voff = lrow * K + 16 * llog;  // < 8 NW K
  // bytes of each slice's rows that lie inside the operand, from the slice's
  // first row (0 .. 64 rows of K bytes); at K-step ks a slice's descriptor
  // starts ks * BK bytes into that row and covers the rest
  int a_rec[SPW], b_rec[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    a_rec[s] = max(0, min(M - (m0 + 8 * NW * s), 8 * NW)) * K;
    b_rec[s] = max(0, min(N - (n0 + 8 * NW * s), 8 * NW)) * K;
  }
  i32x4 ra[SPW], rb[SPW];
#pragma unroll
  for (int s = 0; s < SPW; ++s) {
    if (s < SPWA) ra[s] = rsrc32(A + int64_t(m0 + 8 * NW * s) * K, a_rec[s]);
    rb[s] = rsrc32(B + int64_t(n0 + 8 * NW * s) * K, b_rec[s]);
  }
  const uint32_t la_base = __builtin_amdgcn_readfirstlane(lds_addr_of(lds_a + 8 * w * BK));
  const uint32_t lb_base = __builtin_amdgcn_readfirstlane(lds_addr_of(lds_b + 8 * w * BK));
  // ks == nk (after the last step): every lane's offset lies past every
  // slice's range (records <= 64 K <= 2^30), so the loads read zeros
  // without touching memory and the loop body needs no branch
  auto gload_slice = [&](int ks, int st, int s) {
    const int vk = ks < nk ? voff + ks * BK : (1 << 30);  // < 8 NW K
    if (s < SPWA) lds_dma16(ra[s], vk, la_base + uint32_t(st * TBM * BK + 8 * NW * s * BK));
    lds_dma16(rb[s], vk, lb_base + uint32_t(st * BN * BK + 8 * NW * s * BK));
  };
  auto gload = [&](int ks, int st) {
#pragma unroll
    for (int s = 0; s < SPW; ++s) gload_slice(ks, st, s);
  };

  // ---- scales, by direct 16-byte buffer loads into LDS as well: one load
  // per row brings the words of kSG consecutive K-steps (one 16-byte piece
  // of a scale row instead of one word of kSG of them), for the group of
  // steps that follows the current one.
  // Lane i of wave w fills slot 64 w + i (waves 0-3 the A rows, 4-7 the B
  // rows).  Lanes with nothing to move read their wave's first scale row
  // into a slot nobody reads.
  constexpr bool kScales = MODE == MODE_FP8G || MODE == MODE_MX;
  static_assert(!kScales || NW == 8, "scale staging assumes 512 threads");
  // Each wave's scale base starts at the first scale row its lanes read
  // (64-bit arithmetic, once per workgroup); a lane's offset from it stays
  // below 256 rows of at most 2^19 bytes, so it fits 32 bits whatever M
  // and N are.
  const uint8_t* sbase = nullptr;  // this wave's scale rows at K-step 0
  int soff_v = 0;                  // this lane's byte offset from sbase
  int64_t s_records = 0;           // bytes from sbase to the end of the scale array
  int s_per = 1;                   // GEN: this wave's K-steps (FP8G) / 32-blocks (MX) per scale
  if (kScales) {
    // waves 0-3 (uniform w < 4) own the A slots, waves 4-7 the B slots
    const bool a_side = w < 4;
    const int r = tid - 256;
    const int esz = MODE == MODE_FP8G ? 4 : 1;
    const uint8_t* SA = static_cast<const uint8_t*>(p.SA) + int64_t(batch) * p.sSA * esz;
    const uint8_t* SB = static_cast<const uint8_t*>(p.SB) + int64_t(batch) * p.sSB * esz;
    // bytes per scale row, scale rows of each operand, and this lane's row
    // next to the wave's first row (rows past the operand read its last row)
    int row_bytes, rows_op, row, row0;
    if (GEN) {
      // general blocks: a scale row holds sc scales; B rows of the FP8G
      // kernel are output columns, gn of them per scale row
      row_bytes = (a_side ? p.sc_a : p.sc_b) * esz;
      s_per = a_side ? p.sg_a : p.sg_b;
      rows_op = a_side ? M : (MODE == MODE_FP8G ? N / p.gn : N);
    } else {
      row_bytes = nk * 4;  // FP8G: one float per K-step; MX: K / 32 bytes
      rows_op = a_side ? M : (MODE == MODE_FP8G && !GN1 ? N / 128 : N);
    }
    if (a_side) {
      row0 = m0;
      row = min(m0 + tid, M - 1);
    } else if (MODE == MODE_MX || GN1) {
      // B scale row per output column
      row0 = MODE == MODE_FP8G && GEN ? n0 / p.gn : n0;
      row = MODE == MODE_FP8G && GEN ? min(n0 + r, N - 1) / p.gn : min(n0 + r, N - 1);
    } else {
      // FP8G with one B scale per 128 (GEN: group_n, a multiple of 128)
      // columns: slots 256 and 257 hold the tile's two column halves
      const int gdiv = GEN ? p.gn : 128;
      row0 = n0 / gdiv;
      row = (r >= 0 && r < 2 && n0 + 128 * r < N) ? (n0 + 128 * r) / gdiv : row0;
    }
    sbase = (a_side ? SA : SB) + int64_t(row0) * row_bytes;
    s_records = int64_t(rows_op - row0) * row_bytes;
    soff_v = (row - row0) * row_bytes;
  }
  const uint32_t ls_base =
      __builtin_amdgcn_readfirstlane(lds_addr_of(reinterpret_cast<const uint8_t*>(&lds_s[0][64 * w * kSG])));
  // group q (steps kSG q .. kSG q + kSG - 1) into buffer q & 1; words past a
  // row's last step are never read
  // GEN: the 16 bytes start at the first scale the group needs (FP8G: a
  // float, 4 per load; MX: its e8m0 byte rounded down to a word, so the
  // group's at most 12 distinct bytes fit)
  auto sload = [&](int q) {
    if (kScales) {
      const int64_t o = !GEN ? 4 * int64_t(kSG) * q
                             : (MODE == MODE_FP8G ? 4 * int64_t((kSG * q) / s_per) : int64_t(((16 * q) / s_per) & ~3));
      lds_dma16(raw_rsrc(sbase + o, s_records - o), soff_v, ls_base + uint32_t((q & 1) * 512 * kSG * 4));
    }
  };

  // ---- wave / lane roles in the MFMA loop
  const int wm = w % WGM, wn = w / WGM;
  const int g = lane >> 4, r16 = lane & 15;
  const int swz = r16 & 7;
  const int c0 = 16 * (g ^ swz), c1 = 16 * ((g + 4) ^ swz);

  typedef typename std::conditional<MODE == MODE_I8, v4i, v4f>::type acc_t;
  acc_t acc[NB][MB];
#pragma unroll
  for (int j = 0; j < NB; ++j)
#pragma unroll
    for (int i = 0; i < MB; ++i) acc[j][i] = acc_t{0, 0, 0, 0};

  gload(0, 0);
  sload(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's direct loads have landed
  __syncthreads();

  // The next step's tiles stream into the idle stage while this one is
  // multiplied: each wave issues its A and B slice for it at the head of
  // column blocks 0 .. SPW-1, between the MFMAs of the first half of the
  // step (all at the head of the step stalls the MFMA issue behind the
  // loads; spread over the whole step, the last ones land late).  The final
  // step issues its loads past the operands' ranges (no memory traffic) so
  // that the body has no branch.
  for (int ks = 0; ks < nk; ++ks) {
    const int st = ks & 1;
    const int kn = ks + 1;
    // the next group's scales during the last step of this group (the
    // buffer they go to was last read kGS steps ago)
    if (ks % kGS == kGS - 1 && ks + 1 < nk) sload((ks + 1) / kGS);

    const uint8_t* ta = lds_a + st * TBM * BK;
    const uint8_t* tb = lds_b + st * BN * BK;
    const uint32_t* ss = &lds_s[(ks / kSG) & 1][ks % kSG];  // + slot * kSG
    // GEN, FP8G: word of this step's A / B scale within the group's 4;
    // MX: byte of this lane's 32-block scale within the group's 16
    const uint32_t* ssa = ss;
    const uint32_t* ssb = ss;
    int mxa = 0, mxb = 0;
    // SUB: the word (FP8G) / byte (MX) of the second sub-block of the step
    // (FP8G: K 64..127; MX: the second 16 elements of the lane's 32-block)
    const uint32_t* ssa1 = ss;
    const uint32_t* ssb1 = ss;
    int mxa1 = 0, mxb1 = 0;
    if (GEN) {
      const int q = ks / kGS;
      if (MODE == MODE_FP8G) {
        // granule = K-step (64-wide half step for SUB); 4 granules per group
        const int gr0 = SUB ? 2 * ks : ks;
        ssa = &lds_s[q & 1][gr0 / p.sg_a - (4 * q) / p.sg_a];
        ssb = &lds_s[q & 1][gr0 / p.sg_b - (4 * q) / p.sg_b];
        if (SUB) {
          ssa1 = &lds_s[q & 1][(gr0 + 1) / p.sg_a - (4 * q) / p.sg_a];
          ssb1 = &lds_s[q & 1][(gr0 + 1) / p.sg_b - (4 * q) / p.sg_b];
        }
      } else {
        // granule = the lane's 32-element block (16-element sub-block for
        // SUB); 16 granules per group
        ssa = ssb = ssa1 = ssb1 = &lds_s[q & 1][0];
        const int gr0 = SUB ? 8 * ks + 2 * g : 4 * ks + g;
        mxa = gr0 / p.sg_a - (((16 * q) / p.sg_a) & ~3);
        mxb = gr0 / p.sg_b - (((16 * q) / p.sg_b) & ~3);
        if (SUB) {
          mxa1 = (gr0 + 1) / p.sg_a - (((16 * q) / p.sg_a) & ~3);
          mxb1 = (gr0 + 1) / p.sg_b - (((16 * q) / p.sg_b) & ~3);
        }
      }
    }
    // LDS reads retire in order, so a wait for one read also waits for all
    // reads issued before it.  The step's scales are therefore read first,
    // then the fragments in the order their MFMAs need them (the first MFMA
    // waits only for the scales and its own two fragments); B fragments
    // stream PF ahead.
    auto afrag = [&](int i) {
      const int row = 16 * MB * wm + 16 * i + r16;
      return lds_frag(ta, row * BK + c0, row * BK + c1);
    };
    auto bfrag = [&](int j) {
      const int rowb = 128 * wn + 16 * j + r16;
      return lds_frag(tb, rowb * BK + c0, rowb * BK + c1);
    };
    float sa[MB], sa1[MB];
    uint32_t qa_w[MB], qb_w[NB], qa_w1[MB];
    float sbg = 0.f, sbg1 = 0.f;
    if (MODE == MODE_FP8G) {
#pragma unroll
      for (int i = 0; i < MB; ++i) sa[i] = __uint_as_float(ssa[(16 * MB * wm + 16 * i + r16) * kSG]);
      if (!GN1) sbg = __uint_as_float(ssb[(256 + wn) * kSG]);
      if (SUB) {
#pragma unroll
        for (int i = 0; i < MB; ++i) sa1[i] = __uint_as_float(ssa1[(16 * MB * wm + 16 * i + r16) * kSG]);
        if (!GN1) sbg1 = __uint_as_float(ssb1[(256 + wn) * kSG]);
      }
    } else if (MODE == MODE_MX) {
#pragma unroll
      for (int i = 0; i < MB; ++i) qa_w[i] = ssa[(16 * MB * wm + 16 * i + r16) * kSG + (GEN ? mxa >> 2 : 0)];
#pragma unroll
      for (int j = 0; j < NB; ++j) qb_w[j] = ssb[(256 + 128 * wn + 16 * j + r16) * kSG + (GEN ? mxb >> 2 : 0)];
      if (SUB) {
#pragma unroll
        for (int i = 0; i < MB; ++i) qa_w1[i] = ssa1[(16 * MB * wm + 16 * i + r16) * kSG + (mxa1 >> 2)];
      }
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the scale reads ahead of the fragment reads
    constexpr int PF = SUB ? 1 : 2;  // B fragments in flight ahead of their MFMAs
    v8i pq[PF];
    pq[0] = bfrag(0);
    v8i q[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) q[i] = afrag(i);
#pragma unroll
    for (int t = 1; t < PF; ++t) pq[t] = bfrag(t);
    // FP8G: the rescale of block j-1 runs on the VALU between the MFMAs of
    // block j, which do not depend on it.
    v4f dprev[MB];
    float sb4p[4];
    auto rescale = [&](int jj, const v4f (&d)[MB], const float (&sb4)[4]) {
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        if (GN1) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[jj][i][r] = fmaf(d[i][r], sa[i] * sb4[r], acc[jj][i][r]);
        } else {
          const float sc = sa[i] * sbg;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[jj][i][r] = fmaf(d[i][r], sc, acc[jj][i][r]);
        }
      }
    };
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      if (j < SPW) gload_slice(kn, st ^ 1, j);
      v8i pnext;
      if (j + PF < NB) pnext = bfrag(j + PF);
      const v8i pb = pq[0];
      if (SUB && MODE == MODE_FP8G) {
        // two 64-wide K groups per step: a lane's first 16 fragment bytes
        // hold K 16g..16g+15 (< 64), its last 16 K 64+16g.. (>= 64), so
        // zeroing one half of the A fragment leaves exactly one group's
        // products; each partial takes its own pair of scales
        float sl[4] = {0.f, 0.f, 0.f, 0.f}, sh[4] = {0.f, 0.f, 0.f, 0.f};
        if (GN1) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            sl[r] = __uint_as_float(ssb[(256 + 128 * wn + 16 * j + 4 * g + r) * kSG]);
            sh[r] = __uint_as_float(ssb1[(256 + 128 * wn + 16 * j + 4 * g + r) * kSG]);
          }
        }
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const v4f zero = {0.f, 0.f, 0.f, 0.f};
          const v8i qlo = {q[i][0], q[i][1], q[i][2], q[i][3], 0, 0, 0, 0};
          const v8i qhi = {0, 0, 0, 0, q[i][4], q[i][5], q[i][6], q[i][7]};
          // zero scale operands: the unscaled MFMA (see the file header)
          const v4f dl = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pb, qlo, zero, 0, 0, 0, 0, 0, 0);
          const v4f dh = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pb, qhi, zero, 0, 0, 0, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float fl = GN1 ? sa[i] * sl[r] : sa[i] * sbg;
            const float fh = GN1 ? sa1[i] * sh[r] : sa1[i] * sbg1;
            acc[j][i][r] = fmaf(dh[r], fh, fmaf(dl[r], fl, acc[j][i][r]));
          }
        }
      } else if (SUB && MODE == MODE_MX) {
        // 16-element blocks: a lane's fragment holds the first halves of its
        // two 32-blocks when g is even, the second halves when g is odd.
        // MFMA h keeps the lanes with g % 2 == h (the others' A bytes are
        // zeroed) and takes the scales of those halves.
        const uint32_t qbw1 = ssb1[(256 + 128 * wn + 16 * j + r16) * kSG + (mxb1 >> 2)];
        const int qb0 = int((qb_w[j] >> (8 * (mxb & 3))) & 0xFFu);
        const int qb1 = int((qbw1 >> (8 * (mxb1 & 3))) & 0xFFu);
        const bool odd = (g & 1) != 0;
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const v8i z = {0, 0, 0, 0, 0, 0, 0, 0};
          const v8i q0 = odd ? z : q[i];
          const v8i q1 = odd ? q[i] : z;
          const int qa0 = int((qa_w[i] >> (8 * (mxa & 3))) & 0xFFu);
          const int qa1 = int((qa_w1[i] >> (8 * (mxa1 & 3))) & 0xFFu);
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pb, q0, acc[j][i], FB, FA, 0, qb0, 0, qa0);
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pb, q1, acc[j][i], FB, FA, 0, qb1, 0, qa1);
        }
      } else if (MODE == MODE_FP8G) {
        float sb4[4] = {0.f, 0.f, 0.f, 0.f};
        if (GN1) {
#pragma unroll
          for (int r = 0; r < 4; ++r) sb4[r] = __uint_as_float(ssb[(256 + 128 * wn + 16 * j + 4 * g + r) * kSG]);
        }
        v4f dcur[MB];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const v4f zero = {0.f, 0.f, 0.f, 0.f};
          // zero scale operands: the unscaled MFMA (see the file header)
          dcur[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(pb, q[i], zero, 0, 0, 0, 0, 0, 0);
        }
        if (j > 0) rescale(j - 1, dprev, sb4p);
#pragma unroll
        for (int i = 0; i < MB; ++i) dprev[i] = dcur[i];
#pragma unroll
        for (int r = 0; r < 4; ++r) sb4p[r] = sb4[r];
      } else if (MODE == MODE_MX) {
        // E8M0 scale bytes: byte g of the row's word covers this lane's
        // 32-element K block (the instruction reads its scale from byte 0)
        const int sha = GEN ? 8 * (mxa & 3) : 8 * g, shb = GEN ? 8 * (mxb & 3) : 8 * g;
        const int qb = int((qb_w[j] >> shb) & 0xFFu);
#pragma unroll
        for (int i = 0; i < MB; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              pb, q[i], acc[j][i], FB, FA, 0, qb, 0, int((qa_w[i] >> sha) & 0xFFu));
      } else if (MODE == MODE_I8) {
        const v4i plo = {pb[0], pb[1], pb[2], pb[3]};
        const v4i phi = {pb[4], pb[5], pb[6], pb[7]};
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const v4i qlo = {q[i][0], q[i][1], q[i][2], q[i][3]};
          const v4i qhi = {q[i][4], q[i][5], q[i][6], q[i][7]};
          acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(plo, qlo, acc[j][i], 0, 0, 0);
          acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(phi, qhi, acc[j][i], 0, 0, 0);
        }
      } else {
        // bf16: each 16-byte half of a fragment is 8 elements of K (the
        // same K positions in the A and the B fragment, so the order of K
        // inside an instruction does not matter)
        const v4i plo = {pb[0], pb[1], pb[2], pb[3]};
        const v4i phi = {pb[4], pb[5], pb[6], pb[7]};
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          const v4i qlo = {q[i][0], q[i][1], q[i][2], q[i][3]};
          const v4i qhi = {q[i][4], q[i][5], q[i][6], q[i][7]};
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, plo),
                                                              __builtin_bit_cast(bf16x8, qlo), acc[j][i], 0, 0, 0);
          acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, phi),
                                                              __builtin_bit_cast(bf16x8, qhi), acc[j][i], 0, 0, 0);
        }
      }
#pragma unroll
      for (int t = 0; t + 1 < PF; ++t) pq[t] = pq[t + 1];
      if (j + PF < NB) pq[PF - 1] = pnext;
      if (MODE == MODE_FP8G && !SUB && j > 0) {
        // issue order: the two prefetch reads, then one MFMA followed by
        // four rescale FMAs, MB times
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < MB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (MODE == MODE_FP8G && !SUB) rescale(NB - 1, dprev, sb4p);

    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
  }

  store_tile<MODE, OUT_BF16, MB>(p, acc, lds_ab, w, lane, batch, m0, n0);
}

// ---------------------------------------------------------------------------
// Small and skinny products (few 256 x 256 tiles): split K inside the
// workgroup.  SKW waves (4; the template allows 8) share one 64 x 64 output
// tile; wave w runs K-steps [w * per, (w + 1) * per) over the whole tile.
// Each wave stages its own A and B tiles of a step (16 KiB) and the step's
// scales (one word per row) in a private LDS region with the big kernel's
// direct loads (8 rows x 128 bytes per instruction: whole cache lines;
// loading MFMA fragments straight into registers reads 64-byte half lines
// of 16 rows per instruction, and ran at a third of the rate) and swizzle;
// nothing is shared, so the K loop has no barrier.  Once a step's
// fragments and scales are in registers the region takes the next step's,
// which are in flight while the step is multiplied; one wait per step
// covers all of them (scales read with ordinary loads made the compiler
// wait for every load in flight before their first use, which cost 30 %
// at 237 x 4096 x 4096).  One region per wave keeps a workgroup at 66 KiB,
// two per CU.  The SKW partial tiles then meet in LDS (the stage area) and
// each output is the sum of the partials in wave order - the result does
// not depend on timing.  Same MFMAs, scales and epilogue arithmetic as
// k_gemm.
constexpr int SK_T = 64;  // output tile edge

template <int MODE, int OUT_BF16, int FA, int FB, int SKW>
__global__ void __launch_bounds__(64 * SKW, 8 / SKW) k_gemm_sk(GemmArgs p) {
  typedef typename std::conditional<MODE == MODE_I8, v4i, v4f>::type acc_t;
  constexpr bool kScales = MODE == MODE_FP8G || MODE == MODE_MX;
  constexpr int kTiles = 2 * SK_T * BK;             // A then B tile of one K-step
  constexpr int kRegion = kTiles + 2 * 64 * 4;      // + A and B scale words of the step
  __shared__ __attribute__((aligned(16))) uint8_t lds_sk[SKW * kRegion];
  static_assert(sizeof(acc_t) * SKW * SK_T * SK_T / 4 <= sizeof(lds_sk), "partials fit the stage area");
  acc_t (*red)[SK_T * SK_T / 4] = reinterpret_cast<acc_t (*)[SK_T * SK_T / 4]>(lds_sk);

  const int tid = threadIdx.x;
  const int batch = blockIdx.z;
  const int m0 = blockIdx.y * SK_T, n0 = blockIdx.x * SK_T;
  const int M = p.M, N = p.N, K = p.K;
  const int nk = K / BK;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int g = lane >> 4, r16 = lane & 15;
  const int per = (nk + SKW - 1) / SKW;
  const int k_begin = min(w * per, nk), k_end = min(k_begin + per, nk);

  const uint8_t* A = p.A + int64_t(batch) * p.sA;
  const uint8_t* B = p.B + int64_t(batch) * p.sB;
  // this wave's LDS region: A rows, B rows, then 64 A and 64 B scale words
  uint8_t* const my = lds_sk + w * kRegion;
  // direct loads: lane i of an 8-row slice fills LDS bytes [16 i, 16 i + 16)
  // of it, i.e. row i / 8, physical chunk i % 8, which holds the logical
  // chunk (i % 8) ^ (row & 7).  One descriptor per operand, built once,
  // covers the tile's rows inside the operand (rows at or past M (N) read
  // as zero); slice and K-step only move the lane offset (< 64 K).
  const int lrow = lane >> 3;
  const int voff = lrow * K + 16 * ((lane & 7) ^ lrow);
  const i32x4 ra = rsrc32(A + int64_t(m0) * K, max(0, min(M - m0, SK_T)) * K);
  const i32x4 rb = rsrc32(B + int64_t(n0) * K, max(0, min(N - n0, SK_T)) * K);
  const uint32_t my_addr = __builtin_amdgcn_readfirstlane(lds_addr_of(my));
  // Scales of a step come in with its tiles, one word per lane: FP8G the
  // A scale of row m0 + lane and the tile's B scale (every lane the same
  // word); MX the A and B words of rows m0 + lane, n0 + lane that hold the
  // step's four 32-block exponents.  Rows past the operand read the last
  // row (never stored).
  const int64_t sa_row = MODE == MODE_FP8G ? int64_t(nk) * 4 : int64_t(K / 32);  // bytes per scale row
  const uint8_t* const SAb = static_cast<const uint8_t*>(p.SA) + int64_t(batch) * p.sSA * (MODE == MODE_FP8G ? 4 : 1);
  const uint8_t* const SBb = static_cast<const uint8_t*>(p.SB) + int64_t(batch) * p.sSB * (MODE == MODE_FP8G ? 4 : 1);
  const int sa_voff = int((min(m0 + lane, M - 1) - m0) * sa_row);
  const int sb_voff = MODE == MODE_MX ? int((min(n0 + lane, N - 1) - n0) * sa_row) : 0;
  const uint8_t* const sa_base = SAb + int64_t(m0) * sa_row;
  const uint8_t* const sb_base = MODE == MODE_MX ? SBb + int64_t(n0) * sa_row : SBb + int64_t(n0 / 128) * sa_row;
  // ks == k_end (after the wave's last step): offsets past every range
  // (records <= 64 K <= 2^30; 2^30 + 56 K < 2^31) and empty scale
  // descriptors: zeros, no memory traffic, no branch
  auto dma_step = [&](int ks) {
    const bool live = ks < k_end;
    const int vk = live ? voff + ks * BK : (1 << 30);
    const uint32_t base = my_addr;
#pragma unroll
    for (int sl = 0; sl < 8; ++sl) {
      lds_dma16(ra, vk + 8 * sl * K, base + uint32_t(sl * 8 * BK));
      lds_dma16(rb, vk + 8 * sl * K, base + uint32_t(SK_T * BK + sl * 8 * BK));
    }
    if (kScales) {
      const int so = 4 * ks;  // the step's word within a scale row (FP8G: its float; MX: its 4 bytes)
      lds_dma4(rsrc32(sa_base + so, live ? 0x7FFFFFFF : 0), sa_voff, base + uint32_t(kTiles));
      lds_dma4(rsrc32(sb_base + so, live ? 0x7FFFFFFF : 0), sb_voff, base + uint32_t(kTiles + 256));
    }
  };
  // fragment reads: row r's logical chunk c sits at physical chunk c ^ (r & 7)
  const int swz = r16 & 7;
  const int c0 = 16 * (g ^ swz), c1 = 16 * ((g + 4) ^ swz);
  auto load_step = [&](v8i (&f)[8], float (&sa)[4], float& sb, int (&qa)[4], int (&qb)[4]) {
    const uint8_t* ta = my;
    const uint8_t* tb = ta + SK_T * BK;
    const uint32_t* sw = reinterpret_cast<const uint32_t*>(ta + kTiles);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = 16 * b + r16;
      f[b] = lds_frag(ta, row * BK + c0, row * BK + c1);
      f[4 + b] = lds_frag(tb, row * BK + c0, row * BK + c1);
    }
    if (MODE == MODE_FP8G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[i] = __uint_as_float(sw[16 * i + r16]);
      sb = __uint_as_float(sw[64]);
    } else if (MODE == MODE_MX) {
      // byte g of a row's word: this lane's 32-element block of the step
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qa[i] = int((sw[16 * i + r16] >> (8 * g)) & 0xFFu);
        qb[i] = int((sw[64 + 16 * i + r16] >> (8 * g)) & 0xFFu);
      }
    }
  };

  acc_t acc[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = acc_t{0, 0, 0, 0};

  if (k_begin < k_end) {
    v8i cur[8];
    float sa[4] = {0.f, 0.f, 0.f, 0.f}, sb = 0.f;
    int qa[4] = {0, 0, 0, 0}, qb[4] = {0, 0, 0, 0};
    dma_step(k_begin);
    for (int ks = k_begin; ks < k_end; ++ks) {
      // this step's tiles and scales have landed; once they are in
      // registers the region takes the next step's
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      load_step(cur, sa, sb, qa, qb);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      dma_step(ks + 1);  // past the last step: out of range, no traffic, no branch
#pragma unroll
      for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (MODE == MODE_FP8G) {
            const v4f zero = {0.f, 0.f, 0.f, 0.f};
            // zero scale operands: the unscaled MFMA (see the file header)
            const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cur[4 + j], cur[i], zero, 0, 0, 0, 0, 0, 0);
            const float sc = sa[i] * sb;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[j][i][r] = fmaf(d[r], sc, acc[j][i][r]);
          } else if (MODE == MODE_MX) {
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cur[4 + j], cur[i], acc[j][i], FB, FA,
                                                                         0, qb[j], 0, qa[i]);
          } else {
            const v4i plo = {cur[4 + j][0], cur[4 + j][1], cur[4 + j][2], cur[4 + j][3]};
            const v4i phi = {cur[4 + j][4], cur[4 + j][5], cur[4 + j][6], cur[4 + j][7]};
            const v4i qlo = {cur[i][0], cur[i][1], cur[i][2], cur[i][3]};
            const v4i qhi = {cur[i][4], cur[i][5], cur[i][6], cur[i][7]};
            acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(plo, qlo, acc[j][i], 0, 0, 0);
            acc[j][i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(phi, qhi, acc[j][i], 0, 0, 0);
          }
        }
      }
    }
  }

  // ---- the partial tiles meet in LDS (over the stage area, once every
  // wave is done with it and its last loads have landed): element (row,
  // col) of wave w's partial at red[w][(row * 64 + col) / 4]; lane holds
  // rows 16 i + r16, columns 16 j + 4 g .. + 3
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w][((16 * i + r16) * SK_T + 16 * j + 4 * g) / 4] = acc[j][i];
  __syncthreads();

  // 64 SKW threads share the 64 x 64 outputs: SKW threads per row, each
  // summing CPT groups of 4 consecutive columns
  constexpr int TPR = SKW;                // threads per row
  constexpr int CPT = SK_T / TPR / 4;     // float4 groups per thread
  static_assert(64 * SKW == SK_T * TPR, "one thread row per tile row");
  const int row = tid / TPR, col0 = 4 * CPT * (tid % TPR);
  const int m = m0 + row;
  if (m >= M) return;
  float xs = 0.f;
  if (MODE == MODE_I8) xs = static_cast<const float*>(p.SA)[int64_t(batch) * p.sSA + m];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int col = col0 + 4 * c;
    const int n = n0 + col;
    if (n >= N) continue;
    const int idx = (row * SK_T + col) / 4;
    acc_t v = red[0][idx];
#pragma unroll
    for (int u = 1; u < SKW; ++u) v += red[u][idx];
    const int64_t o = int64_t(batch) * p.sC + int64_t(m) * N + n;
    float y[4];
    if (MODE == MODE_I8) {
      const float4 ws = *reinterpret_cast<const float4*>(static_cast<const float*>(p.SB) +
                                                         int64_t(batch) * p.sSB + n);
      const float wsv[4] = {ws.x, ws.y, ws.z, ws.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = float(v[r]) * (xs * wsv[r]);
      if (p.acc_out != nullptr) *reinterpret_cast<int4*>(p.acc_out + o) = make_int4(v[0], v[1], v[2], v[3]);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) y[r] = float(v[r]);
    }
    if (OUT_BF16) {
      const uint32_t lo = encode_bf16(y[0]) | (encode_bf16(y[1]) << 16);
      const uint32_t hi = encode_bf16(y[2]) | (encode_bf16(y[3]) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<float4*>(static_cast<float*>(p.out) + o) = make_float4(y[0], y[1], y[2], y[3]);
    }
  }
}

__global__ void k_zero_bytes(uint32_t* __restrict__ p, int64_t n_words) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n_words; i += int64_t(gridDim.x) * 256)
    p[i] = 0u;
}

bsq_status zero_fill(void* p, int64_t bytes, hipStream_t st) {
  if (bytes == 0) return ok();
  const int64_t words = bytes / 4;
  int64_t grid = (words + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(k_zero_bytes, unsigned(grid), 256, 0, st, static_cast<uint32_t*>(p), words);
  return launch_status("zero fill");
}

// Tile height of the big kernel: 256, 192 or 128 rows by 256 columns, one
// workgroup per CU, so the time is about (passes over the 256 CUs) x (time
// of one tile).  A shorter tile moves more operand bytes per flop; measured
// at n = 2048 and 4096, one pass of 192-row tiles takes 0.86-0.90 and of
// 128-row tiles 0.74-0.79 of a pass of 256-row tiles (weights below, in
// hundredths).  The height with the smallest passes x weight wins, the
// taller on a tie: e.g. m = 3072, n = 4096 gives 192 tiles of 256 rows
// (one pass, part idle) but exactly 256 of 192 rows (66.8 -> 59.5 us).
constexpr int kCUs = 256;
int tile_rows_for(int64_t M, int64_t N, int64_t batch) {
  const int64_t cols = (N + BN - 1) / BN * batch;
  const int rows[3] = {256, 192, 128};
  const int weight[3] = {100, 88, 78};
  int best = 256;
  int64_t best_cost = -1;
  for (int i = 0; i < 3; ++i) {
    const int64_t tiles = (M + rows[i] - 1) / rows[i] * cols;
    const int64_t cost = (tiles + kCUs - 1) / kCUs * weight[i];
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = rows[i];
    }
  }
  return best;
}

// Fewer 256 x 256 tiles than this and the split-K kernel is used instead
// (the big-tile kernel would leave most of the 256 CUs idle).
constexpr int64_t kSkinnyTiles = 64;

// Launches a GEMM kernel; when the caller asked for timing events
// (bsq_time_next_gemm), through hipExtLaunchKernel so that the events
// record this kernel's own start and end.
template <typename Kernel, typename... Args>
void launch_gemm_kernel(Kernel k, dim3 grid, dim3 block, hipStream_t st, Args... args) {
  const GemmEvents ev = take_gemm_events();
  if (ev.start != nullptr || ev.stop != nullptr)
    hipExtLaunchKernelGGL(k, grid, block, 0, st, ev.start, ev.stop, 0, args...);
  else
    hipLaunchKernelGGL(k, grid, block, 0, st, args...);
}

template <int MODE, int OUT_BF16, int FA, int FB, int GN1, int GEN = 0, int SUB = 0>
bsq_status run(const GemmArgs& a, int batch, hipStream_t st) {
  const int64_t tiles = int64_t((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN) * batch;
  // big-tile grids: all tiles of a product along x, the batch along z
  auto big_grid = [&](int rows) {
    return dim3(unsigned(((a.M + rows - 1) / rows) * ((a.N + BN - 1) / BN)), 1u, unsigned(batch));
  };
  if (int64_t((a.M + 127) / 128) * ((a.N + BN - 1) / BN) > int64_t(0x7FFFFFFF) || batch > 65535)
    return fail(BSQ_ERR_UNSUPPORTED, "more than 2^31 - 1 tiles, or a batch over 65535");
  if constexpr (GEN != 0) {
    // general scale blocks: the big-tile kernel at every size
    const dim3 grid = big_grid(BM);
    launch_gemm_kernel(k_gemm<MODE, OUT_BF16, FA, FB, GN1, 8, 256, 1, SUB>, grid, dim3(512), st, a);
    return launch_status("gemm (general scale blocks)");
  }
  if constexpr (MODE != MODE_BF16) {
    if (tiles < kSkinnyTiles && !GN1) {
      dim3 grid(unsigned((a.N + SK_T - 1) / SK_T), unsigned((a.M + SK_T - 1) / SK_T), unsigned(batch));
      // 4 waves (66 KiB, two workgroups per CU).  With the scales brought
      // in by the tile loads, 8 waves (K split finer) and a second LDS
      // region per wave (two steps in flight) were slower on every shape
      // measured (64 .. 1024 rows, K 512 .. 8192).
      launch_gemm_kernel(k_gemm_sk<MODE, OUT_BF16, FA, FB, 4>, grid, dim3(256), st, a);
      return launch_status("gemm (split K)");
    }
  }
  constexpr int NW = 8;
  const int rows = tile_rows_for(a.M, a.N, batch);
  const dim3 grid = big_grid(rows);
  if (rows == 128)
    launch_gemm_kernel(k_gemm<MODE, OUT_BF16, FA, FB, GN1, NW, 128>, grid, dim3(64 * NW), st, a);
  else if (rows == 192)
    launch_gemm_kernel(k_gemm<MODE, OUT_BF16, FA, FB, GN1, NW, 192>, grid, dim3(64 * NW), st, a);
  else
    launch_gemm_kernel(k_gemm<MODE, OUT_BF16, FA, FB, GN1, NW, 256>, grid, dim3(64 * NW), st, a);
  return launch_status("gemm");
}

__global__ void __launch_bounds__(256) k_int8_small(const int8_t* __restrict__ xq,
                                                    const int8_t* __restrict__ wqT,
                                                    const float* __restrict__ xs,
                                                    const float* __restrict__ ws,
                                                    float* __restrict__ y, int32_t* __restrict__ acc,
                                                    int64_t Bn, int64_t D_in, int64_t D_out) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= Bn * D_out) return;
  const int64_t b = idx / D_out, j = idx % D_out;
  const int8_t* xr = xq + b * D_in;
  const int8_t* wr = wqT + j * D_in;
  int32_t a = 0;
  for (int64_t i = 0; i < D_in; ++i) a += int32_t(xr[i]) * int32_t(wr[i]);
  y[idx] = float(a) * (xs[b] * ws[j]);
  if (acc != nullptr) acc[idx] = a;
}

}  // namespace

bsq_status launch_int8_matmul_small(int64_t B, int64_t D_in, int64_t D_out, const int8_t* xq,
                                    const int8_t* wqT, const float* xs, const float* ws, float* y,
                                    int32_t* acc, hipStream_t st) {
  const int64_t n = B * D_out;
  if (n == 0) return ok();
  launch_gemm_kernel(k_int8_small, dim3(unsigned((n + 255) / 256)), dim3(256), st, xq, wqT, xs, ws, y,
                     acc, B, D_in, D_out);
  return launch_status("int8_matmul (small shapes)");
}

bsq_status launch_gemm(const GemmLaunch& L, hipStream_t st) {
  const int64_t out_elem = L.out_bf16 ? 2 : 4;
  if (L.batch == 0 || L.M == 0 || L.N == 0) return ok();
  if (L.K == 0) {
    bsq_status s = zero_fill(L.out, L.batch * L.M * L.N * out_elem, st);
    if (s == BSQ_OK && L.acc_out) s = zero_fill(L.acc_out, L.batch * L.M * L.N * 4, st);
    return s;
  }
  GemmArgs a;
  a.A = static_cast<const uint8_t*>(L.A);
  a.B = static_cast<const uint8_t*>(L.B);
  a.SA = L.SA;
  a.SB = L.SB;
  a.out = L.out;
  a.acc_out = L.acc_out;
  a.M = int(L.M);
  a.N = int(L.N);
  a.K = int(L.K);
  a.sA = L.M * L.K;
  a.sB = L.N * L.K;
  a.sC = L.M * L.N;
  a.sc_a = L.sc_a; a.sc_b = L.sc_b; a.sg_a = L.sg_a; a.sg_b = L.sg_b; a.gn = L.gn;
  if (L.gen && L.mode == MODE_FP8G) {
    a.sSA = L.M * L.sc_a;
    a.sSB = (L.N / L.gn) * L.sc_b;
    const int sel = (L.gn % 128 == 0 ? 0 : 1) | (L.out_bf16 ? 2 : 0) | (L.sub ? 4 : 0);
    switch (sel) {  // gn % 128 == 0: one B scale per wave's 128 columns
      case 0: return run<MODE_FP8G, 0, 0, 0, 0, 1>(a, int(L.batch), st);
      case 1: return run<MODE_FP8G, 0, 0, 0, 1, 1>(a, int(L.batch), st);
      case 2: return run<MODE_FP8G, 1, 0, 0, 0, 1>(a, int(L.batch), st);
      case 3: return run<MODE_FP8G, 1, 0, 0, 1, 1>(a, int(L.batch), st);
      case 4: return run<MODE_FP8G, 0, 0, 0, 0, 1, 1>(a, int(L.batch), st);
      case 5: return run<MODE_FP8G, 0, 0, 0, 1, 1, 1>(a, int(L.batch), st);
      case 6: return run<MODE_FP8G, 1, 0, 0, 0, 1, 1>(a, int(L.batch), st);
      default: return run<MODE_FP8G, 1, 0, 0, 1, 1, 1>(a, int(L.batch), st);
    }
  }
  if (L.gen && L.mode == MODE_MX) {
    a.sSA = L.M * L.sc_a;
    a.sSB = L.N * L.sc_b;
    const int sel = (L.fa_e5m2 ? 1 : 0) | (L.fb_e5m2 ? 2 : 0) | (L.out_bf16 ? 4 : 0);
    if (L.sub) {
      switch (sel) {
        case 0: return run<MODE_MX, 0, 0, 0, 0, 1, 1>(a, int(L.batch), st);
        case 1: return run<MODE_MX, 0, 1, 0, 0, 1, 1>(a, int(L.batch), st);
        case 2: return run<MODE_MX, 0, 0, 1, 0, 1, 1>(a, int(L.batch), st);
        case 3: return run<MODE_MX, 0, 1, 1, 0, 1, 1>(a, int(L.batch), st);
        case 4: return run<MODE_MX, 1, 0, 0, 0, 1, 1>(a, int(L.batch), st);
        case 5: return run<MODE_MX, 1, 1, 0, 0, 1, 1>(a, int(L.batch), st);
        case 6: return run<MODE_MX, 1, 0, 1, 0, 1, 1>(a, int(L.batch), st);
        default: return run<MODE_MX, 1, 1, 1, 0, 1, 1>(a, int(L.batch), st);
      }
    }
    switch (sel) {
      case 0: return run<MODE_MX, 0, 0, 0, 0, 1>(a, int(L.batch), st);
      case 1: return run<MODE_MX, 0, 1, 0, 0, 1>(a, int(L.batch), st);
      case 2: return run<MODE_MX, 0, 0, 1, 0, 1>(a, int(L.batch), st);
      case 3: return run<MODE_MX, 0, 1, 1, 0, 1>(a, int(L.batch), st);
      case 4: return run<MODE_MX, 1, 0, 0, 0, 1>(a, int(L.batch), st);
      case 5: return run<MODE_MX, 1, 1, 0, 0, 1>(a, int(L.batch), st);
      case 6: return run<MODE_MX, 1, 0, 1, 0, 1>(a, int(L.batch), st);
      default: return run<MODE_MX, 1, 1, 1, 0, 1>(a, int(L.batch), st);
    }
  }
  switch (L.mode) {
    case MODE_FP8G:
      a.sSA = L.M * (L.K / 128);
      a.sSB = (L.gn1 ? L.N : L.N / 128) * (L.K / 128);
      if (L.gn1) return L.out_bf16 ? run<MODE_FP8G, 1, 0, 0, 1>(a, int(L.batch), st)
                                   : run<MODE_FP8G, 0, 0, 0, 1>(a, int(L.batch), st);
      return L.out_bf16 ? run<MODE_FP8G, 1, 0, 0, 0>(a, int(L.batch), st)
                        : run<MODE_FP8G, 0, 0, 0, 0>(a, int(L.batch), st);
    case MODE_MX: {
      a.sSA = L.M * (L.K / 32);
      a.sSB = L.N * (L.K / 32);
      const int sel = (L.fa_e5m2 ? 1 : 0) | (L.fb_e5m2 ? 2 : 0) | (L.out_bf16 ? 4 : 0);
      switch (sel) {
        case 0: return run<MODE_MX, 0, 0, 0, 0>(a, int(L.batch), st);
        case 1: return run<MODE_MX, 0, 1, 0, 0>(a, int(L.batch), st);
        case 2: return run<MODE_MX, 0, 0, 1, 0>(a, int(L.batch), st);
        case 3: return run<MODE_MX, 0, 1, 1, 0>(a, int(L.batch), st);
        case 4: return run<MODE_MX, 1, 0, 0, 0>(a, int(L.batch), st);
        case 5: return run<MODE_MX, 1, 1, 0, 0>(a, int(L.batch), st);
        case 6: return run<MODE_MX, 1, 0, 1, 0>(a, int(L.batch), st);
        default: return run<MODE_MX, 1, 1, 1, 0>(a, int(L.batch), st);
      }
    }
    case MODE_I8:
      a.sSA = L.M;
      a.sSB = L.N;
      return run<MODE_I8, 0, 0, 0, 0>(a, int(L.batch), st);
    case MODE_BF16:
      // the kernel walks rows in bytes: 2 K bytes, 64 elements per step
      a.K = int(2 * L.K);
      a.sA = L.M * 2 * L.K;
      a.sB = L.N * 2 * L.K;
      a.sSA = a.sSB = 0;
      return L.out_bf16 ? run<MODE_BF16, 1, 0, 0, 0>(a, int(L.batch), st)
                        : run<MODE_BF16, 0, 0, 0, 0>(a, int(L.batch), st);
  }
  return fail(BSQ_ERR_UNSUPPORTED, "unknown gemm mode");
}

}  // namespace bsq
