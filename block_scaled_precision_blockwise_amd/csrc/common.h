// Internal helpers shared by the HIP translation units of libbsq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "bsq.h"

namespace bsq {

// ------------------------------------------------------------ status ----

// Records `msg` as this thread's last error and returns `st`.
bsq_status fail(bsq_status st, const std::string& msg);
// Clears this thread's last error and returns BSQ_OK.
bsq_status ok();
// BSQ_OK when the current HIP device is gfx950 (cached per device).
bsq_status require_gfx950();
// Maps the result of a kernel launch to a status.
bsq_status launch_status(const char* what);

// Events that the next GEMM kernel launched on this thread records at its
// start and end (set by bsq_time_next_gemm); taking them clears them.
struct GemmEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
GemmEvents take_gemm_events();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define BSQ_CHECK_PTR(p)                                                     \
  do {                                                                       \
    if ((p) == nullptr) return ::bsq::fail(BSQ_ERR_NULL, #p " is NULL");      \
    if (!::bsq::aligned16(p))                                                \
      return ::bsq::fail(BSQ_ERR_ALIGN, #p " is not 16-byte aligned");       \
  } while (0)

#define BSQ_CHECK(cond, st, msg)                                             \
  do {                                                                       \
    if (!(cond)) return ::bsq::fail((st), (msg));                            \
  } while (0)

// -------------------------------------------------- device arithmetic ----

// float32 -> bfloat16 bits, nearest with ties to even (finite inputs).
__device__ __forceinline__ uint32_t encode_bf16(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float decode_bf16(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Streaming (non-temporal) 16-byte loads: data read once should not
// displace reused data in the caches.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float4 ldnt(const float4* p) {
  const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  return make_float4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint4 ldnt(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// float32(1e-10): the lower clamp of the fp32 block scales.
__device__ __forceinline__ float scale_floor() { return __uint_as_float(0x2EDBE6FFu); }

}  // namespace bsq
