// Internal helpers shared by the libpf translation units (host validation,
// error reporting, bf16 bit conversions, gfx950 vector types).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "pf.h"

namespace pf {

// ---- host-side status reporting (thread-local message) ----
pf_status fail(pf_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pf_status ok();
pf_status launch_status(const char* what);   // maps hipGetLastError() after a launch

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define PF_REQUIRE(cond, st, ...) \
  do {                            \
    if (!(cond)) return ::pf::fail((st), __VA_ARGS__); \
  } while (0)

#define PF_REQUIRE_PTR(p) PF_REQUIRE((p) != nullptr, PF_ERR_NULL, "%s is NULL", #p)
#define PF_REQUIRE_ALIGNED(p) \
  PF_REQUIRE(::pf::aligned16(p), PF_ERR_MISALIGNED, "%s is not 16-byte aligned", #p)

// ---- device vector types ----
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short short4v;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (the hardware conversion honours the default mode).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

}  // namespace pf
