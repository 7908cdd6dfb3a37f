// Internal helpers shared by the libmla_fp8 sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_fp8.h"

namespace mla {

// Records a thread-local error text and returns `status`.
int fail(int status, const char* fmt, ...);
// Clears the thread-local error text and returns MLA_OK.
int ok();
// Maps the last HIP launch error to a status.
int check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Unsigned 32-bit division by a runtime constant d >= 1 (round-up method with a
// 33-bit magic): q = (umulhi(n, magic) + n) >> shift, valid for n < 2^31.
struct FastDiv {
  uint32_t d;
  uint32_t magic;
  uint32_t shift;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  f.shift = s;
  // magic = floor(2^32 * (2^s - d) / d) + 1
  f.magic = static_cast<uint32_t>(((1ull << 32) * ((1ull << s) - d)) / d + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  uint32_t hi = __umulhi(n, f.magic);
  return (hi + n) >> f.shift;
}

// bf16 (round to nearest even) of a finite or infinite fp32 value; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
  uint32_t b = __float_as_uint(x);
  uint32_t r = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
  return (x != x) ? ((b >> 16) | 0x40u) : r;
}

}  // namespace mla
